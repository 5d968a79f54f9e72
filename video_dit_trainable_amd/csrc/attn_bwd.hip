// Backward of the block-sparse attention with the selection held fixed (the
// router takes no gradient: paper §2.1-§2.2).  Dense mode serves the coarse
// branch's attention over the pooled cube tokens.
//
// Deterministic by construction -- every output row is owned by one block:
//  * k_bwd_dkdv: one block (2 waves x 32 keys) per KV cube j, looping over the
//    query cubes that selected it (CSC list, ascending).  Per query tile it
//    recomputes S = Q K^T and P = exp(S - LSE), then dV += P^T dO,
//    dP = dO V^T, dS = P (dP - delta), dK += dS^T Q.  K and V stay in
//    registers; Q and dO tiles go through swizzled LDS, their transposes are
//    read with ds_read_b64_tr_b16.
//  * k_bwd_dq: one block (2 waves x 32 queries) per query cube i over its KV
//    list (CSR): S^T, P^T, dP^T = V dO^T, dS^T, dQ += dS K (K^T fragments by
//    transposing reads of the K tile).
// The row statistics (lse * log2 e, -delta) with delta = rowsum(dO * O) are
// computed by the dQ kernel, which holds every query row's dO anyway; it runs
// first and the dK/dV kernel reads them.  Per-cube gradient rows
// (the coarse branch's dQ_c, dK_c, dV_c) are added as row/64 to every token of
// the cube before the single rounding to the storage type.  On a padded grid
// (§2.2 "Kernel Implementation") pad tokens take no part: as keys they are
// masked, as queries their row statistics make P = 0, their gradient rows are
// zero, and the per-cube rows go as row/n to the n real tokens.
#include <cmath>

#include "common.h"
#include "launch.h"

namespace vsa2 {

// Row statistics of the fine branch for the backward kernels: stats[2t] =
// lse_t * log2(e) (+inf for a row with no selected key, so its P is 0) and
// stats[2t + 1] = -delta_t = -(dO_t . O_t), the initial value of the dP
// accumulators, so that they end at dP - delta.

// One (query cube, KV cube) pair of the dK/dV kernel for one wave: keys 32kh..
// (K, V fragments kf, vf in registers) against queries 32qh.. of the Q / dO
// tiles qs, dos and their row statistics sts (pairs lse2, delta) in LDS.
// Fragment reads of a swizzled 64 x D tile: row-major (row r, k-step s) and
// transposed (rows r0 .., columns col0 ..).  bf16 takes the per-lane bases
// (sw_row_base for row 16qb + cc of the wave's half, sw_tr_base for rows r0);
// fp32 (test precision) computes each address in full.
template <typename T, int D>
__device__ __forceinline__ Frag<T> rd_row(const T* t, int base, int r, int s, int g) {
  if constexpr (sizeof(T) == 2) return sw_frag_at<T>(t, base + (r & ~15) * D, s);
  else return sw_frag<T, D>(t, r, s, g);
}
template <typename T, int D>
__device__ __forceinline__ Frag<T> rd_tr(const T* t, int base, int r0, int col0, int g, int c) {
  if constexpr (sizeof(T) == 2) return sw_frag_tr_at<T, D>(t, base, col0);
  else return sw_frag_tr<T, D>(t, r0, col0, g, c);
}

// One (query cube, KV cube) pair of the dK/dV kernel for one wave: keys 32kh..
// (K, V fragments kf, vf in registers) against queries 32qh.. of the Q / dO
// tiles qs, dos and their row statistics sts (pairs lse2, delta) in LDS.
// Query rows 32qh + 16qb + 4g + r (qb = 0, 1 in turn) meet keys 32kh + 16kb + cc;
// P and dS of each 16-query block go straight into the low (qb = 0) or high
// (qb = 1) half of the bf16 B fragments of the dV and dK products, so only one
// 16 x 32 block of S and dP is live at a time.
template <typename T, int D, bool DENSE>
__device__ __forceinline__ void dkdv_pair(const T* qs, const T* dos, const float* sts, int brow, int btr,
                                          const Frag<T> (&kf)[2][D / 32], const Frag<T> (&vf)[2][D / 32],
                                          const bool (&kv_ok)[2], f32x4 (&dka)[D / 16][2], f32x4 (&dva)[D / 16][2],
                                          int qh, int g, int cc, float c) {
  opaque(brow);
  opaque(btr);
  Frag<T> pf[2], sf[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = 32 * qh + 16 * qb + cc;
    // row statistics of queries 32qh + 16qb + 4g + r: lse2 and -delta, the
    // latter the starting value of the dP accumulators (they end at dP - delta)
    const float* sp = sts + 2 * (32 * qh + 16 * qb + 4 * g);
    const f32x4 s01 = *reinterpret_cast<const f32x4*>(sp);
    const f32x4 s23 = *reinterpret_cast<const f32x4*>(sp + 4);
    const float l2[4] = {s01[0], s01[2], s23[0], s23[2]};
    const f32x4 ndl = {s01[1], s01[3], s23[1], s23[3]};
    f32x4 p[2], dp[2] = {ndl, ndl};
    {
      const Frag<T> a = rd_row<T, D>(qs, brow, row, 0, g);
      p[0] = mma0(a, kf[0][0]);
      p[1] = mma0(a, kf[1][0]);
      const Frag<T> b = rd_row<T, D>(dos, brow, row, 0, g);
      mma(dp[0], b, vf[0][0]);
      mma(dp[1], b, vf[1][0]);
    }
#pragma unroll
    for (int s = 1; s < D / 32; ++s) {
      const Frag<T> a = rd_row<T, D>(qs, brow, row, s, g);
      mma(p[0], a, kf[0][s]);
      mma(p[1], a, kf[1][s]);
      const Frag<T> b = rd_row<T, D>(dos, brow, row, s, g);
      mma(dp[0], b, vf[0][s]);
      mma(dp[1], b, vf[1][s]);
    }
    // P = exp2(S c - lse2), dS = P (dP - delta)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pe = kv_ok[kb] ? fast_exp2(fmaf(p[kb][r], c, -l2[r])) : 0.f;
        pf[kb].v[4 * qb + r] = from_f32<T>(pe);
        sf[kb].v[4 * qb + r] = from_f32<T>(pe * dp[kb][r]);
      }
  }
  // dV^T += dO^T P, dK^T += Q^T dS over these 32 queries; the transposed
  // fragments of step db + 1 are read while the products of step db run
  Frag<T> ao[2], aq[2];
  ao[0] = rd_tr<T, D>(dos, btr, 32 * qh, 0, g, cc);
  aq[0] = rd_tr<T, D>(qs, btr, 32 * qh, 0, g, cc);
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    if (db + 1 < D / 16) {
      ao[(db + 1) & 1] = rd_tr<T, D>(dos, btr, 32 * qh, 16 * (db + 1), g, cc);
      aq[(db + 1) & 1] = rd_tr<T, D>(qs, btr, 32 * qh, 16 * (db + 1), g, cc);
    }
    mma(dva[db][0], ao[db & 1], pf[0]);
    mma(dva[db][1], ao[db & 1], pf[1]);
    mma(dka[db][0], aq[db & 1], sf[0]);
    mma(dka[db][1], aq[db & 1], sf[1]);
  }
}

// dK, dV: one 256-thread block per KV cube j over its CSC list of query cubes.
// Wave w takes keys 32 (w & 1) .. and queries 32 (w >> 1) .. of every pair;
// the two query halves are summed through LDS at the end (fixed order).  The
// Q / dO tiles and row statistics of the next pair are copied LDS-direct into
// the other of two stages while the current pair is computed; the stages are
// distinct arrays and the loop is unrolled by two, so the compiler can tell
// the copy into one stage from the reads of the other.
// PAD (fine branch on a padded grid): the cube's pad keys get P = 0, so their
// dK, dV rows are zero; pad query rows arrive with lse2 = +inf (P = 0).
// BS: 2^BS cubes per attention block; the CSC lists query blocks, and list
// position n is query cube (entry << BS) + (n mod 2^BS).
// TEXT (MMDiT conditioning): ntc text cubes (ntext tokens) follow the video
// cubes; a video KV cube's list continues with every text query cube (text
// attends to all video), a text KV cube's list is every video and text query
// cube.  The text KV cubes take the first blocks of the grid.
// QB = 2 (128-token blocks): a workgroup takes both KV cubes of a block (waves
// 0, 1 the first cube, 2, 3 the second), which share the block's list; each
// wave runs both query halves of every staged Q / dO tile itself, so the
// tiles are staged once for 128 keys and no query-half reduction is needed.
// SCHED (64-token blocks): the grid holds as many workgroups as fit on the
// device; each takes KV cubes from the work schedule's queues (its XCD's
// first) until they are empty, and runs each exactly as a one-cube workgroup
// would.
template <typename T, typename TO, int D, bool DENSE, bool PAD, int BS, bool TEXT, int QB = 1, bool SCHED = false>
__global__ __launch_bounds__(256, 2) void k_bwd_dkdv(const T* __restrict__ q, const T* __restrict__ k,
                                                     const T* __restrict__ v, const T* __restrict__ d_o,
                                                     const float* __restrict__ stats,
                                                     const int32_t* __restrict__ col_ptr,
                                                     const int32_t* __restrict__ row_idx,
                                                     const float* __restrict__ dk_add,
                                                     const float* __restrict__ dv_add, TO* __restrict__ dk,
                                                     TO* __restrict__ dv, int nq, int nkv, int seq, int ld,
                                                     int out_rows, int64_t kph, float scale, float c, PadGrid pad,
                                                     int ntc, int ntext, int nbh,
                                                     const int32_t* __restrict__ sk_hdr = nullptr,
                                                     const int32_t* __restrict__ sk_items = nullptr,
                                                     int32_t* __restrict__ sk_ctr = nullptr) {
  static_assert(!(DENSE && PAD), "padding applies to the fine branch");
  static_assert(!DENSE || BS == 0, "the dense mode has one cube per block");
  static_assert(!(DENSE && TEXT), "text rows apply to the fine branch");
  static_assert(QB == 1 || (QB == 2 && BS == 1 && !TEXT && !DENSE), "whole-block workgroups for 128-token blocks");
  static_assert(!SCHED || (((QB == 1 && BS == 0) || (QB == 2 && !TEXT)) && !DENSE),
                "the schedule serves cubes (text cubes too) or whole 128-token blocks");
  constexpr int TILE = 64 * D;
  __shared__ __align__(16) T tA[2 * TILE];  // stage A: Q tile | dO tile
  __shared__ __align__(16) T tB[2 * TILE];  // stage B
  __shared__ __align__(16) float sA[128];   // stage A row statistics: [row][lse2, delta]
  __shared__ __align__(16) float sB[128];
  __shared__ int s_item;                    // SCHED: the item the workgroup runs next
  for (int iter = 0;; ++iter) {
  int bh, j;
  bool textk = false;  // a text KV cube
  if constexpr (SCHED) {
    __syncthreads();  // every wave is done with the previous item's tiles and s_item
    const int nitem = nkv / QB + (TEXT ? ntc : 0);  // KV cubes (QB = 2: KV blocks), then text cubes
    if (threadIdx.x == 0) s_item = sched_take(sk_hdr, sk_items, sk_ctr, nbh * nitem);
    __syncthreads();
    const int code = s_item;
    if (code < 0) break;
    bh = code / nitem;
    j = code - bh * nitem;  // text cube t: nkv + t, as in the row numbering
    if constexpr (QB == 2) j = (j << 1) + ((int)threadIdx.x >> 7);  // this wave's KV cube
    if constexpr (TEXT) textk = j >= nkv;
  } else if (iter > 0) {
    break;
  } else if constexpr (TEXT) {
    const int tblk = (ntc * nbh + 7) & ~7;  // a multiple of 8 keeps the video blocks' XCD map
    if ((int)blockIdx.x < tblk) {
      if ((int)blockIdx.x >= ntc * nbh) return;
      bh = blockIdx.x / ntc;
      j = nkv + blockIdx.x % ntc;
      textk = true;
    } else {
      if (!xcd_work(blockIdx.x - tblk, nkv, bh, j)) return;
    }
  } else if constexpr (QB == 2) {
    int jb;
    if (!xcd_work(blockIdx.x, nkv >> 1, bh, jb)) return;
    j = (jb << 1) + ((int)threadIdx.x >> 7);  // this wave's KV cube
  } else {
    if (!xcd_work(blockIdx.x, nkv, bh, j)) return;
  }
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, cc = lane & 15;
  const int kh = w & 1, qh = QB == 2 ? 0 : w >> 1;  // QB = 2: every wave runs both query halves
  const size_t hoff = (size_t)bh * ld * D;

  int cnt, nsel = 0;  // list length; nsel = selected entries before the text query cubes
  const int32_t* rows = nullptr;
  if constexpr (DENSE) {
    cnt = nq;
  } else if (TEXT && textk) {
    cnt = nq + ntc;
  } else {
    const int32_t* cp = col_ptr + (size_t)bh * ((nkv >> BS) + 1);
    const int64_t start = min<int64_t>(max(cp[j >> BS], 0), kph);
    const int64_t end = min<int64_t>(max<int64_t>(cp[(j >> BS) + 1], start), kph);
    cnt = (int)(end - start) << BS;
    rows = row_idx + (size_t)bh * kph + start;
    nsel = cnt;
    if constexpr (TEXT) cnt += ntc;
  }
  // list entry of position n (DENSE: the query tile n); read one step before
  // its copy is started, so the load is complete at the wait that precedes
  // the copy
  auto entry = [&](int n) -> int {
    if constexpr (DENSE) return n;
    if constexpr (TEXT) {
      if (textk || n >= nsel) return 0;  // positions past the selection need no load
    }
    return rows[n >> BS];
  };
  // query cube of an entry at list position pos (whose low BS bits are `sub`:
  // stage A takes the even positions, stage B the odd ones); a corrupt sparse
  // entry is fetched as cube 0 and skipped.  The entry stays in a vector
  // register until here (opaque), so its load is only waited for after the
  // copies issued behind it have been waited for anyway.
  auto cube_of = [&](int raw, int sub, int pos, bool& ok) -> int {
    if constexpr (TEXT) {
      if (textk || pos >= nsel) {
        ok = true;
        return textk ? pos : nq + (pos - nsel);
      }
    }
    if constexpr (!DENSE) opaque(raw);
    raw = __builtin_amdgcn_readfirstlane(raw);
    if constexpr (BS > 0) raw = (int)(((unsigned)raw << BS) | (unsigned)sub);
    ok = (unsigned)raw < (unsigned)nq;
    return ok ? raw : 0;
  };
  const float* stats_bh = stats + 2 * (size_t)bh * ld;
#define VSA2_FETCH_QDO(ii, tbuf, sbuf)                                                             \
  {                                                                                                \
    dma_tile<64, D, T, 256>(q + hoff + (size_t)(ii) * TILE, tbuf, tid);                            \
    dma_tile<64, D, T, 256>(d_o + hoff + (size_t)(ii) * TILE, tbuf + TILE, tid);                   \
    if (tid < 32) {                                                                                \
      int so_ = 16 * tid;                                                                          \
      opaque(so_);                                                                                 \
      lds_copy16(reinterpret_cast<const char*>(stats_bh + (size_t)(ii) * 128) + (uint32_t)so_,     \
                 (VSA2_LDS void*)(sbuf));                                                          \
    }                                                                                              \
  }

  Frag<T> kf[2][D / 32], vf[2][D / 32];
  bool kv_ok[2];
  uint64_t km = ~0ull;  // PAD / TEXT: real slots of cube j
  if constexpr (TEXT) {
    if (textk) {
      const int nr = ntext - 64 * (j - nkv);
      km = nr >= 64 ? ~0ull : (1ull << nr) - 1;
    }
  }
  if constexpr (PAD) {
    if (!textk) km = cube_slots(j, pad);
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = j * 64 + 32 * kh + 16 * kb + cc;
    kv_ok[kb] = (PAD || TEXT) ? (bool)((km >> (32 * kh + 16 * kb + cc)) & 1) : (!DENSE || key < seq);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      kf[kb][s] = frag_global<T, D>(k + hoff, key, s, g);
      vf[kb][s] = frag_global<T, D>(v + hoff, key, s, g);
    }
  }
  // dK^T, dV^T partial sums over this wave's query half: rows d = 16db + 4g + r, column key 16kb + cc
  f32x4 dka[D / 16][2], dva[D / 16][2];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    dka[db][0] = dka[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    dva[db][0] = dva[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  int brow = 0, btr = 0, btr1 = 0;  // per-lane parts of the bf16 fragment addresses
  if constexpr (sizeof(T) == 2) {
    brow = sw_row_base<T, D>(cc, g);  // rows 16m + cc add 16m D (the swizzle sees only r & 15)
    btr = sw_tr_base<T, D>(32 * qh, g, cc);
    if constexpr (QB == 2) btr1 = sw_tr_base<T, D>(32, g, cc);
  }
  bool ok_a = false, ok_b = false;
  int raw = 0;  // list entry whose copy starts next
  if (cnt > 0) {
    const int ii0 = cube_of(entry(0), 0, 0, ok_a);
    VSA2_FETCH_QDO(ii0, tA, sA);
    if (cnt > 1) raw = entry(1);
  }
  for (int n = 0; n < cnt; n += 2) {
    wait_vm0();
    __syncthreads();  // stage A holds entry n; every wave is done with stage B
    if (n + 1 < cnt) {
      const int ii = cube_of(raw, 1, n + 1, ok_b);
      if (n + 2 < cnt) raw = entry(n + 2);
      VSA2_FETCH_QDO(ii, tB, sB);
    }
    if (ok_a) {
      dkdv_pair<T, D, DENSE>(tA, tA + TILE, sA, brow, btr, kf, vf, kv_ok, dka, dva, qh, g, cc, c);
      if constexpr (QB == 2)  // the other query half
        dkdv_pair<T, D, DENSE>(tA, tA + TILE, sA, brow, btr1, kf, vf, kv_ok, dka, dva, 1, g, cc, c);
    }
    if (n + 1 >= cnt) break;
    wait_vm0();
    __syncthreads();  // stage B holds entry n + 1; every wave is done with stage A
    if (n + 2 < cnt) {
      const int ii = cube_of(raw, 0, n + 2, ok_a);
      if (n + 3 < cnt) raw = entry(n + 3);
      VSA2_FETCH_QDO(ii, tA, sA);
    }
    if (ok_b) {
      dkdv_pair<T, D, DENSE>(tB, tB + TILE, sB, brow, btr, kf, vf, kv_ok, dka, dva, qh, g, cc, c);
      if constexpr (QB == 2)
        dkdv_pair<T, D, DENSE>(tB, tB + TILE, sB, brow, btr1, kf, vf, kv_ok, dka, dva, 1, g, cc, c);
    }
  }
#undef VSA2_FETCH_QDO

  if constexpr (QB == 2) {  // each wave holds its keys' whole sums
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) dka[db][kb][r] *= scale;
  } else {
  // sum the two query halves: waves with qh = 1 hand their partials to qh = 0 through LDS
  __syncthreads();
  constexpr int PART = (D / 16) * 2 * 4 * 64;  // floats per wave and tensor
  static_assert(2 * PART * sizeof(float) <= sizeof(tA), "reduction buffer must fit a stage");
  float* mine = reinterpret_cast<float*>(kh ? tB : tA);  // [dK | dV][db][kb][r][lane]
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int o = ((db * 2 + kb) * 4 + r) * 64 + lane;
          mine[o] = dka[db][kb][r];
          mine[PART + o] = dva[db][kb][r];
        }
  }
  __syncthreads();
  if (qh == 1) continue;  // this wave's part is handed over (the next item starts at a barrier)
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = ((db * 2 + kb) * 4 + r) * 64 + lane;
        dka[db][kb][r] = (dka[db][kb][r] + mine[o]) * scale;
        dva[db][kb][r] += mine[PART + o];
      }
  }
  // the coarse branch's per-block gradient rows, 1/n to each of the block's
  // n real tokens (n = 64 2^BS unless the grid is padded)
  if (dk_add && !textk) {
    const float* ka = dk_add + ((size_t)bh * (nkv >> BS) + (j >> BS)) * D;
    const float* va = dv_add + ((size_t)bh * (nkv >> BS) + (j >> BS)) * D;
    float wk[2] = {1.0f / (float)(64 << BS), 1.0f / (float)(64 << BS)};
    if constexpr (PAD) {
      const int n = __popcll(km) + (BS ? __popcll(cube_slots(j ^ 1, pad)) : 0);
      const float inv_n = 1.0f / (float)n;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) wk[kb] = kv_ok[kb] ? inv_n : 0.f;
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(ka + 16 * db + 4 * g);
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(va + 16 * db + 4 * g);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          dka[db][kb][r] += a4[r] * wk[kb];
          dva[db][kb][r] += b4[r] * wk[kb];
        }
    }
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int kvrow = j * 64 + 32 * kh + 16 * kb + cc;
    const bool live = DENSE ? (kvrow < seq && kvrow < out_rows) : (kvrow < out_rows);
    if (!live) continue;
    TO* krow = dk + ((size_t)bh * out_rows + kvrow) * D;
    TO* vrow = dv + ((size_t)bh * out_rows + kvrow) * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      Vec4<TO> a4, b4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        a4.v[r] = from_f32<TO>(dka[db][kb][r]);
        b4.v[r] = from_f32<TO>(dva[db][kb][r]);
      }
      store4(krow + 16 * db + 4 * g, a4);
      store4(vrow + 16 * db + 4 * g, b4);
    }
  }
  }  // items
}

// One (query cube, KV cube) pair of the dQ kernel for one wave: queries 32qh..
// (Q, dO fragments qf, of in registers, row statistics l2 and ndl = -delta,
// the starting value of the dP^T accumulators) against keys
// 32kh.. of the K / V tiles ks, vs in LDS; keys at or beyond lim are masked
// (PAD: keys whose bit in km is clear).
template <typename T, int D, bool PAD>
__device__ __forceinline__ void dq_pair(const T* ks, const T* vs, int brow, int btr, int lim, uint64_t km,
                                        const Frag<T> (&qf)[2][D / 32], const Frag<T> (&of)[2][D / 32],
                                        const float (&l2)[2], const float (&ndl)[2], f32x4 (&dqa)[D / 16][2], int kh,
                                        int g, int cc, float c) {
  opaque(brow);
  opaque(btr);
  // S^T = K Q^T, dP^T = V dO^T: [kb][qb] holds keys 32kh + 16kb + 4g + r against query 32qh + 16qb + cc
  Frag<T> sf[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = 32 * kh + 16 * kb + cc;
    f32x4 p[2], dp[2] = {f32x4{ndl[0], ndl[0], ndl[0], ndl[0]}, f32x4{ndl[1], ndl[1], ndl[1], ndl[1]}};
    {
      const Frag<T> a = rd_row<T, D>(ks, brow, row, 0, g);
      p[0] = mma0(a, qf[0][0]);
      p[1] = mma0(a, qf[1][0]);
      const Frag<T> b = rd_row<T, D>(vs, brow, row, 0, g);
      mma(dp[0], b, of[0][0]);
      mma(dp[1], b, of[1][0]);
    }
#pragma unroll
    for (int s = 1; s < D / 32; ++s) {
      const Frag<T> a = rd_row<T, D>(ks, brow, row, s, g);
      mma(p[0], a, qf[0][s]);
      mma(p[1], a, qf[1][s]);
      const Frag<T> b = rd_row<T, D>(vs, brow, row, s, g);
      mma(dp[0], b, of[0][s]);
      mma(dp[1], b, of[1][s]);
    }
    // dS^T = P^T (dP^T - delta) straight into the low (kb = 0) / high (kb = 1) half of the B fragments
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 32 * kh + 16 * kb + 4 * g + r;
      const bool kin = PAD ? (bool)((km >> key) & 1) : key < lim;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float pe = kin ? fast_exp2(fmaf(p[qb][r], c, -l2[qb])) : 0.f;
        sf[qb].v[4 * kb + r] = from_f32<T>(pe * dp[qb][r]);
      }
    }
  }
  // dQ^T += K^T dS^T over these 32 keys
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    const Frag<T> a = rd_tr<T, D>(ks, btr, 32 * kh, 16 * db, g, cc);
    mma(dqa[db][0], a, sf[0]);
    mma(dqa[db][1], a, sf[1]);
  }
}

// dQ: one 256-thread block per query cube i over its CSR list of KV cubes.
// Wave w takes queries 32 (w & 1) .. and keys 32 (w >> 1) .. of every pair; the
// key halves are summed through LDS at the end.  K / V tiles of the next pair
// are copied LDS-direct into the other stage while the current pair runs
// (distinct stage arrays, loop unrolled by two, as in the dK/dV kernel).
// PAD (fine branch on a padded grid): pad keys are masked; pad query rows get
// the statistics (+inf, 0), so their P is 0 here and in the dK/dV kernel.
// BS: 2^BS cubes per attention block; the CSR lists KV blocks, and list
// position n is KV cube (entry << BS) + (n mod 2^BS).
// TEXT (MMDiT conditioning): ntc text cubes (ntext tokens) follow the nq video
// cubes; a video query cube's list continues with every text cube, a text
// query cube's list is every video and text cube.  The text query cubes take
// the first blocks of the grid.
// QB = 2 (128-token blocks): a workgroup takes both query cubes of a block
// (waves 0, 1 the first cube, 2, 3 the second); each wave runs both key
// halves of every staged K / V tile itself, so the tiles are staged once for
// 128 query rows and no key-half reduction is needed.
// SCHED (64-token blocks): as in the dK/dV kernel, over the schedule's
// query-cube queues.
template <typename T, typename TO, int D, bool DENSE, bool STATS, bool PAD, int BS, bool TEXT, int QB = 1,
          bool SCHED = false>
__global__ __launch_bounds__(256, 2) void k_bwd_dq(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, const T* __restrict__ d_o,
                                                   const T* __restrict__ o, const float* __restrict__ lse,
                                                   float* __restrict__ stats_out, const float* __restrict__ stats,
                                                   const int32_t* __restrict__ row_ptr,
                                                   const int32_t* __restrict__ col_idx,
                                                   const float* __restrict__ dq_add, TO* __restrict__ dq, int nq,
                                                   int nkv, int seq, int ld, int out_rows, int64_t kph, float scale,
                                                   float c, int ct, int cy, int cx, PadGrid pad, int ntc, int ntext,
                                                   int nbh, const int32_t* __restrict__ sq_hdr = nullptr,
                                                   const int32_t* __restrict__ sq_items = nullptr,
                                                   int32_t* __restrict__ sq_ctr = nullptr) {
  static_assert(!PAD || (STATS && !DENSE), "padding applies to the fine branch");
  static_assert(!DENSE || BS == 0, "the dense mode has one cube per block");
  static_assert(!TEXT || (STATS && !DENSE), "text rows apply to the fine branch");
  static_assert(QB == 1 || (QB == 2 && BS == 1 && !TEXT && !DENSE), "whole-block workgroups for 128-token blocks");
  static_assert(!SCHED || (((QB == 1 && BS == 0) || (QB == 2 && !TEXT)) && !DENSE && STATS),
                "the schedule serves cubes (text cubes too) or whole 128-token blocks");
  constexpr int TILE = 64 * D;
  __shared__ __align__(16) T tA[2 * TILE];  // stage A: K tile | V tile
  __shared__ __align__(16) T tB[2 * TILE];  // stage B
  __shared__ int s_item;                    // SCHED: the item the workgroup runs next
  for (int iter = 0;; ++iter) {
  int bh, i;
  bool textq = false;  // a text query cube
  if constexpr (SCHED) {
    __syncthreads();  // every wave is done with the previous item's tiles and s_item
    const int nitem = nq / QB + (TEXT ? ntc : 0);  // query cubes (QB = 2: query blocks), then text cubes
    if (threadIdx.x == 0) s_item = sched_take(sq_hdr, sq_items, sq_ctr, nbh * nitem);
    __syncthreads();
    const int code = s_item;
    if (code < 0) break;
    bh = code / nitem;
    i = code - bh * nitem;  // text cube t: nq + t, as in the row numbering
    if constexpr (QB == 2) i = (i << 1) + ((int)threadIdx.x >> 7);  // this wave's query cube
    if constexpr (TEXT) textq = i >= nq;
  } else if (iter > 0) {
    break;
  } else if constexpr (TEXT) {
    const int tblk = (ntc * nbh + 7) & ~7;  // a multiple of 8 keeps the video blocks' XCD map
    if ((int)blockIdx.x < tblk) {
      if ((int)blockIdx.x >= ntc * nbh) return;
      bh = blockIdx.x / ntc;
      i = nq + blockIdx.x % ntc;
      textq = true;
    } else {
      if (!xcd_work(blockIdx.x - tblk, nq, bh, i)) return;
      if (ct > 0) i = blocked_cube(i, ct, cy, cx);
    }
  } else if constexpr (QB == 2) {
    int ib;
    if (!xcd_work(blockIdx.x, nq >> 1, bh, ib)) return;
    if (ct > 0) ib = blocked_cube(ib, ct, cy, cx >> 1);
    i = (ib << 1) + ((int)threadIdx.x >> 7);  // this wave's query cube
  } else {
    if (!xcd_work(blockIdx.x, nq, bh, i)) return;
    if (ct > 0) i = blocked_cube(i, ct, cy, cx);
  }
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, cc = lane & 15;
  const int qh = w & 1, kh = QB == 2 ? 0 : w >> 1;  // QB = 2: every wave runs both key halves
  const size_t hoff = (size_t)bh * ld * D;

  int cnt, nsel = 0;  // list length; nsel = selected entries before the text cubes
  const int32_t* cols = nullptr;
  if constexpr (DENSE) {
    cnt = nkv;
  } else if (TEXT && textq) {
    cnt = nkv + ntc;
  } else {
    const int32_t* rp = row_ptr + (size_t)bh * ((nq >> BS) + 1);
    const int64_t start = min<int64_t>(max(rp[i >> BS], 0), kph);
    const int64_t end = min<int64_t>(max<int64_t>(rp[(i >> BS) + 1], start), kph);
    cnt = (int)(end - start) << BS;
    cols = col_idx + (size_t)bh * kph + start;
    nsel = cnt;
    if constexpr (TEXT) cnt += ntc;
  }
  // list entry of position n (DENSE: the KV tile n), read one step before its copy starts
  auto entry = [&](int n) -> int {
    if constexpr (DENSE) return n;
    if constexpr (TEXT) {
      if (textq || n >= nsel) return 0;  // positions past the selection need no load
    }
    return cols[n >> BS];
  };
  // KV cube of an entry at list position pos (whose low BS bits are `sub`),
  // and how many of its keys are valid (0 for a corrupt entry)
  auto cube_of = [&](int raw, int sub, int pos, int& lim) -> int {
    if constexpr (DENSE) {
      lim = min(64, seq - raw * 64);
      return raw;
    } else {
      if constexpr (TEXT) {
        if (textq || pos >= nsel) {
          const int jj = textq ? pos : nkv + (pos - nsel);
          lim = jj < nkv ? 64 : min(64, ntext - 64 * (jj - nkv));
          return jj;
        }
      }
      opaque(raw);
      raw = __builtin_amdgcn_readfirstlane(raw);
      if constexpr (BS > 0) raw = (int)(((unsigned)raw << BS) | (unsigned)sub);
      const bool ok = (unsigned)raw < (unsigned)nkv;
      lim = ok ? 64 : 0;
      return ok ? raw : 0;
    }
  };
#define VSA2_FETCH_KV(jj, tbuf)                                                       \
  {                                                                                   \
    dma_tile<64, D, T, 256>(k + hoff + (size_t)(jj) * TILE, tbuf, tid);               \
    dma_tile<64, D, T, 256>(v + hoff + (size_t)(jj) * TILE, tbuf + TILE, tid);        \
  }

  // this wave's 32 queries: Q and dO rows as B fragments (column = query 32qh + 16qb + cc)
  Frag<T> qf[2][D / 32], of[2][D / 32];
  float l2[2], ndl[2];
  uint64_t qm = ~0ull;  // PAD / TEXT: real rows of query cube i
  if constexpr (TEXT) {
    if (textq) {
      const int nr = ntext - 64 * (i - nq);
      qm = nr >= 64 ? ~0ull : (1ull << nr) - 1;
    }
  }
  if constexpr (PAD) {
    if (!textq) qm = cube_slots(i, pad);
  }
  bool qreal[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = i * 64 + 32 * qh + 16 * qb + cc;
    qreal[qb] = !(PAD || TEXT) || ((qm >> (32 * qh + 16 * qb + cc)) & 1);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      qf[qb][s] = frag_global<T, D>(q + hoff, qrow, s, g);
      of[qb][s] = frag_global<T, D>(d_o + hoff, qrow, s, g);
    }
    if constexpr (STATS) {
      // delta = dO . O over the row: this lane's 4 x 8 elements, then the 4 lanes g
      float part = 0.f;
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const Frag<T> of8 = frag_global<T, D>(o + hoff, qrow, s, g);
#pragma unroll
        for (int e = 0; e < 8; ++e) part = fmaf(to_f32(of[qb][s].v[e]), to_f32(of8.v[e]), part);
      }
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      const float l = lse[(size_t)bh * ld + qrow];
      l2[qb] = (l == -INFINITY || !qreal[qb]) ? INFINITY : l * LOG2E;
      ndl[qb] = qreal[qb] ? -part : 0.f;
      if (kh == 0 && g == 0) {
        stats_out[2 * ((size_t)bh * ld + qrow)] = l2[qb];
        stats_out[2 * ((size_t)bh * ld + qrow) + 1] = ndl[qb];
      }
    } else {
      l2[qb] = stats[2 * ((size_t)bh * ld + qrow)];
      ndl[qb] = stats[2 * ((size_t)bh * ld + qrow) + 1];
    }
  }
  // dQ^T partial over this wave's key half: rows d = 16db + 4g + r, column query 16qb + cc
  f32x4 dqa[D / 16][2];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) dqa[db][0] = dqa[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  int brow = 0, btr = 0, btr1 = 0;
  if constexpr (sizeof(T) == 2) {
    brow = sw_row_base<T, D>(cc, g);  // rows 16m + cc add 16m D (the swizzle sees only r & 15)
    btr = sw_tr_base<T, D>(32 * kh, g, cc);
    if constexpr (QB == 2) btr1 = sw_tr_base<T, D>(32, g, cc);
  }
  int lim_a = 0, lim_b = 0, raw = 0;
  uint64_t km_a = ~0ull, km_b = ~0ull;  // PAD: real slots of the staged KV cubes
  auto slots_of = [&](int jj, int lim) -> uint64_t {
    if constexpr (PAD) {
      if (TEXT && jj >= nkv) return lim >= 64 ? ~0ull : (1ull << lim) - 1;  // a text cube's tail
      return lim > 0 ? cube_slots(jj, pad) : 0ull;
    } else {
      return ~0ull;
    }
  };
  if (cnt > 0) {
    const int j0 = cube_of(entry(0), 0, 0, lim_a);
    km_a = slots_of(j0, lim_a);
    VSA2_FETCH_KV(j0, tA);
    if (cnt > 1) raw = entry(1);
  }
  for (int n = 0; n < cnt; n += 2) {
    wait_vm0();
    __syncthreads();  // stage A holds entry n; every wave is done with stage B
    if (n + 1 < cnt) {
      const int jj = cube_of(raw, 1, n + 1, lim_b);
      km_b = slots_of(jj, lim_b);
      if (n + 2 < cnt) raw = entry(n + 2);
      VSA2_FETCH_KV(jj, tB);
    }
    if (lim_a > 32 * kh)
      dq_pair<T, D, PAD>(tA, tA + TILE, brow, btr, lim_a, km_a, qf, of, l2, ndl, dqa, kh, g, cc, c);
    if constexpr (QB == 2) {  // the other key half
      if (lim_a > 32) dq_pair<T, D, PAD>(tA, tA + TILE, brow, btr1, lim_a, km_a, qf, of, l2, ndl, dqa, 1, g, cc, c);
    }
    if (n + 1 >= cnt) break;
    wait_vm0();
    __syncthreads();  // stage B holds entry n + 1; every wave is done with stage A
    if (n + 2 < cnt) {
      const int jj = cube_of(raw, 0, n + 2, lim_a);
      km_a = slots_of(jj, lim_a);
      if (n + 3 < cnt) raw = entry(n + 3);
      VSA2_FETCH_KV(jj, tA);
    }
    if (lim_b > 32 * kh)
      dq_pair<T, D, PAD>(tB, tB + TILE, brow, btr, lim_b, km_b, qf, of, l2, ndl, dqa, kh, g, cc, c);
    if constexpr (QB == 2) {
      if (lim_b > 32) dq_pair<T, D, PAD>(tB, tB + TILE, brow, btr1, lim_b, km_b, qf, of, l2, ndl, dqa, 1, g, cc, c);
    }
  }
#undef VSA2_FETCH_KV

  if constexpr (QB == 2) {  // each wave holds its queries' whole sums
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) dqa[db][qb][r] *= scale;
  } else {
  // sum the two key halves through LDS
  __syncthreads();
  constexpr int PART = (D / 16) * 2 * 4 * 64;
  static_assert(PART * sizeof(float) <= sizeof(tA), "reduction buffer must fit a stage");
  float* mine = reinterpret_cast<float*>(qh ? tB : tA);
  if (kh == 1) {
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mine[((db * 2 + qb) * 4 + r) * 64 + lane] = dqa[db][qb][r];
  }
  __syncthreads();
  if (kh == 1) continue;  // this wave's part is handed over (the next item starts at a barrier)
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dqa[db][qb][r] = (dqa[db][qb][r] + mine[((db * 2 + qb) * 4 + r) * 64 + lane]) * scale;
  }
  if (dq_add && !textq) {  // the coarse branch's per-block gradient row, 1/n to each of the n real tokens
    const float* qa = dq_add + ((size_t)bh * (nq >> BS) + (i >> BS)) * D;
    float wq[2] = {1.0f / (float)(64 << BS), 1.0f / (float)(64 << BS)};
    if constexpr (PAD) {
      const int n = __popcll(qm) + (BS ? __popcll(cube_slots(i ^ 1, pad)) : 0);
      const float inv_n = 1.0f / (float)n;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) wq[qb] = qreal[qb] ? inv_n : 0.f;
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(qa + 16 * db + 4 * g);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) dqa[db][qb][r] += a4[r] * wq[qb];
    }
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = i * 64 + 32 * qh + 16 * qb + cc;
    const bool live = DENSE ? (qrow < seq && qrow < out_rows) : (qrow < out_rows);
    if (!live) continue;
    TO* dst = dq + ((size_t)bh * out_rows + qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      Vec4<TO> a4;
#pragma unroll
      for (int r = 0; r < 4; ++r) a4.v[r] = from_f32<TO>(dqa[db][qb][r]);
      store4(dst + 16 * db + 4 * g, a4);
    }
  }
  }  // items
}

// The fine backward over the work schedule: dQ over the query-cube queues
// (it writes the row statistics), then dK/dV over the KV-cube queues; with
// 128-token blocks (BS = 1) the items are blocks and the workgroups whole-block.
template <typename T, int D, bool PAD, int BS, bool TEXT = false>
hipError_t launch_bwd_sched(const AttnBwdArgs& a, hipStream_t st) {
  constexpr int QB = BS ? 2 : 1;
  static_assert(!(TEXT && BS), "text rows with 128-token blocks run per cube, off the schedule");
  const int ntc = TEXT ? a.ntc : 0;
  hipError_t e = launch_fill_u32((uint32_t*)a.sq_ctr, 0u, 16, st);
  if (e != hipSuccess) return e;
  const auto fq = k_bwd_dq<T, T, D, false, true, PAD, BS, TEXT, QB, true>;
  timer_before(TK_BWD_DQ, st);
  hipLaunchKernelGGL(fq, dim3(resident_grid((const void*)fq, 256, a.bh * (a.nq / QB + ntc))), dim3(256), 0, st,
                     (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.d_o, (const T*)a.o, a.lse, a.stats_out,
                     nullptr, a.row_ptr, a.col_idx, a.dq_add, (T*)a.dq, a.nq, a.nkv, a.seq, a.ld, a.out_rows, a.kph,
                     a.scale, a.scale_log2, a.ct, a.cy, a.cx, a.pad, ntc, a.ntext, a.bh, a.sq_hdr, a.sq_items,
                     a.sq_ctr);
  timer_after(TK_BWD_DQ, st);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const auto fk = k_bwd_dkdv<T, T, D, false, PAD, BS, TEXT, QB, true>;
  timer_before(TK_BWD_DKDV, st);
  hipLaunchKernelGGL(fk, dim3(resident_grid((const void*)fk, 256, a.bh * (a.nkv / QB + ntc))), dim3(256), 0, st,
                     (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.d_o, a.stats_out, a.col_ptr, a.row_idx,
                     a.dk_add, a.dv_add, (T*)a.dk, (T*)a.dv, a.nq, a.nkv, a.seq, a.ld, a.out_rows, a.kph, a.scale,
                     a.scale_log2, a.pad, ntc, a.ntext, a.bh, a.sk_hdr, a.sk_items, a.sq_ctr + 8);
  timer_after(TK_BWD_DKDV, st);
  return hipGetLastError();
}

template <typename T, typename TO, int D, bool DENSE, bool PAD, int BS, bool TEXT, int QB = 1>
hipError_t launch_bwd_tt(const AttnBwdArgs& a, hipStream_t st) {
  // dQ first: in sparse mode it writes the row statistics the dK/dV kernel reads
  const int tblk = TEXT ? (a.ntc * a.bh + 7) & ~7 : 0;  // text cubes take the first blocks
  if (!DENSE) timer_before(TK_BWD_DQ, st);
  if constexpr (DENSE)
    hipLaunchKernelGGL((k_bwd_dq<T, TO, D, DENSE, false, false, 0, false>), dim3(xcd_grid(a.nq, a.bh)), dim3(256),
                       0, st, (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.d_o, nullptr, nullptr, nullptr,
                       a.stats, a.row_ptr, a.col_idx, a.dq_add, (TO*)a.dq, a.nq, a.nkv, a.seq, a.ld, a.out_rows, a.kph,
                       a.scale, a.scale_log2, a.ct, a.cy, a.cx, a.pad, 0, 0, a.bh);
  else
    hipLaunchKernelGGL((k_bwd_dq<T, TO, D, DENSE, true, PAD, BS, TEXT, QB>), dim3(tblk + xcd_grid(a.nq / QB, a.bh)),
                       dim3(256), 0, st, (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.d_o, (const T*)a.o,
                       a.lse, a.stats_out, nullptr, a.row_ptr, a.col_idx, a.dq_add, (TO*)a.dq, a.nq, a.nkv, a.seq,
                       a.ld, a.out_rows, a.kph, a.scale, a.scale_log2, a.ct, a.cy, a.cx, a.pad, a.ntc, a.ntext, a.bh);
  if (!DENSE) timer_after(TK_BWD_DQ, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!DENSE) timer_before(TK_BWD_DKDV, st);
  hipLaunchKernelGGL((k_bwd_dkdv<T, TO, D, DENSE, PAD, BS, TEXT, QB>), dim3(tblk + xcd_grid(a.nkv / QB, a.bh)), dim3(256),
                     0, st, (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.d_o,
                     DENSE ? a.stats : a.stats_out, a.col_ptr, a.row_idx, a.dk_add, a.dv_add, (TO*)a.dk, (TO*)a.dv,
                     a.nq, a.nkv, a.seq, a.ld, a.out_rows, a.kph, a.scale, a.scale_log2, a.pad, a.ntc, a.ntext, a.bh);
  if (!DENSE) timer_after(TK_BWD_DKDV, st);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_t(const AttnBwdArgs& a, hipStream_t st) {
  if (a.dense) return launch_bwd_tt<T, float, D, true, false, 0, false>(a, st);
  if (a.sq_hdr && !(a.bs && a.ntc)) {  // the work schedule's queues
    if (a.bs) return a.pad.on ? launch_bwd_sched<T, D, true, 1>(a, st) : launch_bwd_sched<T, D, false, 1>(a, st);
    if (a.ntc)
      return a.pad.on ? launch_bwd_sched<T, D, true, 0, true>(a, st) : launch_bwd_sched<T, D, false, 0, true>(a, st);
    return a.pad.on ? launch_bwd_sched<T, D, true, 0>(a, st) : launch_bwd_sched<T, D, false, 0>(a, st);
  }
#define VSA2_BWD(PAD, BS)                                                                              \
  return a.ntc ? launch_bwd_tt<T, T, D, false, PAD, BS, true>(a, st)                                  \
               : launch_bwd_tt<T, T, D, false, PAD, BS, false>(a, st)
  if (a.bs && !a.ntc)  // whole 128-token blocks per workgroup
    return a.pad.on ? launch_bwd_tt<T, T, D, false, true, 1, false, 2>(a, st)
                    : launch_bwd_tt<T, T, D, false, false, 1, false, 2>(a, st);
  if (a.bs) {  // with text rows: per-cube workgroups
    if (a.pad.on) return launch_bwd_tt<T, T, D, false, true, 1, true>(a, st);
    return launch_bwd_tt<T, T, D, false, false, 1, true>(a, st);
  }
  if (a.pad.on) VSA2_BWD(true, 0);
  VSA2_BWD(false, 0);
#undef VSA2_BWD
}

hipError_t launch_attn_bwd(const AttnBwdArgs& a, hipStream_t st) {
  if (a.bf16) return a.d == 128 ? launch_bwd_t<bf16, 128>(a, st) : launch_bwd_t<bf16, 64>(a, st);
  return a.d == 128 ? launch_bwd_t<float, 128>(a, st) : launch_bwd_t<float, 64>(a, st);
}

}  // namespace vsa2
