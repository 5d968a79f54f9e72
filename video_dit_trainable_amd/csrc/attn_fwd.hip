// Block-sparse flash attention forward: the fine branch of VSA2 (paper §2.2
// Eq.(12), the -inf block mask of §2.1 applied by skipping unselected tiles).
// The same kernel in "dense" mode runs the coarse branch's attention over the
// nb pooled cube tokens (Eq.(2)-(3)), with a ragged last tile.  On a padded
// grid (§2.2 "Kernel Implementation") pad keys are masked and pad query rows
// give zeros.  MMDiT text rows (after Eq.(12)) join the fine branch as cubes
// every video query attends to, and whose queries attend to everything.
//
// Work split: one block (2 waves) per query cube; each wave owns 32 queries as
// MFMA B fragments in registers, so every K/V byte read from LDS feeds two
// 16-query MFMA blocks.  The selected K and V cubes are gathered through the
// CSR list into chunk-swizzled row-major LDS tiles; the next cube's loads are
// in flight (in registers) while the current one is computed.  S^T = K Q^T
// leaves, per lane, 4 keys of one query per 16-key block, so the online
// softmax is lane-local apart from a 4-lane max, and the exponentials feed
// O^T += V^T P^T straight from the accumulators: the accumulators of key
// blocks 2h, 2h+1 form the B operand with the k-slot order
// pi(g, e) = 4g + e (e < 4), 16 + 4g + e - 4 (e >= 4) of keys 32h.., and the
// V^T A operand is read in the same order by transposing LDS reads.  The O
// rescale is lazy: the running max is only moved when a tile exceeds it by
// more than 2^8, which keeps every exponential <= 256 and the result exact.
#include <climits>
#include <cmath>

#include "common.h"
#include "launch.h"

namespace vsa2 {

// PAD (fine branch on a padded grid): pad slots of a KV cube are masked like
// keys past the end; pad query rows are written as O_f = 0, LSE = -inf.
// BS: 2^BS cubes per attention block.  The CSR lists blocks; query cube i
// takes the list of its block i >> BS, and list position n is cube
// (entry << BS) + (n mod 2^BS) of the selected block.
// TEXT (MMDiT conditioning): ntc text cubes (ntext tokens, rows past them are
// padding) follow the nq video cubes.  A video query cube attends to its
// selected cubes and then to every text cube; a text query cube attends to
// every video and text cube.  The text query cubes take the first blocks of
// the grid, so their long lists start first.
// QB = 2 with BS = 1 (128-token blocks): a 256-thread workgroup takes both
// query cubes of a block (waves 0, 1 the first cube, 2, 3 the second), which
// share the block's KV list, so every gathered K / V tile is staged once for
// 128 query rows.
// SCHED: the grid holds as many workgroups as fit on the device; each takes
// items from the work schedule's queues (its XCD's first) until they are
// empty, and runs each exactly as a workgroup of the one-item launch would.
// QB = 2 with BS = 0 (PAIR, on the schedule, text rows too): a workgroup takes
// two consecutive items of a queue, two query cubes of one head with lists of
// their own (waves 0, 1 the first, 2, 3 the second).  It walks the merge of
// the two lists, staging each KV cube in either list once; the waves of a cube
// compute the tiles of its own list, in the list's order, so each cube's
// result is the one-cube workgroup's bit for bit.
// QB = 2 stages K / V tiles LDS-direct into two stages (the copy of the next
// step runs while this one is computed); the one-cube kernel stages the next
// tile through registers into a single LDS tile.
template <typename T, typename TO, int D, bool DENSE, bool PAD, int BS, bool TEXT, int QB = 1, bool SCHED = false>
__global__ __launch_bounds__(128 * QB, 2) void k_attn_fwd(const T* __restrict__ q, const T* __restrict__ k,
                                                  const T* __restrict__ v, const int32_t* __restrict__ row_ptr,
                                                  const int32_t* __restrict__ col_idx, TO* __restrict__ o,
                                                  float* __restrict__ lse, int nq, int nkv, int seq, int ld,
                                                  int out_rows, int64_t kph, float c, int ct, int cy, int cx,
                                                  PadGrid pad, int ntc, int ntext, int nbh,
                                                  const int32_t* __restrict__ sq_hdr = nullptr,
                                                  const int32_t* __restrict__ sq_items = nullptr,
                                                  int32_t* __restrict__ sq_ctr = nullptr) {
  static_assert(!(DENSE && PAD), "padding applies to the fine branch");
  static_assert(!(DENSE && TEXT), "text rows apply to the fine branch");
  static_assert(QB == 1 || (QB == 2 && (BS == 1 || SCHED) && !(TEXT && BS) && !DENSE),
                "whole-block workgroups for 128-token blocks, pairs of cubes on the schedule");
  constexpr bool PAIR = QB == 2 && BS == 0;  // two query cubes with lists of their own
  constexpr bool STAGED = QB == 2;           // two LDS-direct stages (pairs and whole blocks)
  static_assert(!SCHED || (((QB == 1 && BS == 0) || (QB == 2 && !(TEXT && BS))) && !DENSE),
                "the schedule serves cubes (text cubes too) or whole 128-token blocks");
  constexpr int TILE = 64 * D;
  // the K and V tiles; STAGED: two stages, ks = stage A (K | V), vs = stage B
  __shared__ __align__(16) T ks[STAGED ? 2 * TILE : TILE];
  __shared__ __align__(16) T vs[STAGED ? 2 * TILE : TILE];
  __shared__ int s_item;  // SCHED: the item the workgroup runs next
  __shared__ int s_item2;  // PAIR: the second query cube's item, or -1
  __shared__ int s_pend;   // PAIR: an item taken with one of another head, run next
  if (PAIR && threadIdx.x == 0) s_pend = -1;
  for (int iter = 0;; ++iter) {
  int bh, i, i2 = -1;
  bool textq = false;  // a text query cube
  if constexpr (SCHED) {
    __syncthreads();  // every wave is done with the previous item's tiles and s_item
    // query cubes (QB = 2: blocks, PAIR: cubes), then text cubes
    const int nitem = (PAIR ? nq : nq / QB) + (TEXT ? ntc : 0);
    if (threadIdx.x == 0) {
      if constexpr (PAIR) {
        int c0 = s_pend, c1 = -1;
        if (c0 >= 0) {
          s_pend = -1;
        } else {
          c0 = sched_take2(sq_hdr, sq_items, sq_ctr, nbh * nitem, c1);
          if (c0 >= 0 && c1 >= 0 && c1 / nitem != c0 / nitem) {  // heads differ: one at a time
            s_pend = c1;
            c1 = -1;
          }
        }
        s_item = c0;
        s_item2 = c1;
      } else {
        s_item = sched_take(sq_hdr, sq_items, sq_ctr, nbh * nitem);
      }
    }
    __syncthreads();
    const int code = s_item;
    if (code < 0) break;
    bh = code / nitem;
    i = code - bh * nitem;  // QB = 2: the block; text cube t: nq + t, as in the row numbering
    if constexpr (PAIR) i2 = s_item2 < 0 ? -1 : s_item2 - bh * nitem;
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
  } else if constexpr (QB == 2 && !PAIR) {
    if (!xcd_work(blockIdx.x, nq >> 1, bh, i)) return;  // i: the block
    if (ct > 0) i = blocked_cube(i, ct, cy, cx >> 1);
  } else {
    if (!xcd_work(blockIdx.x, nq, bh, i)) return;
    if (ct > 0) i = blocked_cube(i, ct, cy, cx);
  }
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, cc = lane & 15;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the wave index, known to be uniform
  // this wave's query cube (PAIR: -1 for the waves of an absent second cube)
  const int qcube = PAIR ? ((wu >> 1) ? i2 : i) : (QB == 2 ? (i << 1) + (w >> 1) : i);
  const int wq = QB == 2 ? (w & 1) : w;  // and its 32-row half
  if constexpr (PAIR && TEXT) textq = qcube >= nq;  // this wave's cube is a text cube
  const size_t hoff = (size_t)bh * ld * D;
  const T* kbase = k + hoff;
  const T* vbase = v + hoff;

  int cnt, nsel = 0;  // list length; nsel = selected entries before the text cubes
  const int32_t* cols = nullptr;
  if constexpr (DENSE) {
    cnt = nkv;
  } else if constexpr (PAIR) {
    cnt = 0;  // the two lists are walked as a merge (below)
  } else if (TEXT && textq) {
    cnt = nkv + ntc;
  } else {
    const int blk = QB == 2 ? i : (i >> BS);
    const int32_t* rp = row_ptr + (size_t)bh * ((nq >> BS) + 1);
    const int64_t start = min<int64_t>(max(rp[blk], 0), kph);
    const int64_t end = min<int64_t>(max<int64_t>(rp[blk + 1], start), kph);
    cnt = (int)(end - start) << BS;
    cols = col_idx + (size_t)bh * kph + start;
    nsel = cnt;
    if constexpr (TEXT) cnt += ntc;
  }
  // PAIR: the lists of the two cubes x = i, i2 as sequences of KV cubes: a
  // video cube's selected cubes, then (TEXT) the text cubes nkv ..; a text
  // cube's list is every cube 0 .. nkv + ntc - 1; an absent cube's is empty
  struct PList {
    const int32_t* cl;  // the selected entries
    int ns, tot;        // how many of them, and the whole length
    bool all;           // every cube in order (a text query cube)
  };
  auto plist = [&](int x) -> PList {
    if (x < 0) return PList{col_idx, 0, 0, false};
    if (TEXT && x >= nq) return PList{col_idx, 0, nkv + ntc, true};
    const int32_t* rp = row_ptr + (size_t)bh * (nq + 1);
    const int64_t start = min<int64_t>(max(rp[x], 0), kph);
    const int64_t end = min<int64_t>(max<int64_t>(rp[x + 1], start), kph);
    const int ns = (int)(end - start);
    return PList{col_idx + (size_t)bh * kph + start, ns, ns + (TEXT ? ntc : 0), false};
  };
  // cube id of list position n; out-of-range ids (corrupt lists) become -1 = masked tile
  auto cube_at = [&](int n) -> int {
    if constexpr (DENSE) return n;
    if constexpr (TEXT) {
      if (textq) return n;
      if (n >= nsel) return nkv + (n - nsel);
    }
    const int jj = cols[n >> BS];
    return (unsigned)jj < (unsigned)(nkv >> BS) ? (jj << BS) + (n & ((1 << BS) - 1)) : -1;
  };
  auto kv_limit = [&](int jj) -> int {  // valid keys of cube jj
    if constexpr (DENSE) return min(64, seq - jj * 64);
    if constexpr (TEXT) {
      if (jj >= nkv) return min(64, ntext - 64 * (jj - nkv));
    }
    return jj >= 0 ? 64 : 0;
  };

  Frag<T> qf[2][D / 32];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      qf[qb][s] = frag_global<T, D>(q + hoff, max(qcube, 0) * 64 + 32 * wq + 16 * qb + cc, s, g);

  f32x4 oacc[D / 16][2];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) oacc[db][0] = oacc[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

  int vtr = 0;  // bf16: this lane's part of the transposed V reads (rows 4g + c/4 of key half 0)
  if constexpr (sizeof(T) == 2) vtr = sw_tr_base<T, D>(0, g, cc);
  // one staged K / V tile (kst, vst) into this wave's running softmax and O;
  // keys at or beyond lim are masked (PAD: and keys whose bit in km is clear)
  auto tile = [&](const T* kst, const T* vst, int lim, uint64_t km) {
    // S^T = K Q^T: acc[kb][qb] holds keys 16kb + 4g + r of query 16qb + cc (of this wave)
    f32x4 acc[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const Frag<T> a = sw_frag<T, D>(kst, 16 * kb + cc, 0, g);
      acc[kb][0] = mma0(a, qf[0][0]);
      acc[kb][1] = mma0(a, qf[1][0]);
    }
#pragma unroll
    for (int s = 1; s < D / 32; ++s)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const Frag<T> a = sw_frag<T, D>(kst, 16 * kb + cc, s, g);
        mma(acc[kb][0], a, qf[0][s]);
        mma(acc[kb][1], a, qf[1][s]);
      }
    if (lim < 64) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * kb + 4 * g + r >= lim) acc[kb][0][r] = acc[kb][1][r] = -INFINITY;
    }
    if constexpr (PAD) {
      if (km != ~0ull) {
        const uint64_t mine = km >> (4 * g);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (!((mine >> (16 * kb + r)) & 1)) acc[kb][0][r] = acc[kb][1][r] = -INFINITY;
      }
    }
    // lane-local maxima; the 4-lane reduction only runs when a lane asks to
    // move its reference maximum (lazy rescale, exponentials stay <= 2^8)
    float mt[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float x = acc[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) x = fmaxf(x, acc[kb][qb][r]);
      mt[qb] = x;
    }
    if (__ballot(mt[0] * c > m[0] * c + 8.f || mt[1] * c > m[1] * c + 8.f)) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float gm = group_max(mt[qb]);
        if (gm * c > m[qb] * c + 8.f) {
          const float alpha = fast_exp2((m[qb] - gm) * c);
          m[qb] = gm;
          l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 16; ++db) oacc[db][qb] *= alpha;
        }
      }
    }
    Frag<T> pf[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float mc = m[qb] == -INFINITY ? 0.f : -m[qb] * c;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(fmaf(acc[kb][qb][r], c, mc));
          acc[kb][qb][r] = p;
          l[qb] += p;
        }
      pf[qb][0] = frag_from_acc<T>(acc[0][qb], acc[1][qb]);
      pf[qb][1] = frag_from_acc<T>(acc[2][qb], acc[3][qb]);
    }
    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        Frag<T> a;
        if constexpr (sizeof(T) == 2) a = sw_frag_tr_at<T, D>(vst, vtr + 32 * h * D, 16 * db);
        else a = sw_frag_tr<T, D>(vst, 32 * h, 16 * db, g, cc);
        mma(oacc[db][0], a, pf[0][h]);
        mma(oacc[db][1], a, pf[1][h]);
      }
  };
  if constexpr (STAGED) {
    // PAIR: the merge of the two lists: the head of each (a corrupt entry
    // reads as -1, a masked tile, like the one-cube kernel's), the smaller
    // goes next, and a KV cube in both lists is staged once for both cubes.
    // Whole blocks: the block's list in order, every tile for all four waves.
    auto head = [&](const PList& L, int p) -> int {
      if (p >= L.tot) return INT_MAX;
      if (TEXT && L.all) return p;
      if (TEXT && p >= L.ns) return nkv + (p - L.ns);
      const int jj = L.cl[p];
      return (unsigned)jj < (unsigned)nkv ? jj : -1;
    };
    PList la{col_idx, 0, 0, false}, lb{col_idx, 0, 0, false};
    int pa = 0, pb = 0;
    int ha = 0, hb = 0;
    if constexpr (PAIR) {
      la = plist(i);
      lb = plist(i2);
      ha = head(la, 0);
      hb = head(lb, 0);
    }
    // the next KV cube and which of the two cubes take it; false at the end
    auto step = [&](int& jj, bool& in_a, bool& in_b) -> bool {
      if constexpr (PAIR) {
        if (ha == INT_MAX && hb == INT_MAX) return false;
        jj = min(ha, hb);
        in_a = ha == jj;
        in_b = hb == jj;
        if (in_a) ha = head(la, ++pa);
        if (in_b) hb = head(lb, ++pb);
      } else {
        if (pa >= cnt) return false;
        jj = cube_at(pa++);
        in_a = in_b = true;
      }
      return true;
    };
    auto fetch = [&](int jj, T* st) {  // LDS-direct copy of K and V cube jj into a stage
      dma_tile<64, D, T, 256>(kbase + (size_t)max(jj, 0) * TILE, st, tid);
      dma_tile<64, D, T, 256>(vbase + (size_t)max(jj, 0) * TILE, st + TILE, tid);
    };
    auto run = [&](const T* st, int jj, bool in_a, bool in_b) {
      if (!((wu >> 1) ? in_b : in_a)) return;  // not in this wave's list
      uint64_t km = ~0ull;  // text cubes: their tail goes by the limit
      if constexpr (PAD) km = jj < 0 ? 0ull : ((TEXT && jj >= nkv) ? ~0ull : cube_slots(jj, pad));
      tile(st, st + TILE, kv_limit(jj), km);
    };
    // stage A takes the even steps, stage B the odd ones; the copy into one
    // stage runs while the other is computed
    int ja = 0, jb = 0;
    bool aa = false, ab = false, ba = false, bb = false;
    bool has_a = step(ja, aa, ab);
    if (has_a) fetch(ja, ks);
    while (has_a) {
      wait_vm0();
      __syncthreads();  // stage A holds its tile; every wave is done with stage B
      const bool has_b = step(jb, ba, bb);
      if (has_b) fetch(jb, vs);
      run(ks, ja, aa, ab);
      if (!has_b) break;
      wait_vm0();
      __syncthreads();  // stage B holds its tile; every wave is done with stage A
      has_a = step(ja, aa, ab);
      if (has_a) fetch(ja, ks);
      run(vs, jb, ba, bb);
    }
  } else if (cnt > 0) {
    SwRegs<64, D, T, 128 * QB> kr, vr;
    int j = cube_at(0);
    sw_load(kr, kbase + (size_t)max(j, 0) * 64 * D, tid);
    sw_load(vr, vbase + (size_t)max(j, 0) * 64 * D, tid);
    for (int n = 0; n < cnt; ++n) {
      sw_store(kr, ks, tid);
      sw_store(vr, vs, tid);
      __syncthreads();
      const int lim = kv_limit(j);
      uint64_t km = ~0ull;  // PAD: real slots of cube j (text cubes: their tail goes by lim)
      if constexpr (PAD) km = j < 0 ? 0ull : ((TEXT && j >= nkv) ? ~0ull : cube_slots(j, pad));
      if (n + 1 < cnt) {
        j = cube_at(n + 1);
        sw_load(kr, kbase + (size_t)max(j, 0) * 64 * D, tid);
        sw_load(vr, vbase + (size_t)max(j, 0) * 64 * D, tid);
      }
      tile(ks, vs, lim, km);
      __syncthreads();
    }
  }

  uint64_t qm = ~0ull;  // PAD / TEXT: real rows of query cube i
  if constexpr (TEXT) {
    if (textq) {
      const int nr = ntext - 64 * (qcube - nq);
      qm = nr >= 64 ? ~0ull : (1ull << nr) - 1;
    }
  }
  if (PAIR && qcube < 0) continue;  // the waves of an absent second cube (the next item starts at a barrier)
  if constexpr (PAD) {
    if (!textq) qm = cube_slots(qcube, pad);
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = qcube * 64 + 32 * wq + 16 * qb + cc;
    const bool real = !(PAD || TEXT) || ((qm >> (32 * wq + 16 * qb + cc)) & 1);
    const float lsum = group_sum(l[qb]);  // every lane takes part in the cross-lane sum
    const float lt = real ? lsum : 0.f;
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const bool live = DENSE ? (qrow < seq && qrow < out_rows) : (qrow < out_rows);
    if (live) {
      TO* orow = o + ((size_t)bh * out_rows + qrow) * D;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        Vec4<TO> r4;
#pragma unroll
        for (int r = 0; r < 4; ++r) r4.v[r] = from_f32<TO>(real ? oacc[db][qb][r] * inv : 0.f);
        store4(orow + 16 * db + 4 * g, r4);
      }
      if (g == 0) lse[(size_t)bh * out_rows + qrow] = lt > 0.f ? (m[qb] * c + __log2f(lt)) * LN2 : -INFINITY;
    }
  }
  }  // items
}

template <typename T, int D>
hipError_t launch_fwd_t(const AttnArgs& a, hipStream_t st) {
  dim3 grid(xcd_grid(a.nq, a.bh));
  if (a.dense) {
    hipLaunchKernelGGL((k_attn_fwd<T, float, D, true, false, 0, false>), grid, dim3(128), 0, st, (const T*)a.q,
                       (const T*)a.k, (const T*)a.v, nullptr, nullptr, (float*)a.o, a.lse, a.nq, a.nkv, a.seq, a.ld,
                       a.out_rows, a.kph, a.scale_log2, 0, 0, 0, a.pad, 0, 0, a.bh);
  } else {
    timer_before(TK_FINE_FWD, st);
    const dim3 tgrid(grid.x + ((a.ntc * a.bh + 7) & ~7));  // text query cubes first
#define VSA2_FWD(PAD, BS, TEXT)                                                                                 \
  hipLaunchKernelGGL((k_attn_fwd<T, T, D, false, PAD, BS, TEXT>), TEXT ? tgrid : grid, dim3(128), 0, st,          \
                     (const T*)a.q, (const T*)a.k, (const T*)a.v, a.row_ptr, a.col_idx, (T*)a.o, a.lse, a.nq, a.nkv, \
                     a.seq, a.ld, a.out_rows, a.kph, a.scale_log2, a.ct, a.cy, a.cx, a.pad, a.ntc, a.ntext, a.bh)
#define VSA2_FWD_T(PAD, BS)                   \
  if (a.ntc) VSA2_FWD(PAD, BS, true);         \
  else VSA2_FWD(PAD, BS, false)
    const dim3 bgrid(xcd_grid(a.nq >> 1, a.bh));  // whole 128-token blocks per workgroup
#define VSA2_FWD_BLOCK(PAD)                                                                                     \
  hipLaunchKernelGGL((k_attn_fwd<T, T, D, false, PAD, 1, false, 2>), bgrid, dim3(256), 0, st, (const T*)a.q,    \
                     (const T*)a.k, (const T*)a.v, a.row_ptr, a.col_idx, (T*)a.o, a.lse, a.nq, a.nkv, a.seq, a.ld, \
                     a.out_rows, a.kph, a.scale_log2, a.ct, a.cy, a.cx, a.pad, 0, 0, a.bh)
#define VSA2_FWD_PAIR_SCHED(PAD, TEXT)                                                                         \
  {                                                                                                            \
    const auto fn = k_attn_fwd<T, T, D, false, PAD, 0, TEXT, 2, true>;                                         \
    hipError_t e_ = launch_fill_u32((uint32_t*)a.sq_ctr, 0u, 8, st);                                           \
    if (e_ != hipSuccess) return e_;                                                                           \
    const dim3 pgrid(resident_grid((const void*)fn, 256, a.bh * ((a.nq + a.ntc + 1) >> 1)));                   \
    hipLaunchKernelGGL(fn, pgrid, dim3(256), 0, st, (const T*)a.q, (const T*)a.k, (const T*)a.v, a.row_ptr,     \
                       a.col_idx, (T*)a.o, a.lse, a.nq, a.nkv, a.seq, a.ld, a.out_rows, a.kph, a.scale_log2,    \
                       a.ct, a.cy, a.cx, a.pad, a.ntc, a.ntext, a.bh, a.sq_hdr, a.sq_items, a.sq_ctr);        \
  }
#define VSA2_FWD_BLOCK_SCHED(PAD)                                                                              \
  {                                                                                                            \
    const auto fn = k_attn_fwd<T, T, D, false, PAD, 1, false, 2, true>;                                        \
    hipError_t e_ = launch_fill_u32((uint32_t*)a.sq_ctr, 0u, 8, st);                                           \
    if (e_ != hipSuccess) return e_;                                                                           \
    const dim3 pgrid(resident_grid((const void*)fn, 256, a.bh * (a.nq >> 1)));                                 \
    hipLaunchKernelGGL(fn, pgrid, dim3(256), 0, st, (const T*)a.q, (const T*)a.k, (const T*)a.v, a.row_ptr,     \
                       a.col_idx, (T*)a.o, a.lse, a.nq, a.nkv, a.seq, a.ld, a.out_rows, a.kph, a.scale_log2,    \
                       a.ct, a.cy, a.cx, a.pad, 0, 0, a.bh, a.sq_hdr, a.sq_items, a.sq_ctr);                  \
  }
    if (a.sq_hdr && !a.bs) {
      if (a.ntc) {
        if (a.pad.on) VSA2_FWD_PAIR_SCHED(true, true) else VSA2_FWD_PAIR_SCHED(false, true)
      } else {
        if (a.pad.on) VSA2_FWD_PAIR_SCHED(true, false) else VSA2_FWD_PAIR_SCHED(false, false)
      }
    } else if (a.sq_hdr && !a.ntc) {  // whole 128-token blocks on the schedule
      if (a.pad.on) VSA2_FWD_BLOCK_SCHED(true) else VSA2_FWD_BLOCK_SCHED(false)
    } else if (a.bs && !a.ntc) {
      if (a.pad.on) { VSA2_FWD_BLOCK(true); } else { VSA2_FWD_BLOCK(false); }
    } else if (a.bs) {  // with text rows: per-cube workgroups
      if (a.pad.on) { VSA2_FWD(true, 1, true); } else { VSA2_FWD(false, 1, true); }
    } else {
      if (a.pad.on) { VSA2_FWD_T(true, 0); } else { VSA2_FWD_T(false, 0); }
    }
#undef VSA2_FWD_PAIR_SCHED
#undef VSA2_FWD_BLOCK_SCHED
#undef VSA2_FWD_BLOCK
#undef VSA2_FWD_T
#undef VSA2_FWD
    timer_after(TK_FINE_FWD, st);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t st) {
  if (a.bf16) return a.d == 128 ? launch_fwd_t<bf16, 128>(a, st) : launch_fwd_t<bf16, 64>(a, st);
  return a.d == 128 ? launch_fwd_t<float, 128>(a, st) : launch_fwd_t<float, 64>(a, st);
}

}  // namespace vsa2
