// Fine-grained router of VSA2, paper §2.2 Eq.(6)-(7) with the fused two-pass
// scheme of its "Kernel Implementation" paragraph: the pooled score matrix
// Q_r K_r^T is computed twice on chip -- pass 1 accumulates each pooled
// query's log-sum-exp, pass 2 recomputes the tiles, normalises them and
// averages the 8 x 8 (query sub-cube, key sub-cube) entries of each cube pair.
// Only the nb x nb block scores reach memory.  On a padded grid (§2.2 "Kernel
// Implementation") pooled tokens that hold no real token are masked.
//
// Work split: a 256-thread block owns 128 pooled queries (16 query cubes);
// wave w holds queries 32w .. 32w+31 as MFMA B fragments in registers and
// streams all pooled keys of the head, 64 at a time, through two LDS stages
// filled by LDS-direct copies (distinct arrays, loop unrolled by two, so a
// copy into one stage never makes the reads of the other wait).
//
// Key order inside a staged tile: LDS row 16 kb + c holds pooled key
//   pi(kb, c) = 32 (kb >> 1) + 4 (kb & 1) + 8 (c >> 2) + (c & 3)
// of the 64-key tile.  The accumulator of S^T = K Q^T for 16-row block kb
// gives lane (g, c) rows 4g .. 4g+3, i.e. keys pi(kb, 4g + r) =
// 8 (4 (kb >> 1) + g) + 4 (kb & 1) + r: over kb = 2h, 2h+1 and r = 0..3 one lane
// holds all 8 keys of key cube 4h + g.  The 8 x 8 pooling is then 7 in-lane
// adds and a 3-step DPP reduction over the 8 query lanes of a query cube.
#include <cmath>

#include "common.h"
#include "launch.h"

namespace vsa2 {

namespace {

constexpr int RQ = 128;  // pooled queries per block
constexpr int RK = 64;   // pooled keys per staged tile

__device__ __forceinline__ int key_of_row(int r) {
  const int kb = r >> 4, c = r & 15;
  return 32 * (kb >> 1) + 4 * (kb & 1) + 8 * (c >> 2) + (c & 3);
}

// Copy keys [k0, k0 + 64) of one head's K_r (rows of D elements) into a
// swizzled LDS tile in the order above; keys at or past nkeys read key
// nkeys - 1 (masked by the caller).
template <typename T, int D>
__device__ __forceinline__ void dma_keys(const T* __restrict__ kr, int k0, int nkeys, T* lds, int tid) {
  using S = SwTile<T, D>;
  constexpr int RSTEP = 256 / S::NCH;
  static_assert(RK * S::NCH % 256 == 0, "tile chunks must split evenly over the block");
  const int wbase = __builtin_amdgcn_readfirstlane(tid & ~63);
  const int pc = tid % S::NCH;
#pragma unroll
  for (int n = 0; n < RK * S::NCH / 256; ++n) {
    const int r = n * RSTEP + tid / S::NCH;
    const int key = min(k0 + key_of_row(r), nkeys - 1);
    int off = (key * D + S::EPC * (pc ^ (S::f(r) & (S::NCH - 1)))) * (int)sizeof(T);
    opaque(off);
    lds_copy16(reinterpret_cast<const char*>(kr) + (uint32_t)off, (VSA2_LDS void*)(lds + (n * 256 + wbase) * S::EPC));
  }
}

// Sum over the 8 lanes c, c^1, .., c^7 of a row-group of 8 (DPP, no LDS).
__device__ __forceinline__ float sum8(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));  // row_half_mirror
  return x;
}

// One 64-key tile for one wave: acc[kb][qb] = S^T block (keys of LDS rows
// 16kb + 4g + r, query 32w + 16qb + c), unscaled.  bf16: bs[s] is this lane's
// element offset of k-step s in row cc of the tile (the swizzle XOR already
// applied), so every read is a base register plus an immediate.
template <typename T, int D>
__device__ __forceinline__ void tile_scores(const T* ks, const int (&bs)[D / 32], const Frag<T> (&qf)[2][D / 32],
                                            int g, int cc, f32x4 (&acc)[4][2]) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    Frag<T> a;
    if constexpr (sizeof(T) == 2) a = frag_from8(load8(ks + bs[0] + 16 * kb * D));
    else a = sw_frag<T, D>(ks, 16 * kb + cc, 0, g);
    acc[kb][0] = mma0(a, qf[0][0]);
    acc[kb][1] = mma0(a, qf[1][0]);
  }
#pragma unroll
  for (int s = 1; s < D / 32; ++s)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      Frag<T> a;
      if constexpr (sizeof(T) == 2) a = frag_from8(load8(ks + bs[s] + 16 * kb * D));
      else a = sw_frag<T, D>(ks, 16 * kb + cc, s, g);
      mma(acc[kb][0], a, qf[0][s]);
      mma(acc[kb][1], a, qf[1][s]);
    }
}

// keys of a tile at or past nkeys get -inf (only the last tile can have them)
__device__ __forceinline__ void mask_tail(f32x4 (&acc)[4][2], int k0, int nkeys, int g) {
  if (k0 + RK <= nkeys) return;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (k0 + key_of_row(16 * kb + 4 * g + r) >= nkeys) acc[kb][0][r] = acc[kb][1][r] = -INFINITY;
}

// Padded grids: keys whose bit in the tile's existence word tm is clear get
// -inf (LDS row 16kb + 4g + r holds key 32 (kb >> 1) + 8g + 4 (kb & 1) + r).
__device__ __forceinline__ void mask_keys(f32x4 (&acc)[4][2], uint64_t tm, int g) {
  if (tm == ~0ull) return;
  const uint64_t mine = tm >> (8 * g);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (!((mine >> (32 * (kb >> 1) + 4 * (kb & 1) + r)) & 1)) acc[kb][0][r] = acc[kb][1][r] = -INFINITY;
}

}  // namespace

// Existence words of the pooled keys of a padded grid: bit b of word t is set
// when pooled key 64t + b (sub-cube b % 8 of cube 8t + b / 8) holds a real
// token, i.e. when its first slot does.  Keys past the last cube are clear.
__global__ void k_route_kmask(uint64_t* __restrict__ kmask, int nb, PadGrid pad) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (8 * nb + RK - 1) / RK) return;
  uint64_t m = 0;
  for (int k = 0; k < 8; ++k) {
    const int c = 8 * t + k;
    if (c >= nb) break;
    const uint64_t real = cube_slots(c, pad);
    for (int s = 0; s < 8; ++s) m |= ((real >> (8 * s)) & 1ull) << (8 * k + s);
  }
  kmask[t] = m;
}

// TAIL: the pooled key count is not a multiple of 64, so the last key tile is
// ragged (masked).  Without it no tile is, and the masking is compiled out.
// PAD: a padded grid; keys and queries that hold no real token are taken from
// the existence words (which also clear the ragged tail): such keys are
// masked, such queries get LSE +inf, so pass 2 gives them no weight.
// BS: 2^BS cubes per attention block (pass 2 averages the 8 2^BS x 8 2^BS
// entries of each block pair; nb counts cubes).
// G1: the VSA router baseline -- one pooled token per attention block (the
// coarse operands Q_c, K_c, hstride rows per head; nb counts blocks), and
// pass 2 writes the probabilities P_c themselves (Eq.(2)).
template <typename T, int D, bool PASS2, bool TAIL, bool PAD, int BS, bool G1 = false>
__global__ __launch_bounds__(256, 2) void k_router(const T* __restrict__ qr, const T* __restrict__ kr,
                                                   float* __restrict__ lse2, float* __restrict__ scores, int nb,
                                                   float c, const uint64_t* __restrict__ kmask, int hstride) {
  static_assert(!(TAIL && PAD), "the existence words cover the ragged tail");
  static_assert(BS == 0 || (BS == 1 && PASS2), "128-token blocks change only the score pass");
  static_assert(!G1 || (!PAD && BS == 0), "the coarse operands have one row per block");
  __shared__ __align__(16) T kA[RK * D];
  __shared__ __align__(16) T kB[RK * D];
  const int Lr = G1 ? nb : 8 * nb;  // pooled tokens per head
  const int nqt = (Lr + RQ - 1) / RQ, nkt = (Lr + RK - 1) / RK;
  int bh, qt;
  if (!xcd_work(blockIdx.x, nqt, bh, qt)) return;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, cc = lane & 15;
  const T* qbase = qr + (size_t)bh * hstride * D;
  const T* kbase = kr + (size_t)bh * hstride * D;

  // this wave's 32 pooled queries as B fragments: query qt*128 + 32w + 16qb + cc
  Frag<T> qf[2][D / 32];
  float lse[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = qt * RQ + 32 * w + 16 * qb + cc;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      if (qrow < Lr) {
        qf[qb][s] = frag_global<T, D>(qbase, qrow, s, g);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[qb][s].v[e] = from_f32<T>(0.f);
      }
    }
    if constexpr (PASS2) lse[qb] = qrow < Lr ? lse2[(size_t)bh * Lr + qrow] : INFINITY;
  }
  int bs[D / 32] = {};  // bf16: per-lane fragment offsets of the k-steps (see tile_scores)
  if constexpr (sizeof(T) == 2) {
    const int brow = sw_row_base<T, D>(cc, g);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      bs[s] = brow ^ (32 * s);
      opaque(bs[s]);
    }
  }
  // key-tile copies: for a full tile the per-lane source offsets are fixed and
  // only the (uniform) tile base moves; a ragged last tile takes dma_keys
  using S = SwTile<T, D>;
  constexpr int RSTEP = 256 / S::NCH;
  constexpr int NCP = RK * S::NCH / 256;
  const int nfull = Lr / RK;
  const int wbase = __builtin_amdgcn_readfirstlane(tid & ~63);
  int coff[NCP];
#pragma unroll
  for (int n = 0; n < NCP; ++n) {
    const int r = n * RSTEP + tid / S::NCH, pc = tid % S::NCH;
    coff[n] = (key_of_row(r) * D + S::EPC * (pc ^ (S::f(r) & (S::NCH - 1)))) * (int)sizeof(T);
  }
  auto copy_tile = [&](int t, T* lds) {
    if (t < nfull) {
      const char* src = reinterpret_cast<const char*>(kbase + (size_t)t * RK * D);
      asm volatile("" : "+s"(src));  // keep the tile base one uniform value (scalar registers)
#pragma unroll
      for (int n = 0; n < NCP; ++n) {
        int off = coff[n];
        opaque(off);  // a 32-bit per-lane offset on a uniform base (saddr form)
        lds_copy16(src + (uint32_t)off, (VSA2_LDS void*)(lds + (n * 256 + wbase) * S::EPC));
      }
    } else {
      dma_keys<T, D>(kbase, t * RK, Lr, lds, tid);
    }
  };
  // pass 2: the lane that stores a block score (the first of each 8 2^BS
  // query lanes; with BS = 1 only even g, whose key cube starts a pair)
  const int nblk = nb >> BS;
  bool qstore[2];
  float* srow[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qcube = (qt * RQ + 32 * w + 16 * qb + cc) >> 3;
    qstore[qb] = (cc & ((8 << BS) - 1)) == 0 && qcube < nb && (BS == 0 || (g & 1) == 0);
    srow[qb] = scores + ((size_t)bh * nblk + (min(qcube, nb - 1) >> BS)) * nblk;
  }

  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};  // pass 1: running max / sum (scaled log2 domain)

  auto consume = [&](const f32x4 (&acc)[4][2], int t) {
    if constexpr (PASS2 && G1) {
      // P_c of query 16qb + cc and keys t*64 + 32 (kb >> 1) + 4 (kb & 1) + 8g + r
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int qrow = qt * RQ + 32 * w + 16 * qb + cc;
        if (qrow >= Lr) continue;
        float* dst = scores + ((size_t)bh * nb + qrow) * nb;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const int key0 = t * RK + 32 * (kb >> 1) + 4 * (kb & 1) + 8 * g;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (key0 + r < nb) dst[key0 + r] = fast_exp2(fmaf(acc[kb][qb][r], c, -lse[qb]));
        }
      }
    } else if constexpr (!PASS2) {
      // The tile's terms are taken against the lane's running maximum m as it
      // stands; m moves (with the exact tile maximum, and l rescaled) only for
      // the first tile with a key, or when the tile's sum leaves [0, 2^64]
      // (a key more than about 58 above m in the log2 domain, or an overflow).
      // The sum stays exact: every term is exp2(s c - m c) for the m that l
      // is kept against, and the final merge over lanes rescales each l once.
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float lt = 0.f;
        if (m[qb] != -INFINITY) {
          const float mc = -m[qb] * c;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) lt += fast_exp2(fmaf(acc[kb][qb][r], c, mc));
        }
        if (m[qb] == -INFINITY || !(lt <= 0x1p64f)) {
          float mt = acc[0][qb][0];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) mt = fmaxf(mt, acc[kb][qb][r]);
          lt = 0.f;
          if (mt > m[qb]) {
            l[qb] *= fast_exp2((m[qb] - mt) * c);
            m[qb] = mt;
          }
          if (m[qb] != -INFINITY) {
            const float mc = -m[qb] * c;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
              for (int r = 0; r < 4; ++r) lt += fast_exp2(fmaf(acc[kb][qb][r], c, mc));
          }
        }
        l[qb] += lt;
      }
    } else {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float s8 = 0.f;
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int r = 0; r < 4; ++r) s8 += fast_exp2(fmaf(acc[2 * h + kk][qb][r], c, -lse[qb]));
          s8 = sum8(s8);
          if constexpr (BS == 1) {
            s8 += __shfl_xor(s8, 8);   // the other query cube of the pair (lanes c ^ 8)
            s8 += __shfl_xor(s8, 16);  // the other key cube of the pair (lanes g ^ 1)
          }
          const int kcube = t * (RK / 8) + 4 * h + g;
          if (qstore[qb] && kcube < nb) srow[qb][kcube >> BS] = s8 * (1.0f / (64 << (2 * BS)));
        }
      }
    }
  };

  copy_tile(0, kA);
  for (int t = 0; t < nkt; t += 2) {
    f32x4 acc[4][2];
    wait_vm0();
    __syncthreads();  // stage A holds tile t; every wave is done with stage B
    if (t + 1 < nkt) copy_tile(t + 1, kB);
    tile_scores<T, D>(kA, bs, qf, g, cc, acc);
    if constexpr (TAIL) mask_tail(acc, t * RK, Lr, g);
    if constexpr (PAD) mask_keys(acc, kmask[t], g);
    consume(acc, t);
    if (t + 1 >= nkt) break;
    wait_vm0();
    __syncthreads();  // stage B holds tile t + 1; every wave is done with stage A
    if (t + 2 < nkt) copy_tile(t + 2, kA);
    tile_scores<T, D>(kB, bs, qf, g, cc, acc);
    if constexpr (TAIL) mask_tail(acc, (t + 1) * RK, Lr, g);
    if constexpr (PAD) mask_keys(acc, kmask[t + 1], g);
    consume(acc, t + 1);
  }

  if constexpr (!PASS2) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qrow = qt * RQ + 32 * w + 16 * qb + cc;
      const float M = group_max(m[qb]);
      const float part = (m[qb] == -INFINITY) ? 0.f : l[qb] * fast_exp2((m[qb] - M) * c);
      const float lt = group_sum(part);
      bool exists = true;
      if constexpr (PAD) exists = qrow < Lr && ((kmask[qrow >> 6] >> (qrow & 63)) & 1);
      if (g == 0 && qrow < Lr) lse2[(size_t)bh * Lr + qrow] = exists ? M * c + __log2f(lt) : INFINITY;
    }
  }
}

template <typename T, int D, bool TAIL, bool PAD>
hipError_t launch_route_tt(const RouteArgs& a, hipStream_t st) {
  static_assert(RQ % 16 == 0 && RK % 16 == 0, "query and key tiles hold whole cube pairs");
  const int nqt = (8 * a.nb + RQ - 1) / RQ;
  dim3 grid(xcd_grid(nqt, a.bh));
  if constexpr (PAD) {
    const int nkt = (8 * a.nb + RK - 1) / RK;
    hipLaunchKernelGGL(k_route_kmask, dim3((nkt + 255) / 256), dim3(256), 0, st, a.kmask, a.nb, a.pad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  timer_before(TK_ROUTER_LSE, st);
  hipLaunchKernelGGL((k_router<T, D, false, TAIL, PAD, 0>), grid, dim3(256), 0, st, (const T*)a.qr, (const T*)a.kr,
                     a.lse2, a.scores, a.nb, a.scale_log2, (const uint64_t*)a.kmask, 8 * a.nb);
  timer_after(TK_ROUTER_LSE, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  timer_before(TK_ROUTER_SCORES, st);
  if (a.bs)
    hipLaunchKernelGGL((k_router<T, D, true, TAIL, PAD, 1>), grid, dim3(256), 0, st, (const T*)a.qr,
                       (const T*)a.kr, a.lse2, a.scores, a.nb, a.scale_log2, (const uint64_t*)a.kmask, 8 * a.nb);
  else
    hipLaunchKernelGGL((k_router<T, D, true, TAIL, PAD, 0>), grid, dim3(256), 0, st, (const T*)a.qr,
                       (const T*)a.kr, a.lse2, a.scores, a.nb, a.scale_log2, (const uint64_t*)a.kmask, 8 * a.nb);
  timer_after(TK_ROUTER_SCORES, st);
  return hipGetLastError();
}

// The VSA router baseline: P_c over the nb coarse tokens (hstride rows per head).
template <typename T, int D, bool TAIL>
hipError_t launch_route_coarse_tt(const RouteArgs& a, hipStream_t st) {
  const int nqt = (a.nb + RQ - 1) / RQ;
  dim3 grid(xcd_grid(nqt, a.bh));
  hipLaunchKernelGGL((k_router<T, D, false, TAIL, false, 0, true>), grid, dim3(256), 0, st, (const T*)a.qr,
                     (const T*)a.kr, a.lse2, a.scores, a.nb, a.scale_log2, nullptr, a.hstride);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_router<T, D, true, TAIL, false, 0, true>), grid, dim3(256), 0, st, (const T*)a.qr,
                     (const T*)a.kr, a.lse2, a.scores, a.nb, a.scale_log2, nullptr, a.hstride);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_route_t(const RouteArgs& a, hipStream_t st) {
  if (a.g1) return a.nb % RK ? launch_route_coarse_tt<T, D, true>(a, st) : launch_route_coarse_tt<T, D, false>(a, st);
  if (a.pad.on) return launch_route_tt<T, D, false, true>(a, st);
  return (8 * a.nb) % RK ? launch_route_tt<T, D, true, false>(a, st) : launch_route_tt<T, D, false, false>(a, st);
}

// Router pool 1: the passes ran over the tokens with sub-cubes as their
// groups, writing the mean over each (query sub-cube, key sub-cube) pair; the
// score of a cube pair is the mean of its 8 x 8 such means (groups of equal
// size).  One workgroup per (query cube, batch*head), fixed summation order.
__global__ __launch_bounds__(256) void k_route_fold(const float* __restrict__ sub, float* __restrict__ scores,
                                                    int nc) {
  const int c = blockIdx.x, bh = blockIdx.y;
  const size_t n8 = 8 * (size_t)nc;
  const float* rows = sub + ((size_t)bh * n8 + 8 * (size_t)c) * n8;
  float* out = scores + ((size_t)bh * nc + c) * nc;
  for (int j = threadIdx.x; j < nc; j += 256) {
    float acc = 0.f;
    for (int s1 = 0; s1 < 8; ++s1)
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) acc += rows[s1 * n8 + 8 * (size_t)j + s2];
    out[j] = acc * (1.0f / 64.0f);
  }
}

hipError_t launch_route_fold(const float* sub, float* scores, int bh, int nc, hipStream_t st) {
  hipLaunchKernelGGL(k_route_fold, dim3(nc, bh), dim3(256), 0, st, sub, scores, nc);
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  if (a.bf16) return a.d == 128 ? launch_route_t<bf16, 128>(a, st) : launch_route_t<bf16, 64>(a, st);
  return a.d == 128 ? launch_route_t<float, 128>(a, st) : launch_route_t<float, 64>(a, st);
}

}  // namespace vsa2
