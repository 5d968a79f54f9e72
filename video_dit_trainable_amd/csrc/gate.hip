// Gated merge of VSA2 (paper §2.2 Eq.(13)-(14)): G = tanh(X W_g), one gate per
// token and head, O = G * Repeat(O_hat_c) + O_f (Eq.(4) broadcast fused), and
// its backward (dW_g, dX, dO_hat_c).  On a padded grid (§2.2 "Kernel
// Implementation") pad rows get G = 0 and O = 0 and take no part in the
// backward (dpre = 0 there, so their dX is 0 and their X adds nothing to dW_g).
//
// X W_g and dpre W_g^T are skinny GEMMs run on MFMA; in bf16 mode the fp32
// operands W_g and dpre are split into a bf16 high part and a bf16 remainder
// (x = hi + lo to ~16 mantissa bits) so the products keep near-fp32 accuracy.
// dW_g = X^T dpre is reduced over token chunks into per-chunk partials that a
// second kernel adds in a fixed order (no float atomics).
#include <algorithm>
#include <cmath>

#include "common.h"
#include "launch.h"

namespace vsa2 {

constexpr int HMAX = 64;   // heads supported by the gate kernels

__host__ __device__ inline int pad_up(int x, int m) { return (x + m - 1) / m * m; }

// Repack W_g [dm, H] fp32 into MFMA operands: F = W_g^T [hp, dm] (hi, lo) and
// Bk = W_g [dm, hk] (hi, lo), zero-padded.
template <typename T>
__global__ void k_gate_prep(const float* __restrict__ w, T* __restrict__ wt, int dm, int H, int hp, int hk) {
  T* fhi = wt;
  T* flo = fhi + (size_t)hp * dm;
  T* bhi = flo + (size_t)hp * dm;
  T* blo = bhi + (size_t)dm * hk;
  const size_t nf = (size_t)hp * dm, nbk = (size_t)dm * hk;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < nf + nbk; idx += (size_t)gridDim.x * blockDim.x) {
    int h, m;
    T *dhi, *dlo;
    size_t o;
    if (idx < nf) {
      h = (int)(idx / dm); m = (int)(idx % dm); dhi = fhi; dlo = flo; o = idx;
    } else {
      const size_t r = idx - nf;
      m = (int)(r / hk); h = (int)(r % hk); dhi = bhi; dlo = blo; o = r;
    }
    const float x = h < H ? w[(size_t)m * H + h] : 0.f;
    const T hi = from_f32<T>(x);
    dhi[o] = hi;
    dlo[o] = from_f32<T>(x - to_f32(hi));
  }
}

template <typename T>
__device__ __forceinline__ void split8(const float* x, Frag<T>& hi, Frag<T>& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const T h = from_f32<T>(x[e]);
    hi.v[e] = h;
    lo.v[e] = from_f32<T>(x[e] - to_f32(h));
  }
}

// One block per (cube, batch): gates of its 64 tokens for every head, then the merge.
template <typename T, int D, int NHB>
__global__ __launch_bounds__(256) void k_gate_fwd(const T* __restrict__ x, const T* __restrict__ wt,
                                                  const float* __restrict__ oc_hat, const T* __restrict__ o_f,
                                                  T* __restrict__ o, float* __restrict__ gout, int H, int nb, int dm,
                                                  int hp, PadGrid pad, int bs, int ld) {
  constexpr bool SPLIT = sizeof(T) == 2;
  __shared__ float gs[64][HMAX + 1];
  const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4,
            cc = lane & 15;
  const uint64_t real = pad.on ? cube_slots(c, pad) : ~0ull;  // padded grid: pad rows get g = 0, O = 0
  const size_t L = (size_t)nb * CUBE;
  const T* fhi = wt;
  const T* flo = wt + (size_t)hp * dm;
  // gate products: wave w takes k-steps [w S/4, (w+1) S/4) of X W_g for all 64
  // tokens (4 blocks of 16), so each wave reads a quarter of W_g; the four
  // partial sums are added through LDS (one head block at a time, fixed order)
  __shared__ float gpart[4][4][4][64];  // [wave][token block][r][lane]
  f32x4 acc[4][NHB];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) acc[tb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int S = dm / 32, s0 = w * S / 4, s1 = (w + 1) * S / 4;
  const T* xblk = x + ((size_t)b * L + (size_t)c * CUBE + cc) * dm;
#pragma unroll 4
  for (int s = s0; s < s1; ++s) {
    Frag<T> a[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) a[tb] = frag_from8(load8(xblk + (size_t)16 * tb * dm + 32 * s + 8 * g));
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const Frag<T> bhi = frag_from8(load8(fhi + (size_t)(16 * hb + cc) * dm + 32 * s + 8 * g));
      Frag<T> blo;
      if constexpr (SPLIT) blo = frag_from8(load8(flo + (size_t)(16 * hb + cc) * dm + 32 * s + 8 * g));
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        mma(acc[tb][hb], a[tb], bhi);
        if constexpr (SPLIT) mma(acc[tb][hb], a[tb], blo);
      }
    }
  }
  // acc[tb][hb] lane (g, c): tokens 16 tb + 4g + r (rows), head 16 hb + c (column)
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int r = 0; r < 4; ++r) gpart[w][tb][r][lane] = acc[tb][hb][r];
    __syncthreads();
    const int tb = w;  // wave w finishes token block w
    const int h = 16 * hb + cc;
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v[r] = tanhf(gpart[0][tb][r][lane] + gpart[1][tb][r][lane] + gpart[2][tb][r][lane] + gpart[3][tb][r][lane]);
      if (!((real >> (16 * tb + 4 * g + r)) & 1)) v[r] = 0.f;
    }
    const size_t t0 = (size_t)c * CUBE + 16 * tb;
#pragma unroll
    for (int r = 0; r < 4; ++r) gs[16 * tb + 4 * g + r][h] = v[r];
    if (h < H)
      *reinterpret_cast<float4*>(gout + ((size_t)b * H + h) * L + t0 + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
    __syncthreads();
  }
  __syncthreads();
  constexpr int UPR = D / 8;  // units per token row
  constexpr int UPT = 64 * UPR / 256;  // units per thread and head
#pragma unroll 2
  for (int h = 0; h < H; ++h) {
    const size_t bh = (size_t)b * H + h;
    const float* oc = oc_hat + (bh * (nb >> bs) + (c >> bs)) * D;  // the coarse token of the cube's block
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + 256 * i;
      const int t = u / UPR, dg = u % UPR;
      const float gv = gs[t][h];
      const size_t off = (bh * ld + (size_t)c * CUBE + t) * D + 8 * dg;
      const Vec8<T> f = load8(o_f + off);
      const float4 a0 = *reinterpret_cast<const float4*>(oc + 8 * dg);
      const float4 a1 = *reinterpret_cast<const float4*>(oc + 8 * dg + 4);
      const float ocv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const bool tok_real = (real >> t) & 1;
      Vec8<T> r;
#pragma unroll
      for (int e = 0; e < 8; ++e) r.v[e] = from_f32<T>(tok_real ? fmaf(gv, ocv[e], to_f32(f.v[e])) : 0.f);
      store8(o + off, r);
    }
  }
}

// One block per (cube, batch): dgate, dpre = dg (1 - g^2), dO_hat_c and its
// rowsum against O_hat_c for every head, then dX = dpre W_g^T.
template <typename T, int D, int NS>
__global__ __launch_bounds__(256) void k_gate_bwd(const T* __restrict__ wt, const float* __restrict__ oc_hat,
                                                  const float* __restrict__ gin, const T* __restrict__ d_o,
                                                  float* __restrict__ dpre, T* __restrict__ doc,
                                                  const float* __restrict__ lse_c, float* __restrict__ stats_c,
                                                  T* __restrict__ dx, int H, int nb,
                                                  int nbp, int dm, int hp, int hk, PadGrid pad, int bs,
                                                  float* __restrict__ doc_part, int ld) {
  constexpr bool SPLIT = sizeof(T) == 2;
  constexpr int UPR = D / 8;
  constexpr int RROWS = 256 / UPR;
  // dps and red during the head loop; afterwards the same bytes stage the dX
  // tiles (one 64-token x 64-column tile per wave)
  constexpr int DPS_BYTES = 64 * (HMAX + 4) * 4, RED_BYTES = RROWS * D * 4;
  constexpr int STAGE_BYTES = 4 * 64 * 64 * (int)sizeof(T);
  constexpr int SMEM = DPS_BYTES + RED_BYTES > STAGE_BYTES ? DPS_BYTES + RED_BYTES : STAGE_BYTES;
  __shared__ __align__(16) char smem[SMEM];
  float(*dps)[HMAX + 4] = reinterpret_cast<float(*)[HMAX + 4]>(smem);
  float(*red)[D] = reinterpret_cast<float(*)[D]>(smem + DPS_BYTES);
  __shared__ float wsum[4];
  const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4,
            cc = lane & 15;
  const size_t L = (size_t)nb * CUBE;
  const uint64_t real = pad.on ? cube_slots(c, pad) : ~0ull;  // padded grid: pad rows get g = 0, dpre = 0
  for (int u = tid; u < 64 * (HMAX + 4); u += 256) dps[u / (HMAX + 4)][u % (HMAX + 4)] = 0.f;
  __syncthreads();
  const int dg = tid % UPR;
  constexpr int TPT = 64 / RROWS;  // tokens per thread and head
  // dO rows and gates of the next head are loaded while the current head is reduced
  Vec8<T> xn[TPT];
  float gn[TPT];
  auto fetch = [&](int h) {
    const size_t bh = (size_t)b * H + h;
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const size_t tok = (size_t)c * CUBE + tid / UPR + RROWS * i;
      xn[i] = load8(d_o + (bh * ld + tok) * D + 8 * dg);
      gn[i] = gin[bh * L + tok];
    }
  };
  if (H > 0) fetch(0);
  for (int h = 0; h < H; ++h) {
    const size_t bh = (size_t)b * H + h;
    Vec8<T> xc[TPT];
    float gc[TPT];
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      xc[i] = xn[i];
      gc[i] = gn[i];
    }
    if (h + 1 < H) fetch(h + 1);
    const float* oc = oc_hat + (bh * (nb >> bs) + (c >> bs)) * D;
    const float4 a0 = *reinterpret_cast<const float4*>(oc + 8 * dg);
    const float4 a1 = *reinterpret_cast<const float4*>(oc + 8 * dg + 4);
    const float ocv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    float pacc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int t = tid / UPR + RROWS * i;
      const size_t tok = (size_t)c * CUBE + t;
      const Vec8<T> x = xc[i];
      const bool tok_real = (real >> t) & 1;
      const float gv = tok_real ? gc[i] : 0.f;
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xv = to_f32(x.v[e]);
        part = fmaf(xv, ocv[e], part);
        pacc[e] = fmaf(gv, xv, pacc[e]);
      }
#pragma unroll
      for (int s = 1; s < UPR; s <<= 1) part += __shfl_xor(part, s);
      if (dg == 0) {
        const float dp = tok_real ? part * (1.f - gv * gv) : 0.f;
        dps[t][h] = dp;
        dpre[bh * L + tok] = dp;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[tid / UPR][8 * dg + e] = pacc[e];
    __syncthreads();
    float prod = 0.f;
    if (tid < D) {
      float s = 0.f;
      for (int r = 0; r < RROWS; ++r) s += red[r][tid];
      if (bs) {  // 128-token blocks: the pair kernel adds the two cubes' sums
        doc_part[(bh * nb + c) * D + tid] = s;
      } else {
        doc[(bh * nbp + c) * D + tid] = from_f32<T>(s);
        prod = s * oc[tid];
      }
    }
    if (!bs) {
      for (int s = 1; s < 64; s <<= 1) prod += __shfl_xor(prod, s);
      if (lane == 0) wsum[w] = prod;
    }
    __syncthreads();
    if (tid == 0 && !bs) {
      stats_c[2 * (bh * nbp + c)] = lse_c[bh * nb + c] * LOG2E;
      stats_c[2 * (bh * nbp + c) + 1] = -(wsum[0] + wsum[1] + wsum[2] + wsum[3]);
    }
  }
  // zero the padding rows of dO_hat_c and mask them in the row statistics
  for (int row = nb + c; row < nbp && !bs; row += nb)
    for (int h = 0; h < H; ++h) {
      const size_t bh = (size_t)b * H + h;
      for (int d = tid; d < D; d += 256) doc[(bh * nbp + row) * D + d] = from_f32<T>(0.f);
      if (tid == 0) {
        stats_c[2 * (bh * nbp + row)] = INFINITY;
        stats_c[2 * (bh * nbp + row) + 1] = 0.f;
      }
    }
  __syncthreads();
  // dX^T[m][t] = sum_h W_g[m][h] dpre[t][h]: wave w takes the column blocks
  // [w dm/64, (w+1) dm/64) for all 64 tokens, so each wave reads a quarter of
  // W_g (its hi and lo parts) and reuses every fragment for 4 token blocks
  const T* bhi = wt + 2 * (size_t)hp * dm;
  const T* blo = bhi + (size_t)dm * hk;
  Frag<T> phi[4][NS], plo[4][NS];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      float v8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v8[e] = dps[16 * tb + cc][32 * s + 8 * g + e];
      split8<T>(v8, phi[tb][s], plo[tb][s]);
    }
  __syncthreads();  // every wave has its dpre fragments: dps may be overwritten
  // Each wave stages 64 tokens x 64 columns (four column blocks) at a time and
  // writes them as whole 128-byte row segments; dm is a multiple of 64.
  T* stage = reinterpret_cast<T*>(smem) + w * 64 * 64;
  T* dxt = dx + ((size_t)b * L + (size_t)c * CUBE) * dm;
  const int nq = dm / 64, q0 = w * nq / 4, q1 = (w + 1) * nq / 4;
  for (int qd = q0; qd < q1; ++qd) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int mb = 4 * qd + j;
      f32x4 acc[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const Frag<T> ahi = frag_from8(load8(bhi + (size_t)(16 * mb + cc) * hk + 32 * s + 8 * g));
        Frag<T> alo;
        if constexpr (SPLIT) alo = frag_from8(load8(blo + (size_t)(16 * mb + cc) * hk + 32 * s + 8 * g));
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          mma(acc[tb], ahi, phi[tb][s]);
          if constexpr (SPLIT) {
            mma(acc[tb], ahi, plo[tb][s]);
            mma(acc[tb], alo, phi[tb][s]);
          }
        }
      }
      // lane (g, c): columns 16j + 4g .. +3 of token 16tb + c; the 8-byte
      // pieces are placed at chunk (2j + g/2) ^ (t & 7) of the token's row
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        Vec4<T> r4;
#pragma unroll
        for (int r = 0; r < 4; ++r) r4.v[r] = from_f32<T>(acc[tb][r]);
        const int t = 16 * tb + cc;
        store4(stage + t * 64 + 8 * ((2 * j + (g >> 1)) ^ (t & 7)) + 4 * (g & 1), r4);
      }
    }
    // 8 lanes per token row: lane l writes chunk l % 8 of rows l / 8 + 8i
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = lane / 8 + 8 * i, ch = lane % 8;
      const Vec8<T> v = load8(stage + t * 64 + 8 * (ch ^ (t & 7)));
      store8(dxt + (size_t)t * dm + 64 * qd + 8 * ch, v);
    }
  }
}

// 128-token blocks: dO_hat_c of a block is the sum of its two cubes' sums,
// and its row statistics (lse_c log2 e, -rowsum(dO_hat_c O_hat_c)) follow as
// in k_gate_bwd; rows nb .. nbp-1 are zeroed and masked.  One workgroup per
// (block, batch * head) and D threads.
template <typename T, int D>
__global__ __launch_bounds__(D) void k_coarse_pair(const float* __restrict__ doc_part,
                                                   const float* __restrict__ oc_hat, const float* __restrict__ lse_c,
                                                   T* __restrict__ doc, float* __restrict__ stats_c, int nblk,
                                                   int nbp) {
  __shared__ float wsum[D / 64];
  const int blk = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const size_t bh = blockIdx.y;
  const float* part = doc_part + (bh * 2 * nblk + 2 * blk) * D;
  const float s = part[tid] + part[D + tid];
  doc[(bh * nbp + blk) * D + tid] = from_f32<T>(s);
  float prod = s * oc_hat[(bh * nblk + blk) * D + tid];
  for (int o = 1; o < 64; o <<= 1) prod += __shfl_xor(prod, o);
  if (lane == 0) wsum[tid >> 6] = prod;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int w = 0; w < D / 64; ++w) t += wsum[w];
    stats_c[2 * (bh * nbp + blk)] = lse_c[bh * nblk + blk] * LOG2E;
    stats_c[2 * (bh * nbp + blk) + 1] = -t;
  }
  for (int row = nblk + blk; row < nbp; row += nblk) {
    doc[(bh * nbp + row) * D + tid] = from_f32<T>(0.f);
    if (tid == 0) {
      stats_c[2 * (bh * nbp + row)] = INFINITY;
      stats_c[2 * (bh * nbp + row) + 1] = 0.f;
    }
  }
}

// dW_g partial over one token chunk: dW[m][h] = sum_t X[t][m] dpre[h][t].
// Block = (64 columns of X, token chunk, batch); X tiles transposed in LDS.
template <typename T>
__global__ __launch_bounds__(256) void k_dwg_part(const T* __restrict__ x, const float* __restrict__ dpre,
                                                  float* __restrict__ part, int H, int nb, int dm, int nchunk) {
  constexpr bool SPLIT = sizeof(T) == 2;
  using G = TileGeom<T, 64>;
  __shared__ T xt[G::TR_ELEMS];
  const int mblk = blockIdx.x, chunk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, cc = lane & 15;
  const size_t L = (size_t)nb * CUBE;
  const int nhb = (H + 15) / 16;
  f32x4 acc[HMAX / 16];
#pragma unroll
  for (int hb = 0; hb < HMAX / 16; ++hb) acc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  TileRegs<T, 64, 256> regs;
  const size_t t_beg = (size_t)chunk * DW_TC, t_end = min(L, (size_t)(chunk + 1) * DW_TC);
  if (t_beg < t_end) tile_load<T, 64, 256>(regs, x + ((size_t)b * L + t_beg) * dm + 64 * mblk, tid, 64, (size_t)dm);
  for (size_t t0 = t_beg; t0 < t_end; t0 += 64) {
    __syncthreads();
    tile_store_tr<T, 64, 256>(regs, xt, tid);
    __syncthreads();
    if (t0 + 64 < t_end)  // next tile's loads overlap this tile's products
      tile_load<T, 64, 256>(regs, x + ((size_t)b * L + t0 + 64) * dm + 64 * mblk, tid, 64, (size_t)dm);
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const Frag<T> a = frag_tr<T, 64>(xt, 16 * w + cc, c2, g);
#pragma unroll
      for (int hb = 0; hb < HMAX / 16; ++hb) {
        if (hb < nhb) {
          const int h = 16 * hb + cc;
          float v8[8];
          if (h < H) {
            const float* src = dpre + ((size_t)b * H + h) * L + t0 + 32 * c2 + 4 * g;
            const float4 lo = *reinterpret_cast<const float4*>(src);
            const float4 hi = *reinterpret_cast<const float4*>(src + 16);
            v8[0] = lo.x; v8[1] = lo.y; v8[2] = lo.z; v8[3] = lo.w;
            v8[4] = hi.x; v8[5] = hi.y; v8[6] = hi.z; v8[7] = hi.w;
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v8[e] = 0.f;
          }
          Frag<T> bhi, blo;
          split8<T>(v8, bhi, blo);
          mma(acc[hb], a, bhi);
          if constexpr (SPLIT) mma(acc[hb], a, blo);
        }
      }
    }
  }
  float* out = part + (((size_t)b * nchunk + chunk) * dm + 64 * mblk) * H;
#pragma unroll
  for (int hb = 0; hb < HMAX / 16; ++hb) {
    const int h = 16 * hb + cc;
    if (hb < nhb && h < H) {
#pragma unroll
      for (int r = 0; r < 4; ++r) out[(size_t)(16 * w + 4 * g + r) * H + h] = acc[hb][r];
    }
  }
}

// The bf16 dW_g partial: dW^T[h][m] = sum_t dpre[h][t] X[t][m] over one token
// chunk.  Each wave owns 64 columns of X and works alone: it copies its
// 64-token x 64-column tiles LDS-direct (row-major, chunk-swizzled, two
// stages in distinct arrays, the loop unrolled by two) and reads them as
// transposed B fragments; the A operand is dpre^T, split into bf16 hi + lo
// (fp32-accurate products), loaded one tile ahead.  NHB = 16-head blocks.
template <int NHB>
__global__ __launch_bounds__(256, 2) void k_dwg_part_bf16(const bf16* __restrict__ x, const float* __restrict__ dpre,
                                                          float* __restrict__ part, int H, int nb, int dm,
                                                          int nchunk) {
  using T = bf16;
  using S = SwTile<T, 64>;
  constexpr int TT = 64 * 64;  // elements per wave tile
  __shared__ __align__(16) T sA[4 * TT];
  __shared__ __align__(16) T sB[4 * TT];
  const int chunk = blockIdx.y, b = blockIdx.z, tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4,
            cc = lane & 15;
  const int m0 = 256 * blockIdx.x + 64 * w;
  if (m0 >= dm) return;  // waves work alone: no barrier follows
  const size_t L = (size_t)nb * CUBE;
  const size_t t_beg = (size_t)chunk * DW_TC, t_end = min(L, (size_t)(chunk + 1) * DW_TC);
  T* tA = sA + w * TT;
  T* tB = sB + w * TT;
  // copy n of this lane fills physical chunk lane % 8 of row 8n + lane / 8
  // with logical chunk (lane % 8) ^ f(row); rows 8n + j share f for n and n + 2
  const int rl = lane >> 3, pc = lane & 7;
  int coff[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int r = 8 * n + rl;
    coff[n] = (r * dm + 8 * (pc ^ (S::f(r) & (S::NCH - 1)))) * (int)sizeof(T);
  }
  const char* xb = reinterpret_cast<const char*>(x + (size_t)b * L * dm + m0);
  auto copy = [&](size_t t0, T* tile) {
    const char* src = xb + t0 * dm * sizeof(T);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      int off = coff[n & 1] + (n >> 1) * 16 * dm * (int)sizeof(T);
      opaque(off);
      lds_copy16(src + (uint32_t)off, (VSA2_LDS void*)(tile + n * 512));
    }
  };
  float4 dp[2][NHB][2], dpn[2][NHB][2];
  auto load_dp = [&](size_t t0, float4 (&d)[2][NHB][2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const int h = 16 * hb + cc;
        if (h < H) {
          const float* src = dpre + ((size_t)b * H + h) * L + t0 + 32 * ks + 4 * g;
          d[ks][hb][0] = *reinterpret_cast<const float4*>(src);
          d[ks][hb][1] = *reinterpret_cast<const float4*>(src + 16);
        } else {
          d[ks][hb][0] = d[ks][hb][1] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
  };
  f32x4 acc[NHB][4];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[hb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int btr = sw_tr_base<T, 64>(0, g, cc);
  auto tile_products = [&](const T* tile, const float4 (&d)[2][NHB][2]) {
    int base = btr;
    opaque(base);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      Frag<T> ahi[NHB], alo[NHB];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const float4 lo = d[ks][hb][0], hi = d[ks][hb][1];
        const float v8[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        split8<T>(v8, ahi[hb], alo[hb]);
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const Frag<T> bx = sw_frag_tr_at<T, 64>(tile, base + 32 * ks * 64, 16 * mb);
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          mma(acc[hb][mb], ahi[hb], bx);
          mma(acc[hb][mb], alo[hb], bx);
        }
      }
    }
  };
  if (t_beg < t_end) {
    copy(t_beg, tA);
    load_dp(t_beg, dp);
  }
  for (size_t t0 = t_beg; t0 < t_end; t0 += 128) {
    wait_vm0();  // tile t0 (stage A) and its dpre values are in
    if (t0 + 64 < t_end) {
      copy(t0 + 64, tB);
      load_dp(t0 + 64, dpn);
    }
    tile_products(tA, dp);
    if (t0 + 64 >= t_end) break;
    wait_vm0();  // tile t0 + 64 (stage B)
    if (t0 + 128 < t_end) {
      copy(t0 + 128, tA);
      load_dp(t0 + 128, dp);
    }
    tile_products(tB, dpn);
  }
  float* out = part + (((size_t)b * nchunk + chunk) * dm + m0) * H;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 16 * hb + 4 * g + r;
        if (h < H) out[(size_t)(16 * mb + cc) * H + h] = acc[hb][mb][r];
      }
}

__global__ void k_dwg_reduce(const float* __restrict__ part, float* __restrict__ dw, int n, int parts) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  float s = 0.f;
  for (int p = 0; p < parts; ++p) s += part[(size_t)p * n + idx];
  dw[idx] = s;
}

template <typename T>
static hipError_t gate_prep(const float* w_g, void* wt, int dm, int H, hipStream_t st) {
  const int hp = pad_up(H, 16), hk = pad_up(H, 32);
  const size_t n = (size_t)(hp + hk) * dm;
  unsigned blocks = (unsigned)((n + 255) / 256);
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL((k_gate_prep<T>), dim3(blocks), dim3(256), 0, st, w_g, (T*)wt, dm, H, hp, hk);
  return hipGetLastError();
}

// MMDiT text rows (after the video slots of each head) have no coarse term:
// O = O_f there.  One thread per 8 elements.
template <typename T>
__global__ __launch_bounds__(256) void k_copy_rows(const T* __restrict__ src, T* __restrict__ dst, size_t row0,
                                                   size_t ld, size_t nrows, size_t rowlen, size_t nbh) {
  const size_t per = nrows * rowlen / 8;
  for (size_t u = (size_t)blockIdx.x * 256 + threadIdx.x; u < per * nbh; u += (size_t)gridDim.x * 256) {
    const size_t bh = u / per, e = (u % per) * 8;
    const size_t off = (bh * ld + row0) * rowlen + e;
    store8(dst + off, load8(src + off));
  }
}

template <typename T, int D>
hipError_t launch_gate_fwd_t(const GateArgs& a, hipStream_t st) {
  hipError_t e = gate_prep<T>(a.w_g, a.wt, a.dm, a.heads, st);
  if (e != hipSuccess) return e;
  const int hp = pad_up(a.heads, 16);
  const dim3 grid(a.nb, a.batch);
#define VSA2_GATE_FWD(NHB)                                                                                     \
  hipLaunchKernelGGL((k_gate_fwd<T, D, NHB>), grid, dim3(256), 0, st, (const T*)a.x, (const T*)a.wt, a.oc_hat, \
                     (const T*)a.o_f, (T*)a.o, a.g, a.heads, a.nb, a.dm, hp, a.pad, a.bs, a.ld)
  switch (hp / 16) {
    case 1: VSA2_GATE_FWD(1); break;
    case 2: VSA2_GATE_FWD(2); break;
    case 3: VSA2_GATE_FWD(3); break;
    default: VSA2_GATE_FWD(4); break;
  }
#undef VSA2_GATE_FWD
  const size_t L = (size_t)a.nb * CUBE;
  if ((size_t)a.ld > L) {
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t bhn = (size_t)a.batch * a.heads, n8 = ((size_t)a.ld - L) * D / 8 * bhn;
    const int blocks = (int)std::min<size_t>((n8 + 255) / 256, 4096);
    hipLaunchKernelGGL((k_copy_rows<T>), dim3(blocks), dim3(256), 0, st, (const T*)a.o_f, (T*)a.o, L, (size_t)a.ld,
                       (size_t)a.ld - L, (size_t)D, bhn);
  }
  return hipGetLastError();
}

hipError_t launch_gate_fwd(const GateArgs& a, hipStream_t st) {
  if (a.bf16) return a.d == 128 ? launch_gate_fwd_t<bf16, 128>(a, st) : launch_gate_fwd_t<bf16, 64>(a, st);
  return a.d == 128 ? launch_gate_fwd_t<float, 128>(a, st) : launch_gate_fwd_t<float, 64>(a, st);
}

template <typename T, int D>
hipError_t launch_gate_bwd_t(const GateBwdArgs& a, hipStream_t st) {
  hipError_t e = gate_prep<T>(a.w_g, a.wt, a.dm, a.heads, st);
  if (e != hipSuccess) return e;
  const int hp = pad_up(a.heads, 16), hk = pad_up(a.heads, 32);
  if (hk <= 32)
    hipLaunchKernelGGL((k_gate_bwd<T, D, 1>), dim3(a.nb, a.batch), dim3(256), 0, st, (const T*)a.wt, a.oc_hat, a.g,
                       (const T*)a.d_o, a.dpre, (T*)a.doc, a.lse_c, a.stats_c, (T*)a.dx, a.heads, a.nb, a.nbp, a.dm,
                       hp, hk, a.pad, a.bs, a.doc_part, a.ld);
  else
    hipLaunchKernelGGL((k_gate_bwd<T, D, 2>), dim3(a.nb, a.batch), dim3(256), 0, st, (const T*)a.wt, a.oc_hat, a.g,
                       (const T*)a.d_o, a.dpre, (T*)a.doc, a.lse_c, a.stats_c, (T*)a.dx, a.heads, a.nb, a.nbp, a.dm,
                       hp, hk, a.pad, a.bs, a.doc_part, a.ld);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.bs) {
    hipLaunchKernelGGL((k_coarse_pair<T, D>), dim3(a.nb >> 1, a.batch * a.heads), dim3(D), 0, st, a.doc_part,
                       a.oc_hat, a.lse_c, (T*)a.doc, a.stats_c, a.nb >> 1, a.nbp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if constexpr (sizeof(T) == 2) {
    const dim3 grid((a.dm + 255) / 256, a.nchunk, a.batch);
    const int nhb = (a.heads + 15) / 16;
    const bf16* xx = (const bf16*)a.x;
    if (nhb == 1) hipLaunchKernelGGL(k_dwg_part_bf16<1>, grid, dim3(256), 0, st, xx, a.dpre, a.dw_part, a.heads, a.nb, a.dm, a.nchunk);
    else if (nhb == 2) hipLaunchKernelGGL(k_dwg_part_bf16<2>, grid, dim3(256), 0, st, xx, a.dpre, a.dw_part, a.heads, a.nb, a.dm, a.nchunk);
    else if (nhb == 3) hipLaunchKernelGGL(k_dwg_part_bf16<3>, grid, dim3(256), 0, st, xx, a.dpre, a.dw_part, a.heads, a.nb, a.dm, a.nchunk);
    else hipLaunchKernelGGL(k_dwg_part_bf16<4>, grid, dim3(256), 0, st, xx, a.dpre, a.dw_part, a.heads, a.nb, a.dm, a.nchunk);
  } else {
    hipLaunchKernelGGL((k_dwg_part<T>), dim3(a.dm / 64, a.nchunk, a.batch), dim3(256), 0, st, (const T*)a.x, a.dpre,
                       a.dw_part, a.heads, a.nb, a.dm, a.nchunk);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = a.dm * a.heads;
  hipLaunchKernelGGL(k_dwg_reduce, dim3((n + 255) / 256), dim3(256), 0, st, a.dw_part, a.dw_g, n,
                     a.batch * a.nchunk);
  return hipGetLastError();
}

hipError_t launch_gate_bwd(const GateBwdArgs& a, hipStream_t st) {
  if (a.bf16) return a.d == 128 ? launch_gate_bwd_t<bf16, 128>(a, st) : launch_gate_bwd_t<bf16, 64>(a, st);
  return a.d == 128 ? launch_gate_bwd_t<float, 128>(a, st) : launch_gate_bwd_t<float, 64>(a, st);
}

}  // namespace vsa2
