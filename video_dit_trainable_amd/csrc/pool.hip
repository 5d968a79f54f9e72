// Mean pooling for the router (paper §2.2 Eq.(5): 2x2x2 windows = 8
// contiguous tokens in cube-tiled order; router pool 1 copies the tokens,
// pool 4 leaves the router to the coarse operands) and for the coarse branch (Eq.(1):
// attention blocks, 4x4x4 cubes = 64 contiguous tokens or 4x4x8 pairs = 128),
// one pass over Q, K and V.  On a padded grid (§2.2 "Kernel Implementation")
// windows average their real tokens.
#include "common.h"
#include "launch.h"

namespace vsa2 {

// One workgroup per (batch*head, attention block of 2^bs cubes).  Unit u =
// (tensor, sub-cube, 8 columns): the 8 tokens of sub-cube s are summed in
// fp32; the block mean is the mean of its sub-cube means.  On a padded grid
// only real tokens are summed: a sub-cube mean divides by its real-token
// count (a sub-cube with none gives a zero row) and the block mean is the
// real-token sum over the block's count.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_pool(const T* __restrict__ q, const T* __restrict__ k,
                                              const T* __restrict__ v, T* __restrict__ qr, T* __restrict__ kr,
                                              T* __restrict__ qc, T* __restrict__ kc, T* __restrict__ vc, int nb,
                                              int nbp, PadGrid pad, int bs, int ld, int rp) {
  __shared__ float sub[3][8][D];
  const int blk = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int nblk = nb >> bs;
  constexpr int CG = D / 8;
  int count = 0;  // real tokens of the block
  for (int cb = 0; cb < (1 << bs); ++cb) {
    const int c = (blk << bs) + cb;
    const size_t tok0 = (size_t)bh * ld + (size_t)c * CUBE;  // ld rows per head (video, then any text rows)
    const uint64_t real = pad.on ? cube_slots(c, pad) : ~0ull;
    count += __popcll(real);
    for (int u = tid; u < 3 * 8 * CG; u += 256) {
      const int tensor = u / (8 * CG), s = (u / CG) % 8, cg = u % CG;
      const T* src = tensor == 0 ? q : (tensor == 1 ? k : v);
      const uint32_t sreal = (uint32_t)(real >> (8 * s)) & 0xFF;
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        Vec8<T> x = load8(src + (tok0 + 8 * s + r) * D + 8 * cg);
        if (rp == 1 && tensor < 2)  // router pool 1: the router's rows are the tokens (64 per cube)
          store8((tensor == 0 ? qr : kr) + ((size_t)bh * nb * 64 + (size_t)c * 64 + 8 * s + r) * D + 8 * cg, x);
        const bool ok = (sreal >> r) & 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += ok ? to_f32(x.v[e]) : 0.f;
      }
      const int n = __popc(sreal);
      Vec8<T> m;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // block sums (padded grid or 2-cube block) or sub-cube means (single
        // full cube: the mean of the eight means, as one scale at the end)
        const float part = (pad.on || bs) ? acc[e] : acc[e] * 0.125f;
        sub[tensor][s][8 * cg + e] = cb ? sub[tensor][s][8 * cg + e] + part : part;
        m.v[e] = from_f32<T>(n == 8 ? acc[e] * 0.125f : (n > 0 ? acc[e] / (float)n : 0.f));
      }
      if (rp == 2 && tensor < 2) {
        T* dst = tensor == 0 ? qr : kr;
        store8(dst + ((size_t)bh * nb * 8 + (size_t)c * 8 + s) * D + 8 * cg, m);
      }
    }
  }
  __syncthreads();
  const float scale = (pad.on || bs) ? 1.0f / (float)count : 0.125f;
  for (int u = tid; u < 3 * D; u += 256) {
    const int tensor = u / D, d = u % D;
    float a = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) a += sub[tensor][s][d];
    T* dst = tensor == 0 ? qc : (tensor == 1 ? kc : vc);
    dst[((size_t)bh * nbp + blk) * D + d] = from_f32<T>(a * scale);
  }
  // zero the padding rows nblk .. nbp-1 of the coarse operands
  for (int row = nblk + blk; row < nbp; row += nblk) {
    for (int u = tid; u < 3 * D; u += 256) {
      T* dst = u / D == 0 ? qc : (u / D == 1 ? kc : vc);
      dst[((size_t)bh * nbp + row) * D + u % D] = from_f32<T>(0.f);
    }
  }
}

template <typename T, int D>
hipError_t launch_pool_t(const PoolArgs& a, hipStream_t st) {
  dim3 grid(a.nb >> a.bs, a.bh);
  hipLaunchKernelGGL((k_pool<T, D>), grid, dim3(256), 0, st, (const T*)a.q, (const T*)a.k, (const T*)a.v,
                     (T*)a.qr, (T*)a.kr, (T*)a.qc, (T*)a.kc, (T*)a.vc, a.nb, a.nbp, a.pad, a.bs, a.ld, a.rp);
  return hipGetLastError();
}

hipError_t launch_pool(const PoolArgs& a, hipStream_t st) {
  if (a.bf16) return a.d == 128 ? launch_pool_t<bf16, 128>(a, st) : launch_pool_t<bf16, 64>(a, st);
  return a.d == 128 ? launch_pool_t<float, 128>(a, st) : launch_pool_t<float, 64>(a, st);
}

}  // namespace vsa2
