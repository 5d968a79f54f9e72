// Mean pooling for the router (paper §2.2 Eq.(5): 2x2x2 windows = 8
// contiguous tokens in cube-tiled order) and for the coarse branch (Eq.(1):
// 4x4x4 cubes = 64 contiguous tokens), one pass over Q, K and V.
#include "common.h"
#include "launch.h"

namespace vsa2 {

// One block per (batch*head, cube).  Unit u = (tensor, sub-cube, 8 columns):
// the 8 tokens of sub-cube s are summed in fp32; the cube mean is the mean of
// the eight sub-cube means.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_pool(const T* __restrict__ q, const T* __restrict__ k,
                                              const T* __restrict__ v, T* __restrict__ qr, T* __restrict__ kr,
                                              T* __restrict__ qc, T* __restrict__ kc, T* __restrict__ vc, int nb,
                                              int nbp) {
  __shared__ float sub[3][8][D];
  const int c = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const size_t L = (size_t)nb * CUBE;
  const size_t tok0 = (size_t)bh * L + (size_t)c * CUBE;
  constexpr int CG = D / 8;
  for (int u = tid; u < 3 * 8 * CG; u += 256) {
    const int tensor = u / (8 * CG), s = (u / CG) % 8, cg = u % CG;
    const T* src = tensor == 0 ? q : (tensor == 1 ? k : v);
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      Vec8<T> x = load8(src + (tok0 + 8 * s + r) * D + 8 * cg);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += to_f32(x.v[e]);
    }
    Vec8<T> m;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[e] *= 0.125f;
      sub[tensor][s][8 * cg + e] = acc[e];
      m.v[e] = from_f32<T>(acc[e]);
    }
    if (tensor < 2) {
      T* dst = tensor == 0 ? qr : kr;
      store8(dst + ((size_t)bh * nb * 8 + (size_t)c * 8 + s) * D + 8 * cg, m);
    }
  }
  __syncthreads();
  for (int u = tid; u < 3 * D; u += 256) {
    const int tensor = u / D, d = u % D;
    float a = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) a += sub[tensor][s][d];
    T* dst = tensor == 0 ? qc : (tensor == 1 ? kc : vc);
    dst[((size_t)bh * nbp + c) * D + d] = from_f32<T>(a * 0.125f);
  }
  // zero the padding rows nb .. nbp-1 of the coarse operands
  for (int row = nb + c; row < nbp; row += nb) {
    for (int u = tid; u < 3 * D; u += 256) {
      T* dst = u / D == 0 ? qc : (u / D == 1 ? kc : vc);
      dst[((size_t)bh * nbp + row) * D + u % D] = from_f32<T>(0.f);
    }
  }
}

template <typename T, int D>
hipError_t launch_pool_t(const PoolArgs& a, hipStream_t st) {
  dim3 grid(a.nb, a.bh);
  hipLaunchKernelGGL((k_pool<T, D>), grid, dim3(256), 0, st, (const T*)a.q, (const T*)a.k, (const T*)a.v,
                     (T*)a.qr, (T*)a.kr, (T*)a.qc, (T*)a.kc, (T*)a.vc, a.nb, a.nbp);
  return hipGetLastError();
}

hipError_t launch_pool(const PoolArgs& a, hipStream_t st) {
  if (a.bf16) return a.d == 128 ? launch_pool_t<bf16, 128>(a, st) : launch_pool_t<bf16, 64>(a, st);
  return a.d == 128 ? launch_pool_t<float, 128>(a, st) : launch_pool_t<float, 64>(a, st);
}

}  // namespace vsa2
