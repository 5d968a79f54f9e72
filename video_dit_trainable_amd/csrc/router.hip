// Fine-grained router of VSA2, paper §2.2 Eq.(6)-(7) with the fused two-pass
// scheme of its "Kernel Implementation" paragraph: the pooled score matrix
// Q_r K_r^T is computed twice on chip -- pass 1 accumulates each pooled
// query's log-sum-exp, pass 2 recomputes the tiles, normalises them and
// averages the 8 x 8 (query sub-cube, key sub-cube) entries of each cube pair.
// Only the nb x nb block scores reach memory.
//
// Work split: a block owns 64 pooled queries (8 query cubes); each of its 4
// waves holds 16 of them as B fragments in registers and streams all pooled
// keys, 64 at a time, through a double-buffered LDS tile.  The accumulator of
// S^T = K_r Q_r^T gives each lane 4 keys x 1 query per 16-key block, so the
// 8 x 8 pooling is 4 in-lane adds + one cross-group and three in-row shuffles.
#include <cmath>

#include "common.h"
#include "launch.h"

namespace vsa2 {

template <typename T, int D, bool PASS2>
__global__ __launch_bounds__(256) void k_router(const T* __restrict__ qr, const T* __restrict__ kr,
                                                float* __restrict__ lse2, float* __restrict__ scores, int nb,
                                                float c) {
  using G = TileGeom<T, D>;
  __shared__ T ks[2][G::RM_ELEMS];
  const int Lr = 8 * nb;
  const int ntile = (Lr + 63) / 64;
  int bh, qt;
  if (!xcd_work(blockIdx.x, ntile, bh, qt)) return;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, cc = lane & 15;
  const int qrow = qt * 64 + 16 * w + cc;
  const T* qbase = qr + (size_t)bh * Lr * D;
  const T* kbase = kr + (size_t)bh * Lr * D;

  Frag<T> qf[D / 32];
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    if (qrow < Lr) {
      qf[s] = frag_global<T, D>(qbase, qrow, s, g);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[s].v[e] = from_f32<T>(0.f);
    }
  }

  TileRegs<T, D, 256> regs;
  tile_load<T, D, 256>(regs, kbase, tid, min(64, Lr));
  tile_store_rm<T, D, 256>(regs, ks[0], tid);
  __syncthreads();

  float m = -INFINITY, l = 0.f;
  float lse = 0.f;
  if constexpr (PASS2) lse = qrow < Lr ? lse2[(size_t)bh * Lr + qrow] : INFINITY;

  for (int t = 0; t < ntile; ++t) {
    if (t + 1 < ntile) tile_load<T, D, 256>(regs, kbase + (size_t)(t + 1) * 64 * D, tid, min(64, Lr - (t + 1) * 64));
    const T* kl = ks[t & 1];
    f32x4 acc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) mma(acc[kb], frag_rm<T, D>(kl, 16 * kb + cc, s, g), qf[s]);
    }
    if (t * 64 + 64 > Lr) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t * 64 + 16 * kb + 4 * g + r >= Lr) acc[kb][r] = -INFINITY;
    }
    if constexpr (!PASS2) {
      float mt = acc[0][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mt = fmaxf(mt, acc[kb][r]);
      if (mt > m) {
        l *= fast_exp2((m - mt) * c);
        m = mt;
      }
      if (m != -INFINITY) {
        const float mc = -m * c;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) l += fast_exp2(fmaf(acc[kb][r], c, mc));
      }
    } else {
      const int qcube = qt * 8 + 2 * w + (cc >> 3);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        float s4 = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) s4 += fast_exp2(fmaf(acc[kb][r], c, -lse));
        s4 += __shfl_xor(s4, 16);
        s4 += __shfl_xor(s4, 1);
        s4 += __shfl_xor(s4, 2);
        s4 += __shfl_xor(s4, 4);
        const int kcube = t * 8 + 2 * kb + (g >> 1);
        if ((g & 1) == 0 && (cc & 7) == 0 && qcube < nb && kcube < nb)
          scores[((size_t)bh * nb + qcube) * nb + kcube] = s4 * (1.0f / 64.0f);
      }
    }
    if (t + 1 < ntile) tile_store_rm<T, D, 256>(regs, ks[(t + 1) & 1], tid);
    __syncthreads();
  }

  if constexpr (!PASS2) {
    const float M = group_max(m);
    const float part = (m == -INFINITY) ? 0.f : l * fast_exp2((m - M) * c);
    const float lt = group_sum(part);
    if (g == 0 && qrow < Lr) lse2[(size_t)bh * Lr + qrow] = M * c + __log2f(lt);
  }
}

template <typename T, int D>
hipError_t launch_route_t(const RouteArgs& a, hipStream_t st) {
  const int ntile = (8 * a.nb + 63) / 64;
  dim3 grid(xcd_grid(ntile, a.bh));
  timer_before(TK_ROUTER_LSE, st);
  hipLaunchKernelGGL((k_router<T, D, false>), grid, dim3(256), 0, st, (const T*)a.qr, (const T*)a.kr, a.lse2,
                     a.scores, a.nb, a.scale_log2);
  timer_after(TK_ROUTER_LSE, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  timer_before(TK_ROUTER_SCORES, st);
  hipLaunchKernelGGL((k_router<T, D, true>), grid, dim3(256), 0, st, (const T*)a.qr, (const T*)a.kr, a.lse2,
                     a.scores, a.nb, a.scale_log2);
  timer_after(TK_ROUTER_SCORES, st);
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  if (a.bf16) return a.d == 128 ? launch_route_t<bf16, 128>(a, st) : launch_route_t<bf16, 64>(a, st);
  return a.d == 128 ? launch_route_t<float, 128>(a, st) : launch_route_t<float, 64>(a, st);
}

}  // namespace vsa2
