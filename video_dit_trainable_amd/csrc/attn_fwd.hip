// Block-sparse flash attention forward: the fine branch of VSA2 (paper §2.2
// Eq.(12), the -inf block mask of §2.1 applied by skipping unselected tiles).
// The same kernel in "dense" mode runs the coarse branch's attention over the
// nb pooled cube tokens (Eq.(2)-(3)), with a ragged last tile.
//
// One block = one query cube (64 queries) of one (batch, head), 4 waves of 16
// queries.  Q stays in registers as B fragments; the selected K/V cubes are
// gathered through the CSR list into a double-buffered LDS stage (K row-major,
// V transposed so both products read 16-byte runs), with the next cube's loads
// in flight while the current one is computed.  S^T = K Q^T puts the 16 keys
// of a lane group against one query per lane, so the online softmax is
// lane-local except a 4-way max across the slot groups, and the exponentials
// feed O^T += V^T P^T directly from the accumulator registers.
#include <cmath>

#include "common.h"
#include "launch.h"

namespace vsa2 {

template <typename T, typename TO, int D, bool DENSE>
__global__ __launch_bounds__(256) void k_attn_fwd(const T* __restrict__ q, const T* __restrict__ k,
                                                  const T* __restrict__ v, const int32_t* __restrict__ row_ptr,
                                                  const int32_t* __restrict__ col_idx, TO* __restrict__ o,
                                                  float* __restrict__ lse, int nq, int nkv, int seq, int ld,
                                                  int out_rows, int64_t kph, float c) {
  using G = TileGeom<T, D>;
  __shared__ T ksm[2][G::RM_ELEMS];
  __shared__ T vsm[2][G::TR_ELEMS];
  int bh, i;
  if (!xcd_work(blockIdx.x, nq, bh, i)) return;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, cc = lane & 15;
  const int qrow = i * 64 + 16 * w + cc;
  const size_t hoff = (size_t)bh * ld * D;
  const T* qb = q + hoff;
  const T* kbase = k + hoff;
  const T* vbase = v + hoff;

  int cnt;
  const int32_t* cols = nullptr;
  if constexpr (DENSE) {
    cnt = nkv;
  } else {
    const int32_t* rp = row_ptr + (size_t)bh * (nq + 1);
    const int64_t start = min<int64_t>(max(rp[i], 0), kph);
    const int64_t end = min<int64_t>(max<int64_t>(rp[i + 1], start), kph);
    cnt = (int)(end - start);
    cols = col_idx + (size_t)bh * kph + start;
  }
  // cube id of list entry n; out-of-range ids (corrupt lists) become -1 = masked tile
  auto cube_at = [&](int n) -> int {
    if constexpr (DENSE) return n;
    const int jj = cols[n];
    return (unsigned)jj < (unsigned)nkv ? jj : -1;
  };
  auto kv_limit = [&](int jj) -> int {  // valid keys of cube jj
    if constexpr (DENSE) return min(64, seq - jj * 64);
    return jj >= 0 ? 64 : 0;
  };

  Frag<T> qf[D / 32];
#pragma unroll
  for (int s = 0; s < D / 32; ++s) qf[s] = frag_global<T, D>(qb, qrow, s, g);

  f32x4 oacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  if (cnt > 0) {
    TileRegs<T, D, 256> kr, vr;
    int j = cube_at(0);
    tile_load<T, D, 256>(kr, kbase + (size_t)max(j, 0) * 64 * D, tid, kv_limit(j));
    tile_load<T, D, 256>(vr, vbase + (size_t)max(j, 0) * 64 * D, tid, kv_limit(j));
    tile_store_rm<T, D, 256>(kr, ksm[0], tid);
    tile_store_tr<T, D, 256>(vr, vsm[0], tid);
    __syncthreads();
    for (int n = 0; n < cnt; ++n) {
      const int buf = n & 1;
      int jn = 0;
      if (n + 1 < cnt) {
        jn = cube_at(n + 1);
        tile_load<T, D, 256>(kr, kbase + (size_t)max(jn, 0) * 64 * D, tid, kv_limit(jn));
        tile_load<T, D, 256>(vr, vbase + (size_t)max(jn, 0) * 64 * D, tid, kv_limit(jn));
      }
      f32x4 acc[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / 32; ++s)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mma(acc[kb], frag_rm<T, D>(ksm[buf], 16 * kb + cc, s, g), qf[s]);
      const int lim = kv_limit(j);
      if (lim < 64) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * kb + 4 * g + r >= lim) acc[kb][r] = -INFINITY;
      }
      float mt = acc[0][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mt = fmaxf(mt, acc[kb][r]);
      mt = group_max(mt);
      const float mnew = fmaxf(m, mt);
      if (mnew != -INFINITY) {
        const float alpha = fast_exp2((m - mnew) * c);
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) oacc[db] *= alpha;
        const float mc = -m * c;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = fast_exp2(fmaf(acc[kb][r], c, mc));
            acc[kb][r] = p;
            l += p;
          }
        const Frag<T> p0 = frag_from_acc<T>(acc[0], acc[1]);
        const Frag<T> p1 = frag_from_acc<T>(acc[2], acc[3]);
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
          mma(oacc[db], frag_tr<T, D>(vsm[buf], 16 * db + cc, 0, g), p0);
          mma(oacc[db], frag_tr<T, D>(vsm[buf], 16 * db + cc, 1, g), p1);
        }
      }
      if (n + 1 < cnt) {
        tile_store_rm<T, D, 256>(kr, ksm[buf ^ 1], tid);
        tile_store_tr<T, D, 256>(vr, vsm[buf ^ 1], tid);
      }
      __syncthreads();
      j = jn;
    }
  }

  const float lt = group_sum(l);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  const bool live = DENSE ? (qrow < seq && qrow < out_rows) : (qrow < out_rows);
  if (live) {
    TO* orow = o + ((size_t)bh * out_rows + qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      Vec4<TO> r4;
#pragma unroll
      for (int r = 0; r < 4; ++r) r4.v[r] = from_f32<TO>(oacc[db][r] * inv);
      store4(orow + 16 * db + 4 * g, r4);
    }
    if (g == 0) lse[(size_t)bh * out_rows + qrow] = lt > 0.f ? (m * c + __log2f(lt)) * LN2 : -INFINITY;
  }
}

template <typename T, int D>
hipError_t launch_fwd_t(const AttnArgs& a, hipStream_t st) {
  dim3 grid(xcd_grid(a.nq, a.bh));
  if (a.dense) {
    hipLaunchKernelGGL((k_attn_fwd<T, float, D, true>), grid, dim3(256), 0, st, (const T*)a.q, (const T*)a.k,
                       (const T*)a.v, nullptr, nullptr, (float*)a.o, a.lse, a.nq, a.nkv, a.seq, a.ld, a.out_rows,
                       a.kph, a.scale_log2);
  } else {
    hipLaunchKernelGGL((k_attn_fwd<T, T, D, false>), grid, dim3(256), 0, st, (const T*)a.q, (const T*)a.k,
                       (const T*)a.v, a.row_ptr, a.col_idx, (T*)a.o, a.lse, a.nq, a.nkv, a.seq, a.ld, a.out_rows,
                       a.kph, a.scale_log2);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t st) {
  if (a.bf16) return a.d == 128 ? launch_fwd_t<bf16, 128>(a, st) : launch_fwd_t<bf16, 64>(a, st);
  return a.d == 128 ? launch_fwd_t<float, 128>(a, st) : launch_fwd_t<float, 64>(a, st);
}

}  // namespace vsa2
