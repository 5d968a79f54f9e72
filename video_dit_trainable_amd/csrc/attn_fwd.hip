// Block-sparse flash attention forward: the fine branch of VSA2 (paper §2.2
// Eq.(12), the -inf block mask of §2.1 applied by skipping unselected tiles).
// The same kernel in "dense" mode runs the coarse branch's attention over the
// nb pooled cube tokens (Eq.(2)-(3)), with a ragged last tile.
//
// Work split: one block (2 waves) per query cube; each wave owns 32 queries as
// MFMA B fragments in registers, so every K/V byte read from LDS feeds two
// 16-query MFMA blocks.  The selected K cubes and the pre-transposed V cubes
// are gathered through the CSR list into chunk-swizzled LDS tiles; the next
// cube's loads are in flight (in registers) while the current one is
// computed.  S^T = K Q^T leaves, per lane, 4 keys of one query per 16-key
// block, so the online softmax is lane-local apart from a 4-lane max, and the
// exponentials feed O^T += V^T P^T straight from the accumulators.  The O
// rescale is lazy: the running max is only moved when a tile exceeds it by
// more than 2^8, which keeps every exponential <= 256 and the result exact.
//
// V is read as V^T: a pre-pass writes each 64-token cube of V transposed to
// [d][64] with the tokens of every 32-token half reordered to the MFMA
// k-slot order pi(g, e) = 4g + e (e < 4), 16 + 4g + e - 4 (e >= 4), so one
// 16-byte LDS read yields a whole A fragment.
#include <cmath>

#include "common.h"
#include "launch.h"

namespace vsa2 {

// V [bh][rows][D] -> VT [bh][rows/64][D][64] (k-slot order inside each 32-token half).
template <typename T, int D>
__global__ __launch_bounds__(256) void k_vt_perm(const T* __restrict__ v, T* __restrict__ vt, int tiles) {
  __shared__ T s[64][D + 8];
  const int t = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const T* src = v + ((size_t)bh * tiles + t) * 64 * D;
  for (int u = tid; u < 64 * D / 8; u += 256) {
    const int r = u / (D / 8), c8 = u % (D / 8);
    store8(&s[r][8 * c8], load8(src + (size_t)r * D + 8 * c8));
  }
  __syncthreads();
  T* dst = vt + ((size_t)bh * tiles + t) * 64 * D;
  for (int u = tid; u < D * 8; u += 256) {      // output chunk: row d, 8 positions 8u'..8u'+7
    const int d = u / 8, p0 = 8 * (u % 8);
    const int half = p0 >> 5, g = (p0 >> 3) & 3;
    Vec8<T> o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o.v[e] = s[32 * half + (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4)][d];
    store8(dst + (size_t)d * 64 + p0, o);
  }
}

template <typename T, typename TO, int D, bool DENSE>
__global__ __launch_bounds__(128, 2) void k_attn_fwd(const T* __restrict__ q, const T* __restrict__ k,
                                                  const T* __restrict__ vt, const int32_t* __restrict__ row_ptr,
                                                  const int32_t* __restrict__ col_idx, TO* __restrict__ o,
                                                  float* __restrict__ lse, int nq, int nkv, int seq, int ld,
                                                  int out_rows, int64_t kph, float c, int ct, int cy, int cx) {
  __shared__ __align__(16) T ks[64 * D];
  __shared__ __align__(16) T vs[D * 64];
  int bh, i;
  if (!xcd_work(blockIdx.x, nq, bh, i)) return;
  if (ct > 0) i = blocked_cube(i, ct, cy, cx);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, cc = lane & 15;
  const size_t hoff = (size_t)bh * ld * D;
  const T* kbase = k + hoff;
  const T* vbase = vt + hoff;

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

  Frag<T> qf[2][D / 32];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qf[qb][s] = frag_global<T, D>(q + hoff, i * 64 + 32 * w + 16 * qb + cc, s, g);

  f32x4 oacc[D / 16][2];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) oacc[db][0] = oacc[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

  if (cnt > 0) {
    SwRegs<64, D, T, 128> kr;
    SwRegs<D, 64, T, 128> vr;
    int j = cube_at(0);
    sw_load(kr, kbase + (size_t)max(j, 0) * 64 * D, tid);
    sw_load(vr, vbase + (size_t)max(j, 0) * 64 * D, tid);
    for (int n = 0; n < cnt; ++n) {
      sw_store(kr, ks, tid);
      sw_store(vr, vs, tid);
      __syncthreads();
      const int lim = kv_limit(j);
      if (n + 1 < cnt) {
        j = cube_at(n + 1);
        sw_load(kr, kbase + (size_t)max(j, 0) * 64 * D, tid);
        sw_load(vr, vbase + (size_t)max(j, 0) * 64 * D, tid);
      }
      // S^T = K Q^T: acc[kb][qb] holds keys 16kb + 4g + r of query 16qb + cc (of this wave)
      f32x4 acc[4][2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const Frag<T> a = sw_frag<T, D>(ks, 16 * kb + cc, 0, g);
        acc[kb][0] = mma0(a, qf[0][0]);
        acc[kb][1] = mma0(a, qf[1][0]);
      }
#pragma unroll
      for (int s = 1; s < D / 32; ++s)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const Frag<T> a = sw_frag<T, D>(ks, 16 * kb + cc, s, g);
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
          const Frag<T> a = sw_frag<T, 64>(vs, 16 * db + cc, h, g);
          mma(oacc[db][0], a, pf[0][h]);
          mma(oacc[db][1], a, pf[1][h]);
        }
      __syncthreads();
    }
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = i * 64 + 32 * w + 16 * qb + cc;
    const float lt = group_sum(l[qb]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const bool live = DENSE ? (qrow < seq && qrow < out_rows) : (qrow < out_rows);
    if (live) {
      TO* orow = o + ((size_t)bh * out_rows + qrow) * D;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        Vec4<TO> r4;
#pragma unroll
        for (int r = 0; r < 4; ++r) r4.v[r] = from_f32<TO>(oacc[db][qb][r] * inv);
        store4(orow + 16 * db + 4 * g, r4);
      }
      if (g == 0) lse[(size_t)bh * out_rows + qrow] = lt > 0.f ? (m[qb] * c + __log2f(lt)) * LN2 : -INFINITY;
    }
  }
}

template <typename T, int D>
hipError_t launch_fwd_t(const AttnArgs& a, hipStream_t st) {
  const int tiles = a.ld / 64;
  hipLaunchKernelGGL((k_vt_perm<T, D>), dim3(tiles, a.bh), dim3(256), 0, st, (const T*)a.v, (T*)a.vt, tiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid(xcd_grid(a.nq, a.bh));
  if (a.dense) {
    hipLaunchKernelGGL((k_attn_fwd<T, float, D, true>), grid, dim3(128), 0, st, (const T*)a.q, (const T*)a.k,
                       (const T*)a.vt, nullptr, nullptr, (float*)a.o, a.lse, a.nq, a.nkv, a.seq, a.ld, a.out_rows,
                       a.kph, a.scale_log2, 0, 0, 0);
  } else {
    timer_before(TK_FINE_FWD, st);
    hipLaunchKernelGGL((k_attn_fwd<T, T, D, false>), grid, dim3(128), 0, st, (const T*)a.q, (const T*)a.k,
                       (const T*)a.vt, a.row_ptr, a.col_idx, (T*)a.o, a.lse, a.nq, a.nkv, a.seq, a.ld, a.out_rows,
                       a.kph, a.scale_log2, a.ct, a.cy, a.cx);
    timer_after(TK_FINE_FWD, st);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t st) {
  if (a.bf16) return a.d == 128 ? launch_fwd_t<bf16, 128>(a, st) : launch_fwd_t<bf16, 64>(a, st);
  return a.d == 128 ? launch_fwd_t<float, 128>(a, st) : launch_fwd_t<float, 64>(a, st);
}

}  // namespace vsa2
