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
// delta = rowsum(dO * O) comes from k_bwd_delta.  Per-cube gradient rows
// (the coarse branch's dQ_c, dK_c, dV_c) are added as row/64 to every token of
// the cube before the single rounding to the storage type.
#include <cmath>

#include "common.h"
#include "launch.h"

namespace vsa2 {

template <typename T, int D>
__global__ __launch_bounds__(256) void k_bwd_delta(const T* __restrict__ o, const T* __restrict__ d_o,
                                                   float* __restrict__ delta, size_t rows) {
  constexpr int LPT = D / 8;  // lanes per row
  const size_t row = ((size_t)blockIdx.x * 256 + threadIdx.x) / LPT;
  const int part = threadIdx.x % LPT;
  float s = 0.f;
  if (row < rows) {
    Vec8<T> a = load8(o + row * D + 8 * part);
    Vec8<T> b = load8(d_o + row * D + 8 * part);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += to_f32(a.v[e]) * to_f32(b.v[e]);
  }
#pragma unroll
  for (int x = 1; x < LPT; x <<= 1) s += __shfl_xor(s, x);
  if (row < rows && part == 0) delta[row] = s;
}

template <typename T, typename TO, int D, bool DENSE>
__global__ __launch_bounds__(128) void k_bwd_dkdv(const T* __restrict__ q, const T* __restrict__ k,
                                                  const T* __restrict__ v, const T* __restrict__ d_o,
                                                  const float* __restrict__ lse, const float* __restrict__ delta,
                                                  const int32_t* __restrict__ col_ptr,
                                                  const int32_t* __restrict__ row_idx,
                                                  const float* __restrict__ dk_add, const float* __restrict__ dv_add,
                                                  TO* __restrict__ dk, TO* __restrict__ dv, int nq, int nkv, int seq,
                                                  int ld, int out_rows, int lse_rows, int64_t kph, float scale,
                                                  float c, int ct, int cy, int cx) {
  __shared__ __align__(16) T qs[64 * D];
  __shared__ __align__(16) T dos[64 * D];
  __shared__ float lse_s[64], del_s[64];
  int bh, j;
  if (!xcd_work(blockIdx.x, nkv, bh, j)) return;
  if (ct > 0) j = blocked_cube(j, ct, cy, cx);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, cc = lane & 15;
  const size_t hoff = (size_t)bh * ld * D;

  int cnt;
  const int32_t* rows = nullptr;
  if constexpr (DENSE) {
    cnt = nq;
  } else {
    const int32_t* cp = col_ptr + (size_t)bh * (nkv + 1);
    const int64_t start = min<int64_t>(max(cp[j], 0), kph);
    const int64_t end = min<int64_t>(max<int64_t>(cp[j + 1], start), kph);
    cnt = (int)(end - start);
    rows = row_idx + (size_t)bh * kph + start;
  }
  // query cube of list entry n (-1 = corrupt entry, masked tile) and its valid rows
  auto cube_at = [&](int n) -> int {
    if constexpr (DENSE) return n;
    const int ii = rows[n];
    return (unsigned)ii < (unsigned)nq ? ii : -1;
  };
  auto q_limit = [&](int ii) -> int {
    if constexpr (DENSE) return min(64, seq - ii * 64);
    return ii >= 0 ? 64 : 0;
  };

  // K, V rows of this wave as B fragments: key 32w + 16kb + cc
  Frag<T> kf[2][D / 32], vf[2][D / 32];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      kf[kb][s] = frag_global<T, D>(k + hoff, j * 64 + 32 * w + 16 * kb + cc, s, g);
      vf[kb][s] = frag_global<T, D>(v + hoff, j * 64 + 32 * w + 16 * kb + cc, s, g);
    }
  bool kv_ok[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) kv_ok[kb] = !DENSE || (j * 64 + 32 * w + 16 * kb + cc < seq);

  f32x4 dka[D / 16][2], dva[D / 16][2];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    dka[db][0] = dka[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    dva[db][0] = dva[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  if (cnt > 0) {
    SwRegs<64, D, T, 128> qr, dr;
    float lse_n = 0.f, del_n = 0.f;
    auto fetch = [&](int n) {
      const int ii = cube_at(n);
      const int valid = q_limit(ii);
      sw_load(qr, q + hoff + (size_t)max(ii, 0) * 64 * D, tid);
      sw_load(dr, d_o + hoff + (size_t)max(ii, 0) * 64 * D, tid);
      if (tid < 64) {
        const bool ok = tid < valid;
        const size_t t = (size_t)max(ii, 0) * 64 + tid;
        lse_n = ok ? lse[(size_t)bh * lse_rows + t] * LOG2E : INFINITY;
        del_n = ok ? delta[(size_t)bh * ld + t] : 0.f;
      }
    };
    fetch(0);
    for (int n = 0; n < cnt; ++n) {
      sw_store(qr, qs, tid);
      sw_store(dr, dos, tid);
      if (tid < 64) {
        lse_s[tid] = lse_n;
        del_s[tid] = del_n;
      }
      __syncthreads();
      if (n + 1 < cnt) fetch(n + 1);

      // S[q][kv]: p[qb][kb] holds queries 16qb + 4g + r against key 32w + 16kb + cc
      f32x4 p[4][2];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const Frag<T> a = sw_frag<T, D>(qs, 16 * qb + cc, 0, g);
        p[qb][0] = mma0(a, kf[0][0]);
        p[qb][1] = mma0(a, kf[1][0]);
      }
#pragma unroll
      for (int s = 1; s < D / 32; ++s)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
          const Frag<T> a = sw_frag<T, D>(qs, 16 * qb + cc, s, g);
          mma(p[qb][0], a, kf[0][s]);
          mma(p[qb][1], a, kf[1][s]);
        }
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float l2 = lse_s[16 * qb + 4 * g + r];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const float pe = fast_exp2(fmaf(p[qb][kb][r], c, -l2));
            p[qb][kb][r] = kv_ok[kb] ? pe : 0.f;
          }
        }
      // dV^T += dO^T P
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const Frag<T> f0 = frag_from_acc<T>(p[2 * h][0], p[2 * h + 1][0]);
        const Frag<T> f1 = frag_from_acc<T>(p[2 * h][1], p[2 * h + 1][1]);
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
          const Frag<T> a = sw_frag_tr<T, D>(dos, 32 * h, 16 * db, g, cc);
          mma(dva[db][0], a, f0);
          mma(dva[db][1], a, f1);
        }
      }
      // dP = dO V^T, dS = P (dP - delta)
      f32x4 dp[4][2];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const Frag<T> a = sw_frag<T, D>(dos, 16 * qb + cc, 0, g);
        dp[qb][0] = mma0(a, vf[0][0]);
        dp[qb][1] = mma0(a, vf[1][0]);
      }
#pragma unroll
      for (int s = 1; s < D / 32; ++s)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
          const Frag<T> a = sw_frag<T, D>(dos, 16 * qb + cc, s, g);
          mma(dp[qb][0], a, vf[0][s]);
          mma(dp[qb][1], a, vf[1][s]);
        }
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float dl = del_s[16 * qb + 4 * g + r];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) dp[qb][kb][r] = p[qb][kb][r] * (dp[qb][kb][r] - dl);
        }
      // dK^T += Q^T dS
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const Frag<T> f0 = frag_from_acc<T>(dp[2 * h][0], dp[2 * h + 1][0]);
        const Frag<T> f1 = frag_from_acc<T>(dp[2 * h][1], dp[2 * h + 1][1]);
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
          const Frag<T> a = sw_frag_tr<T, D>(qs, 32 * h, 16 * db, g, cc);
          mma(dka[db][0], a, f0);
          mma(dka[db][1], a, f1);
        }
      }
      __syncthreads();
    }
  }

#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int kvrow = j * 64 + 32 * w + 16 * kb + cc;
    const bool live = DENSE ? (kvrow < seq && kvrow < out_rows) : (kvrow < out_rows);
    if (!live) continue;
    TO* krow = dk + ((size_t)bh * out_rows + kvrow) * D;
    TO* vrow = dv + ((size_t)bh * out_rows + kvrow) * D;
    const float* ka = dk_add ? dk_add + ((size_t)bh * nkv + j) * D : nullptr;
    const float* va = dv_add ? dv_add + ((size_t)bh * nkv + j) * D : nullptr;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      Vec4<TO> a4, b4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = 16 * db + 4 * g + r;
        a4.v[r] = from_f32<TO>(dka[db][kb][r] * scale + (ka ? ka[d] * (1.0f / 64.0f) : 0.f));
        b4.v[r] = from_f32<TO>(dva[db][kb][r] + (va ? va[d] * (1.0f / 64.0f) : 0.f));
      }
      store4(krow + 16 * db + 4 * g, a4);
      store4(vrow + 16 * db + 4 * g, b4);
    }
  }
}

template <typename T, typename TO, int D, bool DENSE>
__global__ __launch_bounds__(128) void k_bwd_dq(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, const T* __restrict__ d_o,
                                                   const float* __restrict__ lse, const float* __restrict__ delta,
                                                   const int32_t* __restrict__ row_ptr,
                                                   const int32_t* __restrict__ col_idx,
                                                   const float* __restrict__ dq_add, TO* __restrict__ dq, int nq,
                                                   int nkv, int seq, int ld, int out_rows, int lse_rows, int64_t kph,
                                                   float scale, float c, int ct, int cy, int cx) {
  __shared__ __align__(16) T ks[64 * D];
  __shared__ __align__(16) T vs[64 * D];
  __shared__ __align__(16) T dos[64 * D];
  int bh, i;
  if (!xcd_work(blockIdx.x, nq, bh, i)) return;
  if (ct > 0) i = blocked_cube(i, ct, cy, cx);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, cc = lane & 15;
  const size_t hoff = (size_t)bh * ld * D;

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
  auto cube_at = [&](int n) -> int {
    if constexpr (DENSE) return n;
    const int jj = cols[n];
    return (unsigned)jj < (unsigned)nkv ? jj : -1;
  };
  auto kv_limit = [&](int jj) -> int {
    if constexpr (DENSE) return min(64, seq - jj * 64);
    return jj >= 0 ? 64 : 0;
  };

  // this cube's dO tile (B fragments of dP^T = V dO^T come from LDS)
  {
    SwRegs<64, D, T, 128> r;
    sw_load(r, d_o + hoff + (size_t)i * 64 * D, tid);
    sw_store(r, dos, tid);
  }
  Frag<T> qf[2][D / 32];
  float lse2[2], del[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = i * 64 + 32 * w + 16 * qb + cc;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qf[qb][s] = frag_global<T, D>(q + hoff, qrow, s, g);
    const bool ok = !DENSE || qrow < seq;
    lse2[qb] = ok ? lse[(size_t)bh * lse_rows + qrow] * LOG2E : INFINITY;
    del[qb] = ok ? delta[(size_t)bh * ld + qrow] : 0.f;
  }
  f32x4 dqa[D / 16][2];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) dqa[db][0] = dqa[db][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (cnt > 0) {
    SwRegs<64, D, T, 128> kr, vr;
    int j = cube_at(0);
    sw_load(kr, k + hoff + (size_t)max(j, 0) * 64 * D, tid);
    sw_load(vr, v + hoff + (size_t)max(j, 0) * 64 * D, tid);
    for (int n = 0; n < cnt; ++n) {
      sw_store(kr, ks, tid);
      sw_store(vr, vs, tid);
      __syncthreads();
      const int lim = kv_limit(j);
      if (n + 1 < cnt) {
        j = cube_at(n + 1);
        sw_load(kr, k + hoff + (size_t)max(j, 0) * 64 * D, tid);
        sw_load(vr, v + hoff + (size_t)max(j, 0) * 64 * D, tid);
      }
      f32x4 p[4][2], dp[4][2];
      {
        const Frag<T> o0 = sw_frag<T, D>(dos, 32 * w + cc, 0, g);
        const Frag<T> o1 = sw_frag<T, D>(dos, 32 * w + 16 + cc, 0, g);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const Frag<T> a = sw_frag<T, D>(ks, 16 * kb + cc, 0, g);
          p[kb][0] = mma0(a, qf[0][0]);
          p[kb][1] = mma0(a, qf[1][0]);
          const Frag<T> b = sw_frag<T, D>(vs, 16 * kb + cc, 0, g);
          dp[kb][0] = mma0(b, o0);
          dp[kb][1] = mma0(b, o1);
        }
      }
#pragma unroll
      for (int s = 1; s < D / 32; ++s) {
        const Frag<T> o0 = sw_frag<T, D>(dos, 32 * w + cc, s, g);
        const Frag<T> o1 = sw_frag<T, D>(dos, 32 * w + 16 + cc, s, g);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const Frag<T> a = sw_frag<T, D>(ks, 16 * kb + cc, s, g);
          mma(p[kb][0], a, qf[0][s]);
          mma(p[kb][1], a, qf[1][s]);
          const Frag<T> b = sw_frag<T, D>(vs, 16 * kb + cc, s, g);
          mma(dp[kb][0], b, o0);
          mma(dp[kb][1], b, o1);
        }
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool kin = 16 * kb + 4 * g + r < lim;
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const float pe = kin ? fast_exp2(fmaf(p[kb][qb][r], c, -lse2[qb])) : 0.f;
            dp[kb][qb][r] = pe * (dp[kb][qb][r] - del[qb]);
          }
        }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const Frag<T> f0 = frag_from_acc<T>(dp[2 * h][0], dp[2 * h + 1][0]);
        const Frag<T> f1 = frag_from_acc<T>(dp[2 * h][1], dp[2 * h + 1][1]);
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
          const Frag<T> a = sw_frag_tr<T, D>(ks, 32 * h, 16 * db, g, cc);
          mma(dqa[db][0], a, f0);
          mma(dqa[db][1], a, f1);
        }
      }
      __syncthreads();
    }
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = i * 64 + 32 * w + 16 * qb + cc;
    const bool live = DENSE ? (qrow < seq && qrow < out_rows) : (qrow < out_rows);
    if (!live) continue;
    TO* dst = dq + ((size_t)bh * out_rows + qrow) * D;
    const float* qa = dq_add ? dq_add + ((size_t)bh * nq + i) * D : nullptr;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      Vec4<TO> a4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = 16 * db + 4 * g + r;
        a4.v[r] = from_f32<TO>(dqa[db][qb][r] * scale + (qa ? qa[d] * (1.0f / 64.0f) : 0.f));
      }
      store4(dst + 16 * db + 4 * g, a4);
    }
  }
}

template <typename T, int D>
hipError_t launch_delta_t(const AttnBwdArgs& a, float* delta, hipStream_t st) {
  const size_t rows = (size_t)a.bh * a.ld;
  const size_t threads = rows * (D / 8);
  hipLaunchKernelGGL((k_bwd_delta<T, D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, (const T*)a.o,
                     (const T*)a.d_o, delta, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_delta(const AttnBwdArgs& a, float* delta, hipStream_t st) {
  if (a.bf16) return a.d == 128 ? launch_delta_t<bf16, 128>(a, delta, st) : launch_delta_t<bf16, 64>(a, delta, st);
  return a.d == 128 ? launch_delta_t<float, 128>(a, delta, st) : launch_delta_t<float, 64>(a, delta, st);
}

template <typename T, typename TO, int D, bool DENSE>
hipError_t launch_bwd_tt(const AttnBwdArgs& a, hipStream_t st) {
  if (!DENSE) timer_before(TK_BWD_DKDV, st);
  hipLaunchKernelGGL((k_bwd_dkdv<T, TO, D, DENSE>), dim3(xcd_grid(a.nkv, a.bh)), dim3(128), 0, st, (const T*)a.q,
                     (const T*)a.k, (const T*)a.v, (const T*)a.d_o, a.lse, a.delta, a.col_ptr, a.row_idx, a.dk_add,
                     a.dv_add, (TO*)a.dk, (TO*)a.dv, a.nq, a.nkv, a.seq, a.ld, a.out_rows, a.lse_rows, a.kph, a.scale,
                     a.scale_log2, 0, 0, 0);
  if (!DENSE) timer_after(TK_BWD_DKDV, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!DENSE) timer_before(TK_BWD_DQ, st);
  hipLaunchKernelGGL((k_bwd_dq<T, TO, D, DENSE>), dim3(xcd_grid(a.nq, a.bh)), dim3(128), 0, st, (const T*)a.q,
                     (const T*)a.k, (const T*)a.v, (const T*)a.d_o, a.lse, a.delta, a.row_ptr, a.col_idx, a.dq_add,
                     (TO*)a.dq, a.nq, a.nkv, a.seq, a.ld, a.out_rows, a.lse_rows, a.kph, a.scale, a.scale_log2, a.ct,
                     a.cy, a.cx);
  if (!DENSE) timer_after(TK_BWD_DQ, st);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_t(const AttnBwdArgs& a, hipStream_t st) {
  return a.dense ? launch_bwd_tt<T, float, D, true>(a, st) : launch_bwd_tt<T, T, D, false>(a, st);
}

hipError_t launch_attn_bwd(const AttnBwdArgs& a, hipStream_t st) {
  if (a.bf16) return a.d == 128 ? launch_bwd_t<bf16, 128>(a, st) : launch_bwd_t<bf16, 64>(a, st);
  return a.d == 128 ? launch_bwd_t<float, 128>(a, st) : launch_bwd_t<float, 64>(a, st);
}

}  // namespace vsa2
