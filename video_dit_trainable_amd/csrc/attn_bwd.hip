// Backward of the block-sparse attention with the selection held fixed (the
// router takes no gradient: paper §2.1-§2.2).  Dense mode serves the coarse
// branch's attention over the pooled cube tokens.
//
// Deterministic by construction -- every output row is owned by one block:
//  * k_bwd_dkdv: one block per KV cube j, looping over the query cubes that
//    selected it (CSC list, ascending).  Per query tile it recomputes
//    S = Q K^T and P = exp(S - LSE), then dV += P^T dO, dP = dO V^T,
//    dS = P (dP - delta), dK += dS^T Q.  K and V stay in registers.
//  * k_bwd_dq: one block per query cube i over its KV list (CSR):
//    S^T, P^T, dP^T = V dO^T, dS^T, dQ += dS K.
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
__global__ __launch_bounds__(256) void k_bwd_dkdv(const T* __restrict__ q, const T* __restrict__ k,
                                                  const T* __restrict__ v, const T* __restrict__ d_o,
                                                  const float* __restrict__ lse, const float* __restrict__ delta,
                                                  const int32_t* __restrict__ col_ptr,
                                                  const int32_t* __restrict__ row_idx,
                                                  const float* __restrict__ dk_add, const float* __restrict__ dv_add,
                                                  TO* __restrict__ dk, TO* __restrict__ dv, int nq, int nkv, int seq,
                                                  int ld, int out_rows, int lse_rows, int64_t kph, float scale,
                                                  float c) {
  using G = TileGeom<T, D>;
  __shared__ T qs[G::RM_ELEMS];
  __shared__ T qt[G::TR_ELEMS];
  __shared__ T ds_[G::RM_ELEMS];
  __shared__ T dt[G::TR_ELEMS];
  __shared__ float lse_s[64], del_s[64];
  int bh, j;
  if (!xcd_work(blockIdx.x, nkv, bh, j)) return;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, cc = lane & 15;
  const int kvrow = j * 64 + 16 * w + cc;
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

  Frag<T> kf[D / 32], vf[D / 32];
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    kf[s] = frag_global<T, D>(k + hoff, kvrow, s, g);
    vf[s] = frag_global<T, D>(v + hoff, kvrow, s, g);
  }
  const bool kv_ok = !DENSE || kvrow < seq;

  f32x4 dka[D / 16], dva[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    dka[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    dva[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  if (cnt > 0) {
    TileRegs<T, D, 256> qr, dr;
    float lse_n = 0.f, del_n = 0.f;
    auto fetch = [&](int n) {
      int i = DENSE ? n : rows[n];
      if (!DENSE && (unsigned)i >= (unsigned)nq) i = -1;   // corrupt list entry: masked tile
      const int valid = DENSE ? min(64, seq - i * 64) : (i >= 0 ? 64 : 0);
      tile_load<T, D, 256>(qr, q + hoff + (size_t)max(i, 0) * 64 * D, tid, valid);
      tile_load<T, D, 256>(dr, d_o + hoff + (size_t)max(i, 0) * 64 * D, tid, valid);
      if (tid < 64) {
        const int t = max(i, 0) * 64 + tid;
        const bool ok = i >= 0 && (!DENSE || t < seq);
        lse_n = ok ? lse[(size_t)bh * lse_rows + t] * LOG2E : INFINITY;
        del_n = ok ? delta[(size_t)bh * ld + t] : 0.f;
      }
    };
    fetch(0);
    for (int n = 0; n < cnt; ++n) {
      tile_store_rm<T, D, 256>(qr, qs, tid);
      tile_store_tr<T, D, 256>(qr, qt, tid);
      tile_store_rm<T, D, 256>(dr, ds_, tid);
      tile_store_tr<T, D, 256>(dr, dt, tid);
      if (tid < 64) {
        lse_s[tid] = lse_n;
        del_s[tid] = del_n;
      }
      __syncthreads();
      if (n + 1 < cnt) fetch(n + 1);

      // S[q][kv] and P, accumulator rows = queries 16qb + 4g + r, column = kv
      f32x4 p[4];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) p[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / 32; ++s)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) mma(p[qb], frag_rm<T, D>(qs, 16 * qb + cc, s, g), kf[s]);
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pe = fast_exp2(fmaf(p[qb][r], c, -lse_s[16 * qb + 4 * g + r]));
          p[qb][r] = kv_ok ? pe : 0.f;
        }
      // dV^T += dO^T P
      {
        const Frag<T> f0 = frag_from_acc<T>(p[0], p[1]);
        const Frag<T> f1 = frag_from_acc<T>(p[2], p[3]);
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
          mma(dva[db], frag_tr<T, D>(dt, 16 * db + cc, 0, g), f0);
          mma(dva[db], frag_tr<T, D>(dt, 16 * db + cc, 1, g), f1);
        }
      }
      // dP = dO V^T, dS = P (dP - delta)
      f32x4 dp[4];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) dp[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / 32; ++s)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) mma(dp[qb], frag_rm<T, D>(ds_, 16 * qb + cc, s, g), vf[s]);
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) dp[qb][r] = p[qb][r] * (dp[qb][r] - del_s[16 * qb + 4 * g + r]);
      // dK^T += Q^T dS
      {
        const Frag<T> f0 = frag_from_acc<T>(dp[0], dp[1]);
        const Frag<T> f1 = frag_from_acc<T>(dp[2], dp[3]);
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
          mma(dka[db], frag_tr<T, D>(qt, 16 * db + cc, 0, g), f0);
          mma(dka[db], frag_tr<T, D>(qt, 16 * db + cc, 1, g), f1);
        }
      }
      __syncthreads();
    }
  }

  const bool live = DENSE ? (kvrow < seq && kvrow < out_rows) : (kvrow < out_rows);
  if (live) {
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
        a4.v[r] = from_f32<TO>(dka[db][r] * scale + (ka ? ka[d] * (1.0f / 64.0f) : 0.f));
        b4.v[r] = from_f32<TO>(dva[db][r] + (va ? va[d] * (1.0f / 64.0f) : 0.f));
      }
      store4(krow + 16 * db + 4 * g, a4);
      store4(vrow + 16 * db + 4 * g, b4);
    }
  }
}

template <typename T, typename TO, int D, bool DENSE>
__global__ __launch_bounds__(256) void k_bwd_dq(const T* __restrict__ q, const T* __restrict__ k,
                                                const T* __restrict__ v, const T* __restrict__ d_o,
                                                const float* __restrict__ lse, const float* __restrict__ delta,
                                                const int32_t* __restrict__ row_ptr,
                                                const int32_t* __restrict__ col_idx,
                                                const float* __restrict__ dq_add, TO* __restrict__ dq, int nq, int nkv,
                                                int seq, int ld, int out_rows, int lse_rows, int64_t kph,
                                                float scale, float c) {
  using G = TileGeom<T, D>;
  __shared__ T ks[G::RM_ELEMS];
  __shared__ T kt[G::TR_ELEMS];
  __shared__ T vs[G::RM_ELEMS];
  int bh, i;
  if (!xcd_work(blockIdx.x, nq, bh, i)) return;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, cc = lane & 15;
  const int qrow = i * 64 + 16 * w + cc;
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

  const bool q_ok = !DENSE || qrow < seq;
  const float lse2 = q_ok ? lse[(size_t)bh * lse_rows + qrow] * LOG2E : INFINITY;
  const float del = q_ok ? delta[(size_t)bh * ld + qrow] : 0.f;

  Frag<T> qf[D / 32], of[D / 32];
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    qf[s] = frag_global<T, D>(q + hoff, qrow, s, g);
    of[s] = frag_global<T, D>(d_o + hoff, qrow, s, g);
  }
  f32x4 dqa[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) dqa[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (cnt > 0) {
    TileRegs<T, D, 256> kr, vr;
    int j = cube_at(0);
    auto fetch = [&](int jj) {
      tile_load<T, D, 256>(kr, k + hoff + (size_t)max(jj, 0) * 64 * D, tid, kv_limit(jj));
      tile_load<T, D, 256>(vr, v + hoff + (size_t)max(jj, 0) * 64 * D, tid, kv_limit(jj));
    };
    fetch(j);
    for (int n = 0; n < cnt; ++n) {
      tile_store_rm<T, D, 256>(kr, ks, tid);
      tile_store_tr<T, D, 256>(kr, kt, tid);
      tile_store_rm<T, D, 256>(vr, vs, tid);
      __syncthreads();
      const int jcur = j;
      if (n + 1 < cnt) {
        j = cube_at(n + 1);
        fetch(j);
      }
      const int lim = kv_limit(jcur);
      f32x4 p[4], dp[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        p[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int s = 0; s < D / 32; ++s)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          mma(p[kb], frag_rm<T, D>(ks, 16 * kb + cc, s, g), qf[s]);
          mma(dp[kb], frag_rm<T, D>(vs, 16 * kb + cc, s, g), of[s]);
        }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float pe = fast_exp2(fmaf(p[kb][r], c, -lse2));
          if (16 * kb + 4 * g + r >= lim) pe = 0.f;
          dp[kb][r] = pe * (dp[kb][r] - del);
        }
      const Frag<T> f0 = frag_from_acc<T>(dp[0], dp[1]);
      const Frag<T> f1 = frag_from_acc<T>(dp[2], dp[3]);
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        mma(dqa[db], frag_tr<T, D>(kt, 16 * db + cc, 0, g), f0);
        mma(dqa[db], frag_tr<T, D>(kt, 16 * db + cc, 1, g), f1);
      }
      __syncthreads();
    }
  }

  const bool live = DENSE ? (qrow < seq && qrow < out_rows) : (qrow < out_rows);
  if (live) {
    TO* qrow_p = dq + ((size_t)bh * out_rows + qrow) * D;
    const float* qa = dq_add ? dq_add + ((size_t)bh * nq + i) * D : nullptr;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      Vec4<TO> a4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = 16 * db + 4 * g + r;
        a4.v[r] = from_f32<TO>(dqa[db][r] * scale + (qa ? qa[d] * (1.0f / 64.0f) : 0.f));
      }
      store4(qrow_p + 16 * db + 4 * g, a4);
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
  hipLaunchKernelGGL((k_bwd_dkdv<T, TO, D, DENSE>), dim3(xcd_grid(a.nkv, a.bh)), dim3(256), 0, st, (const T*)a.q,
                     (const T*)a.k, (const T*)a.v, (const T*)a.d_o, a.lse, a.delta, a.col_ptr, a.row_idx, a.dk_add,
                     a.dv_add, (TO*)a.dk, (TO*)a.dv, a.nq, a.nkv, a.seq, a.ld, a.out_rows, a.lse_rows, a.kph, a.scale,
                     a.scale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_bwd_dq<T, TO, D, DENSE>), dim3(xcd_grid(a.nq, a.bh)), dim3(256), 0, st, (const T*)a.q,
                     (const T*)a.k, (const T*)a.v, (const T*)a.d_o, a.lse, a.delta, a.row_ptr, a.col_idx, a.dq_add,
                     (TO*)a.dq, a.nq, a.nkv, a.seq, a.ld, a.out_rows, a.lse_rows, a.kph, a.scale, a.scale_log2);
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
