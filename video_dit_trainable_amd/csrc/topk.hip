// Per-sequence TopK of VSA2 (paper §2.2 Eq.(8)-(9)): for each (batch, head)
// keep the k = nb*K largest of the nb*nb block scores; each query cube then
// holds a variable number of KV cubes.
//
// Exact selection without sorting.  Non-negative fp32 values order like their
// uint32 bit patterns, so the k-th largest pattern tau is found by a 3-pass
// radix select (digits of 12, 12 and 8 bits; per-head histograms with integer
// atomics, whose totals do not depend on ordering).  Then every row counts
// its entries > tau and == tau, a per-head scan hands the ties at tau to the
// lowest flat indices, and each row is compacted in ascending column order
// (wave ballots), which also records a selection bitmap and column counts.
// The CSC form is built from the bitmap with no atomics: 4 waves split the
// rows of a 64-column strip, count, offset by an exclusive scan, and write.
#include <cmath>

#include "common.h"
#include "launch.h"

namespace vsa2 {

__device__ __forceinline__ uint32_t score_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? 0u : u;  // scores are >= 0; -0.0 ranks as +0.0
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (lane == 0) ? 0ull : (~0ull >> (64 - lane)); }

__global__ void k_fill_u32(uint32_t* __restrict__ p, uint32_t val, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = val;
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t val, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, st, p, val, n);
  return hipGetLastError();
}

// Histogram of digit (u >> SHIFT) & (2^BITS - 1) over the entries whose bits
// above SHIFT+BITS equal the prefix found by the previous passes.  Each thread
// reads 4 consecutive scores per step (n is a multiple of 4 for every head:
// n = nb^2 is, or the head offset breaks alignment and the scalar path runs).
template <int SHIFT, int BITS>
__global__ __launch_bounds__(256) void k_hist(const float* __restrict__ scores, uint32_t* __restrict__ hist,
                                              const uint32_t* __restrict__ state, size_t n) {
  constexpr int NBIN = 1 << BITS;
  __shared__ uint32_t h[NBIN];
  const int bh = blockIdx.y, tid = threadIdx.x;
  for (int b = tid; b < NBIN; b += 256) h[b] = 0;
  __syncthreads();
  const uint32_t prefix = (SHIFT + BITS < 32) ? state[bh * 4 + 0] : 0u;
  const float* s = scores + (size_t)bh * n;
  auto add = [&](float x) {
    const uint32_t u = score_bits(x);
    bool ok = true;
    if constexpr (SHIFT + BITS < 32) ok = (u >> (SHIFT + BITS)) == (prefix >> (SHIFT + BITS));
    if (ok) atomicAdd(&h[(u >> SHIFT) & (NBIN - 1)], 1u);
  };
  if ((n & 3) == 0) {
    const float4* s4 = reinterpret_cast<const float4*>(s);
    const size_t n4 = n / 4;
    for (size_t i = (size_t)blockIdx.x * 256 + tid; i < n4; i += (size_t)gridDim.x * 256) {
      const float4 v = s4[i];
      add(v.x); add(v.y); add(v.z); add(v.w);
    }
  } else {
    for (size_t i = (size_t)blockIdx.x * 256 + tid; i < n; i += (size_t)gridDim.x * 256) add(s[i]);
  }
  __syncthreads();
  for (int b = tid; b < NBIN; b += 256)
    if (h[b]) atomicAdd(&hist[(size_t)bh * 4096 + b], h[b]);
}

// Pick the digit holding the `need`-th largest remaining entry.
// state = {prefix, need, count strictly above the prefix region, -}.
template <int SHIFT, int BITS>
__global__ __launch_bounds__(256) void k_select(const uint32_t* __restrict__ hist, uint32_t* __restrict__ state,
                                                uint32_t k_first) {
  constexpr int NBIN = 1 << BITS, PER = NBIN / 256;
  __shared__ uint32_t part[256];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const uint32_t* hb = hist + (size_t)bh * 4096;
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) s += hb[tid * PER + i];
  part[tid] = s;
  __syncthreads();
  if (tid == 0) {
    const bool first = (SHIFT + BITS == 32);
    uint32_t need = first ? k_first : state[bh * 4 + 1];
    uint32_t above = first ? 0u : state[bh * 4 + 2];
    uint32_t prefix = first ? 0u : state[bh * 4 + 0];
    uint32_t acc = 0;
    int t = 255;
    for (; t > 0; --t) {
      if (acc + part[t] >= need) break;
      acc += part[t];
    }
    int b = t * PER + PER - 1;
    for (; b > t * PER; --b) {
      if (acc + hb[b] >= need) break;
      acc += hb[b];
    }
    state[bh * 4 + 0] = prefix | ((uint32_t)b << SHIFT);
    state[bh * 4 + 1] = need - acc;
    state[bh * 4 + 2] = above + acc;
  }
}

// Per row: entries > tau and == tau (one wave per row; 4 columns per lane and
// step when rows are 16-byte aligned, nb % 4 == 0).
__global__ __launch_bounds__(256) void k_rowcount(const float* __restrict__ scores, const uint32_t* __restrict__ state,
                                                  uint32_t* __restrict__ rowcnt, int nb) {
  const int bh = blockIdx.y, row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= nb) return;
  const uint32_t tau = state[bh * 4 + 0];
  const float* s = scores + ((size_t)bh * nb + row) * nb;
  uint32_t gt = 0, eq = 0;
  if ((nb & 3) == 0) {
    for (int j0 = 0; j0 < nb; j0 += 256) {
      const int j = j0 + 4 * lane;
      if (j < nb) {
        const float4 v = *reinterpret_cast<const float4*>(s + j);
        const uint32_t u[4] = {score_bits(v.x), score_bits(v.y), score_bits(v.z), score_bits(v.w)};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gt += u[e] > tau;
          eq += u[e] == tau;
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      gt += __shfl_xor(gt, o);
      eq += __shfl_xor(eq, o);
    }
  } else {
    for (int j0 = 0; j0 < nb; j0 += 64) {
      const int j = j0 + lane;
      const uint32_t u = j < nb ? score_bits(s[j]) : 0u;
      gt += __popcll(__ballot(j < nb && u > tau));
      eq += __popcll(__ballot(j < nb && u == tau));
    }
  }
  if (lane == 0) {
    rowcnt[((size_t)bh * 2 + 0) * nb + row] = gt;
    rowcnt[((size_t)bh * 2 + 1) * nb + row] = eq;
  }
}

// Block-wide exclusive scan of one value per thread (1024 threads); returns
// the exclusive prefix and sets `total`.
// Ties at tau go to the lowest flat indices: row i takes
// clamp(need - (ties in rows < i), 0, ties in row i).  Builds row_ptr.
__global__ __launch_bounds__(1024) void k_rowalloc(const uint32_t* __restrict__ rowcnt,
                                                   const uint32_t* __restrict__ state, uint32_t* __restrict__ take,
                                                   int32_t* __restrict__ row_ptr, int nb) {
  __shared__ uint32_t sh[17];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const uint32_t need = state[bh * 4 + 1];
  const uint32_t* gt = rowcnt + (size_t)bh * 2 * nb;
  const uint32_t* eq = gt + nb;
  uint32_t carry_eq = 0, carry_sel = 0;
  for (int i0 = 0; i0 < nb; i0 += 1024) {
    const int i = i0 + tid;
    const uint32_t e = i < nb ? eq[i] : 0u;
    uint32_t tot;
    const uint32_t before = carry_eq + block_scan_1024(e, tot, sh);
    carry_eq += tot;
    const uint32_t tk = need > before ? min(need - before, e) : 0u;
    const uint32_t sel = i < nb ? gt[i] + tk : 0u;
    const uint32_t pos = carry_sel + block_scan_1024(sel, tot, sh);
    carry_sel += tot;
    if (i < nb) {
      take[(size_t)bh * nb + i] = tk;
      row_ptr[(size_t)bh * (nb + 1) + i] = (int32_t)pos;
    }
  }
  if (tid == 0) row_ptr[(size_t)bh * (nb + 1) + nb] = (int32_t)carry_sel;
}

// Compact each row in ascending column order; with csc, record the bitmap the
// CSC is built from.
__global__ __launch_bounds__(256) void k_compact(const float* __restrict__ scores, const uint32_t* __restrict__ state,
                                                 const uint32_t* __restrict__ take, const int32_t* __restrict__ row_ptr,
                                                 int32_t* __restrict__ col_idx, uint32_t* __restrict__ bitmap,
                                                 int nb, int64_t kph, int words, int csc) {
  const int bh = blockIdx.y, row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= nb) return;
  const uint32_t tau = state[bh * 4 + 0];
  const uint32_t tk = take[(size_t)bh * nb + row];
  const float* s = scores + ((size_t)bh * nb + row) * nb;
  int32_t* out = col_idx + (size_t)bh * kph + row_ptr[(size_t)bh * (nb + 1) + row];
  uint32_t* bm = bitmap + ((size_t)bh * nb + row) * words;
  uint32_t eq_seen = 0, written = 0;
  const uint64_t lt = lanemask_lt(lane);
  const int64_t row0 = row_ptr[(size_t)bh * (nb + 1) + row];
  if ((nb & 3) == 0) {
    // 16-byte rows: lane l reads columns 4l .. 4l + 3 of each 256-column
    // step in one load (the next step's load is issued before this one is
    // ranked).  Ranks in column order: the entries of lower lanes, then the
    // lane's own lower columns.
    float4 cur = make_float4(0.f, 0.f, 0.f, 0.f), nxt = cur;
    if (4 * lane < nb) cur = *reinterpret_cast<const float4*>(s + 4 * lane);
    for (int j1 = 0; j1 < nb; j1 += 256) {
      const int j = j1 + 4 * lane;
      if (j + 256 < nb) nxt = *reinterpret_cast<const float4*>(s + j + 256);
      const bool in = j < nb;  // nb % 4 == 0: all four columns or none
      const uint32_t u[4] = {score_bits(cur.x), score_bits(cur.y), score_bits(cur.z), score_bits(cur.w)};
      bool is_eq[4], sel[4];
      uint64_t eqm[4], selm[4];
      uint32_t eq_lower = 0;  // equal entries of the lower lanes of this step
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        is_eq[e] = in && u[e] == tau;
        eqm[e] = __ballot(is_eq[e]);
        eq_lower += __popcll(eqm[e] & lt);
      }
      uint32_t rank = eq_seen + eq_lower, sel_lower = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sel[e] = in && (u[e] > tau || (is_eq[e] && rank < tk));
        rank += is_eq[e];
        selm[e] = __ballot(sel[e]);
        sel_lower += __popcll(selm[e] & lt);
      }
      uint32_t pos = written + sel_lower;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (sel[e] && row0 + pos < kph) out[pos] = j + e;
        pos += sel[e];
      }
      // bitmap word k of the step (columns j1 + 32k ..) holds lanes 8k .. 8k + 7,
      // four columns each: bit 4i + e is element e of lane 8k + i
      if (csc && lane < 8 && j1 + 64 * (lane >> 1) < nb) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t x = (uint32_t)(selm[e] >> (8 * lane)) & 0xFFu;  // spread bit i to bit 4i
          x = (x | (x << 12)) & 0x000F000Fu;
          x = (x | (x << 6)) & 0x03030303u;
          x = (x | (x << 3)) & 0x11111111u;
          word |= x << e;
        }
        bm[(j1 >> 5) + lane] = word;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        eq_seen += __popcll(eqm[e]);
        written += __popcll(selm[e]);
      }
      cur = nxt;
    }
    return;
  }
  // four 64-column chunks per step, compacted in column order; the next
  // step's four are loaded while this step's are ranked
  uint32_t uu[4], un[4];
  auto load4 = [&](int j1, uint32_t (&d)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = j1 + 64 * q + lane;
      d[q] = j < nb ? score_bits(s[j]) : 0u;
    }
  };
  load4(0, uu);
  for (int j1 = 0; j1 < nb; j1 += 256) {
    if (j1 + 256 < nb) load4(j1 + 256, un);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j0 = j1 + 64 * q;
      if (j0 >= nb) break;
      const int j = j0 + lane;
      const uint32_t u = uu[q];
      const bool is_eq = j < nb && u == tau;
      const uint64_t eqm = __ballot(is_eq);
      const uint32_t rank = eq_seen + __popcll(eqm & lt);
      const bool sel = j < nb && (u > tau || (is_eq && rank < tk));
      const uint64_t selm = __ballot(sel);
      const uint32_t before = __popcll(selm & lt);
      if (sel && row0 + written + before < kph) out[written + before] = j;
      if (csc && lane < 2) bm[(j0 >> 5) + lane] = (uint32_t)(selm >> (32 * lane));
      eq_seen += __popcll(eqm);
      written += __popcll(selm);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) uu[q] = un[q];
  }
}

// Selection given as CSR: bitmap + column counts.  A column that appears
// twice in a row sets its bit once and is counted once, so the column counts
// always match the bitmap the CSC is filled from.
__global__ __launch_bounds__(256) void k_csr_scatter(const int32_t* __restrict__ row_ptr,
                                                     const int32_t* __restrict__ col_idx, uint32_t* __restrict__ bitmap,
                                                     uint32_t* __restrict__ colcnt, int nb, int64_t kph, int words) {
  const int bh = blockIdx.y, row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= nb) return;
  const int32_t* rp = row_ptr + (size_t)bh * (nb + 1);
  const int32_t* ci = col_idx + (size_t)bh * kph;
  const int64_t n0 = min<int64_t>(max(rp[row], 0), kph), n1 = min<int64_t>(max<int64_t>(rp[row + 1], n0), kph);
  for (int64_t n = n0 + lane; n < n1; n += 64) {
    const int j = ci[n];
    if ((unsigned)j >= (unsigned)nb) continue;   // corrupt entry: ignored
    const uint32_t bit = 1u << (j & 31);
    const uint32_t was = atomicOr(&bitmap[((size_t)bh * nb + row) * words + (j >> 5)], bit);
    if (!(was & bit)) atomicAdd(&colcnt[(size_t)bh * nb + j], 1u);
  }
}

__global__ __launch_bounds__(1024) void k_colptr(const uint32_t* __restrict__ colcnt, int32_t* __restrict__ col_ptr,
                                                 int nb) {
  __shared__ uint32_t sh[17];
  const int bh = blockIdx.x, tid = threadIdx.x;
  uint32_t carry = 0;
  for (int i0 = 0; i0 < nb; i0 += 1024) {
    const int i = i0 + tid;
    uint32_t tot;
    const uint32_t pos = carry + block_scan_1024(i < nb ? colcnt[(size_t)bh * nb + i] : 0u, tot, sh);
    carry += tot;
    if (i < nb) col_ptr[(size_t)bh * (nb + 1) + i] = (int32_t)pos;
  }
  if (tid == 0) col_ptr[(size_t)bh * (nb + 1) + nb] = (int32_t)carry;
}

// Column counts of the selection from its bitmap: block = (64-column strip,
// bh), wave w counts rows [w*R, (w+1)*R), lane = column; fixed order, no
// atomics.
__global__ __launch_bounds__(1024) void k_colcount(const uint32_t* __restrict__ bitmap,
                                                   uint32_t* __restrict__ colcnt, int nb, int words) {
  constexpr int NW = 16;
  __shared__ uint32_t cnt[NW][64];
  const int bh = blockIdx.y, strip = blockIdx.x, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = strip * 64 + lane;
  const int R = (nb + NW - 1) / NW;
  const int r0 = min(nb, w * R), r1 = min(nb, r0 + R);
  const uint32_t* bm = bitmap + (size_t)bh * nb * words + 2 * strip;
  const bool hi_half = lane >= 32;
  const uint32_t bit = 1u << (lane & 31);
  uint32_t c = 0;
  for (int rb = r0; rb < r1; rb += 64) {
    // lane l loads the strip's two words of row rb + l; readlane hands them to every lane
    const int r = rb + lane;
    uint32_t lo = 0u, hi = 0u;
    if (r < r1) {
      lo = bm[(size_t)r * words];
      hi = bm[(size_t)r * words + 1];
    }
    const int n = min(64, r1 - rb);
    for (int i = 0; i < n; ++i) {
      const uint32_t a = __builtin_amdgcn_readlane(lo, i), b = __builtin_amdgcn_readlane(hi, i);
      c += ((hi_half ? b : a) & bit) ? 1u : 0u;
    }
  }
  cnt[w][lane] = c;
  __syncthreads();
  if (w == 0 && j < nb) {
    uint32_t t = 0;
    for (int ww = 0; ww < NW; ++ww) t += cnt[ww][lane];
    colcnt[(size_t)bh * nb + j] = t;
  }
}

// CSC rows in ascending order from the bitmap: block = (64-column strip, bh),
// wave w scans rows [w*R, (w+1)*R), lane = column.
__global__ __launch_bounds__(1024) void k_csc_fill(const uint32_t* __restrict__ bitmap, const int32_t* __restrict__ col_ptr,
                                                   int32_t* __restrict__ row_idx, int nb, int64_t kph, int words) {
  constexpr int NW = 16;  // waves per strip, each over nb / NW consecutive rows
  __shared__ uint32_t cnt[NW][64];
  const int bh = blockIdx.y, strip = blockIdx.x, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = strip * 64 + lane;
  const int R = (nb + NW - 1) / NW;
  const int r0 = min(nb, w * R), r1 = min(nb, r0 + R);
  // Rows go through the wave 64 at a time: lane l loads the strip's two
  // bitmap words of row rb + l, and readlane hands each row's words to every
  // lane in row order. readlane reads a lane whether or not it is active, so
  // every lane stays in both passes; only the columns past nb write nothing.
  const uint32_t* bm = bitmap + (size_t)bh * nb * words + 2 * strip;
  const bool hi_half = lane >= 32;
  const uint32_t bit = 1u << (lane & 31);
  auto load_rows = [&](int rb, uint32_t& lo, uint32_t& hi) {
    const int r = rb + lane;
    lo = hi = 0u;
    if (r < r1) {
      lo = bm[(size_t)r * words];
      hi = bm[(size_t)r * words + 1];
    }
  };
  auto has = [&](uint32_t lo, uint32_t hi, int i) -> bool {  // does row rb + i select column j
    const uint32_t a = __builtin_amdgcn_readlane(lo, i), b = __builtin_amdgcn_readlane(hi, i);
    return ((hi_half ? b : a) & bit) != 0u;
  };
  uint32_t c = 0;
  for (int rb = r0; rb < r1; rb += 64) {
    uint32_t lo, hi;
    load_rows(rb, lo, hi);
    const int n = min(64, r1 - rb);
    for (int i = 0; i < n; ++i) c += has(lo, hi, i) ? 1u : 0u;
  }
  cnt[w][lane] = c;
  __syncthreads();
  const bool live = j < nb;
  uint32_t base = live ? (uint32_t)col_ptr[(size_t)bh * (nb + 1) + j] : 0u;
  for (int ww = 0; ww < w; ++ww) base += cnt[ww][lane];
  int32_t* out = row_idx + (size_t)bh * kph;
  for (int rb = r0; rb < r1; rb += 64) {
    uint32_t lo, hi;
    load_rows(rb, lo, hi);
    const int n = min(64, r1 - rb);
    for (int i = 0; i < n; ++i)
      if (has(lo, hi, i) && live && base < kph) out[base++] = rb + i;
  }
}

static hipError_t csc_from_bitmap(const TopkArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_colptr, dim3(a.bh), dim3(1024), 0, st, a.ws.colcnt, a.col_ptr, a.nb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_csc_fill, dim3(a.ws.words / 2, a.bh), dim3(1024), 0, st, a.ws.bitmap, a.col_ptr, a.row_idx,
                     a.nb, a.k, a.ws.words);
  return hipGetLastError();
}

#define VSA2_CHECK(x)                      \
  do {                                     \
    hipError_t e_ = (x);                   \
    if (e_ != hipSuccess) return e_;       \
  } while (0)

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  const size_t n = (size_t)a.nb * a.nb;
  int chunks = (int)((n + 256 * 64 - 1) / (256 * 64));
  if (chunks > 128) chunks = 128;
  if (chunks < 1) chunks = 1;
  const dim3 hgrid(chunks, a.bh);
  const dim3 rgrid((a.nb + 3) / 4, a.bh);
  VSA2_CHECK(launch_fill_u32(a.ws.hist, 0u, (size_t)a.bh * 4096, st));
  hipLaunchKernelGGL((k_hist<20, 12>), hgrid, dim3(256), 0, st, a.scores, a.ws.hist, a.ws.state, n);
  VSA2_CHECK(hipGetLastError());
  hipLaunchKernelGGL((k_select<20, 12>), dim3(a.bh), dim3(256), 0, st, a.ws.hist, a.ws.state, (uint32_t)a.k);
  VSA2_CHECK(hipGetLastError());
  VSA2_CHECK(launch_fill_u32(a.ws.hist, 0u, (size_t)a.bh * 4096, st));
  hipLaunchKernelGGL((k_hist<8, 12>), hgrid, dim3(256), 0, st, a.scores, a.ws.hist, a.ws.state, n);
  VSA2_CHECK(hipGetLastError());
  hipLaunchKernelGGL((k_select<8, 12>), dim3(a.bh), dim3(256), 0, st, a.ws.hist, a.ws.state, 0u);
  VSA2_CHECK(hipGetLastError());
  VSA2_CHECK(launch_fill_u32(a.ws.hist, 0u, (size_t)a.bh * 4096, st));
  hipLaunchKernelGGL((k_hist<0, 8>), hgrid, dim3(256), 0, st, a.scores, a.ws.hist, a.ws.state, n);
  VSA2_CHECK(hipGetLastError());
  hipLaunchKernelGGL((k_select<0, 8>), dim3(a.bh), dim3(256), 0, st, a.ws.hist, a.ws.state, 0u);
  VSA2_CHECK(hipGetLastError());
  hipLaunchKernelGGL(k_rowcount, rgrid, dim3(256), 0, st, a.scores, a.ws.state, a.ws.rowcnt, a.nb);
  VSA2_CHECK(hipGetLastError());
  hipLaunchKernelGGL(k_rowalloc, dim3(a.bh), dim3(1024), 0, st, a.ws.rowcnt, a.ws.state, a.ws.take, a.row_ptr, a.nb);
  VSA2_CHECK(hipGetLastError());
  const int csc = a.col_ptr != nullptr;  // forward-only callers need no CSC
  hipLaunchKernelGGL(k_compact, rgrid, dim3(256), 0, st, a.scores, a.ws.state, a.ws.take, a.row_ptr, a.col_idx,
                     a.ws.bitmap, a.nb, a.k, a.ws.words, csc);
  VSA2_CHECK(hipGetLastError());
  if (!csc) return hipSuccess;
  hipLaunchKernelGGL(k_colcount, dim3(a.ws.words / 2, a.bh), dim3(1024), 0, st, a.ws.bitmap, a.ws.colcnt, a.nb,
                     a.ws.words);
  VSA2_CHECK(hipGetLastError());
  return csc_from_bitmap(a, st);
}

// The VSA router baseline's selection (paper §1, Figure 1 left): every query
// block keeps its own kr largest scores, ties to the lower column.  One
// workgroup per (row, batch * head): a 4-pass radix select over 8-bit digits
// of the bit patterns (LDS histogram) finds the kr-th largest pattern tau and
// how many entries equal to tau to take; the row is then compacted in column
// order (wave ballots, per-wave totals through LDS).  Writes the CSR.
__global__ __launch_bounds__(256) void k_row_topk(const float* __restrict__ scores, int32_t* __restrict__ row_ptr,
                                                  int32_t* __restrict__ col_idx, int nb, int kr) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sel_state[2];
  __shared__ uint32_t wcnt[4][2];
  const int row = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* s = scores + ((size_t)bh * nb + row) * nb;
  uint32_t prefix = 0, need = (uint32_t)kr;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0u;
    __syncthreads();
    for (int j = tid; j < nb; j += 256) {
      const uint32_t u = score_bits(s[j]);
      if (pass == 0 || (u >> (shift + 8)) == (prefix >> (shift + 8))) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t acc = 0;
      int b = 255;
      for (; b > 0; --b) {
        if (acc + hist[b] >= need) break;
        acc += hist[b];
      }
      sel_state[0] = prefix | ((uint32_t)b << shift);
      sel_state[1] = need - acc;
    }
    __syncthreads();
    prefix = sel_state[0];
    need = sel_state[1];
    __syncthreads();  // every thread has the state before the next pass clears the histogram
  }
  const uint32_t tau = prefix;  // take every entry above tau and the first `need` equal to it
  const uint64_t lt = lanemask_lt(lane);
  int32_t* out = col_idx + ((size_t)bh * nb + row) * kr;
  uint32_t gt_seen = 0, eq_seen = 0;
  for (int j0 = 0; j0 < nb; j0 += 256) {
    const int j = j0 + tid;
    const uint32_t u = j < nb ? score_bits(s[j]) : 0u;
    const bool gt = j < nb && u > tau, eq = j < nb && u == tau;
    const uint64_t gtm = __ballot(gt), eqm = __ballot(eq);
    if (lane == 0) {
      wcnt[w][0] = (uint32_t)__popcll(gtm);
      wcnt[w][1] = (uint32_t)__popcll(eqm);
    }
    __syncthreads();
    uint32_t gtb = gt_seen + (uint32_t)__popcll(gtm & lt), eqb = eq_seen + (uint32_t)__popcll(eqm & lt);
    uint32_t gtt = 0, eqt = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (v < w) {
        gtb += wcnt[v][0];
        eqb += wcnt[v][1];
      }
      gtt += wcnt[v][0];
      eqt += wcnt[v][1];
    }
    const bool sel = gt || (eq && eqb < need);
    const uint32_t pos = gtb + min(eqb, need);  // selected entries before column j
    if (sel && pos < (uint32_t)kr) out[pos] = j;
    gt_seen += gtt;
    eq_seen += eqt;
    __syncthreads();  // the per-wave totals are rewritten next chunk
  }
  if (tid == 0) {
    row_ptr[(size_t)bh * (nb + 1) + row] = row * kr;
    if (row == nb - 1) row_ptr[(size_t)bh * (nb + 1) + nb] = nb * kr;
  }
}

hipError_t launch_topk_rows(const TopkArgs& a, hipStream_t st) {
  const int kr = (int)(a.k / a.nb);
  hipLaunchKernelGGL(k_row_topk, dim3(a.nb, a.bh), dim3(256), 0, st, a.scores, a.row_ptr, a.col_idx, a.nb, kr);
  VSA2_CHECK(hipGetLastError());
  return a.col_ptr ? launch_plan(a, st) : hipSuccess;  // forward-only callers need no CSC
}

hipError_t launch_plan(const TopkArgs& a, hipStream_t st) {
  VSA2_CHECK(launch_fill_u32(a.ws.colcnt, 0u, (size_t)a.bh * a.nb, st));
  VSA2_CHECK(launch_fill_u32(a.ws.bitmap, 0u, (size_t)a.bh * a.nb * a.ws.words, st));
  hipLaunchKernelGGL(k_csr_scatter, dim3((a.nb + 3) / 4, a.bh), dim3(256), 0, st, a.row_ptr, a.col_idx, a.ws.bitmap,
                     a.ws.colcnt, a.nb, a.k, a.ws.words);
  VSA2_CHECK(hipGetLastError());
  return csc_from_bitmap(a, st);
}

}  // namespace vsa2
