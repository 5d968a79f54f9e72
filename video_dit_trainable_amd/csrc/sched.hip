// Work schedule of the fine branch: in what order, and on which XCD, the
// per-cube work items of the forward and dQ passes (query cubes) and of the
// dK/dV pass (KV cubes) run.
//
// Per-sequence TopK (paper §2.2 Eq.(8)-(9)) leaves every query cube with its
// own number of KV cubes, and the blog's reproduction notes (its §12) leave
// the scheduler of these unequal lists to the implementer; its §10 counts the
// resulting imbalance and the block-sparse memory traffic among the gap
// between the ideal and the measured speed-up.  At 720p the lists of one
// (batch, head) run up to ~220 blocks per query cube and up to ~800 query
// cubes per KV cube, with a quarter of the lists empty.  The schedule:
//  * orders the cubes of each (batch, head) by a min-hash of their lists: a
//    cube's key is the minimum, over its list, of two fixed bijections of the
//    ids (16 bits each); two cubes share the first half with probability equal
//    to the Jaccard overlap of their lists, so cubes that gather the same
//    tiles sit next to each other;
//  * cuts that order into 8 contiguous ranges of equal work (list length plus
//    a fixed cost per item), one per XCD, so neighbours in the order share an
//    L2 and every XCD gets the same work;
//  * puts the long lists of each range first (by length class, then the
//    min-hash order), so the short and the empty ones end each XCD's queue;
//  * appends each (batch, head)'s range for XCD x to queue x, in (batch,
//    head) order.
// Both sides are built in the same launches, as 2 x (batch x head) lists of
// lists: (batch, head) entry v < nbh is the query side of v, entry nbh + v
// the KV side of v.
// The kernels run as many workgroups as fit on the device at once; each takes
// items from the queue of its XCD (workgroup b runs on XCD b mod 8) and, when
// that queue is empty, from the others.  An item is computed the same way
// whoever takes it, so results do not depend on the order items are taken.
#include "common.h"
#include "launch.h"

namespace vsa2 {

// Two bijections of [0, 2^16) (an odd multiplier is invertible modulo 2^16).
__device__ __forceinline__ uint32_t mh1(uint32_t j) { return (j * 40503u + 12345u) & 0xFFFFu; }
__device__ __forceinline__ uint32_t mh2(uint32_t j) { return ((j ^ 0x5A5Au) * 52429u + 777u) & 0xFFFFu; }

__device__ __forceinline__ int list_len(const int32_t* __restrict__ ptr, int c, int64_t kph) {
  const int64_t s = min<int64_t>(max(ptr[c], 0), kph);
  const int64_t e = min<int64_t>(max<int64_t>(ptr[c + 1], s), kph);
  return (int)(e - s);
}

// The lists of side entry v (see above): (ptr0, idx0) for v < nbh (the CSR),
// (ptr1, idx1) for the others (the CSC).
__device__ __forceinline__ const int32_t* side_ptr(const int32_t* ptr0, const int32_t* ptr1, int v, int nbh, int n) {
  return v < nbh ? ptr0 + (size_t)v * (n + 1) : ptr1 + (size_t)(v - nbh) * (n + 1);
}

// Min-hash key of every list: (min mh1 << 16 | min mh2), 0xFFFFFFFF when the
// list holds no valid id.  One wave per list.
__global__ __launch_bounds__(256) void k_sched_keys(const int32_t* __restrict__ ptr0, const int32_t* __restrict__ idx0,
                                                    const int32_t* __restrict__ ptr1, const int32_t* __restrict__ idx1,
                                                    uint32_t* __restrict__ keys, int n, int64_t kph, int nbh) {
  const int bh = blockIdx.y, c = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (c >= n) return;
  const int32_t* pb = side_ptr(ptr0, ptr1, bh, nbh, n);
  const int64_t s = min<int64_t>(max(pb[c], 0), kph);
  const int64_t e = min<int64_t>(max<int64_t>(pb[c + 1], s), kph);
  const int32_t* li = bh < nbh ? idx0 + (size_t)bh * kph : idx1 + (size_t)(bh - nbh) * kph;
  uint32_t a = 0xFFFFu, b = 0xFFFFu;
  bool any = false;
  for (int64_t p = s + lane; p < e; p += 64) {
    const int j = li[p];
    if ((unsigned)j < (unsigned)n) {
      a = min(a, mh1((uint32_t)j));
      b = min(b, mh2((uint32_t)j));
      any = true;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    a = min(a, (uint32_t)__shfl_xor((int)a, o));
    b = min(b, (uint32_t)__shfl_xor((int)b, o));
  }
  any = __ballot(any) != 0ull;
  if (lane == 0) keys[(size_t)bh * n + c] = any ? ((a << 16) | b) : 0xFFFFFFFFu;
}

constexpr int SCHED_TILE = 4096;   // keys per LDS tile of the rank count
constexpr int SCHED_OVH = 4;       // fixed cost of an item, in list entries
constexpr int SCHED_FASTN = 8192;  // lists per (batch, head) the in-LDS sorts take

// Ascending bitonic sort of m 64-bit values in LDS (m a power of two, at most
// SCHED_FASTN) by one 1024-thread workgroup; the caller has synchronised
// after writing them.  Values equal to each other end up adjacent, so with
// distinct values (an id in the low bits) the order is unique.
__device__ void lds_bitonic(uint64_t* a, int m) {
  for (int k = 2; k <= m; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < m; i += 1024) {
        const int l = i ^ j;
        if (l > i) {
          const uint64_t x = a[i], y = a[l];
          if ((x > y) == ((i & k) == 0)) {
            a[i] = y;
            a[l] = x;
          }
        }
      }
      __syncthreads();
    }
}

__device__ __forceinline__ int pow2_at_least(int n) {
  int m = 2;
  while (m < n) m <<= 1;
  return m;
}

// The (key, id) order of up to SCHED_FASTN lists, one workgroup per (batch,
// head): (key << 32 | id) sorted in LDS, order[rank] = id.
__global__ __launch_bounds__(1024) void k_sched_sort(const uint32_t* __restrict__ keys, int32_t* __restrict__ order,
                                                     int n) {
  __shared__ uint64_t a[SCHED_FASTN];
  const int bh = blockIdx.x, m = pow2_at_least(n);
  for (int i = threadIdx.x; i < m; i += 1024)
    a[i] = i < n ? ((uint64_t)keys[(size_t)bh * n + i] << 32 | (uint32_t)i) : ~0ull;
  __syncthreads();
  lds_bitonic(a, m);
  for (int r = threadIdx.x; r < n; r += 1024) order[(size_t)bh * n + r] = (int32_t)(uint32_t)a[r];
}

// Rank of every cube in (key, id) order, order[rank] = cube.  One thread per
// cube counts the keys below its own; the keys of the (batch, head) pass
// through LDS in tiles, read four at a time.
__global__ __launch_bounds__(256) void k_sched_rank(const uint32_t* __restrict__ keys, int32_t* __restrict__ order,
                                                    int n) {
  __shared__ __align__(16) uint32_t kt[SCHED_TILE];
  const int bh = blockIdx.y, tid = threadIdx.x, e = blockIdx.x * 256 + tid;
  const uint32_t* kb = keys + (size_t)bh * n;
  const uint32_t ke = e < n ? kb[e] : 0u;
  uint32_t rank = 0;
  for (int f0 = 0; f0 < n; f0 += SCHED_TILE) {
    const int nt = min(SCHED_TILE, n - f0);
    __syncthreads();
    for (int f = tid; f < SCHED_TILE; f += 256) kt[f] = f < nt ? kb[f0 + f] : 0xFFFFFFFFu;
    __syncthreads();
    // key f0 + f ranks below ke when smaller, or equal with a lower id; the
    // pad entries past nt (0xFFFFFFFF, id beyond every cube) never do
    const int lim = e - f0;  // ids below e, in this tile's numbering
    const int nt4 = (nt + 3) & ~3;
#pragma unroll 4
    for (int f = 0; f < nt4; f += 4) {
      const uint4 k4 = *reinterpret_cast<const uint4*>(&kt[f]);
      rank += (k4.x < ke || (k4.x == ke && f < lim)) ? 1u : 0u;
      rank += (k4.y < ke || (k4.y == ke && f + 1 < lim)) ? 1u : 0u;
      rank += (k4.z < ke || (k4.z == ke && f + 2 < lim)) ? 1u : 0u;
      rank += (k4.w < ke || (k4.w == ke && f + 3 < lim)) ? 1u : 0u;
    }
  }
  if (e < n) order[(size_t)bh * n + rank] = e;
}

// One workgroup per (batch, head): the work of each position of the order
// (list length + SCHED_OVH), an exclusive scan, and the XCD of a position =
// the eighth of the total its work's midpoint falls in, so the ranges are
// contiguous in the order.  px[bh][p] = XCD << 5 | length class, with class
// floor(log2(length + 1)) + 1 <= 16; rng[bh][0..8] = range starts (rng[8] = n).
__global__ __launch_bounds__(1024) void k_sched_cut(const int32_t* __restrict__ ptr0, const int32_t* __restrict__ ptr1,
                                                    const int32_t* __restrict__ order, uint8_t* __restrict__ px,
                                                    int32_t* __restrict__ rng_out, int n, int64_t kph, int nbh) {
  __shared__ uint32_t sh[17];
  __shared__ int rng[9];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int32_t* pb = side_ptr(ptr0, ptr1, bh, nbh, n);
  const int32_t* ob = order + (size_t)bh * n;
  uint32_t total = 0;
  for (int p0 = 0; p0 < n; p0 += 1024) {
    const int p = p0 + tid;
    const uint32_t w = p < n ? (uint32_t)(list_len(pb, ob[p], kph) + SCHED_OVH) : 0u;
    uint32_t tot;
    (void)block_scan_1024(w, tot, sh);
    total += tot;
  }
  if (tid < 9) rng[tid] = 0;
  __syncthreads();
  uint32_t carry = 0;
  for (int p0 = 0; p0 < n; p0 += 1024) {
    const int p = p0 + tid;
    const int len = p < n ? list_len(pb, ob[p], kph) : 0;
    const uint32_t w = p < n ? (uint32_t)(len + SCHED_OVH) : 0u;
    uint32_t tot;
    const uint32_t before = carry + block_scan_1024(w, tot, sh);
    carry += tot;
    if (p < n) {
      const uint64_t mid2 = 2ull * before + w;                        // twice the midpoint
      const int x = (int)min<uint64_t>(7ull, (8ull * mid2) / (2ull * (uint64_t)total));
      const int c = 32 - __clz((unsigned)len + 1u);                   // floor(log2(len + 1)) + 1
      px[(size_t)bh * n + p] = (uint8_t)((x << 5) | c);
      atomicAdd(&rng[x + 1], 1);
    }
  }
  __syncthreads();
  if (tid == 0) {
    for (int x = 0; x < 8; ++x) rng[x + 1] += rng[x];
  }
  __syncthreads();
  if (tid < 9) rng_out[(size_t)bh * 9 + tid] = rng[tid];
}

// Long lists first inside each XCD's range: the position of p within its
// range = entries of the range with a higher class, plus those of the same
// class earlier in the order.  tmp[bh][range start + that] = cube;
// cnt[bh][x] = items of XCD x.  The head's classes pass through LDS.
__global__ __launch_bounds__(256) void k_sched_place(const uint8_t* __restrict__ px, const int32_t* __restrict__ rng,
                                                     const int32_t* __restrict__ order, int32_t* __restrict__ tmp,
                                                     int32_t* __restrict__ cnt, int n) {
  __shared__ uint8_t pl[SCHED_MAXN];
  const int bh = blockIdx.y, tid = threadIdx.x, p = blockIdx.x * 256 + tid;
  const uint8_t* pxb = px + (size_t)bh * n;
  for (int q = tid; q < n; q += 256) pl[q] = pxb[q];
  __syncthreads();
  if (blockIdx.x == 0 && tid < 8) cnt[(size_t)bh * 8 + tid] = rng[(size_t)bh * 9 + tid + 1] - rng[(size_t)bh * 9 + tid];
  if (p >= n) return;
  const int x = pl[p] >> 5, c = pl[p] & 31;
  const int r0 = rng[(size_t)bh * 9 + x], r1 = rng[(size_t)bh * 9 + x + 1];
  int pos = 0;
  for (int q = r0; q < r1; ++q) {
    const int cq = pl[q] & 31;
    pos += (cq > c || (cq == c && q < p)) ? 1 : 0;
  }
  tmp[(size_t)bh * n + r0 + pos] = order[(size_t)bh * n + p];
}

// The placement of k_sched_place for up to SCHED_FASTN lists, one workgroup
// per (batch, head): positions sorted by (XCD, class descending, position) put
// each XCD's range at its start in the order (the ranges are contiguous) and
// the range long-first, which is the same placement.
__global__ __launch_bounds__(1024) void k_sched_place_sort(const uint8_t* __restrict__ px,
                                                           const int32_t* __restrict__ rng,
                                                           const int32_t* __restrict__ order,
                                                           int32_t* __restrict__ tmp, int32_t* __restrict__ cnt,
                                                           int n) {
  __shared__ uint64_t a[SCHED_FASTN];
  const int bh = blockIdx.x, tid = threadIdx.x, m = pow2_at_least(n);
  const uint8_t* pxb = px + (size_t)bh * n;
  for (int p = tid; p < m; p += 1024) {
    if (p < n) {
      const uint32_t x = pxb[p] >> 5, c = pxb[p] & 31;
      a[p] = (uint64_t)((x << 5) | (31u - c)) << 32 | (uint32_t)p;
    } else {
      a[p] = ~0ull;
    }
  }
  if (tid < 8) cnt[(size_t)bh * 8 + tid] = rng[(size_t)bh * 9 + tid + 1] - rng[(size_t)bh * 9 + tid];
  __syncthreads();
  lds_bitonic(a, m);
  for (int i = tid; i < n; i += 1024) tmp[(size_t)bh * n + i] = order[(size_t)bh * n + (int)(uint32_t)a[i]];
}

// MMDiT text cubes: text cubes 2u, 2u + 1 of (batch, head) h go next to each
// other into queue (h ceil(ntc / 2) + u) mod 8, so the forward, which takes
// two consecutive items at a time, runs them together.
__device__ __forceinline__ int sched_text_queue(int h, int t, int ntc) {
  return (h * ((ntc + 1) >> 1) + (t >> 1)) & 7;
}
// Text items of heads 0 .. nh - 1 in queue x.
__device__ inline int sched_text_count(int nh, int ntc, int x) {
  int c = 0;
  for (int h = 0; h < nh; ++h)
    for (int t = 0; t < ntc; ++t) c += sched_text_queue(h, t, ntc) == x;
  return c;
}

// Queue offsets: queue x holds first its text items, head by head (MMDiT text
// rows: each of their lists holds every cube, tens of times a video list, so
// all of them start at once), then, for every (batch, head) in turn, that
// head's range for XCD x.  hdr[x] = start of queue x in the item array,
// hdr[8 + x] its length, hdr[16] the item count bh (n + ntc) and hdr[17]
// SCHED_MAGIC; hoff[bh][x] = where (batch, head) bh's range starts.  One
// workgroup per side (hdr0 the query side's header, hdr1 the KV side's).
__global__ __launch_bounds__(64) void k_sched_queues(const int32_t* __restrict__ cnt_, int32_t* __restrict__ hdr0,
                                                     int32_t* __restrict__ hdr1, int32_t* __restrict__ hoff_, int bh,
                                                     int n, int ntc) {
  __shared__ int tot[8];
  const int x = threadIdx.x;
  const int32_t* cnt = cnt_ + (size_t)blockIdx.x * bh * 8;
  int32_t* hoff = hoff_ + (size_t)blockIdx.x * bh * 8;
  int32_t* hdr = blockIdx.x ? hdr1 : hdr0;
  const int tx = x < 8 ? sched_text_count(bh, ntc, x) : 0;
  if (x < 8) {
    int s = tx;
    for (int h = 0; h < bh; ++h) s += cnt[(size_t)h * 8 + x];
    tot[x] = s;
  }
  __syncthreads();
  if (x < 8) {
    int head = 0;
    for (int y = 0; y < x; ++y) head += tot[y];
    hdr[x] = head;
    hdr[8 + x] = tot[x];
    if (x == 0) {  // what the fine kernels check before trusting the queues
      hdr[16] = bh * (n + ntc);
      hdr[17] = SCHED_MAGIC;
    }
    int o = head + tx;
    for (int h = 0; h < bh; ++h) {
      hoff[(size_t)h * 8 + x] = o;
      o += cnt[(size_t)h * 8 + x];
    }
  }
}

// Items into their queues: item code = bh (n + ntc) + cube, text cube t being
// item n + t; the text items of queue x sit before hoff[0][x], head by head
// and in the order of t.
__global__ __launch_bounds__(256) void k_sched_fill(const int32_t* __restrict__ tmp, const int32_t* __restrict__ cnt,
                                                    const int32_t* __restrict__ hoff, int32_t* __restrict__ items0,
                                                    int32_t* __restrict__ items1, int n, int ntc, int nbh) {
  const int bh = blockIdx.y, t = blockIdx.x * 256 + threadIdx.x;  // bh: the side entry
  const int side = bh >= nbh ? 1 : 0, h = bh - side * nbh;        // h: the (batch, head)
  int32_t* items = side ? items1 : items0;
  const int64_t base = (int64_t)h * (n + ntc);
  if (blockIdx.x == 0) {
    const int32_t* hoff0 = hoff + (size_t)side * nbh * 8;  // the side's head 0
    for (int u = threadIdx.x; u < ntc; u += 256) {
      const int x = sched_text_queue(h, u, ntc);
      int at = hoff0[x] - sched_text_count(nbh, ntc, x) + sched_text_count(h, ntc, x);
      for (int v = 0; v < u; ++v) at += sched_text_queue(h, v, ntc) == x;
      items[at] = (int32_t)(base + n + u);
    }
  }
  if (t >= n) return;
  int s = 0, x = 0;
  for (; x < 7; ++x) {
    const int c = cnt[(size_t)bh * 8 + x];
    if (t < s + c) break;
    s += c;
  }
  items[hoff[(size_t)bh * 8 + x] + (t - s)] = (int32_t)(base + tmp[(size_t)bh * n + t]);
}

// The schedule from the CSR (query side) and, with a CSC, the KV side, both in
// the same launches.
hipError_t launch_sched(const SchedArgs& a, hipStream_t st) {
  if (a.n > SCHED_MAXN) return hipErrorInvalidValue;
  const int n = a.n;
  const int sides = a.col_ptr ? 2 : 1;  // no CSC (forward only): the query side alone
  const int nv = sides * a.bh;           // side entries
  hipLaunchKernelGGL(k_sched_keys, dim3((n + 3) / 4, nv), dim3(256), 0, st, a.row_ptr, a.col_idx, a.col_ptr,
                     a.row_idx, a.keys, n, a.kph, a.bh);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool fast = n <= SCHED_FASTN;  // the in-LDS sorts; beyond, the counting kernels
  if (fast)
    hipLaunchKernelGGL(k_sched_sort, dim3(nv), dim3(1024), 0, st, a.keys, a.order, n);
  else
    hipLaunchKernelGGL(k_sched_rank, dim3((n + 255) / 256, nv), dim3(256), 0, st, a.keys, a.order, n);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sched_cut, dim3(nv), dim3(1024), 0, st, a.row_ptr, a.col_ptr, a.order, a.px, a.rng, n, a.kph,
                     a.bh);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (fast)
    hipLaunchKernelGGL(k_sched_place_sort, dim3(nv), dim3(1024), 0, st, a.px, a.rng, a.order, a.tmp, a.cnt, n);
  else
    hipLaunchKernelGGL(k_sched_place, dim3((n + 255) / 256, nv), dim3(256), 0, st, a.px, a.rng, a.order, a.tmp,
                       a.cnt, n);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sched_queues, dim3(sides), dim3(64), 0, st, a.cnt, a.row_hdr, a.col_hdr, a.hoff, a.bh, n,
                     a.ntc);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sched_fill, dim3((n + 255) / 256, nv), dim3(256), 0, st, a.tmp, a.cnt, a.hoff, a.row_items,
                     a.col_items, n, a.ntc, a.bh);
  return hipGetLastError();
}

}  // namespace vsa2
