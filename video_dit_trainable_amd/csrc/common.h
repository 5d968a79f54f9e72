// Device-side building blocks shared by the VSA2 kernels (gfx950 / CDNA4).
//
// MFMA fragment convention used everywhere (wave64, 16x16 output tiles):
//   * a "k-step" contracts 32 values.  For bf16 it is one
//     v_mfma_f32_16x16x32_bf16; for fp32 it is eight v_mfma_f32_16x16x4_f32
//     issued on the eight elements of the same fragment, so both element types
//     share one fragment layout.
//   * lane l = 16*g + c (g = 0..3, c = 0..15).  The A operand row and the B
//     operand column are c; the 8 values a lane supplies belong to the k-slots
//     (g, e), e = 0..7.  The hardware pairs A slot (g, e) with B slot (g, e), so
//     any bijection between the 32 slots and the 32 contracted indices gives
//     the same product as long as A and B use the same one.
//   * the accumulator of a 16x16 tile: lane l holds rows 4g + r (r = 0..3) of
//     column c.
// The accumulator of S^T = K Q^T therefore holds, per lane, four keys of one
// query; fed back as the B operand of O^T = V^T P^T it needs the key<->slot map
//   pi(g, e) = 4g + e (e < 4),  16 + 4g + (e - 4) (e >= 4)
// within each 32-key chunk, and the V^T operand is read with the same map.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace vsa2 {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int CUBE = 64;   // tokens per 4x4x4 cube = rows of one attention tile
constexpr int SUBC = 8;    // tokens per 2x2x2 router sub-cube
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x8 v; };

__device__ __forceinline__ void mma(f32x4& c, const Frag<bf16>& a, const Frag<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
}

// product with a zero accumulator (lets the compiler use the inline constant)
__device__ __forceinline__ f32x4 mma0(const Frag<bf16>& a, const Frag<bf16>& b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma0(const Frag<float>& a, const Frag<float>& b) {
  f32x4 c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[0], b.v[0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
  for (int e = 1; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
  return c;
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 8 consecutive elements in registers (16 B of bf16 or 32 B of fp32)
template <typename T> struct Vec8 { T v[8]; };

template <typename T>
__device__ __forceinline__ Vec8<T> load8(const T* p) {
  Vec8<T> r;
  if constexpr (sizeof(T) == 2) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    __builtin_memcpy(&r, &u, 16);
  } else {
    uint4 u0 = reinterpret_cast<const uint4*>(p)[0];
    uint4 u1 = reinterpret_cast<const uint4*>(p)[1];
    __builtin_memcpy(&r, &u0, 16);
    __builtin_memcpy(reinterpret_cast<char*>(&r) + 16, &u1, 16);
  }
  return r;
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const Vec8<T>& r) {
  if constexpr (sizeof(T) == 2) {
    uint4 u;
    __builtin_memcpy(&u, &r, 16);
    *reinterpret_cast<uint4*>(p) = u;
  } else {
    uint4 u0, u1;
    __builtin_memcpy(&u0, &r, 16);
    __builtin_memcpy(&u1, reinterpret_cast<const char*>(&r) + 16, 16);
    reinterpret_cast<uint4*>(p)[0] = u0;
    reinterpret_cast<uint4*>(p)[1] = u1;
  }
}

// 4 consecutive elements (8 B of bf16 / 16 B of fp32)
template <typename T> struct Vec4 { T v[4]; };
template <typename T>
__device__ __forceinline__ Vec4<T> load4(const T* p) {
  Vec4<T> r;
  if constexpr (sizeof(T) == 2) {
    uint2 u = *reinterpret_cast<const uint2*>(p);
    __builtin_memcpy(&r, &u, 8);
  } else {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    __builtin_memcpy(&r, &u, 16);
  }
  return r;
}
template <typename T>
__device__ __forceinline__ void store4(T* p, const Vec4<T>& r) {
  if constexpr (sizeof(T) == 2) {
    uint2 u;
    __builtin_memcpy(&u, &r, 8);
    *reinterpret_cast<uint2*>(p) = u;
  } else {
    uint4 u;
    __builtin_memcpy(&u, &r, 16);
    *reinterpret_cast<uint4*>(p) = u;
  }
}

template <typename T>
__device__ __forceinline__ Frag<T> frag_from8(const Vec8<T>& a) {
  Frag<T> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = a.v[e];
  return f;
}

// Fragment from two 4-element runs (the pi map: slots e<4 from lo, e>=4 from hi).
template <typename T>
__device__ __forceinline__ Frag<T> frag_from44(const Vec4<T>& lo, const Vec4<T>& hi) {
  Frag<T> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) { f.v[e] = lo.v[e]; f.v[4 + e] = hi.v[e]; }
  return f;
}

// Fragment from two accumulator tiles (the pi map) converted to T.
template <typename T>
__device__ __forceinline__ Frag<T> frag_from_acc(const f32x4& lo, const f32x4& hi) {
  Frag<T> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) { f.v[e] = from_f32<T>(lo[e]); f.v[4 + e] = from_f32<T>(hi[e]); }
  return f;
}

// ---------------------------------------------------------------------------
// 64 x D tiles staged through registers into a transposed LDS layout (the
// fp32-storage dW_g kernel).  A "unit" is 4 rows x 8 columns; thread t owns
// units t, t + NT, ...  The transposed tile holds D rows of 64 tokens; the
// 4-token runs of row d are XOR-swizzled by sw(d), so the scatter of a unit
// (8 rows, one 4-token run each) and the fragment reads (16 rows, one run
// each) both spread over the banks:
//   element (d, t) lives at d*TS + 4*((t >> 2) ^ sw(d)) + (t & 3).
// ---------------------------------------------------------------------------
template <typename T, int D> struct TileGeom {
  static constexpr bool WIDE = (sizeof(T) == 2 && D == 128);
  static constexpr int UNITS = (CUBE / 4) * (D / 8);
  static constexpr int TS = WIDE ? 72 : 64;     // transposed row stride (elements)
  static constexpr int TR_ELEMS = D * TS;
  __device__ static constexpr int sw(int d) { return WIDE ? ((d >> 3) & 15) : (((d >> 3) ^ d) & 15); }
};

template <typename T, int D, int NT>
struct TileRegs {
  static constexpr int NU = (TileGeom<T, D>::UNITS + NT - 1) / NT;
  Vec8<T> r[NU][4];
};

// Load a 64 x D tile (row stride ld elements); rows >= valid_rows are zero.
template <typename T, int D, int NT>
__device__ __forceinline__ void tile_load(TileRegs<T, D, NT>& R, const T* __restrict__ src, int tid, int valid_rows,
                                          size_t ld = D) {
#pragma unroll
  for (int n = 0; n < TileRegs<T, D, NT>::NU; ++n) {
    const int u = tid + n * NT;
    if (u < TileGeom<T, D>::UNITS) {
      const int rg = u / (D / 8), cg = u % (D / 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * rg + r;
        if (row < valid_rows) {
          R.r[n][r] = load8(src + (size_t)row * ld + 8 * cg);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) R.r[n][r].v[e] = from_f32<T>(0.f);
        }
      }
    }
  }
}

template <typename T, int D, int NT>
__device__ __forceinline__ void tile_store_tr(const TileRegs<T, D, NT>& R, T* lds, int tid) {
  constexpr int TS = TileGeom<T, D>::TS;
#pragma unroll
  for (int n = 0; n < TileRegs<T, D, NT>::NU; ++n) {
    const int u = tid + n * NT;
    if (u < TileGeom<T, D>::UNITS) {
      const int rg = u / (D / 8), cg = u % (D / 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        Vec4<T> c;
#pragma unroll
        for (int r = 0; r < 4; ++r) c.v[r] = R.r[n][r].v[e];
        const int d = 8 * cg + e;
        store4(lds + d * TS + 4 * (rg ^ TileGeom<T, D>::sw(d)), c);
      }
    }
  }
}

// A fragment of a transposed LDS tile (row = feature d, k = token) with the pi
// map over token chunk c (32 tokens).
template <typename T, int D>
__device__ __forceinline__ Frag<T> frag_tr(const T* lds, int drow, int c, int g) {
  const T* row = lds + drow * TileGeom<T, D>::TS;
  const int s = TileGeom<T, D>::sw(drow);
  return frag_from44(load4(row + 4 * ((8 * c + g) ^ s)), load4(row + 4 * ((8 * c + 4 + g) ^ s)));
}

// Fragment straight from global memory: row `row` of a row-major [*, D] array.
template <typename T, int D>
__device__ __forceinline__ Frag<T> frag_global(const T* __restrict__ base, int row, int ks, int g) {
  return frag_from8(load8(base + (size_t)row * D + 32 * ks + 8 * g));
}

// ---------------------------------------------------------------------------
// Chunk-swizzled LDS tiles (R rows x W elements, stored as a contiguous R*W
// block in global memory).  Thread t loads the 16-byte chunks t + NT*n of the
// tile (coalesced) and stores logical chunk ch of row r at physical chunk
// ch ^ f(r) of that row; a wave's stores cover whole rows, so they never
// conflict.  f spreads both fragment reads over the banks: the 16-byte reads
// of 16 consecutive rows (one chunk each) and the 8-byte transposing reads of
// 4 rows x 4 runs (ds_read_b64_tr_b16).  f was chosen with the LDS bank
// conflict counter of gfx950: on linear and swizzled read patterns it fits
// 128 banks with the 16-byte reads served in 16-lane groups and 64 banks with
// the transposing reads served 32 lanes at a time.  Among the swizzles that
// are linear in the bits of r & 15, the ones below give no conflict for either
// read under every grouping consistent with the counts (and measure zero
// conflict cycles on both patterns):
//   16+ chunks per row: f(r) = 2 (r & 7) ^ 15 [r & 8]
//   8 chunks per row:   f(r) = (r & 6) ^ 7 [r & 8]
// f depends on r & 15 only, so rows r and r + 16m share a swizzle and a
// fragment address moves by 16m rows with a plain add.
// ---------------------------------------------------------------------------
template <typename T, int W> struct SwTile {
  static constexpr int NCH = W * (int)sizeof(T) / 16;  // 16-byte chunks per row
  static constexpr int EPC = 16 / (int)sizeof(T);      // elements per chunk
  __device__ static constexpr int f(int r) {
    return NCH >= 16 ? (((r & 7) << 1) ^ (((r >> 3) & 1) * 15)) : ((r & 6) ^ (((r >> 3) & 1) * 7));
  }
  __device__ static constexpr int off(int r, int ch) { return r * W + EPC * (ch ^ (f(r) & (NCH - 1))); }
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int R, int W, typename T, int NT> struct SwRegs {
  static constexpr int N = R * SwTile<T, W>::NCH / NT;
  static_assert(N * NT == R * SwTile<T, W>::NCH, "tile chunks must split evenly over the block");
  u32x4 c[N];
};

// Global -> registers, linear chunk order (chunk p = tid + NT*n, fully
// coalesced).  The whole tile is always read: callers point masked tiles at
// valid memory and mask their scores instead.
template <int R, int W, typename T, int NT>
__device__ __forceinline__ void sw_load(SwRegs<R, W, T, NT>& g, const T* __restrict__ src, int tid) {
  using S = SwTile<T, W>;
  static_assert(NT % S::NCH == 0, "a block must cover whole rows");
  const u32x4* s4 = reinterpret_cast<const u32x4*>(src) + tid;
#pragma unroll
  for (int n = 0; n < SwRegs<R, W, T, NT>::N; ++n) g.c[n] = s4[NT * n];
}
// Registers -> LDS at the swizzled position of each chunk.
template <int R, int W, typename T, int NT>
__device__ __forceinline__ void sw_store(const SwRegs<R, W, T, NT>& g, T* lds, int tid) {
  using S = SwTile<T, W>;
  constexpr int RSTEP = NT / S::NCH;
  const int r0 = tid / S::NCH, ch = tid % S::NCH;
#pragma unroll
  for (int n = 0; n < SwRegs<R, W, T, NT>::N; ++n) {
    const int r = r0 + RSTEP * n;
    *reinterpret_cast<u32x4*>(lds + r * W + S::EPC * (ch ^ (S::f(r) & (S::NCH - 1)))) = g.c[n];
  }
}
// MFMA fragment (8 elements = k-slots (g, 0..7)) of row r, k-step s of a swizzled tile.
template <typename T, int W>
__device__ __forceinline__ Frag<T> sw_frag(const T* lds, int r, int s, int g) {
  using S = SwTile<T, W>;
  if constexpr (sizeof(T) == 2) {
    return frag_from8(load8(lds + S::off(r, 4 * s + g)));
  } else {
    Vec8<T> v;
    const Vec4<T> a = load4(lds + S::off(r, 8 * s + 2 * g));
    const Vec4<T> b = load4(lds + S::off(r, 8 * s + 2 * g + 1));
#pragma unroll
    for (int e = 0; e < 4; ++e) { v.v[e] = a.v[e]; v.v[4 + e] = b.v[e]; }
    return frag_from8(v);
  }
}

// Transposed MFMA fragment from a swizzled row-major tile: lane (g, c) gets
// tile[r0 + pi(g, e)][col0 + c] for the 8 slots e, i.e. the A operand whose
// rows are tile columns and whose contraction runs over 32 tile rows r0.. .
// bf16: two ds_read_b64_tr_b16.  Within each 16-lane group that instruction
// returns to lane i, element e, the element i % 4 of the 8 bytes addressed by
// lane 4e + i / 4; so lane j addresses row r0 + 4g + j / 4 (+16 for the upper
// 4 slots), columns col0 + 4 (j % 4) .. +3.  fp32: eight scalar reads.
#define VSA2_LDS __attribute__((address_space(3)))
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
// the two halves of a bf16 fragment as one register quad (a plain vector
// concatenation: element-wise copies make the compiler insert bit-field moves)
template <typename T>
__device__ __forceinline__ Frag<T> frag_join(s16x4 lo, s16x4 hi) {
  static_assert(sizeof(T) == 2, "bf16 fragments only");
  Frag<T> f;
  f.v = __builtin_bit_cast(decltype(f.v), __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  return f;
}
template <typename T, int W>
__device__ __forceinline__ Frag<T> sw_frag_tr(const T* lds, int r0, int col0, int g, int c) {
  using S = SwTile<T, W>;
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
    const int col = col0 + 4 * (c & 3);
    const int ra = r0 + 4 * g + (c >> 2), rb = ra + 16;
    const T* pa = lds + S::off(ra, col / S::EPC) + (col % S::EPC);
    const T* pb = lds + S::off(rb, col / S::EPC) + (col % S::EPC);
    const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((VSA2_LDS s16x4*)(pa));
    const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((VSA2_LDS s16x4*)(pb));
    f = frag_join<T>(va, vb);
  } else {
    const int col = col0 + c;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = r0 + (e < 4 ? 4 * g + e : 16 + 4 * g + e - 4);
      f.v[e] = lds[S::off(r, col / S::EPC) + (col % S::EPC)];
    }
  }
  return f;
}

// Direct global -> LDS copy of a swizzled R x W tile (global_load_lds_dwordx4,
// no staging registers).  One instruction of a wave fills 1 KiB of LDS in lane
// order (lane i writes bytes 16i .. 16i+15 after the wave's base), so the lane
// that fills physical chunk pc of row r fetches logical chunk pc ^ f(r) -- the
// same layout sw_store makes.  The copy is asynchronous: the caller waits with
// wait_vm0() and then a barrier before any wave reads the tile.
// Keeps the compiler from hoisting address arithmetic on x out of a loop
// (an empty statement that claims to update the register).
__device__ __forceinline__ void opaque(int& x) { asm volatile("" : "+v"(x)); }

// one 16-byte LDS-direct load per lane (kept out of templates: the host pass
// cannot resolve the builtin inside a dependent context)
__device__ __forceinline__ void lds_copy16(const void* g, VSA2_LDS void* l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}
template <int R, int W, typename T, int NT>
__device__ __forceinline__ void dma_tile(const T* __restrict__ src, T* lds, int tid) {
  using S = SwTile<T, W>;
  constexpr int CH = R * S::NCH;
  static_assert(CH % NT == 0 && NT % 64 == 0 && NT % S::NCH == 0, "tile chunks must split evenly over whole waves");
  // Row r = n (NT / NCH) + tid / NCH: when NT / NCH is a multiple of 16 the
  // low four bits of r, and so the swizzle term, are the same for every n and
  // the per-lane offset is computed once.
  constexpr int RSTEP = NT / S::NCH;
  const int r0 = tid / S::NCH, pc = tid % S::NCH;
  int lane_off = (r0 * W + S::EPC * (pc ^ (S::f(r0) & (S::NCH - 1)))) * (int)sizeof(T);
  opaque(lane_off);  // keeps "base + lane_off" from being hoisted as a 64-bit per-lane pointer
  const int wbase = __builtin_amdgcn_readfirstlane(tid & ~63);
#pragma unroll
  for (int n = 0; n < CH / NT; ++n) {
    uint32_t off;
    if constexpr (RSTEP % 16 == 0) {
      off = (uint32_t)lane_off + (uint32_t)(n * RSTEP * W * sizeof(T));
    } else {
      const int r = r0 + n * RSTEP;
      off = (uint32_t)(r * W + S::EPC * (pc ^ (S::f(r) & (S::NCH - 1)))) * sizeof(T);
    }
    T* lbase = lds + (n * NT + wbase) * S::EPC;  // wave-uniform
    lds_copy16(reinterpret_cast<const char*>(src) + off, (VSA2_LDS void*)lbase);
  }
}
// Wait until every vector-memory load of this wave (including LDS-direct
// copies) has completed: s_waitcnt vmcnt(0), other counters untouched.
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// The same two fragment reads for bf16 tiles with the per-lane part of the
// address computed once.  For a row-major swizzled tile the k-step s of
// sw_frag(r, s, g) sits at element (base ^ 32 s) with base = sw_row_base(r, g),
// and the columns col0 (a multiple of 16) of sw_frag_tr(r0, col0, g, c) at
// (base ^ col0) with base = sw_tr_base(r0, g, c): the swizzle only permutes
// 16-byte chunks inside a row, so the step's contribution is a pure XOR.
template <typename T, int W>
__device__ __forceinline__ int sw_row_base(int r, int g) {
  using S = SwTile<T, W>;
  static_assert(sizeof(T) == 2 && S::EPC == 8, "bf16 tiles only");
  const int f = S::f(r) & (S::NCH - 1);
  return r * W + 8 * (f & ~3) + 8 * (g ^ (f & 3));
}
template <typename T, int W>
__device__ __forceinline__ int sw_tr_base(int r0, int g, int c) {
  using S = SwTile<T, W>;
  static_assert(sizeof(T) == 2 && S::EPC == 8, "bf16 tiles only");
  const int ra = r0 + 4 * g + (c >> 2);
  const int f = S::f(ra) & (S::NCH - 1);
  return ra * W + 8 * (f & ~1) + 8 * (((c >> 1) & 1) ^ (f & 1)) + 4 * (c & 1);
}
template <typename T>
__device__ __forceinline__ Frag<T> sw_frag_at(const T* lds, int base, int s) {
  return frag_from8(load8(lds + (base ^ (32 * s))));
}
// rows ra (from the base) and ra + 16 of the transposed read; W = row length
template <typename T, int W>
__device__ __forceinline__ Frag<T> sw_frag_tr_at(const T* lds, int base, int col0) {
  const T* pa = lds + (base ^ col0);
  const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((VSA2_LDS s16x4*)(pa));
  const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((VSA2_LDS s16x4*)(pa + 16 * W));
  return frag_join<T>(va, vb);
}
// Butterfly reductions over the four slot groups (lanes c, c+16, c+32, c+48).
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float group_sum(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Block -> work-item map that gives each XCD a contiguous slice of every
// (batch, head): consecutive block ids go round-robin over the 8 XCDs, so
// block b runs on XCD b % 8.  Returns false for the padding blocks.
__device__ __forceinline__ bool xcd_work(int bid, int items_per_bh, int& bh, int& item) {
  const int per = (items_per_bh + 7) >> 3;
  const int xcd = bid & 7, s = bid >> 3;
  bh = s / per;
  item = xcd * per + (s - bh * per);
  return item < items_per_bh;
}
// Visiting order of the cubes of one head: 4x4x4 blocks of cubes in raster
// order, cubes inside a block in raster order (edge blocks are smaller).
// Maps position p in [0, ct*cy*cx) to a cube index (c_t * cy + c_y) * cx + c_x,
// so consecutive positions are spatial neighbours in all three axes.
__host__ __device__ inline int blocked_cube(int p, int ct, int cy, int cx) {
  constexpr int B = 4;
  int t0 = 0;
  for (;;) {  // t-slab
    const int st = min(B, ct - t0), slab = st * cy * cx;
    if (p < slab || t0 + st >= ct) break;
    p -= slab;
    t0 += st;
  }
  const int st = min(B, ct - t0);
  int y0 = 0;
  for (;;) {  // y-row of blocks inside the slab
    const int sy = min(B, cy - y0), row = st * sy * cx;
    if (p < row || y0 + sy >= cy) break;
    p -= row;
    y0 += sy;
  }
  const int sy = min(B, cy - y0);
  int x0 = 0;
  for (;;) {  // block inside the row
    const int sx = min(B, cx - x0), blk = st * sy * sx;
    if (p < blk || x0 + sx >= cx) break;
    p -= blk;
    x0 += sx;
  }
  const int sx = min(B, cx - x0);
  const int dx = p % sx, dy = (p / sx) % sy, dt = p / (sx * sy);
  return ((t0 + dt) * cy + (y0 + dy)) * cx + (x0 + dx);
}

// Slots of a cube (slot 8s + u: sub-cube s, position u, each raster over
// 2x2x2) whose coordinate along `axis` (0 t, 1 y, 2 x) is below v: the
// coordinate is 2 * bit(5 - axis) + bit(2 - axis) of the slot.
__host__ __device__ constexpr uint64_t axis_slots(int axis, int v) {
  uint64_t m = 0;
  for (int s = 0; s < 64; ++s)
    if (2 * ((s >> (5 - axis)) & 1) + ((s >> (2 - axis)) & 1) < v) m |= 1ull << s;
  return m;
}
template <int AXIS>
__device__ __forceinline__ uint64_t axis_mask(int v) {
  constexpr uint64_t m1 = axis_slots(AXIS, 1), m2 = axis_slots(AXIS, 2), m3 = axis_slots(AXIS, 3);
  return v >= 4 ? ~0ull : (v == 3 ? m3 : (v == 2 ? m2 : (v == 1 ? m1 : 0ull)));
}

// Real extents (0..4) of cube c.  The quotients use float reciprocals: for
// c < 2^16 (c + 0.5) / n lies at least 0.5 / n from an integer, far beyond
// the rounding error of the two float roundings, so the truncation is exact.
__device__ __forceinline__ void cube_extent(int c, const PadGrid& p, int& vt, int& vy, int& vx) {
  const int a = (int)(((float)c + 0.5f) * p.inv_nyx);
  const int rem = c - a * p.ny * p.nx;
  const int b = (int)(((float)rem + 0.5f) * p.inv_nx);
  const int x = rem - b * p.nx;
  vt = min(4, max(0, p.rt - 4 * a));
  vy = min(4, max(0, p.ry - 4 * b));
  vx = min(4, max(0, p.rx - 4 * x));
}

// Bit s set for the slots of cube c that hold a real token.
__device__ __forceinline__ uint64_t cube_slots(int c, const PadGrid& p) {
  int vt, vy, vx;
  cube_extent(c, p, vt, vy, vx);
  return axis_mask<0>(vt) & axis_mask<1>(vy) & axis_mask<2>(vx);
}

// Number of real tokens of cube c.
__device__ __forceinline__ int cube_count(int c, const PadGrid& p) {
  int vt, vy, vx;
  cube_extent(c, p, vt, vy, vx);
  return vt * vy * vx;
}

// Exclusive prefix sum over a 1024-thread block (every thread takes part);
// total gets the block's sum.  sh: 17 words of LDS.
__device__ inline uint32_t block_scan_1024(uint32_t x, uint32_t& total, uint32_t* sh) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint32_t inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  if (tid == 0) {
    uint32_t a = 0;
    for (int i = 0; i < 16; ++i) {
      const uint32_t t = sh[i];
      sh[i] = a;
      a += t;
    }
    sh[16] = a;
  }
  __syncthreads();
  const uint32_t r = sh[w] + inc - x;
  total = sh[16];
  __syncthreads();
  return r;
}

// Written by the schedule build into word 17 of each side's header, beside
// the item count in word 16.
constexpr int32_t SCHED_MAGIC = 0x53434844;

// Next work item of the schedule for this workgroup: from the queue of its
// XCD (workgroup b runs on XCD b mod 8), then from the others in turn; -1
// when every queue is empty.  hdr = {queue starts[8], queue lengths[8], item
// count, SCHED_MAGIC}; ctr = one counter per queue, zero before the launch;
// total = the launch's item count.  A header that no build of this size
// wrote (a buffer never built, or built for another problem) makes the
// workgroups take the items 0..total-1 in plain order off ctr[0], so every
// item still runs once; queue slots and items outside [0, total) are never
// dereferenced or returned.  Called by one thread.
__device__ inline int sched_take(const int32_t* __restrict__ hdr, const int32_t* __restrict__ items, int32_t* ctr,
                                 int total) {
  if (hdr[16] != total || hdr[17] != SCHED_MAGIC) {
    const int t = atomicAdd(&ctr[0], 1);
    return t < total ? t : -1;
  }
  const int x0 = (int)(blockIdx.x & 7u);
  for (int s = 0; s < 8; ++s) {
    const int x = (x0 + s) & 7;
    const int len = hdr[8 + x];
    if (__hip_atomic_load(&ctr[x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= len) continue;
    const int t = atomicAdd(&ctr[x], 1);
    if (t < len) {
      const int at = hdr[x] + t;
      if ((unsigned)at >= (unsigned)total) return -1;
      const int item = items[at];
      return (unsigned)item < (unsigned)total ? item : -1;
    }
  }
  return -1;
}

// Two consecutive items of one queue (pairs of query cubes): returns the first
// (-1 when every queue is empty) and sets `second` to the one after it in the
// same queue, or -1.  Each queue is taken two items at a time, so the pairs
// are the same whichever workgroup takes them; an unbuilt schedule gives the
// pairs (2t, 2t + 1) of the plain order.
__device__ inline int sched_take2(const int32_t* __restrict__ hdr, const int32_t* __restrict__ items, int32_t* ctr,
                                  int total, int& second) {
  second = -1;
  if (hdr[16] != total || hdr[17] != SCHED_MAGIC) {
    const int t = atomicAdd(&ctr[0], 2);
    if (t >= total) return -1;
    if (t + 1 < total) second = t + 1;
    return t;
  }
  const int x0 = (int)(blockIdx.x & 7u);
  for (int s = 0; s < 8; ++s) {
    const int x = (x0 + s) & 7;
    const int len = hdr[8 + x];
    if (__hip_atomic_load(&ctr[x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= len) continue;
    const int t = atomicAdd(&ctr[x], 2);
    if (t < len) {
      const int at = hdr[x] + t;
      if ((unsigned)at >= (unsigned)total) return -1;
      const int item = items[at];
      if ((unsigned)item >= (unsigned)total) return -1;
      if (t + 1 < len && (unsigned)(at + 1) < (unsigned)total) {
        const int it2 = items[at + 1];
        if ((unsigned)it2 < (unsigned)total) second = it2;
      }
      return item;
    }
  }
  return -1;
}

__host__ __device__ inline int xcd_grid(int items_per_bh, int bh_total) {
  return 8 * ((items_per_bh + 7) >> 3) * bh_total;
}

}  // namespace vsa2
