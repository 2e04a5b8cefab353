// Device helpers shared by the MSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr float LN2 = 0.69314718055994531f;    // ln 2: log2-domain values to natural log
constexpr float LOG2E = 1.44269504088896341f;  // log2 e: natural log to log2 domain

// 2^x on the hardware's v_exp_f32 (about 1 ulp), without the library's rescaling for results
// below 2^-126: softmax weights that small only ever round to zero or a denormal, which no
// sum notices.  exp2_hw(-inf) = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- element types -------------------------------------------------------------------
// bf16 is carried as its 16-bit pattern: the upper half of an IEEE float32.
typedef uint16_t bf16_t;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float32 -> bf16, round to nearest, ties to even (NaN stays NaN): gfx950 converts in
// hardware, two values per v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// two floats -> packed bf16 pair (a in the low half)
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Unpack 8 bf16 (one 16-byte word) into floats.
__device__ __forceinline__ void unpack8(const uint4& w, float* f) {
  f[0] = __uint_as_float(w.x << 16); f[1] = __uint_as_float(w.x & 0xffff0000u);
  f[2] = __uint_as_float(w.y << 16); f[3] = __uint_as_float(w.y & 0xffff0000u);
  f[4] = __uint_as_float(w.z << 16); f[5] = __uint_as_float(w.z & 0xffff0000u);
  f[6] = __uint_as_float(w.w << 16); f[7] = __uint_as_float(w.w & 0xffff0000u);
}

__device__ __forceinline__ void unpack4(const uint2& w, float* f) {
  f[0] = __uint_as_float(w.x << 16); f[1] = __uint_as_float(w.x & 0xffff0000u);
  f[2] = __uint_as_float(w.y << 16); f[3] = __uint_as_float(w.y & 0xffff0000u);
}

__device__ __forceinline__ uint4 pack8(const float* f) {
  uint4 w;
  w.x = f32x2_to_bf16x2(f[0], f[1]);
  w.y = f32x2_to_bf16x2(f[2], f[3]);
  w.z = f32x2_to_bf16x2(f[4], f[5]);
  w.w = f32x2_to_bf16x2(f[6], f[7]);
  return w;
}

__device__ __forceinline__ uint2 pack4(const float* f) {
  uint2 w;
  w.x = f32x2_to_bf16x2(f[0], f[1]);
  w.y = f32x2_to_bf16x2(f[2], f[3]);
  return w;
}

// Load / store n contiguous elements (n = 4 or 8) as floats, for either storage type.
template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static void load8(const float* p, float* f) {
    float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  __device__ __forceinline__ static void load4(const float* p, float* f) {
    float4 a = *reinterpret_cast<const float4*>(p);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  }
  __device__ __forceinline__ static void store8(float* p, const float* f) {
    *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
  }
  __device__ __forceinline__ static void store4(float* p, const float* f) {
    *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static void load8(const bf16_t* p, float* f) {
    unpack8(*reinterpret_cast<const uint4*>(p), f);
  }
  __device__ __forceinline__ static void load4(const bf16_t* p, float* f) {
    unpack4(*reinterpret_cast<const uint2*>(p), f);
  }
  __device__ __forceinline__ static void store8(bf16_t* p, const float* f) {
    *reinterpret_cast<uint4*>(p) = pack8(f);
  }
  __device__ __forceinline__ static void store4(bf16_t* p, const float* f) {
    *reinterpret_cast<uint2*>(p) = pack4(f);
  }
};

// ---- routing-key bank layout ------------------------------------------------------------
// bf16 routing keys (Kr-bar) are stored in tiles of 16 bank rows, laid out for the matrix
// cores: tile T holds rows 16T..16T+15 as H x (D/32) blocks of 512 elements, in (head,
// 32-dim slice) order.  Block (h, s) is the B operand of v_mfma_f32_16x16x32_bf16 for head
// h, dims 32s..32s+31 of the tile's rows: lane l = 16 g + r holds the 8 elements of dims
// 32s + 8g .. 32s + 8g + 7 of row 16T + r.  A bank of C rows occupies ceil(C/16) whole
// tiles; the rows past C in the last tile are padding (zero when the library writes them).
// Each 1 KB block is one contiguous load instruction of a wave, and a tile is 16 rows of
// every head in one contiguous run.  float32 routing keys stay row-major [C, H, D].
__host__ __device__ __forceinline__ int64_t kr_tiles(int64_t n_rows) { return (n_rows + 15) >> 4; }

// Element offset of element i = h * D + e of bank row c in the tiled layout.  Elements
// i .. i+7 with i % 8 == 0 are contiguous.
template <int D>
__device__ __forceinline__ int64_t kr_tiled(int64_t c, int i, int H) {
  const int h = i / D, e = i % D;
  return (c >> 4) * ((int64_t)16 * H * D) + (int64_t)((h * (D / 32) + (e >> 5)) << 9) +
         (((((e & 31) >> 3) << 4) | (int)(c & 15)) << 3) + (e & 7);
}

// ---- order-preserving score keys -------------------------------------------------------
// Maps a float to a uint32 whose unsigned order is the float order (-0.0 folded into
// +0.0).  Key 0 sorts below every non-NaN float and marks "no score yet".
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  if (k == 0u) return -INFINITY;  // never scored (a query with no tokens)
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// ---- wave64 reductions ------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---- DPP reductions (gfx9 data-parallel primitives, no LDS traffic) ----------------------
// dpp_ctrl codes: row_shr:n = 0x110 + n, row_bcast:15 = 0x142, row_bcast:31 = 0x143.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_keep(float v) {  // lanes without a source keep v
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL,
                                                    ROW_MASK, 0xf, false));
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_zero(float v) {  // lanes without a source read 0
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
// Sum over groups of N consecutive lanes (N = 2..16 dividing 16): the group's last lane
// receives the total.
template <int N>
__device__ __forceinline__ float group_sum_last(float v) {
  if (N > 1) v += dpp_zero<0x111>(v);
  if (N > 2) v += dpp_zero<0x112>(v);
  if (N > 4) v += dpp_zero<0x114>(v);
  if (N > 8) v += dpp_zero<0x118>(v);
  return v;
}
// Double-precision variants (the two 32-bit halves move together).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_zero(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xffffffff), CTRL, ROW_MASK, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, ROW_MASK, 0xf, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
template <int N>
__device__ __forceinline__ double group_sum_last(double v) {
  if (N > 1) v += dpp_zero<0x111>(v);
  if (N > 2) v += dpp_zero<0x112>(v);
  if (N > 4) v += dpp_zero<0x114>(v);
  if (N > 8) v += dpp_zero<0x118>(v);
  return v;
}
__device__ __forceinline__ double wave_sum_last(double v) {
  v = group_sum_last<16>(v);
  v += dpp_zero<0x142, 0xa>(v);
  v += dpp_zero<0x143, 0xc>(v);
  return v;
}

// Sum over the whole wave; lane 63 receives the total.
__device__ __forceinline__ float wave_sum_last(float v) {
  v = group_sum_last<16>(v);
  v += dpp_zero<0x142, 0xa>(v);
  v += dpp_zero<0x143, 0xc>(v);
  return v;
}
// Max over groups of 32 lanes: lanes 31 and 63 receive their half's maximum.
__device__ __forceinline__ float half_max_last(float v) {
  v = fmaxf(v, dpp_keep<0x111>(v));
  v = fmaxf(v, dpp_keep<0x112>(v));
  v = fmaxf(v, dpp_keep<0x114>(v));
  v = fmaxf(v, dpp_keep<0x118>(v));
  v = fmaxf(v, dpp_keep<0x142, 0xa>(v));
  return v;
}
// Max over the wave, broadcast to every lane.
__device__ __forceinline__ float wave_max_all(float v) {
  v = half_max_last(v);
  v = fmaxf(v, dpp_keep<0x143, 0xc>(v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// bf16 pair dot product accumulated in float32 (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                         c, false);
}

// Workgroup barrier that waits only for LDS traffic, so global loads issued earlier
// (prefetches) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Index of the document owning bank row c: the largest d with chunk_off[d] <= c, found by
// one wave with 64-way search (a few dependent loads instead of log2(N)).  All lanes
// return the same value.
__device__ __forceinline__ int find_doc_wave(const int64_t* chunk_off, int n_docs, int64_t c) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = n_docs;  // invariant: chunk_off[lo] <= c, answer in [lo, hi)
  while (hi - lo > 1) {
    const int span = hi - lo;
    // span <= 64: one lane per candidate; else 64 strictly increasing sample points.
    const int p = (span <= 64) ? lo + lane : lo + (int)(((int64_t)span * lane) / 64);
    const bool ok = (p < hi) && (chunk_off[p] <= c);
    const uint64_t m = __ballot(ok);              // lane 0 (p = lo) is always set
    const int best = 63 - __clzll((long long)m);  // highest lane with chunk_off[p] <= c
    if (span <= 64) return lo + best;
    const int pn = (best == 63) ? hi : lo + (int)(((int64_t)span * (best + 1)) / 64);
    lo = lo + (int)(((int64_t)span * best) / 64);
    hi = pn;
  }
  return lo;
}

// Documents [d0, d1) of part p out of P: the part starts at the first document whose first
// bank row is >= p * C / P, so every document belongs to exactly one part and parts hold
// nearly equal numbers of rows.  Wave-collective (all lanes must call).
__device__ __forceinline__ int part_first_doc(const int64_t* chunk_off, int n_docs,
                                              int64_t n_chunks, int64_t p, int64_t P) {
  if (p <= 0) return 0;
  if (p >= P) return n_docs;
  const int64_t x = n_chunks * p / P;
  const int d = find_doc_wave(chunk_off, n_docs, x);
  return (chunk_off[d] == x) ? d : d + 1;
}

// Part and query of this workgroup in a (parts x queries) grid.  Workgroups go to the
// eight XCDs round-robin in linear order (x fastest).  With several queries and a part
// count divisible by 8, the linear id is remapped so that the queries of one part run on
// the same XCD one after another: after the first reads a part's rows from HBM, the others
// find them in that XCD's L2.  Otherwise the grid coordinates are used as they are.
__device__ __forceinline__ void part_and_query(int& part, int& query) {
  const unsigned P = gridDim.x, B = gridDim.y;
  if (B == 1 || (P & 7u)) {
    part = (int)blockIdx.x;
    query = (int)blockIdx.y;
    return;
  }
  const unsigned L = blockIdx.y * P + blockIdx.x;
  const unsigned slot = L >> 3;  // position in this XCD's sequence
  part = (int)((slot / B) * 8u + (L & 7u));
  query = (int)(slot % B);
}

}  // namespace msa
