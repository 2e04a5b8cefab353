// Step A -- offline memory encoding: document-wise RoPE + chunk-mean pooling.
//
// hysenlabs.com "EverMind-AI/MSA: routing top-k compressed documents inside attention ...",
// sections "Memory must be encoded offline before a query can reach it" (one pass over the
// corpus caches chunk-pooled K, V, Kr) and "Document-wise RoPE resets every document to
// position zero"; yeyulingfeng.com "深度分析MSA ..." section 三 (mean pooling of each
// 64-token chunk into K-bar / V-bar / Kr-bar; a partial last chunk still counts).
//
// Design (HBM-bound streaming read, ~6 KB per token for the Qwen3-4B-like layer):
//  * The token rows are split over workgroups by bank rows, each workgroup taking a
//    contiguous range of whole chunks.  A thread owns one 8-element "unit" of a token row -- 8
//    consecutive elements, or for a rotated tensor 4 rotation pairs (i..i+3 together with
//    i+d/2..i+d/2+3) -- and streams its unit through the range token by token, 8 tokens
//    per batch with the next batch's loads in flight, so the workgroup reads its range as
//    one coalesced stream.  The sum runs in float32 registers, in token order.
//  * Chunk and document boundaries are the same for every thread of the workgroup: when
//    the stream reaches the end of a chunk, the chunk's mean is stored and the sum
//    restarts.
//  * Rotation by in-document position p = s + r (s = first position of the chunk) is split
//    as R(s) * R(r): each token is rotated by R(r) from a per-workgroup LDS table
//    (cos/sin of r*theta_i, r < chunk, evaluated in double precision), and R(s) is applied
//    once to the chunk sum.  R(s) is kept in double precision and advanced by R(chunk) from
//    chunk to chunk of a document (identity at its start), so every row is computed the
//    same way whatever range holds it.  Both are rotations, so the result is the same mean
//    up to float32 rounding.
//  * The mean divides by the number of real tokens with an IEEE division (a constant chunk
//    pools to itself bit for bit), then rounds once to the storage type.
//  * Row c of document d's chunk j is chunk_off[d] + j: offsets that start past 0 write new
//    documents after the rows a bank already holds.  bf16 routing keys are written in the
//    tiled layout of common.hpp: workgroup ranges start on multiples of 16 rows, and each
//    routing-key wave collects 8 consecutive rows in its own 8 KB of LDS, then writes them
//    as whole 128-byte lines of the tile (16-byte stores per thread scattered over the
//    tile cost 8% of the pass; this leaves about 1%).  Rows of a group of 8 that a range
//    shares with the previous bank contents or ends inside go straight out.  Only the rows
//    of the given documents are written.

#include "common.hpp"
#include "launch.hpp"

namespace msa {
namespace {

// One lane's unit of one token row, as stored (converted to float when used).
template <typename T> struct Raw;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <> struct Raw<bf16_t> {
  uint4 v;
  // Token rows are read once: the non-temporal hint keeps them from displacing other lines
  // (10.8 ms instead of 11.7 ms for the 10M-token encode; on the rotated K's 8-byte halves
  // it was slower, so those keep ordinary loads).
  __device__ __forceinline__ void load8(const bf16_t* p) {
    v = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
  }
  __device__ __forceinline__ void load4x2(const bf16_t* lo, const bf16_t* hi) {
    const uint2 x = *reinterpret_cast<const uint2*>(lo), y = *reinterpret_cast<const uint2*>(hi);
    v = make_uint4(x.x, x.y, y.x, y.y);
  }
  __device__ __forceinline__ void get(float* f) const { unpack8(v, f); }
};
template <> struct Raw<float> {
  float4 x, y;
  __device__ __forceinline__ void load8(const float* p) {
    x = *reinterpret_cast<const float4*>(p);
    y = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void load4x2(const float* lo, const float* hi) {
    x = *reinterpret_cast<const float4*>(lo);
    y = *reinterpret_cast<const float4*>(hi);
  }
  __device__ __forceinline__ void get(float* f) const {
    f[0] = x.x; f[1] = x.y; f[2] = x.z; f[3] = x.w; f[4] = y.x; f[5] = y.y; f[6] = y.z; f[7] = y.w;
  }
};

constexpr int PT = 8;  // tokens per batch

// A workgroup-uniform int64 read through the scalar cache, waited for in the same asm
// block.  The document offsets are read this way inside the stream: the compiler cannot
// prove that the kernel's own stores leave them alone, and a vector load there would make
// the stream wait for every load in flight.
__device__ __forceinline__ int64_t scalar_load_i64(const int64_t* p) {
  int64_t v;
  asm volatile("s_load_dwordx2 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

// First token of workgroup range w of W.  Range boundaries fall on bank rows that are
// multiples of 16 (whole tiles of the routing keys; ranges hold whole chunks), spread evenly
// over the rows written.  Also returns the document owning that token.  Wave-collective.
__device__ __forceinline__ int64_t range_start(const PoolArgs& a, int64_t w, int64_t W, int& doc) {
  if (w <= 0) { doc = 0; return 0; }
  if (w >= W) { doc = a.n_docs; return a.n_tokens; }
  const int64_t r0 = a.chunk_off[0];
  const int64_t r = (r0 + a.n_chunks * w / W) & ~(int64_t)15;
  if (r <= r0) { doc = 0; return 0; }
  doc = __builtin_amdgcn_readfirstlane(find_doc_wave(a.chunk_off, a.n_docs, r));
  return a.doc_tok_off[doc] + (r - a.chunk_off[doc]) * a.chunk;
}

// Bank row of token p, the first token of a chunk of document doc (doc == n_docs: the end).
__device__ __forceinline__ int64_t row_of(const PoolArgs& a, int64_t p, int doc) {
  if (doc >= a.n_docs) return a.chunk_off[a.n_docs];
  return a.chunk_off[doc] + (p - a.doc_tok_off[doc]) / a.chunk;
}

// State of one thread's stream.  The chunk fields are the same in every thread of the
// workgroup: current chunk [cst, bnd) of document doc ([doc_s, doc_e)), bank row c.
struct PoolStream {
  float acc[8];
  // cos / sin of s * theta_q for the current chunk start s (double); the step rotation
  // by one chunk, chunk * theta_q
  double rc[4], rs[4], stc[4], sts[4];
  int64_t cst, bnd, c, doc_s, doc_e;
  int doc;
  bool tiled;  // destination is a bf16 routing-key bank in the tiled layout
  int heads;   // heads of the destination tensor
  // Tiled destination staged in LDS, 8 rows at a time (null: stores go straight out).  A
  // wave's 64 units of a row are 16 whole 512-element blocks of a tile (first_blk ..), so
  // 8 rows of them fill 16 x 4 whole 128-byte lines of the tile.
  bf16_t* stage;          // this wave's staging region in LDS
  int first_blk, n_blk;   // the wave's blocks of a tile row
  int64_t row0, row1;     // bank rows of the workgroup's range
};

// Mean of the finished chunk [cst, bnd) -> bank row c, then move to the next chunk.
template <bool rotate, typename T, int D>
__device__ __forceinline__ void pool_flush(PoolStream& st, const PoolArgs& a, T* dst, int row_elems,
                                           int e_lo, int e_hi, bool store) {
  if constexpr (rotate) {  // R(s), s = first in-document position of the chunk (identity at s = 0)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float c32 = (float)st.rc[q], s32 = (float)st.rs[q];
      const float x = st.acc[q], y = st.acc[4 + q];
      st.acc[q] = x * c32 - y * s32;
      st.acc[4 + q] = y * c32 + x * s32;
    }
  }
  const float fn = (float)(st.bnd - st.cst);
#pragma unroll
  for (int q = 0; q < 8; ++q) st.acc[q] = st.acc[q] / fn;
  // the unit's place in the row: row-major, or (bf16 routing keys) its 16-byte slot of the
  // row's tile, where 4 or 8 consecutive elements of one head stay contiguous
  const int64_t grp = st.c & ~(int64_t)7;  // the row's group of 8 rows
  if constexpr (sizeof(T) == 2) {
    if (st.stage != nullptr && grp >= st.row0 && grp + 8 <= st.row1) {  // uniform
      // staged: the group's 8 rows leave together, as whole 128-byte lines of the tile
      const int r = (int)(st.c & 7);
      // region element offset of element e of row r: piece (block e/32 of the wave's, group
      // (e%32)/8, row r), then e%8
      auto region = [&](int e) { return (((e >> 5) - st.first_blk) * 4 + ((e >> 3) & 3)) * 64 + r * 8 + (e & 7); };
      if (store) {
        if constexpr (rotate) {
          Elem<T>::store4((T*)st.stage + region(e_lo), st.acc);
          Elem<T>::store4((T*)st.stage + region(e_hi), st.acc + 4);
        } else {
          Elem<T>::store8((T*)st.stage + region(e_lo), st.acc);
        }
      }
      if (r == 7) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's staged rows are in LDS
        const int lane = threadIdx.x & 63;
        T* tile = dst + (grp >> 4) * ((int64_t)16 * row_elems);
#pragma unroll 1
        for (int p = lane; p < st.n_blk * 32; p += 64) {  // 16-byte piece p: block p/32, group (p/8)%4, row p%8
          const int slot = (st.first_blk + (p >> 5)) * 64 + ((p >> 3) & 3) * 16 + (int)(grp & 15) + (p & 7);
          *reinterpret_cast<uint4*>(tile + slot * 8) = *reinterpret_cast<const uint4*>((const T*)st.stage + p * 8);
        }
      }
    } else {
      const int64_t o_lo = st.tiled ? kr_tiled<D>(st.c, e_lo, st.heads) : st.c * row_elems + e_lo;
      const int64_t o_hi = st.tiled ? kr_tiled<D>(st.c, e_hi, st.heads) : st.c * row_elems + e_hi;
      if (store) {
        if constexpr (rotate) {
          Elem<T>::store4(dst + o_lo, st.acc);
          Elem<T>::store4(dst + o_hi, st.acc + 4);
        } else {
          Elem<T>::store8(dst + o_lo, st.acc);
        }
      }
    }
  } else {
    (void)grp;
    const int64_t o_lo = st.c * row_elems + e_lo, o_hi = st.c * row_elems + e_hi;
    if (store) {
      if constexpr (rotate) {
        Elem<T>::store4(dst + o_lo, st.acc);
        Elem<T>::store4(dst + o_hi, st.acc + 4);
      } else {
        Elem<T>::store8(dst + o_lo, st.acc);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) st.acc[q] = 0.f;
  ++st.c;
  st.cst = st.bnd;
  if (st.cst == st.doc_e && st.doc + 1 < a.n_docs) {  // next document: positions restart
    ++st.doc;
    st.doc_s = st.doc_e;
    st.doc_e = scalar_load_i64(a.doc_tok_off + st.doc + 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) { st.rc[q] = 1.0; st.rs[q] = 0.0; }
  } else {  // next chunk of the same document: s advances by one chunk
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const double c0 = st.rc[q], s0 = st.rs[q];
      st.rc[q] = c0 * st.stc[q] - s0 * st.sts[q];
      st.rs[q] = s0 * st.stc[q] + c0 * st.sts[q];
    }
  }
  st.bnd = min(st.cst + a.chunk, st.doc_e);
}

// Tokens t0 .. t0 + PT - 1 of this thread's unit (past the range: its last token again).
template <bool rotate, typename T>
__device__ __forceinline__ void pool_load(Raw<T> (&X)[PT], const T* src, int64_t t0, int64_t p1,
                                          int row_elems, int e_lo, int e_hi) {
#pragma unroll
  for (int k = 0; k < PT; ++k) {
    const int64_t t = min(t0 + k, p1 - 1);
    const T* p = src + t * row_elems;
    if constexpr (rotate) X[k].load4x2(p + e_lo, p + e_hi);
    else X[k].load8(p + e_lo);
  }
}

template <bool rotate, typename T, int D>
__device__ __forceinline__ void pool_batch(PoolStream& st, const Raw<T> (&X)[PT], int64_t t0, int64_t p1,
                                           const PoolArgs& a, T* dst, int row_elems, int e_lo, int e_hi,
                                           bool store, const float* rope_tab, int half, int i0) {
#pragma unroll
  for (int k = 0; k < PT; ++k) {
    const int64_t t = t0 + k;
    if (t >= p1) break;  // uniform
    if (t == st.bnd) pool_flush<rotate, T, D>(st, a, dst, row_elems, e_lo, e_hi, store);
    float v[8];
    X[k].get(v);
    if constexpr (rotate) {
      const int r = (int)(t - st.cst);
      const float4 cs = *reinterpret_cast<const float4*>(rope_tab + r * half + i0);
      const float4 sn = *reinterpret_cast<const float4*>(rope_tab + a.chunk * half + r * half + i0);
      const float cq[4] = {cs.x, cs.y, cs.z, cs.w}, sq[4] = {sn.x, sn.y, sn.z, sn.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float x = v[q], y = v[4 + q];
        st.acc[q] += x * cq[q] - y * sq[q];
        st.acc[4 + q] += y * cq[q] + x * sq[q];
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) st.acc[q] += v[q];
    }
  }
}

// The stream of one thread's unit through token range [p0, p1) (whole chunks, starting in
// document doc0).
template <bool rotate, typename T, int D>
__device__ __forceinline__ void pool_stream(const PoolArgs& a, const T* src, T* dst, int64_t p0, int64_t p1,
                                            int doc0, int row_elems, int e_lo, int e_hi, int i0, bool valid,
                                            const float* rope_tab, bool tiled, bf16_t* stage, int first_unit,
                                            int n_units, int64_t row0, int64_t row1) {
  PoolStream st;
  st.tiled = tiled;
  st.heads = row_elems / D;
  st.stage = stage;
  st.row0 = __builtin_amdgcn_readfirstlane(row0);
  st.row1 = __builtin_amdgcn_readfirstlane(row1);
  st.first_blk = first_unit / 4;
  st.n_blk = (n_units + 3) / 4;
#pragma unroll
  for (int q = 0; q < 8; ++q) st.acc[q] = 0.f;
  st.doc = doc0;
  st.doc_s = a.doc_tok_off[doc0];
  st.doc_e = a.doc_tok_off[doc0 + 1];
  st.cst = p0;
  st.bnd = min(p0 + a.chunk, st.doc_e);
  st.c = a.chunk_off[doc0] + (p0 - st.doc_s) / a.chunk;
  // The one-chunk step rotation, and R(s) of the first chunk reached by that same recurrence
  // from the document's start, so a row's value does not depend on where ranges begin
  // (pooling documents in several calls, or with another grid, gives the same bits).
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    st.rc[q] = 1.0; st.rs[q] = 0.0; st.stc[q] = 1.0; st.sts[q] = 0.0;
    if constexpr (rotate) {
      const double th = pow((double)a.rope_base, -2.0 * (double)(i0 + q) / (double)D);
      sincos((double)a.chunk * th, &st.sts[q], &st.stc[q]);
    }
  }
  if constexpr (rotate) {
    for (int64_t j = (p0 - st.doc_s) / a.chunk; j > 0; --j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double c0 = st.rc[q], s0 = st.rs[q];
        st.rc[q] = c0 * st.stc[q] - s0 * st.sts[q];
        st.rs[q] = s0 * st.stc[q] + c0 * st.sts[q];
      }
    }
  }

  // Two batches: one summed while the other is in flight.  Loads are unconditional
  // (clamped to the range) so each wait targets the older batch only.
  Raw<T> X0[PT], X1[PT];
  pool_load<rotate>(X0, src, p0, p1, row_elems, e_lo, e_hi);
  pool_load<rotate>(X1, src, p0 + PT, p1, row_elems, e_lo, e_hi);
  for (int64_t t0 = p0; t0 < p1; t0 += 2 * PT) {
    pool_batch<rotate, T, D>(st, X0, t0, p1, a, dst, row_elems, e_lo, e_hi, valid, rope_tab, D / 2, i0);
    pool_load<rotate>(X0, src, t0 + 2 * PT, p1, row_elems, e_lo, e_hi);
    if (t0 + PT < p1)
      pool_batch<rotate, T, D>(st, X1, t0 + PT, p1, a, dst, row_elems, e_lo, e_hi, valid, rope_tab, D / 2, i0);
    pool_load<rotate>(X1, src, t0 + 3 * PT, p1, row_elems, e_lo, e_hi);
  }
  pool_flush<rotate, T, D>(st, a, dst, row_elems, e_lo, e_hi, valid);  // the range ends at a chunk end
}

template <typename T, int D>
__global__ __launch_bounds__(512) void pool_kernel(PoolArgs a) {
  extern __shared__ float rope_tab[];  // [chunk][D/2] cos, then [chunk][D/2] sin
  const int tid = threadIdx.x, lane = tid & 63;
  const int units_per_head = D / 8;
  const int half = D / 2;
  // Waves are assigned whole to one tensor (K, then V, then Kr; each tensor's units padded
  // to a whole number of waves), so the tensor, its pointers and whether it is rotated are
  // the same across a wave.
  const int nk = a.h_kv * units_per_head, nr = a.h_r * units_per_head;
  const int wk = (nk + 63) / 64, wr = (nr + 63) / 64;
  const int gw = __builtin_amdgcn_readfirstlane(blockIdx.y * (blockDim.x >> 6) + (tid >> 6));
  int tensor, first;  // first unit of this wave within its tensor
  if (gw < wk) { tensor = 0; first = gw * 64; }
  else if (gw < 2 * wk) { tensor = 1; first = (gw - wk) * 64; }
  else { tensor = 2; first = (gw - 2 * wk) * 64; }
  const int n_t = tensor == 2 ? nr : nk;
  const bool valid = gw < 2 * wk + wr && first + lane < n_t;
  const int unit = min(first + lane, n_t - 1);  // lanes past the tensor load its last unit
  const T* src = tensor == 0 ? (const T*)a.K : tensor == 1 ? (const T*)a.V : (const T*)a.Kr;
  T* dst = tensor == 0 ? (T*)a.Kbar : tensor == 1 ? (T*)a.Vbar : (T*)a.Krbar;
  const int heads = tensor == 2 ? a.h_r : a.h_kv;
  const int head = unit / units_per_head, piece = unit % units_per_head;
  const bool rotate = (a.rope_mask >> tensor) & 1u;  // uniform
  // Element offsets of the unit inside one token row of its tensor.
  const int e_lo = head * D + (rotate ? piece * 4 : piece * 8);
  const int e_hi = e_lo + half;  // second half of the rotation pairs
  const int i0 = piece * 4;      // first pair index when rotating
  const int row_elems = heads * D;

  // LDS: the table below, then (bf16 routing keys) 8 KB of staging per routing-key wave
  bf16_t* stage = nullptr;
  if (sizeof(T) == 2 && tensor == 2 && a.stage_waves > 0) {
    const int kr_first = max(2 * wk, (int)blockIdx.y * (int)(blockDim.x >> 6));  // first routing-key wave here
    stage = reinterpret_cast<bf16_t*>(reinterpret_cast<unsigned char*>(rope_tab) + a.stage_offset) +
            (size_t)(gw - kr_first) * (8 * 64 * 8);
  }

  // Per-workgroup table of R(r): angles r * theta_i, r < chunk, in double precision.
  if (a.rope_mask) {
    for (int e = tid; e < a.chunk * half; e += blockDim.x) {
      const int r = e / half, i = e % half;
      const double th = pow((double)a.rope_base, -2.0 * (double)i / (double)D);
      double sn, cs;
      sincos((double)r * th, &sn, &cs);
      rope_tab[e] = (float)cs;
      rope_tab[a.chunk * half + e] = (float)sn;
    }
  }
  __syncthreads();

  // Token range [p0, p1) of this workgroup; every lane takes part in the searches.
  int doc0, doc1;
  const int64_t p0 = range_start(a, blockIdx.x, gridDim.x, doc0);
  const int64_t p1 = range_start(a, (int64_t)blockIdx.x + 1, gridDim.x, doc1);
  if (p0 >= p1 || gw >= 2 * wk + wr) return;

  const bool tiled = tensor == 2 && sizeof(T) == 2;  // bf16 routing keys: tiled bank layout
  const int64_t row0 = row_of(a, p0, doc0), row1 = row_of(a, p1, doc1);
  const int n_units = min(64, n_t - first);
  if (rotate)
    pool_stream<true, T, D>(a, src, dst, p0, p1, doc0, row_elems, e_lo, e_hi, i0, valid, rope_tab, tiled, stage, first,
                            n_units, row0, row1);
  else
    pool_stream<false, T, D>(a, src, dst, p0, p1, doc0, row_elems, e_lo, e_hi, i0, valid, rope_tab, tiled, stage, first,
                             n_units, row0, row1);
}

template <typename T, int D>
hipError_t launch_pool_t(const PoolArgs& a, hipStream_t s) {
  const int nk = a.h_kv * (D / 8), nr = a.h_r * (D / 8);
  const int waves = 2 * ((nk + 63) / 64) + (nr + 63) / 64;  // whole waves per tensor
  int wpg = waves < 8 ? waves : 8;                          // waves per workgroup
  const int ygroups = (waves + wpg - 1) / wpg;
  const int threads = 64 * wpg;
  // Token ranges of one 16-row tile of the routing keys each (ranges hold whole tiles): many
  // short ranges keep the last round of workgroups small (2,048 longer ranges over the 768
  // that fit at once left a last round two-thirds full: 10.7-10.9 ms against 10.2-10.3 ms on
  // the 10M-token encode).
  const int64_t tiles = (a.n_chunks + 15) / 16 + 1;
  int64_t wgs = tiles;
  if (wgs < 1) wgs = 1;
  PoolArgs k = a;
  size_t lds = a.rope_mask ? (size_t)a.chunk * D * sizeof(float) : 0;
  k.stage_waves = 0;
  k.stage_offset = 0;
  if (sizeof(T) == 2) {
    // routing-key waves of the workgroup holding the most of them: 8 KB of staging each
    const int wk = (nk + 63) / 64, wr = (nr + 63) / 64;
    int most = 0;
    for (int y = 0; y < ygroups; ++y) {
      const int lo = y * wpg > 2 * wk ? y * wpg : 2 * wk, hi = (y + 1) * wpg < 2 * wk + wr ? (y + 1) * wpg : 2 * wk + wr;
      if (hi - lo > most) most = hi - lo;
    }
    const size_t off = (lds + 15) & ~(size_t)15;
    if (most <= 8 && off + (size_t)most * 8 * 64 * 16 <= 64 * 1024) {
      k.stage_offset = (int)off;
      k.stage_waves = most;
      lds = (size_t)k.stage_offset + (size_t)most * 8 * 64 * 16;
    }
  }
  dim3 grid((unsigned)wgs, (unsigned)ygroups);
  hipLaunchKernelGGL((pool_kernel<T, D>), grid, dim3(threads), lds, s, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const PoolArgs& a, hipStream_t s) {
  if (a.n_chunks == 0) return hipSuccess;
  if (a.dtype == 0) {
    switch (a.d) {
      case 32: return launch_pool_t<float, 32>(a, s);
      case 64: return launch_pool_t<float, 64>(a, s);
      default: return launch_pool_t<float, 128>(a, s);
    }
  }
  switch (a.d) {
    case 32: return launch_pool_t<bf16_t, 32>(a, s);
    case 64: return launch_pool_t<bf16_t, 64>(a, s);
    default: return launch_pool_t<bf16_t, 128>(a, s);
  }
}

}  // namespace msa
