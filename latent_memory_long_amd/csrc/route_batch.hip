// Step B for a batch of queries -- the router's scan of many queries in one pass.
//
// hysenlabs.com "EverMind-AI/MSA: routing top-k compressed documents inside attention ...",
// section "Routing happens inside attention ...": a document's relevance is the cosine of
// the query's routing vectors with the pooled routing keys, averaged over heads and
// maximised over the query's tokens; yeyulingfeng.com "深度分析MSA ..." section 五 step 2.
// The scores are those of route.hip:
//   s(t, c) = sum_h dot(Qr[t,h], Kb[c,h]) * rs[t,h] * cs[c,h],
//   rs = 1 / (H |Qr[t,h]|), cs = 1 / |Kb[c,h]|   (0 for a zero vector),
//   document score = max over its rows c and the query's tokens t.
//
// With many query rows the scan is a matrix product (query rows x bank rows, inner length
// H x 128) with a per-head scale and a max epilogue, so it is laid out for the matrix
// cores rather than for the bank read:
//  * Each wave keeps 16 bank rows of 8 heads (32 rows of 4 heads) in registers as MFMA B
//    operands for the whole launch, with their per-head 1/|k|: 128 registers, so two
//    waves share a SIMD.  The bank is in the tiled layout (common.hpp): each B operand is
//    one contiguous 1 KB block of a 16-row tile.  A workgroup is eight such waves and covers 128 (256) bank
//    rows; the bank is read from HBM once.
//  * Every query of the batch, padded to 16-row tiles, streams past those registers
//    through LDS in stages of two tiles (32 rows, all heads), double-buffered: the next
//    stage's rows are loaded into registers while the current stage is multiplied, then
//    written to LDS with their per-head 1/(H |q|).  LDS rows are padded by 32 bytes: a
//    16-byte LDS read is served 32 lanes at a time, and the MFMA operand pattern (16
//    rows x 2 column groups per 32 lanes) then touches 32 distinct 16-byte slots.
//  * v_mfma_f32_16x16x32_bf16 products (exact bf16 products, float32 sums) are scaled by
//    rs and cs in float32 and summed over heads in registers, as a pipeline over heads
//    (one head's products, the next head's LDS reads and the previous head's scaling in
//    flight together): no head exchange through LDS.  Each lane folds the maximum of its
//    four query rows of the tile into a running maximum while the tiles belong to one
//    query; the lanes of a bank row are combined once per query.
//  * When the query changes, each bank row's maximum is reduced over the rows of its
//    document inside the wave (a segmented max over lanes) and merged into the document
//    score with an integer atomic max/min on the float bits, after a fill of -inf.  The
//    maximum does not depend on the order of the merges.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace msa {
namespace {

constexpr int BD = 128;               // head dim
constexpr int BWAVES = 8;             // waves per workgroup, two per SIMD
constexpr int SQ = 32;                // query rows per stage: two 16-row tiles
constexpr int KS = BD / 32;           // 32-wide k steps per head
constexpr int BTHREADS = BWAVES * 64;

// 16-row bank tiles per wave: 128 registers of B operands whatever the head count
template <int H> constexpr int bank_tiles() { return 8 / H; }
template <int H> constexpr int bank_rows_per_group() { return BWAVES * bank_tiles<H>() * 16; }

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

struct BatchK {
  const bf16_t* Qr;
  const int32_t* q_off;
  const bf16_t* Krb;
  const int64_t* chunk_off;
  float* scores;  // [n_queries, n_docs], filled with -inf first
  float* row_scores;  // ARG: [n_queries, n_chunks] every bank row's max over the tokens
  int32_t* row_arg;   // ARG: [n_queries, n_chunks] the first token reaching it
  int64_t n_chunks;
  int n_docs;
  int n_queries;
};

// A 16-row tile of one query (wave-uniform): query b (n_queries when past the end),
// first token t0, query length lq, first row of the query in Qr.
struct Tile {
  int b, t0, lq, off;
};

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ Tile query_start(const BatchK& a, int b) {
  Tile t{b, 0, 0, 0};
  while (t.b < a.n_queries) {
    t.off = uni(a.q_off[t.b]);
    t.lq = uni(a.q_off[t.b + 1]) - t.off;
    if (t.lq > 0) break;
    ++t.b;
  }
  return t;
}

__device__ __forceinline__ Tile next_tile(const BatchK& a, const Tile& t) {
  if (t.b >= a.n_queries) return t;
  if (t.t0 + 16 < t.lq) return Tile{t.b, t.t0 + 16, t.lq, t.off};
  return query_start(a, t.b + 1);
}

// Float max through integer atomics: non-negative floats order like their int bits,
// negative ones reversely like their unsigned bits.  The target starts at -inf.
__device__ __forceinline__ void atomic_max_f32(float* p, float v) {
  if (!(v == v)) return;
  if (__float_as_int(v) >= 0) atomicMax(reinterpret_cast<int*>(p), __float_as_int(v));
  else atomicMin(reinterpret_cast<unsigned int*>(p), __float_as_uint(v));
}

// ARG: also record every bank row's score and the first query token reaching it (for the
// router's backward); the document scores are then left to the caller's -inf fill.
template <int H, bool ARG>
__global__ __launch_bounds__(BTHREADS) void route_scan_batch(BatchK a) {
  constexpr int BNT = bank_tiles<H>();
  constexpr int BROWS = bank_rows_per_group<H>();
  constexpr int HD = H * BD;
  constexpr int RS = HD + 16;           // LDS row stride in elements (32 B of padding)
  constexpr int CPR = HD / 8;           // 16-byte chunks per query row
  constexpr int CPT = SQ * CPR / BTHREADS;  // chunks per thread per stage
  static_assert(CPT * BTHREADS == SQ * CPR, "stage chunks must split evenly");
  __shared__ __align__(16) bf16_t Abuf[2][SQ * RS];
  __shared__ __align__(16) float rsb[2][H][SQ];

  const int tid = threadIdx.x, lane = tid & 63, w = uni(tid >> 6);
  const int cl = lane & 15, g = lane >> 4;
  const int64_t C = a.n_chunks;
  const int64_t base = (int64_t)blockIdx.x * BROWS + w * (BNT * 16);
  const bool has_rows = base < C;  // wave-uniform

  // ---- this wave's bank rows: B operands, 1/|k| per head, document of each column ----
  bf16x8_t Bt[BNT][H][KS];
  float cs[BNT][H];
  int doc[BNT];
  const int64_t last_tile = kr_tiles(C) - 1;
#pragma unroll
  for (int j = 0; j < BNT; ++j) {
    // tile of rows base + 16 j ..: one 1 KB block per (head, 32-dim slice), lane l holding
    // its B operand slot (columns past the bank are padding, masked through doc = -1)
    const int64_t c = base + j * 16 + cl;
    const bool valid = c < C;
    const bf16_t* p = a.Krb + min((base >> 4) + j, last_tile) * (16 * HD) + lane * 8;
#pragma unroll
    for (int h = 0; h < H; ++h)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        Bt[j][h][ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p + (h * KS + ks) * 512));
    // the norms read the rows a second time (from cache), so the B operands have no use
    // but the matrix products and may live in accumulation registers
#pragma unroll
    for (int h = 0; h < H; ++h) {
      float ss = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p + (h * KS + ks) * 512));
        ss = dot2_bf16(v.x, v.x, ss);
        ss = dot2_bf16(v.y, v.y, ss);
        ss = dot2_bf16(v.z, v.z, ss);
        ss = dot2_bf16(v.w, v.w, ss);
      }
      ss += __shfl_xor(ss, 16, 64);
      ss += __shfl_xor(ss, 32, 64);
      cs[j][h] = (valid && ss > 0.f) ? __builtin_amdgcn_rsqf(ss) : 0.f;
    }
    doc[j] = -1;
  }
  if (has_rows) {
    int d = find_doc_wave(a.chunk_off, a.n_docs, base);
#pragma unroll
    for (int j = 0; j < BNT; ++j) {
      const int64_t c = base + j * 16 + cl;
      if (c < C) {
        while (a.chunk_off[d + 1] <= c) ++d;
        doc[j] = d;
      }
    }
  }

  // ---- query stages ----
  // Wave w stages rows w*4 .. w*4+3 of the stage (all heads), so its rows lie in one tile
  // (waves 0..3: the first, 4..7: the second).  Load i of a lane holds 16 bytes of the
  // (row, head) pair p = (i / 2) * 8 + lane / 8 of the wave: its chunk (lane & 7) + 8 (i & 1).
  // The eight lanes of a pair and the lane's two loads of it cover the pair's 256 bytes,
  // so every load instruction reads eight whole 128-byte lines, and a pair's squared norm
  // is summed in the lane and over eight lanes.  A row past its query's end re-reads the
  // tile's last row: its scores are masked out before any maximum.
  static_assert(BWAVES * 4 == SQ && CPT * 64 == 4 * H * 16 && CPT % 4 == 0, "stage split");
  // The stage is loaded and committed in two halves (the wave's rows w*4, w*4+1, then
  // w*4+2, w*4+3): each half's loads are in flight during one tile's products, and only
  // half the stage occupies registers at a time.
  constexpr int CPH = CPT / 2;  // loads per half
  uint4 stage_regs[CPH];
  auto load_half = [&](const Tile& t0, const Tile& t1, int half) __attribute__((always_inline)) {
    const Tile& t = (w < BWAVES / 2) ? t0 : t1;  // uniform
    if (t.b >= a.n_queries) return;              // uniform: no such tile
    const char* tb = reinterpret_cast<const char*>(a.Qr + (int64_t)(t.off + t.t0) * HD);  // uniform
    const int last = t.lq - t.t0 - 1;
#pragma unroll
    for (int k = 0; k < CPH; ++k) {
      const int i = half * CPH + k;
      const int p = (i / 2) * 8 + (lane >> 3);
      const int row = (w * 4 + p / H) & 15, head = p % H, chunk = (lane & 7) + 8 * (i & 1);
      const uint32_t off = (uint32_t)(min(row, last) * (HD * 2) + head * (BD * 2) + chunk * 16);
      stage_regs[k] = *reinterpret_cast<const uint4*>(tb + off);
    }
  };
  auto commit_half = [&](const Tile& t0, const Tile& t1, int buf, int half) __attribute__((always_inline)) {
    if (((w < BWAVES / 2) ? t0 : t1).b >= a.n_queries) return;  // uniform: nothing was loaded
#pragma unroll
    for (int k = 0; k < CPH; k += 2) {
      const int i = half * CPH + k;
      const int p = (i / 2) * 8 + (lane >> 3);
      const int row = w * 4 + p / H, head = p % H, chunk = lane & 7;
      bf16_t* dst = &Abuf[buf][row * RS + head * BD + chunk * 8];
      const uint4 v0 = stage_regs[k], v1 = stage_regs[k + 1];
      *reinterpret_cast<uint4*>(dst) = v0;
      *reinterpret_cast<uint4*>(dst + 64) = v1;
      float ss = dot2_bf16(v0.x, v0.x, 0.f);
      ss = dot2_bf16(v0.y, v0.y, ss);
      ss = dot2_bf16(v0.z, v0.z, ss);
      ss = dot2_bf16(v0.w, v0.w, ss);
      ss = dot2_bf16(v1.x, v1.x, ss);
      ss = dot2_bf16(v1.y, v1.y, ss);
      ss = dot2_bf16(v1.z, v1.z, ss);
      ss = dot2_bf16(v1.w, v1.w, ss);
      ss = group_sum_last<8>(ss);  // the eight lanes of the pair
      if ((lane & 7) == 7) rsb[buf][head][row] = ss > 0.f ? __builtin_amdgcn_rsqf(ss) / (float)H : 0.f;
    }
  };

  float run[BNT];  // running max of each bank row over the current query's tiles
  int run_arg[BNT];  // ARG: the query-local token of that maximum
  int run_b = -1;
#pragma unroll
  for (int j = 0; j < BNT; ++j) {
    run[j] = -INFINITY;
    run_arg[j] = 0;
  }

  // Each lane's running maximum covers its own four rows of every tile; the four lane
  // groups of a column are combined once per query, here.  ARG keeps the first token: a
  // lane's tokens rise with its rows and tiles, and equal maxima take the smaller token.
  auto flush = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < BNT; ++j) {
      float x = run[j];
      int xi = run_arg[j];
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        const float ox = __shfl_xor(x, o, 64);
        if constexpr (ARG) {
          const int oi = __shfl_xor(xi, o, 64);
          if (ox > x || (ox == x && oi < xi)) {
            x = ox;
            xi = oi;
          }
        } else {
          x = fmaxf(x, ox);
        }
      }
      run[j] = x;
      run_arg[j] = xi;
    }
    if constexpr (ARG) {
#pragma unroll
      for (int j = 0; j < BNT; ++j) {
        const int64_t c = base + j * 16 + cl;
        if (lane < 16 && c < C) {
          a.row_scores[(int64_t)run_b * C + c] = run[j];
          a.row_arg[(int64_t)run_b * C + c] = run_arg[j];
        }
      }
      return;
    }
    float* sc = a.scores + (int64_t)run_b * a.n_docs;
#pragma unroll
    for (int j = 0; j < BNT; ++j) {
      // segmented max over the 16 columns of the tile, runs = documents
      float v = run[j];
      const int d = doc[j];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float ov = __shfl_up(v, o, 16);
        const int od = __shfl_up(d, o, 16);
        if (cl >= o && od == d) v = fmaxf(v, ov);
      }
      const int dn = __shfl_down(d, 1, 16);
      const bool last = (cl == 15) || dn != d;
      if (lane < 16 && d >= 0 && last) atomic_max_f32(sc + d, v);
    }
  };

  auto compute_tile = [&](const Tile& t, int buf, int tt) __attribute__((always_inline)) {
    const bf16_t* arow = &Abuf[buf][(tt * 16 + cl) * RS + g * 8];
    const float* rrow = &rsb[buf][0][tt * 16 + g * 4];
    float tot[BNT][4];
#pragma unroll
    for (int j = 0; j < BNT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) tot[j][i] = 0.f;
    // Software pipeline over heads: head h's products run while head h + 2's operands
    // load from LDS and head h - 1's products are scaled into the total (a ring of three
    // operand slots; head h - 1's slot takes head h + 2's operands once its products are
    // issued, so its row scales are copied out first).
    bf16x8_t A[3][KS];
    float4 r4[3];
    f32x4_t acc[2][BNT];
#pragma unroll
    for (int h = 0; h < 2 && h < H; ++h) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) A[h][ks] = *reinterpret_cast<const bf16x8_t*>(arow + h * BD + ks * 32);
      r4[h] = *reinterpret_cast<const float4*>(rrow + h * SQ);
    }
#pragma unroll
    for (int h = 0; h <= H; ++h) {
      const int cur = h % 3, prv = (h + 2) % 3;
      const int ac = h & 1, ap = ac ^ 1;
      const float4 rr = r4[prv];  // head h - 1's row scales
      if (h + 2 < H) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          A[prv][ks] = *reinterpret_cast<const bf16x8_t*>(arow + (h + 2) * BD + ks * 32);
        r4[prv] = *reinterpret_cast<const float4*>(rrow + (h + 2) * SQ);
      }
      if (h < H) {
#pragma unroll
        for (int j = 0; j < BNT; ++j) {
          acc[ac][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            acc[ac][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[cur][ks], Bt[j][h][ks], acc[ac][j], 0, 0, 0);
        }
      }
      if (h > 0) {
#pragma unroll
        for (int j = 0; j < BNT; ++j) {
          const float c = cs[j][h - 1];
          tot[j][0] += acc[ap][j][0] * rr.x * c;
          tot[j][1] += acc[ap][j][1] * rr.y * c;
          tot[j][2] += acc[ap][j][2] * rr.z * c;
          tot[j][3] += acc[ap][j][3] * rr.w * c;
        }
      }
    }
    // this lane's maximum over its four rows g*4 + i of the tile, past the query's end
    // masked (only a query's last tile has such rows: a uniform branch)
    const int nv = t.lq - t.t0;
    float m[BNT];
    int mi[BNT];  // ARG: the first row reaching it
#pragma unroll
    for (int j = 0; j < BNT; ++j) {
      float x = tot[j][0];
      int xi = 0;
      if (nv >= 16) {
#pragma unroll
        for (int i = 1; i < 4; ++i) {
          if (ARG) {
            if (tot[j][i] > x) {
              x = tot[j][i];
              xi = i;
            }
          } else {
            x = fmaxf(x, tot[j][i]);
          }
        }
      } else {
        x = (g * 4 < nv) ? x : -INFINITY;
#pragma unroll
        for (int i = 1; i < 4; ++i) {
          if (ARG) {
            if (g * 4 + i < nv && tot[j][i] > x) {
              x = tot[j][i];
              xi = i;
            }
          } else {
            x = (g * 4 + i < nv) ? fmaxf(x, tot[j][i]) : x;
          }
        }
      }
      m[j] = x;
      mi[j] = t.t0 + g * 4 + xi;
    }
    if (t.b != run_b) {
      if (run_b >= 0) flush();
      run_b = t.b;
#pragma unroll
      for (int j = 0; j < BNT; ++j) {
        run[j] = m[j];
        run_arg[j] = mi[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < BNT; ++j) {
        if (ARG) {
          if (m[j] > run[j]) {  // strictly: an earlier tile keeps a tie
            run[j] = m[j];
            run_arg[j] = mi[j];
          }
        } else {
          run[j] = fmaxf(run[j], m[j]);
        }
      }
    }
  };

  Tile t0 = query_start(a, 0);
  Tile t1 = next_tile(a, t0);
  if (t0.b >= a.n_queries) return;  // no query has tokens (uniform over the grid)
  load_half(t0, t1, 0);
  commit_half(t0, t1, 0, 0);
  load_half(t0, t1, 1);
  commit_half(t0, t1, 0, 1);
  __syncthreads();
  int cur = 0;
  while (t0.b < a.n_queries) {
    const Tile n0 = next_tile(a, t1);
    const Tile n1 = next_tile(a, n0);
    const bool more = n0.b < a.n_queries;
    // the other buffer is free: every wave finished the previous stage before the barrier
    if (more) load_half(n0, n1, 0);  // in flight during the first tile's products
    if (has_rows) compute_tile(t0, cur, 0);
    if (more) {
      commit_half(n0, n1, cur ^ 1, 0);
      load_half(n0, n1, 1);  // in flight during the second tile's products
    }
    if (has_rows && t1.b < a.n_queries) compute_tile(t1, cur, 1);
    if (more) commit_half(n0, n1, cur ^ 1, 1);
    __syncthreads();
    t0 = n0;
    t1 = n1;
    cur ^= 1;
  }
  if (has_rows && run_b >= 0) flush();
}

__global__ void fill_neg_inf(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = -INFINITY;
}

}  // namespace

// A fill kernel rather than a memset, so that the call can be captured in a graph.
hipError_t launch_fill_neg_inf(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_neg_inf, dim3((unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)), dim3(256), 0, s,
                     p, n);
  return hipGetLastError();
}

bool route_batch_supported(const RouteArgs& r) {
  return r.dtype == 1 && r.d == BD && (r.h_r == 4 || r.h_r == 8);
}

template <int H>
hipError_t launch_h(const RouteArgs& r, const BatchK& k, hipStream_t s) {
  const dim3 grid((unsigned)((r.n_chunks + bank_rows_per_group<H>() - 1) / bank_rows_per_group<H>()));
  if (k.row_scores) hipLaunchKernelGGL((route_scan_batch<H, true>), grid, dim3(BTHREADS), 0, s, k);
  else hipLaunchKernelGGL((route_scan_batch<H, false>), grid, dim3(BTHREADS), 0, s, k);
  return hipGetLastError();
}

hipError_t launch_route_scan_batch(const RouteArgs& r, hipStream_t s) {
  BatchK k{(const bf16_t*)r.Qr, r.q_off, (const bf16_t*)r.Krbar, r.chunk_off, r.scores, r.row_scores,
           r.row_arg, r.n_chunks, r.n_docs, r.n_queries};
  // -inf: the value of an empty maximum (documents without rows, queries without tokens,
  // and, with row scores, every document: the router's backward reads the rows only)
  const hipError_t e = launch_fill_neg_inf(r.scores, (int64_t)r.n_queries * r.n_docs, s);
  if (e != hipSuccess) return e;
  return r.h_r == 8 ? launch_h<8>(r, k, s) : launch_h<4>(r, k, s);
}

}  // namespace msa
