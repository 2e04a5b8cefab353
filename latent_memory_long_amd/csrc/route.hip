// Step B -- the router's scan of a query's routing vectors against every bank row.
//
// hysenlabs.com "EverMind-AI/MSA: routing top-k compressed documents inside attention ...",
// section "Routing happens inside attention ...": relevance is the cosine similarity of the
// query's routing vectors with the pooled routing keys, averaged over heads and then
// maximised over the query's tokens; yeyulingfeng.com "深度分析MSA ..." section 五 step 2
// (Q_r against Kr-bar gives a document score used for top-k).  A document's score is the
// maximum over its rows (the pages leave the chunk-to-document rule open; max keeps the
// token-wise maximum's spirit and makes max over (token, row) one reduction).
//
//   s(t, c) = sum_h dot(Qr[t,h], Kb[c,h]) * rs[t,h] * cs[c,h],
//   rs = 1 / (H * |Qr[t,h]|), cs = 1 / |Kb[c,h]|   (0 when the norm is 0),
//   S(c) = max_t s(t, c),  D(d) = max_{c in d} S(c).
//
// Work is split into document-aligned parts (each part starts at a document boundary), so
// every document's score is produced by exactly one wave with a plain store: no atomics,
// no initialisation pass, and the result does not depend on scheduling.
//
// The scan reads each bank row once (H * d * 2 bytes per row in bf16) and does
// 2 * Lq * H * d flops on it, so it is bound by HBM bandwidth unless Lq is in the
// hundreds.  Two kernels:
//  * route_scan_mfma (bf16 banks in the tiled layout of common.hpp, up to 8 routing heads,
//    any query length, a pass per 64 query rows): eight waves per part.  Each wave owns
//    whole 16-row tiles (its part's tiles w, w + 8, ...) and computes every head of them,
//    so waves never wait for one another inside a window.  The query rows of every head
//    sit in LDS as MFMA A operands (v_mfma_f32_16x16x32_bf16) with their 1/(H |q|); a
//    tile's head blocks stream from HBM straight into registers as B operands, one 1 KB
//    contiguous load per instruction, through a ring of four (tile, head) blocks with the
//    non-temporal hint.  Row norms are the diagonal of B^T B (one more MFMA chain on the
//    same registers), broadcast to the column's lanes; scaled head products are summed in
//    registers, and the maximum over the query's tokens is reduced across the column's
//    lanes.  Row scores collect in one of two LDS windows of rows, folded into documents
//    by all waves once per window.
//  * route_scan_dot (float32 banks, row-major; bf16 banks with more than 8 routing heads,
//    tiled): each wave streams its own range of rows, four rows per step with the next
//    four in flight; a lane holds 8 elements of a row, head sums and the head mean use DPP
//    lane shifts.
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace msa {
namespace {

struct ScanK {
  const void* Qr;
  const int32_t* q_off;
  const void* Krb;
  const int64_t* chunk_off;
  float* scores;      // [n_queries, n_docs]
  float* row_scores;  // [n_queries, n_chunks] or null: max over the query's tokens per bank row
  int32_t* row_arg;   // [n_queries, n_chunks], with row_scores: the first token reaching it
  int64_t n_chunks;
  int n_docs;
  int H;
};

__device__ __forceinline__ int64_t load_window(const int64_t* chunk_off, int n_docs, int wb) {
  const int di = wb + 1 + (int)(threadIdx.x & 63);
  return (di <= n_docs) ? chunk_off[di] : INT64_MAX;
}

// ------------------------------------------------------------------------------------
// MFMA scan of a bf16 bank in the tiled layout.
// ------------------------------------------------------------------------------------
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
// Bank tiles are read once: the non-temporal hint streams them past the caches (measured on
// the 100M-token bank: a plain read of this pattern reaches 76% of peak, with the hint 86%).
__device__ __forceinline__ bf16x8_t load_nt(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8_t, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}

constexpr int SCAN_WAVES = 8;  // waves per workgroup of the MFMA scan
constexpr int SCAN_RING = 4;   // (tile, head) blocks of loads per wave: three in flight during one
template <int MT, int D, bool ARG>
__global__ __launch_bounds__(512) void route_scan_mfma(ScanK a) {
  constexpr int KK = D / 32;
  constexpr int HMAX = 8;
  constexpr int WINR = ARG ? 1024 : 2048;  // rows per score window (two windows in LDS)
  constexpr int WTILES = WINR / 16;
  constexpr int R = SCAN_RING;
  __shared__ __align__(16) bf16_t Aq[HMAX * MT * KK * 512];
  __shared__ __align__(16) float rsq_t[HMAX][MT * 16];
  __shared__ float scw_all[2][WINR];
  __shared__ int ag_all[ARG ? 2 : 1][ARG ? WINR : 1];
  __shared__ float carry[2];

  const int H = a.H;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int w = tid >> 6, lane = tid & 63;
  const int cl = lane & 15, g = lane >> 4;
  int part, b;
  part_and_query(part, b);
  const int q0 = a.q_off[b];
  const int Lq = a.q_off[b + 1] - q0;
  const int d_begin = part_first_doc(a.chunk_off, a.n_docs, a.n_chunks, part, gridDim.x);
  const int d_end = part_first_doc(a.chunk_off, a.n_docs, a.n_chunks, part + 1, gridDim.x);
  if (d_begin >= d_end) return;
  float* scores = a.scores + (int64_t)b * a.n_docs;
  if (Lq <= 0) {
    for (int d = d_begin + tid; d < d_end; d += nthr) scores[d] = -INFINITY;
    return;
  }
  const int64_t c_begin = a.chunk_off[d_begin];
  const int64_t c_end = a.chunk_off[d_end];
  const bf16_t* Qr = (const bf16_t*)a.Qr;
  const bf16_t* Kb = (const bf16_t*)a.Krb;
  const int64_t tile_elems = (int64_t)16 * H * D;
  const int64_t T_begin = c_begin >> 4;
  const int ntiles = (int)(((c_end + 15) >> 4) - T_begin);
  const int nwin = (ntiles + WTILES - 1) / WTILES;
  const int n_my = ntiles > w ? (ntiles - w + 7) / 8 : 0;   // this wave's tiles: w, w + 8, ...
  const int n_steps = n_my * H;                              // one step per (tile, head)

  for (int rb = 0; rb < Lq; rb += MT * 16) {
    const int rows = min(MT * 16, Lq - rb);
    __syncthreads();  // the previous pass is done with Aq
    for (int u = tid; u < H * MT * KK * 64; u += nthr) {
      const int L = u & 63;
      int rest = u >> 6;
      const int kk = rest % KK;
      rest /= KK;
      const int m = rest % MT, h = rest / MT;
      const int t = rb + m * 16 + (L & 15);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (t < Lq) v = *reinterpret_cast<const uint4*>(Qr + ((int64_t)(q0 + t) * H + h) * D + kk * 32 + (L >> 4) * 8);
      *reinterpret_cast<uint4*>(&Aq[(size_t)u * 8]) = v;
    }
    for (int u = tid; u < H * MT * 16; u += nthr) {
      const int h = u / (MT * 16), tl = u - h * (MT * 16);
      const int t = rb + tl;
      float rr = 0.f;
      if (t < Lq) {
        const bf16_t* q = Qr + ((int64_t)(q0 + t) * H + h) * D;
        float sg[4];
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          float ss = 0.f;
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            const uint4 wq = *reinterpret_cast<const uint4*>(q + kk * 32 + gg * 8);
            ss = dot2_bf16(wq.x, wq.x, ss);
            ss = dot2_bf16(wq.y, wq.y, ss);
            ss = dot2_bf16(wq.z, wq.z, ss);
            ss = dot2_bf16(wq.w, wq.w, ss);
          }
          sg[gg] = ss;
        }
        const float ss = (sg[0] + sg[1]) + (sg[2] + sg[3]);
        rr = ss > 0.f ? __builtin_amdgcn_rsqf(ss) / (float)H : 0.f;
      }
      rsq_t[h][tl] = rr;
    }
    __syncthreads();

    // Loads are issued unconditionally, with the tile clamped into the part's tiles (a wave
    // without tiles of its own, in a part of fewer than eight tiles, reads the part's last
    // tile), so the compiler waits for exactly the oldest ring slot instead of draining the
    // queue.
    const int64_t T_last = T_begin + ntiles - 1;
    auto load = [&](bf16x8_t (&B)[KK], int k, int h) {
      const int64_t T = min(T_begin + w + (int64_t)max(k, 0) * 8, T_last);
      const bf16_t* p = Kb + T * tile_elems + (int64_t)h * (KK * 512) + lane * 8;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) B[kk] = load_nt(p + kk * 512);
    };
    bf16x8_t B[R][KK];
    // load position (lk, lh) runs R steps ahead of the processing position (pk, ph)
    int lk = 0, lh = 0;
    auto advance = [&](int& k, int& h) {
      if (++h == H) { h = 0; ++k; }
    };
    auto clamp_load = [&](bf16x8_t (&Bx)[KK]) {
      const bool in = lk < n_my;
      load(Bx, in ? lk : n_my - 1, in ? lh : H - 1);
      advance(lk, lh);
    };
    // prologue: slot r's loads in slot order (the loop waits for the oldest slot only if
    // the loads entering it are pending in the same order as on its back edge)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      clamp_load(B[r]);
      __builtin_amdgcn_sched_barrier(0);
    }
    int pk = 0, ph = 0;
    float total[MT][4];
    int d_first = d_begin;
    int st = 0;
    for (int wi = 0; wi < nwin; ++wi) {
      const int64_t base_row = (T_begin + (int64_t)wi * WTILES) * 16;
      const int64_t w0 = max(c_begin, base_row);
      const int64_t w1 = min(c_end, base_row + (int64_t)WINR);
      float* scw = scw_all[wi & 1];
      int* agw = ag_all[ARG ? (wi & 1) : 0];
      const int s_end = min(n_steps, (wi + 1) * (WTILES / 8) * H);
      for (; st < s_end; st += R) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (st + r < s_end) {
            const int h = ph;
            if (h == 0) {
#pragma unroll
              for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) total[m][i] = 0.f;
            }
            // 1/|k| of each column (bank row) for this head: Gram diagonal, broadcast from
            // the lane holding element (cl, cl) to the column's four lanes
            f32x4_t gram = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
              gram = __builtin_amdgcn_mfma_f32_16x16x32_bf16(B[r][kk], B[r][kk], gram, 0, 0, 0);
            const int e = cl & 3;
            const float dg = e == 0 ? gram[0] : e == 1 ? gram[1] : e == 2 ? gram[2] : gram[3];
            const float nrm = __shfl(dg, (cl >> 2) * 16 + cl, 64);
            const float cs = nrm > 0.f ? __builtin_amdgcn_rsqf(nrm) : 0.f;
            const bf16_t* Ah = Aq + (size_t)h * (MT * KK * 512) + lane * 8;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int kk = 0; kk < KK; ++kk) {
                const bf16x8_t A = *reinterpret_cast<const bf16x8_t*>(Ah + (m * KK + kk) * 512);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B[r][kk], acc, 0, 0, 0);
              }
              const float4 rv = *reinterpret_cast<const float4*>(&rsq_t[h][m * 16 + g * 4]);
              total[m][0] = fmaf(acc[0] * rv.x, cs, total[m][0]);
              total[m][1] = fmaf(acc[1] * rv.y, cs, total[m][1]);
              total[m][2] = fmaf(acc[2] * rv.z, cs, total[m][2]);
              total[m][3] = fmaf(acc[3] * rv.w, cs, total[m][3]);
            }
            if (h == H - 1) {
              // the column's maximum over the block's valid tokens (ARG: first token reaching it)
              float best = -INFINITY;
              int bt = 0;
#pragma unroll
              for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int tl = m * 16 + g * 4 + i;
                  if (tl < rows && total[m][i] > best) {
                    best = total[m][i];
                    bt = tl;
                  }
                }
#pragma unroll
              for (int o = 16; o < 64; o <<= 1) {
                const float ob = __shfl_xor(best, o, 64);
                if constexpr (ARG) {
                  const int ot = __shfl_xor(bt, o, 64);
                  if (ob > best || (ob == best && ot < bt)) bt = ot;
                }
                best = fmaxf(best, ob);
              }
              const int64_t row = (T_begin + w + (int64_t)pk * 8) * 16 + cl;
              if (g == 0 && row >= w0 && row < w1) {
                scw[row - base_row] = best;
                if constexpr (ARG) agw[row - base_row] = rb + bt;
              }
            }
            advance(pk, ph);
          }
          clamp_load(B[r]);
        }
      }
      lds_barrier();  // every wave's row scores of this window are in LDS
      if constexpr (ARG) {
        for (int64_t r = w0 + tid; r < w1; r += nthr) {
          const float v = scw[r - base_row];
          const int64_t o = (int64_t)b * a.n_chunks + r;
          if (rb == 0 || v > a.row_scores[o]) {  // an earlier block keeps a tie
            a.row_scores[o] = v;
            a.row_arg[o] = agw[r - base_row];
          }
        }
      }
      const int cin = wi & 1, cout = cin ^ 1;
      for (int d = d_first + w; d < d_end; d += SCAN_WAVES) {
        const int64_t r0 = a.chunk_off[d], r1 = a.chunk_off[d + 1];
        if (r0 >= w1) break;
        const int lo = (int)(max(r0, w0) - base_row), hi = (int)(min(r1, w1) - base_row);
        float m = -INFINITY;
        for (int i = lo + lane; i < hi; i += 64) m = fmaxf(m, scw[i]);
        m = wave_max_all(m);
        if (r0 < w0) m = fmaxf(m, carry[cin]);
        if (lane == 0) {
          if (r1 <= w1) scores[d] = (rb == 0) ? m : fmaxf(m, scores[d]);
          else carry[cout] = m;
        }
      }
      if (w1 < c_end) d_first = find_doc_wave(a.chunk_off, a.n_docs, w1);
    }
  }
}

// ------------------------------------------------------------------------------------
// Dot-product scan for short queries.  Each wave owns a document-aligned range of rows,
// reads them four at a time with the next four in flight, and folds row scores into
// documents itself (its documents belong to it alone).  Query rows (raw) and their
// scales rs[t,h] wait in LDS, in blocks of up to QB tokens.
// ------------------------------------------------------------------------------------
constexpr int QB = 16;
constexpr int DOT_WAVES = 4;
constexpr int U = 4;  // rows per group

template <typename T>
struct RowSlot;  // one lane's 8 elements of one 512-element slice of a row
// bf16 rows accumulate in float (bf16 products are exact in float); float32 rows in
// double (float products are exact in double), which keeps near-cancelling cosines of
// float32 inputs within a few float ulps.
template <> struct RowSlot<bf16_t> {
  typedef float acc_t;
  uint4 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ float sumsq() const {
    float s = dot2_bf16(v.x, v.x, 0.f);
    s = dot2_bf16(v.y, v.y, s);
    s = dot2_bf16(v.z, v.z, s);
    return dot2_bf16(v.w, v.w, s);
  }
  __device__ __forceinline__ float dot(const void* q) const {
    const uint4 w = *reinterpret_cast<const uint4*>(q);
    float s = dot2_bf16(v.x, w.x, 0.f);
    s = dot2_bf16(v.y, w.y, s);
    s = dot2_bf16(v.z, w.z, s);
    return dot2_bf16(v.w, w.w, s);
  }
};
template <> struct RowSlot<float> {
  typedef double acc_t;
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ static double d(float x) { return (double)x; }
  __device__ __forceinline__ double sumsq() const {
    return d(a.x) * a.x + d(a.y) * a.y + d(a.z) * a.z + d(a.w) * a.w + d(b.x) * b.x + d(b.y) * b.y +
           d(b.z) * b.z + d(b.w) * b.w;
  }
  __device__ __forceinline__ double dot(const void* q) const {
    const float4 u = reinterpret_cast<const float4*>(q)[0], w = reinterpret_cast<const float4*>(q)[1];
    return d(a.x) * u.x + d(a.y) * u.y + d(a.z) * u.z + d(a.w) * u.w + d(b.x) * w.x + d(b.y) * w.y +
           d(b.z) * w.z + d(b.w) * w.w;
  }
};

template <typename T, int D, int P>
__global__ __launch_bounds__(256) void route_scan_dot(ScanK a) {
  extern __shared__ __align__(16) unsigned char dot_lds[];
  constexpr int LPH = D / 8;  // lanes per head within a 512-element slice
  const int H = a.H;
  const int R = H * D;
  // P = slices of 512 elements per row (template, 1..4)
  typedef typename RowSlot<T>::acc_t acc_t;
  T* qs = reinterpret_cast<T*>(dot_lds);                           // [QB][R] raw query rows
  acc_t* rsl = reinterpret_cast<acc_t*>(dot_lds + (size_t)QB * R * sizeof(T));  // [QB][H]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int part, b;
  part_and_query(part, b);
  const int q0 = a.q_off[b];
  const int Lq = a.q_off[b + 1] - q0;
  const int64_t gw = (int64_t)part * DOT_WAVES + w;
  const int64_t nw = (int64_t)gridDim.x * DOT_WAVES;
  const int d_begin = part_first_doc(a.chunk_off, a.n_docs, a.n_chunks, gw, nw);
  const int d_end = part_first_doc(a.chunk_off, a.n_docs, a.n_chunks, gw + 1, nw);
  float* scores = a.scores + (int64_t)b * a.n_docs;
  const T* Qr = (const T*)a.Qr;
  const T* Kb = (const T*)a.Krb;
  if (Lq <= 0) {  // uniform over the workgroup
    for (int d = d_begin + lane; d < d_end; d += 64) scores[d] = -INFINITY;
    return;
  }
  const int64_t c_begin = (d_begin < d_end) ? a.chunk_off[d_begin] : 0;
  const int64_t c_end = (d_begin < d_end) ? a.chunk_off[d_end] : 0;
  const bool head_last = (lane % LPH) == LPH - 1;

  for (int tb = 0; tb < Lq; tb += QB) {
    const int nt = min(QB, Lq - tb);
    __syncthreads();  // previous block's readers are done with qs
    for (int i = threadIdx.x; i < nt * R; i += blockDim.x) qs[i] = Qr[(int64_t)(q0 + tb) * R + i];
    for (int th = w; th < nt * H; th += DOT_WAVES) {  // one wave per (token, head) norm
      const int t = th / H, h = th % H;
      const T* q = Qr + ((int64_t)(q0 + tb + t) * H + h) * D;
      acc_t ss = 0;
      for (int e = lane; e < D; e += 64) {
        acc_t x;
        if constexpr (sizeof(T) == 4) x = ((const float*)q)[e];
        else x = bf16_to_f32(((const bf16_t*)q)[e]);
        ss += x * x;
      }
      ss = wave_sum_last(ss);
      if (lane == 63) rsl[t * H + h] = ss > 0 ? (acc_t)1 / ((acc_t)H * sqrt(ss)) : (acc_t)0;
    }
    __syncthreads();
    if (c_begin >= c_end) continue;
    // The first token block stores document scores; later blocks (queries longer than QB
    // rows) combine with them.  The two cases are separate loops so the streaming loop of
    // the common case holds no global read that would make it wait for its prefetches.
    auto run_rows = [&](auto first_tag) {
      constexpr bool FIRST = decltype(first_tag)::value;
      int cur = d_begin;
      int wb = cur;
      int64_t win = load_window(a.chunk_off, a.n_docs, wb);
      int64_t nb = __shfl(win, 0);  // end row of document `cur`
      float run = -INFINITY;
      auto emit = [&](int doc, float v) {
        if (lane == 0) {
          if (FIRST) scores[doc] = v;
          else scores[doc] = fmaxf(v, scores[doc]);
        }
      };

      auto load = [&](RowSlot<T> (&X)[U][P], int64_t c0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          int64_t c = c0 + u;
          c = c < c_end ? c : c_end - 1;
#pragma unroll
          for (int p = 0; p < P; ++p) {  // lanes past the row end re-read its last 8 elements
            const int e0 = min(p * 512 + lane * 8, R - 8);
            if constexpr (sizeof(T) == 2) X[u][p].load(Kb + kr_tiled<D>(c, e0, H));  // bf16: tiled bank
            else X[u][p].load(Kb + c * R + e0);
          }
        }
      };
      auto process = [&](RowSlot<T> (&X)[U][P], int64_t c0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t c = c0 + u;
          if (c >= c_end) break;  // uniform
          acc_t cs[P];
#pragma unroll
          for (int p = 0; p < P; ++p) {
            const int e0 = p * 512 + lane * 8;
            acc_t ss = (e0 < R) ? X[u][p].sumsq() : (acc_t)0;
            ss = group_sum_last<LPH>(ss);  // head total on the head's last lane
            cs[p] = (head_last && ss > 0) ? (acc_t)1 / sqrt(ss) : (acc_t)0;
          }
          float best = -INFINITY;
          int arg = 0;  // first maximising token (lane 63)
          for (int t = 0; t < nt; ++t) {
            acc_t contrib = 0;
#pragma unroll
            for (int p = 0; p < P; ++p) {
              const int e0 = p * 512 + lane * 8;
              if (e0 < R) {
                acc_t d0 = X[u][p].dot(qs + t * R + e0);
                d0 = group_sum_last<LPH>(d0);
                contrib += d0 * cs[p] * rsl[t * H + e0 / D];
              }
            }
            contrib = wave_sum_last(contrib);
            if ((float)contrib > best) arg = t;
            best = fmaxf(best, (float)contrib);
          }
          best = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(best), 63));
          if (a.row_scores) {
            arg = __builtin_amdgcn_readlane(arg, 63);
            if (lane == 0) {
              float* rsc = a.row_scores + (int64_t)b * a.n_chunks + c;
              if (FIRST || best > *rsc) {  // an earlier token block keeps a tie
                *rsc = best;
                a.row_arg[(int64_t)b * a.n_chunks + c] = tb + arg;
              }
            }
          }
          // fold into documents (wave-uniform control flow)
          while (c >= nb) {
            emit(cur, run);
            run = -INFINITY;
            ++cur;
            if (cur - wb >= 63) {
              wb = cur;
              win = load_window(a.chunk_off, a.n_docs, wb);
              nb = __shfl(win, 0);
            } else {
              nb = __shfl(win, cur - wb);
            }
          }
          run = fmaxf(run, best);
        }
      };

      // Two groups of U rows: one computed while the other is in flight.  Loads are issued
      // unconditionally (rows clamped to the range) so waits target the oldest group only.
      RowSlot<T> X0[U][P], X1[U][P];
      load(X0, c_begin);
      load(X1, c_begin + U);
      for (int64_t c0 = c_begin; c0 < c_end; c0 += 2 * U) {
        process(X0, c0);
        load(X0, c0 + 2 * U);
        if (c0 + U < c_end) process(X1, c0 + U);
        load(X1, c0 + 3 * U);
      }
      emit(cur, run);  // the range ends at a document end
    };
    if (tb == 0) run_rows(std::true_type{});
    else run_rows(std::false_type{});
  }
}

// Parts of a scan: max_parts, fewer for small banks (at least rows_per_part rows each).
// With several queries the count is rounded down to a multiple of 8 so that all queries
// of a part can share one XCD (part_and_query).
int route_parts(int64_t n_chunks, int64_t rows_per_part, int64_t max_parts, int n_queries) {
  int64_t p = max_parts;
  const int64_t mx = (n_chunks + rows_per_part - 1) / rows_per_part;
  if (p > mx) p = mx;
  if (n_queries > 1 && p >= 8) p &= ~(int64_t)7;
  if (p < 1) p = 1;
  return (int)p;
}

template <int D>
hipError_t launch_mfma(const RouteArgs& r, const ScanK& k, hipStream_t s) {
  const int mt = min(4, (r.max_q_len + 15) / 16);
  // one part per CU: a workgroup's LDS (the query operands of every head, up to 146 KB) leaves
  // room for one per CU, so 256 parts run in a single round
  dim3 grid((unsigned)route_parts(r.n_chunks, 64, 256, r.n_queries), (unsigned)r.n_queries);
  dim3 block(64 * SCAN_WAVES);
  if (k.row_scores) {
    switch (mt) {
      case 1: hipLaunchKernelGGL((route_scan_mfma<1, D, true>), grid, block, 0, s, k); break;
      case 2: hipLaunchKernelGGL((route_scan_mfma<2, D, true>), grid, block, 0, s, k); break;
      case 3: hipLaunchKernelGGL((route_scan_mfma<3, D, true>), grid, block, 0, s, k); break;
      default: hipLaunchKernelGGL((route_scan_mfma<4, D, true>), grid, block, 0, s, k); break;
    }
    return hipGetLastError();
  }
  switch (mt) {
    case 1: hipLaunchKernelGGL((route_scan_mfma<1, D, false>), grid, block, 0, s, k); break;
    case 2: hipLaunchKernelGGL((route_scan_mfma<2, D, false>), grid, block, 0, s, k); break;
    case 3: hipLaunchKernelGGL((route_scan_mfma<3, D, false>), grid, block, 0, s, k); break;
    default: hipLaunchKernelGGL((route_scan_mfma<4, D, false>), grid, block, 0, s, k); break;
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_dot(const RouteArgs& r, const ScanK& k, hipStream_t s) {
  const size_t R = (size_t)r.h_r * D;
  const size_t lds = QB * R * sizeof(T) + QB * r.h_r * (sizeof(T) == 4 ? sizeof(double) : sizeof(float));
  dim3 grid((unsigned)route_parts(r.n_chunks, 8 * DOT_WAVES, 2048, r.n_queries), (unsigned)r.n_queries);
  dim3 block(64 * DOT_WAVES);
  switch ((R + 511) / 512) {
    case 1: hipLaunchKernelGGL((route_scan_dot<T, D, 1>), grid, block, lds, s, k); break;
    case 2: hipLaunchKernelGGL((route_scan_dot<T, D, 2>), grid, block, lds, s, k); break;
    case 3: hipLaunchKernelGGL((route_scan_dot<T, D, 3>), grid, block, lds, s, k); break;
    default: hipLaunchKernelGGL((route_scan_dot<T, D, 4>), grid, block, lds, s, k); break;
  }
  return hipGetLastError();
}

// Each document's score as the largest of its rows' scores (-inf for a document without
// rows): one wave per (query, document).
__global__ __launch_bounds__(256) void docs_from_rows(const float* rows, const int64_t* chunk_off, float* scores,
                                                      int n_docs, int64_t n_chunks) {
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (n >= n_docs) return;
  const int64_t c0 = chunk_off[n], c1 = chunk_off[n + 1];
  const float* r = rows + (int64_t)b * n_chunks;
  float m = -INFINITY;
  for (int64_t c = c0 + lane; c < c1; c += 64) m = fmaxf(m, r[c]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (lane == 0) scores[(int64_t)b * n_docs + n] = m;
}

}  // namespace

// Query rows from which the batched scan (route_batch.hip) takes over.  Below it the scan
// is bound by the bank read and the streaming kernels above are as fast or faster (10M-
// token bank: 64 rows 94 us streaming vs 98 us batched; 128 rows 164 vs 128 us).
constexpr int64_t BATCH_MIN_ROWS = 128;

static hipError_t launch_scan_paths(const RouteArgs& r, hipStream_t s) {
  ScanK k{r.Qr, r.q_off, r.Krbar, r.chunk_off, r.scores, r.row_scores, r.row_arg, r.n_chunks, r.n_docs, r.h_r};
  // bf16: the MFMA scan at any query length (a short query pads its 16-row tile; the
  // scan stays bound by the bank read and beats the dot-product scan even for one row).
  if (route_batch_supported(r) && (r.force_path == 3 || (r.force_path == 0 && r.total_q >= BATCH_MIN_ROWS)))
    return launch_route_scan_batch(r, s);
  bool mfma = (r.dtype == 1) && (r.h_r <= 8);
  if (r.force_path == 1) mfma = false;
  if (r.force_path == 2 && r.dtype == 1 && r.h_r <= 8) mfma = true;
  if (mfma) {
    switch (r.d) {
      case 32: return launch_mfma<32>(r, k, s);
      case 64: return launch_mfma<64>(r, k, s);
      default: return launch_mfma<128>(r, k, s);
    }
  }
  if (r.dtype == 0) {
    switch (r.d) {
      case 32: return launch_dot<float, 32>(r, k, s);
      case 64: return launch_dot<float, 64>(r, k, s);
      default: return launch_dot<float, 128>(r, k, s);
    }
  }
  switch (r.d) {
    case 32: return launch_dot<bf16_t, 32>(r, k, s);
    case 64: return launch_dot<bf16_t, 64>(r, k, s);
    default: return launch_dot<bf16_t, 128>(r, k, s);
  }
}

// With row outputs the rows start at -inf (a query without tokens leaves them so), the
// scan writes each row's maximum and first maximising token, and the document scores are
// then taken as their rows' maxima: the same floats the scan maximises, so they equal the
// scores of a scan without row outputs.
hipError_t launch_route_scan(const RouteArgs& r, hipStream_t s) {
  if (r.row_scores == nullptr) return launch_scan_paths(r, s);
  hipError_t e = launch_fill_neg_inf(r.row_scores, (int64_t)r.n_queries * r.n_chunks, s);
  if (e == hipSuccess) e = launch_scan_paths(r, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(docs_from_rows, dim3((unsigned)((r.n_docs + 3) / 4), (unsigned)r.n_queries), dim3(256), 0, s,
                     r.row_scores, r.chunk_off, r.scores, r.n_docs, r.n_chunks);
  return hipGetLastError();
}

}  // namespace msa
