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
//  * route_scan_mfma (bf16, queries of >= 16 rows): one wave per routing head.  The wave
//    keeps its head's query rows as MFMA A operands (v_mfma_f32_16x16x32_bf16, rows padded
//    to 16) and streams 16-row tiles of its head's Kr-bar slice as B operands straight
//    from HBM into registers, one tile ahead.  Column norms come from the same registers.
//    The scaled per-head scores meet in LDS (double-buffered, one barrier per tile) for
//    the head sum and token max; wave 0 then folds the 16 row scores into documents.
//  * route_scan_dot (any dtype, short queries): one wave per row; each lane holds 8
//    elements of the row and multiplies them with pre-scaled query vectors from LDS,
//    reducing across the wave.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace msa {
namespace {

struct ScanK {
  const void* Qr;
  const int32_t* q_off;
  const void* Krb;
  const int64_t* chunk_off;
  float* scores;  // [n_queries, n_docs]
  int64_t n_chunks;
  int n_docs;
  int H;
};

__device__ __forceinline__ int64_t load_window(const int64_t* chunk_off, int n_docs, int wb) {
  const int di = wb + 1 + (int)(threadIdx.x & 63);
  return (di <= n_docs) ? chunk_off[di] : INT64_MAX;
}

// ------------------------------------------------------------------------------------
// Wave-0 helper of the MFMA scan: fold 16 consecutive row scores (lane l < 16 holds row
// c_first + l) into document maxima.  `win` holds chunk_off[wb + 1 + lane], a window of
// document ends that must cover the tile; it is rebased when the tile runs past it.
// `carry` is the running maximum of document `cur_doc`, which began in an earlier tile.
// A document's score is stored once its last row has been seen; on a later pass over the
// same rows (query rows beyond the first block) it is combined with the stored value.
// ------------------------------------------------------------------------------------
__device__ __forceinline__ void fold_tile_docs(const ScanK& a, float* scores, int64_t c_first,
                                               int64_t c_end, float s, bool first_pass,
                                               int& cur_doc, int& wb, int64_t& win,
                                               float& carry) {
  const int lane = threadIdx.x & 63;
  const int64_t c_last = min(c_first + 15, c_end - 1);
  const int nvalid = (int)(c_last - c_first + 1);
  if (!(c_last < __shfl(win, 63))) {
    wb = cur_doc;
    win = load_window(a.chunk_off, a.n_docs, wb);
  }
  const int64_t c = c_first + lane;
  const bool valid = lane < nvalid;
  int pos = 0;  // #{j : win[j] <= c}, win strictly increasing
#pragma unroll
  for (int step = 32; step >= 1; step >>= 1) {
    const int64_t v = __shfl(win, pos + step - 1);
    if (v <= c) pos += step;
  }
  const int doc = wb + pos;
  const int64_t doc_end = __shfl(win, pos);  // chunk_off[doc + 1]
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) {  // segmented inclusive max
    const float os = __shfl_up(s, off);
    const int od = __shfl_up(doc, off);
    if (lane >= off && od == doc) s = fmaxf(s, os);
  }
  if (doc == cur_doc) s = fmaxf(s, carry);
  if (valid && c + 1 == doc_end) {  // last row of its document
    const float v = first_pass ? s : fmaxf(s, scores[doc]);
    scores[doc] = v;
  }
  const int ld = __shfl(doc, nvalid - 1);
  const float ls = __shfl(s, nvalid - 1);
  const int64_t lend = __shfl(doc_end, nvalid - 1);
  if (c_last + 1 == lend) { cur_doc = ld + 1; carry = -INFINITY; }
  else { cur_doc = ld; carry = ls; }
}

template <int MT, int D>
__global__ __launch_bounds__(512) void route_scan_mfma(ScanK a) {
  constexpr int KK = D / 32;          // 32-wide k steps per head
  constexpr int ROWS = MT * 16;       // query rows per block
  constexpr int STRIDE = ROWS + 4;    // padded LDS row (floats)
  __shared__ float red[2][8][16][STRIDE];
  __shared__ float sc[2][16];

  const int H = a.H;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cl = lane & 15, g = lane >> 4;
  const int b = blockIdx.y;
  const int q0 = a.q_off[b];
  const int Lq = a.q_off[b + 1] - q0;
  const int d_begin = part_first_doc(a.chunk_off, a.n_docs, a.n_chunks, blockIdx.x, gridDim.x);
  const int d_end = part_first_doc(a.chunk_off, a.n_docs, a.n_chunks, blockIdx.x + 1, gridDim.x);
  if (d_begin >= d_end) return;
  float* scores = a.scores + (int64_t)b * a.n_docs;
  if (Lq <= 0) {  // a query without tokens scores -inf everywhere
    for (int d = d_begin + threadIdx.x; d < d_end; d += blockDim.x) scores[d] = -INFINITY;
    return;
  }
  const int64_t c_begin = a.chunk_off[d_begin];
  const int64_t c_end = a.chunk_off[d_end];
  const bf16_t* Qr = (const bf16_t*)a.Qr;
  const bf16_t* Kb = (const bf16_t*)a.Krb;
  const int64_t ntiles = (c_end - c_begin + 15) / 16;

  for (int rb = 0; rb < Lq; rb += ROWS) {
    const int rows = min(ROWS, Lq - rb);
    int cur_doc = d_begin, wb = d_begin;
    int64_t win = load_window(a.chunk_off, a.n_docs, wb);
    float carry = -INFINITY;
    // ---- A operands: this head's query rows, and their scales ----
    bf16x8_t A[MT][KK];
    float rs[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int r = rb + m * 16 + cl;
      float ss = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (r < Lq) {
          const uint4 wq = *reinterpret_cast<const uint4*>(
              Qr + ((int64_t)(q0 + r) * H + w) * D + kk * 32 + g * 8);
          A[m][kk] = __builtin_bit_cast(bf16x8_t, wq);
          float f[8];
          unpack8(wq, f);
#pragma unroll
          for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
        } else {
          A[m][kk] = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
        }
      }
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      const float rrow = ss > 0.f ? 1.0f / ((float)H * sqrtf(ss)) : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) rs[m][i] = __shfl(rrow, g * 4 + i);
    }

    // ---- stream 16-row tiles, one tile of loads in flight ahead ----
    bf16x8_t Bn[KK];
    auto load_tile = [&](int64_t t, bf16x8_t* Bf) {
      const int64_t c = c_begin + t * 16 + cl;
      if (c < c_end) {
        const bf16_t* p = Kb + (c * H + w) * D + g * 8;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          Bf[kk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p + kk * 32));
      } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) Bf[kk] = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
      }
    };
    load_tile(0, Bn);
    int buf = 0;
    for (int64_t t = 0; t < ntiles; ++t) {
      bf16x8_t Bc[KK];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) Bc[kk] = Bn[kk];
      if (t + 1 < ntiles) load_tile(t + 1, Bn);

      float ss = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        float f[8];
        unpack8(__builtin_bit_cast(uint4, Bc[kk]), f);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
      }
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      const float cs = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;

#pragma unroll
      for (int m = 0; m < MT; ++m) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[m][kk], Bc[kk], acc, 0, 0, 0);
        // lane holds rows m*16 + g*4 + i of column cl
        float4 v;
        v.x = acc[0] * rs[m][0] * cs;
        v.y = acc[1] * rs[m][1] * cs;
        v.z = acc[2] * rs[m][2] * cs;
        v.w = acc[3] * rs[m][3] * cs;
        *reinterpret_cast<float4*>(&red[buf][w][cl][m * 16 + g * 4]) = v;
      }
      lds_barrier();

      // head sum, then max over this block's query rows; wave w takes rows w, w+H, ...
      for (int cc = w; cc < 16; cc += H) {
        float s = -INFINITY;
        if (lane < rows) {
          float sum = 0.f;
          for (int h = 0; h < H; ++h) sum += red[buf][h][cc][lane];
          s = sum;
        }
        s = wave_max(s);
        if (lane == 0) sc[buf][cc] = s;
      }
      if (w == 0 && t > 0) {
        const float s = (lane < 16) ? sc[buf ^ 1][lane] : -INFINITY;
        fold_tile_docs(a, scores, c_begin + (t - 1) * 16, c_end, s, rb == 0, cur_doc, wb, win, carry);
      }
      buf ^= 1;
    }
    lds_barrier();
    if (w == 0) {
      const float s = (lane < 16) ? sc[buf ^ 1][lane] : -INFINITY;
      fold_tile_docs(a, scores, c_begin + (ntiles - 1) * 16, c_end, s, rb == 0, cur_doc, wb, win, carry);
    }
    lds_barrier();
  }
}

// ------------------------------------------------------------------------------------
// Dot-product scan.  Each wave owns a document-aligned range of rows and folds row scores
// into documents itself.  Query rows are handled in blocks of up to QB tokens held in LDS
// as float, pre-multiplied by rs[t,h].
// ------------------------------------------------------------------------------------
constexpr int QB = 16;
constexpr int DOT_WAVES = 4;

template <typename T, int D>
__global__ __launch_bounds__(256) void route_scan_dot(ScanK a) {
  extern __shared__ float qs[];  // [QB][H*D]
  const int H = a.H;
  const int R = H * D;
  const int P = (R + 511) / 512;  // 8-element slots per lane
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const int q0 = a.q_off[b];
  const int Lq = a.q_off[b + 1] - q0;
  const int64_t gw = (int64_t)blockIdx.x * DOT_WAVES + w;
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

  for (int tb = 0; tb < Lq; tb += QB) {
    const int nt = min(QB, Lq - tb);
    __syncthreads();  // previous block's readers are done with qs
    // pre-scaled query rows: one wave per (token, head) norm
    for (int th = w; th < nt * H; th += DOT_WAVES) {
      const int t = th / H, h = th % H;
      const T* q = Qr + ((int64_t)(q0 + tb + t) * H + h) * D;
      float ss = 0.f;
      for (int e = lane; e < D; e += 64) {
        float x;
        if constexpr (sizeof(T) == 4) x = ((const float*)q)[e];
        else x = bf16_to_f32(((const bf16_t*)q)[e]);
        ss += x * x;
      }
      ss = wave_sum(ss);
      const float r = ss > 0.f ? 1.0f / ((float)H * sqrtf(ss)) : 0.f;
      for (int e = lane; e < D; e += 64) {
        float x;
        if constexpr (sizeof(T) == 4) x = ((const float*)q)[e];
        else x = bf16_to_f32(((const bf16_t*)q)[e]);
        qs[t * R + h * D + e] = x * r;
      }
    }
    __syncthreads();
    if (c_begin >= c_end) continue;
    const bool first_pass = tb == 0;

    int cur = d_begin;
    int wb = cur;
    int64_t win = load_window(a.chunk_off, a.n_docs, wb);
    int64_t nb = __shfl(win, 0);  // end row of document `cur`
    float run = -INFINITY;
    auto emit = [&](int doc, float v) {
      if (lane == 0) scores[doc] = first_pass ? v : fmaxf(v, scores[doc]);
    };

    float xn[4][8];
    auto load_row = [&](int64_t c, float (*x)[8]) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int e0 = p * 512 + lane * 8;
        if (p < P && e0 < R && c < c_end) Elem<T>::load8(Kb + c * R + e0, x[p]);
        else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[p][e] = 0.f;
        }
      }
    };
    load_row(c_begin, xn);
    for (int64_t c = c_begin; c < c_end; ++c) {
      float x[4][8];
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[p][e] = xn[p][e];
      if (c + 1 < c_end) load_row(c + 1, xn);

      // per-head inverse norms: reduce over the D/8 lanes of a head
      float cs[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += x[p][e] * x[p][e];
#pragma unroll
        for (int o = 1; o < D / 8; o <<= 1) ss += __shfl_xor(ss, o);
        cs[p] = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
      }
      float best = -INFINITY;
      for (int t = 0; t < nt; ++t) {
        float dsum = 0.f;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int e0 = p * 512 + lane * 8;
          if (p < P && e0 < R) {
            const float4 qa = *reinterpret_cast<const float4*>(&qs[t * R + e0]);
            const float4 qb = *reinterpret_cast<const float4*>(&qs[t * R + e0 + 4]);
            float d0 = x[p][0] * qa.x + x[p][1] * qa.y + x[p][2] * qa.z + x[p][3] * qa.w +
                       x[p][4] * qb.x + x[p][5] * qb.y + x[p][6] * qb.z + x[p][7] * qb.w;
            dsum += d0 * cs[p];
          }
        }
        best = fmaxf(best, wave_sum(dsum));
      }
      // fold into documents (wave-uniform control flow)
      while (c >= nb) {
        emit(cur, run);
        run = -INFINITY;
        ++cur;
        if (cur - wb >= 63) {
          wb = cur;
          win = load_window(a.chunk_off, a.n_docs, wb);
        }
        nb = __shfl(win, cur - wb);
      }
      run = fmaxf(run, best);
    }
    emit(cur, run);  // the range ends at a document end
  }
}

int route_parts(int64_t n_chunks, int64_t rows_per_part) {
  int64_t p = 2048;
  const int64_t mx = (n_chunks + rows_per_part - 1) / rows_per_part;
  if (p > mx) p = mx;
  if (p < 1) p = 1;
  return (int)p;
}

template <int D>
hipError_t launch_mfma(const RouteArgs& r, const ScanK& k, hipStream_t s) {
  const int mt = min(4, (r.max_q_len + 15) / 16);
  // 2 workgroups per CU on 256 CUs, several times over; >= 4 tiles per workgroup.
  dim3 grid((unsigned)route_parts(r.n_chunks, 64), (unsigned)r.n_queries);
  dim3 block(64 * r.h_r);
  switch (mt) {
    case 1: hipLaunchKernelGGL((route_scan_mfma<1, D>), grid, block, 0, s, k); break;
    case 2: hipLaunchKernelGGL((route_scan_mfma<2, D>), grid, block, 0, s, k); break;
    case 3: hipLaunchKernelGGL((route_scan_mfma<3, D>), grid, block, 0, s, k); break;
    default: hipLaunchKernelGGL((route_scan_mfma<4, D>), grid, block, 0, s, k); break;
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_dot(const RouteArgs& r, const ScanK& k, hipStream_t s) {
  const size_t lds = (size_t)QB * r.h_r * D * sizeof(float);
  dim3 grid((unsigned)route_parts(r.n_chunks, 4 * DOT_WAVES), (unsigned)r.n_queries);
  hipLaunchKernelGGL((route_scan_dot<T, D>), grid, dim3(64 * DOT_WAVES), lds, s, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_scan(const RouteArgs& r, hipStream_t s) {
  ScanK k{r.Qr, r.q_off, r.Krbar, r.chunk_off, r.scores, r.n_chunks, r.n_docs, r.h_r};
  bool mfma = (r.dtype == 1) && (r.max_q_len >= 16) && (r.h_r <= 8);
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

}  // namespace msa
