// Backward of steps B -- the router's gradient for a routing loss on document scores.
//
// yeyulingfeng.com "深度分析MSA ..." section 四 (training): a routing auxiliary loss (BCE or
// InfoNCE) supervises the document scores; its gradient reaches the routing vectors Qr and
// the pooled routing keys Kr-bar.  A document score is one maximum over (query token, bank
// row) of s(t, c) = (1/H) sum_h cos(Qr[t,h], Kb[c,h]), so dL/dD[b,d] reaches only the
// maximising pair (first row of the document with the largest row score, then the first
// token with the largest score on that row):
//   dQr[t*, h] += g / H * (khat - cos_h qhat) / |q|,  dKb[c*, h] += g / H * (qhat - cos_h khat) / |k|
// (no gradient for a head whose query or key vector is zero).
//
// Kernels:
//  * the forward scan (route.hip), writing each bank row's max over the query's tokens and
//    the first token reaching it;
//  * route_bwd_pair: one wave per (query, document): the maximising row, its token, the key
//    gradient (added atomically: a row can be the maximiser for several queries), and a
//    record (t*, row, per-head cosine and 1/|k|) for the query gradient;
//  * bf16 banks with d = 128 and 4 or 8 heads: route_bwd_doc_b16 (one workgroup per
//    document: every query's maximising row and token, the records, and the rows' key
//    gradients added once per distinct row in a fixed order, without atomics) and
//    route_bwd_dq_b16 (each record's row, which the per-document kernel writes contiguously
//    to the workspace, read with 16-byte loads, several matches in flight);
//  * route_bwd_dq: one workgroup per (query, token) (strided when a query is longer than the
//    grid): gathers the records that name the
//    token (filtered a block of documents at a time through LDS) and writes its gradient
//    (zero for a token that no document's maximum reached).
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace msa {
namespace {

struct RouteBwdK {
  const void* Qr;
  const int32_t* q_off;
  const void* Krb;
  const int64_t* chunk_off;
  const float* dD;          // [B, N]
  const float* row_scores;  // [B, C]
  const int32_t* row_arg;   // [B, C]
  float* dQr;               // [total_q, H, D]
  float* dKrb;              // [C, H, D] row-major, added to
  int32_t* tstar;           // [B, N]: maximising token (query-local), -1 if no gradient
  int64_t* cstar;           // [B, N]: maximising row
  float* cosv;              // [B, N, H]
  float* kinv;              // [B, N, H]: 1/|k| (0 when either vector is zero)
  bf16_t* krec;             // [B, N, H * 128] (bf16 banks of 4 or 8 heads): the record's row
  int64_t n_chunks;
  int n_docs, n_queries, H;
};

template <typename T> __device__ __forceinline__ float ld(const T* p, int64_t i);
template <> __device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld<bf16_t>(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

// Element i = h * D + e of routing-key row c: bf16 banks are in the tiled layout of
// common.hpp, float32 banks row-major.
template <typename T, int D>
__device__ __forceinline__ float ld_key(const T* K, int64_t c, int i, int H) {
  if constexpr (sizeof(T) == 2) return bf16_to_f32(K[kr_tiled<D>(c, i, H)]);
  else return K[c * (int64_t)H * D + i];
}

template <typename T, int D>
__global__ __launch_bounds__(256) void route_bwd_pair(RouteBwdK a) {
  const int lane = threadIdx.x & 63;
  const int d = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (d >= a.n_docs) return;
  const int64_t rec = (int64_t)b * a.n_docs + d;
  const int q0 = a.q_off[b], Lq = a.q_off[b + 1] - q0;
  const float gd = a.dD[rec];
  const int64_t c0 = a.chunk_off[d];
  const int nc = (int)(a.chunk_off[d + 1] - c0);
  const float* rs = a.row_scores + (int64_t)b * a.n_chunks + c0;
  // maximising row: the first with the largest row score
  float best = -INFINITY;
  int bc = nc;
  if (gd != 0.f && Lq > 0) {
    for (int c = lane; c < nc; c += 64) {
      const float v = rs[c];
      if (v > best) { best = v; bc = c; }  // c ascending: a tie keeps the first
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oc = __shfl_xor(bc, o, 64);
    if (ov > best || (ov == best && oc < bc)) { best = ov; bc = oc; }
  }
  if (bc >= nc) {  // no gradient, an empty query or document, or no finite row score
    if (lane == 0) a.tstar[rec] = -1;
    return;
  }
  const int H = a.H;
  const int64_t cs = c0 + bc;
  const int ts = a.row_arg[(int64_t)b * a.n_chunks + cs];  // the scan's first maximising token
  const T* q = (const T*)a.Qr + (int64_t)(q0 + ts) * H * D;
  const T* K = (const T*)a.Krb;
  float* dk = a.dKrb + cs * H * D;  // the gradient is row-major in every dtype
  const float gH = gd / (float)H;
  // gradient of the pair, head by head, lanes over elements
  for (int h = 0; h < H; ++h) {
    float dot = 0.f, qn = 0.f, kn = 0.f;
    for (int e = lane; e < D; e += 64) {
      const float x = ld(q, h * D + e), y = ld_key<T, D>(K, cs, h * D + e, H);
      dot += x * y;
      qn += x * x;
      kn += y * y;
    }
    dot = wave_sum(dot);
    qn = wave_sum(qn);
    kn = wave_sum(kn);
    const bool ok = qn > 0.f && kn > 0.f;
    const float iq = ok ? 1.f / sqrtf(qn) : 0.f, ik = ok ? 1.f / sqrtf(kn) : 0.f;
    const float cosv = dot * iq * ik;
    if (ok) {
      for (int e = lane; e < D; e += 64)
        atomicAdd(dk + h * D + e, gH * (ld(q, h * D + e) * iq - cosv * ld_key<T, D>(K, cs, h * D + e, H) * ik) * ik);
    }
    if (lane == 0) {
      a.cosv[rec * H + h] = cosv;
      a.kinv[rec * H + h] = ik;
    }
  }
  if (lane == 0) {
    a.tstar[rec] = ts;
    a.cstar[rec] = cs;
  }
}

constexpr int DQ_THREADS = 256;
constexpr int DQ_BLOCK = DQ_THREADS;  // documents filtered per step in route_bwd_dq

template <typename T, int D>
__global__ __launch_bounds__(DQ_THREADS) void route_bwd_dq(RouteBwdK a) {
  constexpr int EPT = (16 * D) / DQ_THREADS;  // elements per thread at the largest head count
  __shared__ int match[DQ_BLOCK];
  __shared__ int wave_hits[DQ_THREADS / 64];
  __shared__ float qn_s[16];
  const int b = blockIdx.y;
  const int q0 = a.q_off[b], Lq = a.q_off[b + 1] - q0;
  const int H = a.H, n_el = H * D;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int t = blockIdx.x; t < Lq; t += gridDim.x) {
    const T* q = (const T*)a.Qr + (int64_t)(q0 + t) * n_el;
    const T* K = (const T*)a.Krb;
    if (tid < H) {  // |q|^2 per head, summed in element order
      float acc = 0.f;
      for (int e = 0; e < D; ++e) {
        const float x = ld(q, tid * D + e);
        acc += x * x;
      }
      qn_s[tid] = acc;
    }
    float acc1[EPT], acc2[EPT];  // sum of g * k / |k|, sum of g * cos
#pragma unroll
    for (int j = 0; j < EPT; ++j) acc1[j] = acc2[j] = 0.f;
    const int32_t* ts = a.tstar + (int64_t)b * a.n_docs;
    for (int d0 = 0; d0 < a.n_docs; d0 += DQ_BLOCK) {
      // the block's documents whose maximum sits on token t, listed in document order
      // (a fixed summation order: the result does not depend on scheduling)
      const int dd = d0 + tid;
      const bool hit = dd < a.n_docs && ts[dd] == t;
      const uint64_t bal = __ballot(hit);
      if (lane == 0) wave_hits[wv] = __popcll(bal);
      __syncthreads();
      int base = 0, nm = 0;
#pragma unroll
      for (int i = 0; i < DQ_THREADS / 64; ++i) {
        base += (i < wv) ? wave_hits[i] : 0;
        nm += wave_hits[i];
      }
      if (hit) match[base + __popcll(bal & ((1ull << lane) - 1))] = dd;
      __syncthreads();
      for (int m = 0; m < nm; ++m) {
        const int64_t rec = (int64_t)b * a.n_docs + match[m];
        const float g = a.dD[rec];
        const int64_t kc = a.cstar[rec];
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
          const int i = tid + j * DQ_THREADS;
          if (i < n_el) {
            const int h = i / D;
            acc1[j] += g * ld_key<T, D>(K, kc, i, H) * a.kinv[rec * H + h];
            acc2[j] += g * a.cosv[rec * H + h];
          }
        }
      }
      __syncthreads();
    }
    float* dq = a.dQr + (int64_t)(q0 + t) * n_el;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int i = tid + j * DQ_THREADS;
      if (i < n_el) {
        const float qn = qn_s[i / D];
        float out = 0.f;
        if (qn > 0.f) {
          const float iq = 1.f / sqrtf(qn);
          out = (acc1[j] - acc2[j] * ld(q, i) * iq) * iq / (float)H;
        }
        dq[i] = out;
      }
    }
    __syncthreads();  // qn_s is rewritten for the next token
  }
}

// ---- bf16, d = 128, 4 or 8 heads: all heads of a pair at once --------------------------
// A lane holds EPL consecutive elements of one head (LPH lanes per head): 16-byte loads of
// the query row and of the tiled key row, per-head sums over the head's lanes.

// Sum over the LPH lanes of each head, returned to every lane of the head.
template <int LPH>
__device__ __forceinline__ float head_sum(float v) {
  v = group_sum_last<LPH>(v);
  return __shfl(v, (int)(threadIdx.x & 63) | (LPH - 1), 64);
}

// One document's share of the router's backward (a bank row belongs to one document, so
// the workgroup owns its rows' key gradients):
//  1. for each query, the maximising row (the first with the largest row score, 16 lanes
//     per query) and its first maximising token;
//  2. the queries with a gradient ordered by (row, query);
//  3. in that order, per record: the per-head cosine and 1/|k| (the record the query
//     gradient reads) and the key-gradient contribution, summed in registers over the
//     records of one row and added to the row once with a plain read-modify-write.
// A thread holds 8 consecutive elements of a row (16 threads per head).  The summation
// order is fixed: the result does not depend on scheduling.
template <int H>
__global__ __launch_bounds__(H * 16) void route_bwd_doc_b16(RouteBwdK a) {
  constexpr int D = 128, NE = H * D, NT = H * 16, QPASS = NT / 16;  // queries per pass
  __shared__ int q_c[64], q_t[64], q_order[64];  // row (relative to the document), token
  __shared__ float q_g[64];
  __shared__ int n_valid;
  const int d = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, sub = tid & 15;
  const int e0 = tid * 8, h = e0 / D;
  const bf16_t* K = (const bf16_t*)a.Krb;
  const int64_t c0 = a.chunk_off[d];
  const int nc = (int)(a.chunk_off[d + 1] - c0);
  for (int b0 = 0; b0 < a.n_queries; b0 += 64) {
    // ---- 1. maximising row and token of each query of the chunk ----
    for (int qi = tid / 16; qi < 64; qi += QPASS) {
      const int b = b0 + qi;
      const bool inq = b < a.n_queries;
      const int bb = inq ? b : a.n_queries - 1;  // addresses stay in bounds
      const int64_t rec = (int64_t)bb * a.n_docs + d;
      const int Lq = a.q_off[bb + 1] - a.q_off[bb];
      const float gd = a.dD[rec];
      float best = -INFINITY;
      int bc = nc;
      if (inq && gd != 0.f && Lq > 0) {
        const float* rs = a.row_scores + (int64_t)bb * a.n_chunks + c0;
        for (int c = sub; c < nc; c += 16) {
          const float v = rs[c];
          if (v > best) { best = v; bc = c; }  // c ascending: a tie keeps the first
        }
      }
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) {
        const float ov = __shfl_xor(best, o, 16);
        const int oc = __shfl_xor(bc, o, 16);
        if (ov > best || (ov == best && oc < bc)) { best = ov; bc = oc; }
      }
      if (sub == 0) {
        const bool v = inq && bc < nc;  // else no gradient (an empty query or document, g = 0)
        q_c[qi] = v ? bc : -1;
        q_t[qi] = v ? a.row_arg[(int64_t)bb * a.n_chunks + c0 + bc] : 0;
        q_g[qi] = gd / (float)H;
        if (inq && !v) a.tstar[rec] = -1;
      }
    }
    __syncthreads();
    // ---- 2. the records with a gradient, ordered by (row, query) ----
    if (tid < 64) {
      const int c = q_c[lane];
      const int key = c >= 0 ? c : INT_MAX;
      int rank = 0;
      for (int o = 0; o < 64; ++o) {
        const int ko = __shfl(key, o, 64);
        rank += (ko < key || (ko == key && o < lane)) ? 1 : 0;
      }
      if (c >= 0) q_order[rank] = lane;
      const int nv = __popcll(__ballot(c >= 0));
      if (lane == 0) n_valid = nv;
    }
    __syncthreads();
    // ---- 3. records and key gradients ----
    const int nv = n_valid;  // q_order[0 .. nv-1]; none read past them
    float acc[8], y[8];
    uint4 yraw = make_uint4(0, 0, 0, 0);  // the thread's 16 bytes of the current row
    float ik_row = 0.f;  // 1/|k| of the current row's head (0 for a zero vector)
    int row = -1;
    auto flush = [&]() __attribute__((always_inline)) {
      float* dk = a.dKrb + (c0 + row) * NE + e0;  // row-major, added to
      const float4 u0 = *reinterpret_cast<const float4*>(dk), u1 = *reinterpret_cast<const float4*>(dk + 4);
      *reinterpret_cast<float4*>(dk) = make_float4(u0.x + acc[0], u0.y + acc[1], u0.z + acc[2], u0.w + acc[3]);
      *reinterpret_cast<float4*>(dk + 4) = make_float4(u1.x + acc[4], u1.y + acc[5], u1.z + acc[6], u1.w + acc[7]);
    };
    // The next record's query slice (and its row's key slice when the row changes) is
    // loaded while the current record is computed: records are a chain of dependent loads.
    auto qslice = [&](int qi) __attribute__((always_inline)) {
      return *reinterpret_cast<const uint4*>((const bf16_t*)a.Qr + (int64_t)(a.q_off[b0 + qi] + q_t[qi]) * NE + e0);
    };
    auto kslice = [&](int c) __attribute__((always_inline)) {
      return *reinterpret_cast<const uint4*>(K + kr_tiled<D>(c0 + c, e0, H));
    };
    uint4 xnext = make_uint4(0, 0, 0, 0), ynext = xnext;
    if (nv > 0) {
      xnext = qslice(q_order[0]);
      ynext = kslice(q_c[q_order[0]]);
    }
    for (int r = 0; r < nv; ++r) {
      const int qi = q_order[r];
      const int b = b0 + qi, c = q_c[qi], t = q_t[qi];
      const int64_t rec = (int64_t)b * a.n_docs + d;
      const uint4 xraw = xnext, ycur = ynext;
      if (r + 1 < nv) {  // uniform
        const int qn1 = q_order[r + 1];
        xnext = qslice(qn1);
        const int c1 = q_c[qn1];
        if (c1 != c) ynext = kslice(c1);  // uniform
      }
      if (c != row) {  // uniform: the next row
        if (row >= 0) flush();
        row = c;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
        yraw = ycur;
        unpack8(yraw, y);
        float kn = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) kn += y[i] * y[i];
        kn = head_sum<16>(kn);
        ik_row = kn > 0.f ? 1.f / sqrtf(kn) : 0.f;
      }
      float x[8];
      unpack8(xraw, x);
      float dot = 0.f, qn = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        dot += x[i] * y[i];
        qn += x[i] * x[i];
      }
      dot = head_sum<16>(dot);
      qn = head_sum<16>(qn);
      const bool ok = qn > 0.f && ik_row > 0.f;  // no gradient for a head with a zero vector
      const float iq = ok ? 1.f / sqrtf(qn) : 0.f, ik = ok ? ik_row : 0.f;
      const float co = dot * iq * ik;
      if (sub == 0) {
        a.cosv[rec * H + h] = co;
        a.kinv[rec * H + h] = ik;
      }
      if (tid == 0) {
        a.tstar[rec] = t;
        a.cstar[rec] = c0 + c;
      }
      // the record's row, contiguous, for the query gradient (which would otherwise gather
      // it from the tiled layout at a 128-byte line per 16-byte piece)
      *reinterpret_cast<uint4*>(a.krec + rec * NE + e0) = yraw;
      const float w = q_g[qi] * ik;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += w * (x[i] * iq - co * y[i] * ik);
    }
    if (row >= 0) flush();
    __syncthreads();  // the chunk's arrays are rewritten for the next chunk of queries
  }
}

// The query gradient of one token: its matches (documents whose maximum sits on it) are
// taken PAR at a time by PAR thread groups, each thread holding 8 consecutive elements of
// the token's row; the groups' partial sums are combined in group order, so the summation
// order is fixed.
template <int H>
__global__ __launch_bounds__(DQ_THREADS) void route_bwd_dq_b16(RouteBwdK a) {
  constexpr int D = 128, NE = H * D, TPM = NE / 8, PAR = DQ_THREADS / TPM;
  static_assert(TPM * PAR == DQ_THREADS, "thread groups must tile the workgroup");
  __shared__ int match[DQ_BLOCK];
  __shared__ int wave_hits[DQ_THREADS / 64];
  __shared__ float part1[PAR > 1 ? PAR - 1 : 1][NE];
  __shared__ float part2[PAR > 1 ? PAR - 1 : 1][H];
  const int b = blockIdx.y;
  const int q0 = a.q_off[b], Lq = a.q_off[b + 1] - q0;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int grp = tid / TPM, e0 = (tid % TPM) * 8, h = e0 / D;
  for (int t = blockIdx.x; t < Lq; t += gridDim.x) {
    float acc1[8], acc2 = 0.f;  // sum of g * k / |k|, sum of g * cos (the thread's head)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc1[i] = 0.f;
    const int32_t* ts = a.tstar + (int64_t)b * a.n_docs;
    for (int d0 = 0; d0 < a.n_docs; d0 += DQ_BLOCK) {
      // the block's documents whose maximum sits on token t, listed in document order
      const int dd = d0 + tid;
      const bool hit = dd < a.n_docs && ts[dd] == t;
      const uint64_t bal = __ballot(hit);
      if (lane == 0) wave_hits[wv] = __popcll(bal);
      __syncthreads();
      int base = 0, nm = 0;
#pragma unroll
      for (int i = 0; i < DQ_THREADS / 64; ++i) {
        base += (i < wv) ? wave_hits[i] : 0;
        nm += wave_hits[i];
      }
      if (hit) match[base + __popcll(bal & ((1ull << lane) - 1))] = dd;
      __syncthreads();
      // group grp takes matches grp, grp + PAR, ..., two at a time (both loads in flight)
      int m = grp;
      for (; m + PAR < nm; m += 2 * PAR) {
        const int64_t r0 = (int64_t)b * a.n_docs + match[m], r1 = (int64_t)b * a.n_docs + match[m + PAR];
        const float g0 = a.dD[r0], g1 = a.dD[r1];
        const float w0 = g0 * a.kinv[r0 * H + h], w1 = g1 * a.kinv[r1 * H + h];
        const float c0v = g0 * a.cosv[r0 * H + h], c1v = g1 * a.cosv[r1 * H + h];
        const uint4 v0 = *reinterpret_cast<const uint4*>(a.krec + r0 * NE + e0);
        const uint4 v1 = *reinterpret_cast<const uint4*>(a.krec + r1 * NE + e0);
        float y0[8], y1[8];
        unpack8(v0, y0);
        unpack8(v1, y1);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc1[i] += w0 * y0[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc1[i] += w1 * y1[i];
        acc2 += c0v;
        acc2 += c1v;
      }
      if (m < nm) {
        const int64_t r0 = (int64_t)b * a.n_docs + match[m];
        const float g0 = a.dD[r0];
        float y0[8];
        unpack8(*reinterpret_cast<const uint4*>(a.krec + r0 * NE + e0), y0);
        const float w0 = g0 * a.kinv[r0 * H + h];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc1[i] += w0 * y0[i];
        acc2 += g0 * a.cosv[r0 * H + h];
      }
      __syncthreads();
    }
    // combine the groups in order: group 0 adds groups 1 .. PAR-1
    if constexpr (PAR > 1) {
      if (grp > 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) part1[grp - 1][e0 + i] = acc1[i];
        if (e0 % D == 0) part2[grp - 1][h] = acc2;
      }
      __syncthreads();
      if (grp == 0) {
#pragma unroll
        for (int p = 0; p < PAR - 1; ++p) {
#pragma unroll
          for (int i = 0; i < 8; ++i) acc1[i] += part1[p][e0 + i];
          acc2 += part2[p][h];
        }
      }
    }
    if (grp == 0) {
      const bf16_t* q = (const bf16_t*)a.Qr + (int64_t)(q0 + t) * NE + e0;
      float x[8];
      unpack8(*reinterpret_cast<const uint4*>(q), x);
      float qn = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) qn += x[i] * x[i];
      qn = head_sum<D / 8 < 64 ? D / 8 : 64>(qn);  // the 16 threads of the head (within a wave)
      float* dq = a.dQr + (int64_t)(q0 + t) * NE + e0;
      const float iq = qn > 0.f ? 1.f / sqrtf(qn) : 0.f;
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = qn > 0.f ? (acc1[i] - acc2 * x[i] * iq) * iq / (float)H : 0.f;
      *reinterpret_cast<float4*>(dq) = make_float4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<float4*>(dq + 4) = make_float4(o[4], o[5], o[6], o[7]);
    }
    __syncthreads();  // the partial-sum buffers are rewritten for the next token
  }
}

template <typename T, int D>
hipError_t launch_t(const RouteBwdArgs& r, const RouteBwdK& k, hipStream_t s) {
  if constexpr (sizeof(T) == 2 && D == 128) {
    if (r.h_r == 4 || r.h_r == 8) {
      dim3 g2((unsigned)(r.max_q_len < 1024 ? r.max_q_len : 1024), (unsigned)r.n_queries);
      if (r.h_r == 8) {
        hipLaunchKernelGGL((route_bwd_doc_b16<8>), dim3((unsigned)r.n_docs), dim3(128), 0, s, k);
        hipLaunchKernelGGL((route_bwd_dq_b16<8>), g2, dim3(DQ_THREADS), 0, s, k);
      } else {
        hipLaunchKernelGGL((route_bwd_doc_b16<4>), dim3((unsigned)r.n_docs), dim3(64), 0, s, k);
        hipLaunchKernelGGL((route_bwd_dq_b16<4>), g2, dim3(DQ_THREADS), 0, s, k);
      }
      return hipGetLastError();
    }
  }
  dim3 g1((unsigned)((r.n_docs + 3) / 4), (unsigned)r.n_queries);
  hipLaunchKernelGGL((route_bwd_pair<T, D>), g1, dim3(256), 0, s, k);
  dim3 g2((unsigned)(r.max_q_len < 1024 ? r.max_q_len : 1024), (unsigned)r.n_queries);
  hipLaunchKernelGGL((route_bwd_dq<T, D>), g2, dim3(DQ_THREADS), 0, s, k);
  return hipGetLastError();
}

}  // namespace

// Bytes per record of the record rows kept for the query gradient: 4 or 8 routing heads
// (bf16 banks of dim 128 take the per-document kernels), 0 otherwise.
static size_t krec_bytes(int h_r) { return (h_r == 4 || h_r == 8) ? (size_t)h_r * 128 * 2 : 0; }

size_t route_bwd_workspace_bytes(int n_queries, int n_docs, int64_t n_chunks, int h_r) {
  const size_t bn = (size_t)n_queries * n_docs;
  return align256(bn * 4) + 2 * align256((size_t)n_queries * n_chunks * 4) + align256(bn * 4) +
         align256(bn * 8) + 2 * align256(bn * h_r * 4) + align256(bn * krec_bytes(h_r));
}

hipError_t launch_route_backward(const RouteBwdArgs& r, hipStream_t s) {
  char* ws = (char*)r.workspace;
  const size_t bn = (size_t)r.n_queries * r.n_docs;
  float* scores = (float*)ws;
  ws += align256(bn * 4);
  float* rows = (float*)ws;
  ws += align256((size_t)r.n_queries * r.n_chunks * 4);
  int32_t* rarg = (int32_t*)ws;
  ws += align256((size_t)r.n_queries * r.n_chunks * 4);
  RouteBwdK k{};
  k.tstar = (int32_t*)ws;
  ws += align256(bn * 4);
  k.cstar = (int64_t*)ws;
  ws += align256(bn * 8);
  k.cosv = (float*)ws;
  ws += align256(bn * r.h_r * 4);
  k.kinv = (float*)ws;
  ws += align256(bn * r.h_r * 4);
  k.krec = krec_bytes(r.h_r) ? (bf16_t*)ws : nullptr;
  const float* row_scores = rows;
  const int32_t* row_arg = rarg;
  if (r.row_scores != nullptr) {
    // the forward scan's rows, passed in
    row_scores = r.row_scores;
    row_arg = r.row_arg;
  } else {
    // the forward scan again, keeping every row's max over the query's tokens
    RouteArgs f{r.dtype, r.n_queries, r.total_q, r.q_off, r.max_q_len, r.Qr, r.h_r, r.d, r.n_docs,
                r.n_chunks, r.chunk_off, r.Krbar, scores, 0};
    f.row_scores = rows;
    f.row_arg = rarg;
    const hipError_t e = launch_route_scan(f, s);
    if (e != hipSuccess) return e;
  }
  k.Qr = r.Qr;
  k.q_off = r.q_off;
  k.Krb = r.Krbar;
  k.chunk_off = r.chunk_off;
  k.dD = r.dD;
  k.row_scores = row_scores;
  k.row_arg = row_arg;
  k.dQr = r.dQr;
  k.dKrb = r.dKrbar;
  k.n_chunks = r.n_chunks;
  k.n_docs = r.n_docs;
  k.n_queries = r.n_queries;
  k.H = r.h_r;
  if (r.dtype == 0) {
    switch (r.d) {
      case 32: return launch_t<float, 32>(r, k, s);
      case 64: return launch_t<float, 64>(r, k, s);
      default: return launch_t<float, 128>(r, k, s);
    }
  }
  switch (r.d) {
    case 32: return launch_t<bf16_t, 32>(r, k, s);
    case 64: return launch_t<bf16_t, 64>(r, k, s);
    default: return launch_t<bf16_t, 128>(r, k, s);
  }
}

}  // namespace msa
