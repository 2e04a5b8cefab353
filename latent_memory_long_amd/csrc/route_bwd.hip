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
  float* dKrb;              // [C, H, D], added to
  int32_t* tstar;           // [B, N]: maximising token (query-local), -1 if no gradient
  int64_t* cstar;           // [B, N]: maximising row
  float* cosv;              // [B, N, H]
  float* kinv;              // [B, N, H]: 1/|k| (0 when either vector is zero)
  int64_t n_chunks;
  int n_docs, n_queries, H;
};

template <typename T> __device__ __forceinline__ float ld(const T* p, int64_t i);
template <> __device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld<bf16_t>(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

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
  const T* k = (const T*)a.Krb + cs * H * D;
  float* dk = a.dKrb + cs * H * D;
  const float gH = gd / (float)H;
  // gradient of the pair, head by head, lanes over elements
  for (int h = 0; h < H; ++h) {
    float dot = 0.f, qn = 0.f, kn = 0.f;
    for (int e = lane; e < D; e += 64) {
      const float x = ld(q, h * D + e), y = ld(k, h * D + e);
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
        atomicAdd(dk + h * D + e, gH * (ld(q, h * D + e) * iq - cosv * ld(k, h * D + e) * ik) * ik);
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
        const T* k = K + a.cstar[rec] * n_el;
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
          const int i = tid + j * DQ_THREADS;
          if (i < n_el) {
            const int h = i / D;
            acc1[j] += g * ld(k, i) * a.kinv[rec * H + h];
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

template <typename T, int D>
hipError_t launch_t(const RouteBwdArgs& r, const RouteBwdK& k, hipStream_t s) {
  dim3 g1((unsigned)((r.n_docs + 3) / 4), (unsigned)r.n_queries);
  hipLaunchKernelGGL((route_bwd_pair<T, D>), g1, dim3(256), 0, s, k);
  dim3 g2((unsigned)(r.max_q_len < 1024 ? r.max_q_len : 1024), (unsigned)r.n_queries);
  hipLaunchKernelGGL((route_bwd_dq<T, D>), g2, dim3(DQ_THREADS), 0, s, k);
  return hipGetLastError();
}

}  // namespace

size_t route_bwd_workspace_bytes(int n_queries, int n_docs, int64_t n_chunks, int h_r) {
  const size_t bn = (size_t)n_queries * n_docs;
  return align256(bn * 4) + 2 * align256((size_t)n_queries * n_chunks * 4) + align256(bn * 4) +
         align256(bn * 8) + 2 * align256(bn * h_r * 4);
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
