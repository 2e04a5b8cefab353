// Internal launchers: one per kernel family, defined next to the kernels.  Each one
// assumes the C-ABI layer already validated its arguments and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

struct PoolArgs {
  int dtype;  // 0 f32, 1 bf16
  int n_docs;
  int64_t n_tokens, n_chunks;
  const int64_t* doc_tok_off;
  const int64_t* chunk_off;
  int h_kv, h_r, d, chunk;
  float rope_base;
  uint32_t rope_mask;
  const void *K, *V, *Kr;
  void *Kbar, *Vbar, *Krbar;
  int stage_waves = 0;   // set by the launcher: LDS staging of tiled routing keys
  int stage_offset = 0;
};
hipError_t launch_pool(const PoolArgs& a, hipStream_t s);

struct RouteArgs {
  int dtype;
  int n_queries;
  int64_t total_q;
  const int32_t* q_off;
  int max_q_len;
  const void* Qr;
  int h_r, d;
  int n_docs;
  int64_t n_chunks;
  const int64_t* chunk_off;
  const void* Krbar;
  float* scores;   // [n_queries, n_docs] output
  int force_path;  // 0 auto, 1 dot, 2 mfma, 3 batch (MSA_ROUTE_PATH environment override)
  float* row_scores = nullptr;  // [n_queries, n_chunks] or null: per-row max over tokens
  int32_t* row_arg = nullptr;   // with row_scores: the first token reaching each row's max
};
hipError_t launch_route_scan(const RouteArgs& a, hipStream_t s);
hipError_t launch_fill_neg_inf(float* p, int64_t n, hipStream_t s);
bool route_batch_supported(const RouteArgs& a);
hipError_t launch_route_scan_batch(const RouteArgs& a, hipStream_t s);

struct RouteBwdArgs {
  int dtype;
  int n_queries;
  int64_t total_q;
  const int32_t* q_off;
  int max_q_len;
  const void* Qr;
  int h_r, d;
  int n_docs;
  int64_t n_chunks;
  const int64_t* chunk_off;
  const void* Krbar;
  const float* dD;  // [n_queries, n_docs] gradient of the loss with respect to the scores
  float* dQr;       // [total_q, h_r, d] overwritten
  float* dKrbar;    // [n_chunks, h_r, d] added to
  void* workspace;
  const float* row_scores = nullptr;  // optional: the forward scan's row outputs (else rescanned)
  const int32_t* row_arg = nullptr;
};
size_t route_bwd_workspace_bytes(int n_queries, int n_docs, int64_t n_chunks, int h_r);
hipError_t launch_route_backward(const RouteBwdArgs& a, hipStream_t s);

struct TopkArgs {
  int n_queries, n_docs, k;
  const float* doc_scores;  // [n_queries, n_docs]
  int32_t* ids;
  float* scores;
};
size_t topk_workspace_bytes(int n_queries, int n_docs, int k);
hipError_t launch_topk(const TopkArgs& a, void* workspace, hipStream_t s);

struct AttnArgs {
  int dtype;
  int n_queries;
  int64_t total_q, total_kv;
  const int32_t *q_off, *kv_off;
  int max_q_len;
  const void *Q, *Kloc, *Vloc;
  int hq, h_kv, d;
  float rope_base, scale;
  int k;
  const int32_t* ids;
  int n_docs;
  int64_t n_chunks;
  const int64_t* chunk_off;
  const void *Kbar, *Vbar;
  void* O;
  float* lse;        // optional [total_q * hq]: natural-log log-sum-exp of each row's logits
  void* workspace;
};
int attn_rows_per_block(int max_q_len, int G);
int attn_fwd_rows(int max_q_len, int G, bool host);
int attn_splits(int n_queries, int max_q_len, int hq, int h_kv);
size_t attn_workspace_bytes(int dtype, int n_queries, int64_t total_q, int64_t total_kv,
                            int max_q_len, int hq, int h_kv, int d);
hipError_t launch_sparse_attn(const AttnArgs& a, hipStream_t s);

struct AttnBwdArgs {
  AttnArgs f;        // the forward call's arguments (f.O unused)
  const void* O;     // forward output
  const float* lse;  // optional: the forward's log-sum-exp per row (else recomputed)
  const void* dO;    // gradient of the loss with respect to O
  float *dQ, *dKloc, *dVloc;  // overwritten
  float *dKbar, *dVbar;       // accumulated
  void* workspace;
};
size_t attn_bwd_workspace_bytes(int64_t total_q, int64_t total_kv, int hq, int h_kv, int d);
hipError_t launch_sparse_attn_backward(const AttnBwdArgs& a, hipStream_t s);

constexpr int AUX_BCE = 0;
constexpr int AUX_INFONCE = 1;
struct AuxArgs {
  int kind;  // AUX_BCE or AUX_INFONCE
  int n_queries, n_docs;
  const float* scores;  // [n_queries, n_docs]
  const float* labels;  // [n_queries, n_docs]
  float temperature;
  float* loss;          // [n_queries]
  float* dD;            // [n_queries, n_docs]
};
hipError_t launch_aux_loss(const AuxArgs& a, hipStream_t s);

// Conversion of routing keys between row-major [n_chunks, h_r, d] and the bank layout
// (tiled for bf16, row-major for float32): pack writes the layout's padding rows as zero.
int64_t krbar_elems(int dtype, int64_t n_chunks, int h_r, int d);
hipError_t launch_krbar_pack(int dtype, int64_t n_chunks, int h_r, int d, const void* rows, void* krbar,
                             hipStream_t s);
hipError_t launch_krbar_unpack(int dtype, int64_t n_chunks, int h_r, int d, const void* krbar, void* rows,
                               hipStream_t s);

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace msa
