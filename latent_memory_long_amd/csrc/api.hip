// C ABI of the MSA hot path: argument validation, workspace layout, kernel launches.
// Declarations and the contract of every entry point are in include/msa.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/msa.h"
#include "launch.hpp"
#include "status.hpp"

thread_local std::string g_last_error;

msa_status fail(msa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

namespace {

msa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MSA_OK;
  return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool head_dim_ok(int32_t d) { return d == 32 || d == 64 || d == 128; }

int route_path_override() {
  const char* v = getenv("MSA_ROUTE_PATH");
  if (!v) return 0;
  if (!strcmp(v, "dot")) return 1;
  if (!strcmp(v, "mfma")) return 2;
  if (!strcmp(v, "batch")) return 3;
  return 0;
}

}  // namespace

extern "C" {

int32_t msa_version(void) { return 1 * 10000 + 0 * 100 + 0; }

const char* msa_status_string(msa_status s) {
  switch (s) {
    case MSA_OK: return "ok";
    case MSA_ERR_INVALID_ARG: return "invalid argument";
    case MSA_ERR_UNSUPPORTED: return "unsupported";
    case MSA_ERR_WORKSPACE: return "workspace too small";
    case MSA_ERR_HIP: return "HIP error";
    case MSA_ERR_IO: return "file error";
  }
  return "unknown status";
}

const char* msa_last_error(void) { return g_last_error.c_str(); }

int64_t msa_chunk_offsets(const int64_t* doc_tok_off, int32_t n_docs, int32_t chunk,
                          int64_t* chunk_off) {
  g_last_error.clear();
  if (!doc_tok_off || !chunk_off) { fail(MSA_ERR_INVALID_ARG, "null pointer"); return -1; }
  if (n_docs < 1) { fail(MSA_ERR_INVALID_ARG, "n_docs must be >= 1 (got %d)", n_docs); return -1; }
  if (chunk < 1) { fail(MSA_ERR_INVALID_ARG, "chunk must be >= 1 (got %d)", chunk); return -1; }
  if (doc_tok_off[0] != 0) { fail(MSA_ERR_INVALID_ARG, "doc_tok_off[0] must be 0"); return -1; }
  int64_t c = 0;
  chunk_off[0] = 0;
  for (int32_t d = 0; d < n_docs; ++d) {
    const int64_t len = doc_tok_off[d + 1] - doc_tok_off[d];
    if (len < 1) { fail(MSA_ERR_INVALID_ARG, "document %d has %lld tokens (need >= 1)", d, (long long)len); return -1; }
    c += (len + chunk - 1) / chunk;
    chunk_off[d + 1] = c;
  }
  return c;
}

int64_t msa_krbar_elems(msa_dtype dtype, int64_t n_chunks, int32_t h_r, int32_t d) {
  g_last_error.clear();
  if (dtype != MSA_F32 && dtype != MSA_BF16) { fail(MSA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype); return -1; }
  if (n_chunks < 0 || h_r < 1 || h_r > 64 || !head_dim_ok(d)) {
    fail(MSA_ERR_INVALID_ARG, "need n_chunks >= 0, h_r in [1, 64], d in {32, 64, 128} (got %lld, %d, %d)",
         (long long)n_chunks, h_r, d);
    return -1;
  }
  return msa::krbar_elems((int)dtype, n_chunks, h_r, d);
}

namespace {
msa_status krbar_convert_call(bool pack, msa_dtype dtype, int64_t n_chunks, int32_t h_r, int32_t d, const void* src,
                              void* dst, msa_stream_t stream) {
  g_last_error.clear();
  if (dtype != MSA_F32 && dtype != MSA_BF16) return fail(MSA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (n_chunks < 0 || h_r < 1 || h_r > 64 || !head_dim_ok(d))
    return fail(MSA_ERR_INVALID_ARG, "need n_chunks >= 0, h_r in [1, 64], d in {32, 64, 128} (got %lld, %d, %d)",
                (long long)n_chunks, h_r, d);
  if (n_chunks == 0) return MSA_OK;
  if (!src || !dst) return fail(MSA_ERR_INVALID_ARG, "null pointer");
  if (src == dst) return fail(MSA_ERR_INVALID_ARG, "source and destination must not overlap");
  const hipError_t e = pack ? msa::launch_krbar_pack((int)dtype, n_chunks, h_r, d, src, dst, (hipStream_t)stream)
                            : msa::launch_krbar_unpack((int)dtype, n_chunks, h_r, d, src, dst, (hipStream_t)stream);
  return hip_status(e, pack ? "msa_krbar_pack launch" : "msa_krbar_unpack launch");
}
}  // namespace

msa_status msa_krbar_pack(msa_dtype dtype, int64_t n_chunks, int32_t h_r, int32_t d, const void* rows, void* Krbar,
                          msa_stream_t stream) {
  return krbar_convert_call(true, dtype, n_chunks, h_r, d, rows, Krbar, stream);
}

msa_status msa_krbar_unpack(msa_dtype dtype, int64_t n_chunks, int32_t h_r, int32_t d, const void* Krbar,
                            void* rows, msa_stream_t stream) {
  return krbar_convert_call(false, dtype, n_chunks, h_r, d, Krbar, rows, stream);
}

msa_status msa_pool(msa_dtype dtype, int32_t n_docs, int64_t n_tokens, int64_t n_chunks,
                    const int64_t* doc_tok_off, const int64_t* chunk_off, int32_t h_kv,
                    int32_t h_r, int32_t d, int32_t chunk, float rope_base, uint32_t rope_mask,
                    const void* K, const void* V, const void* Kr, void* Kbar, void* Vbar,
                    void* Krbar, msa_stream_t stream) {
  g_last_error.clear();
  if (dtype != MSA_F32 && dtype != MSA_BF16) return fail(MSA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (n_docs < 1) return fail(MSA_ERR_INVALID_ARG, "n_docs must be >= 1 (got %d)", n_docs);
  if (n_tokens < n_docs) return fail(MSA_ERR_INVALID_ARG, "n_tokens (%lld) < n_docs (%d): every document needs a token", (long long)n_tokens, n_docs);
  if (n_chunks < n_docs || n_chunks > n_tokens) return fail(MSA_ERR_INVALID_ARG, "n_chunks (%lld) must lie in [n_docs, n_tokens]", (long long)n_chunks);
  if (!doc_tok_off || !chunk_off) return fail(MSA_ERR_INVALID_ARG, "null offset array");
  if (!K || !V || !Kr || !Kbar || !Vbar || !Krbar) return fail(MSA_ERR_INVALID_ARG, "null tensor pointer");
  if (h_kv < 1 || h_kv > 64 || h_r < 1 || h_r > 64) return fail(MSA_ERR_UNSUPPORTED, "h_kv and h_r must lie in [1, 64] (got %d, %d)", h_kv, h_r);
  if (!head_dim_ok(d)) return fail(MSA_ERR_UNSUPPORTED, "head dim %d not in {32, 64, 128}", d);
  if (chunk < 1 || chunk > 128) return fail(MSA_ERR_UNSUPPORTED, "chunk %d not in [1, 128]", chunk);
  if (rope_mask > 7u) return fail(MSA_ERR_INVALID_ARG, "rope_mask 0x%x has unknown bits", rope_mask);
  if (rope_mask && !(rope_base > 0.f && isfinite(rope_base))) return fail(MSA_ERR_INVALID_ARG, "rope_base must be finite and > 0");
  if (msa::debug_validate_enabled()) {
    const msa_status v = msa::debug_validate_pool(n_docs, n_tokens, n_chunks, chunk, doc_tok_off, chunk_off,
                                                  (hipStream_t)stream);
    if (v != MSA_OK) return v;
  }
  msa::PoolArgs a{(int)dtype, n_docs, n_tokens, n_chunks, doc_tok_off, chunk_off, h_kv, h_r, d,
                  chunk, rope_base, rope_mask, K, V, Kr, Kbar, Vbar, Krbar};
  return hip_status(msa::launch_pool(a, (hipStream_t)stream), "msa_pool launch");
}

size_t msa_topk_workspace(int32_t n_queries, int32_t n_docs, int32_t k) {
  if (n_queries < 1 || n_docs < 1 || k < 1 || k > 1024) return 0;
  return msa::topk_workspace_bytes(n_queries, n_docs, k);
}

size_t msa_route_topk_workspace(int32_t n_queries, int32_t n_docs, int32_t k) {
  if (n_queries < 1 || n_docs < 1 || k < 1 || k > 1024) return 0;
  return msa::align256((size_t)n_queries * (size_t)n_docs * sizeof(float)) +
         msa::topk_workspace_bytes(n_queries, n_docs, k);
}

namespace {

msa_status check_route(msa_dtype dtype, int32_t n_queries, int64_t total_q, const int32_t* q_off,
                       int32_t max_q_len, const void* Qr, int32_t h_r, int32_t d, int32_t n_docs,
                       int64_t n_chunks, const int64_t* chunk_off, const void* Krbar) {
  if (dtype != MSA_F32 && dtype != MSA_BF16) return fail(MSA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (n_queries < 1 || n_queries > 65535) return fail(MSA_ERR_INVALID_ARG, "n_queries %d not in [1, 65535]", n_queries);
  if (total_q < 0 || total_q > INT32_MAX) return fail(MSA_ERR_INVALID_ARG, "total_q %lld out of range", (long long)total_q);
  if (max_q_len < 1) return fail(MSA_ERR_INVALID_ARG, "max_q_len must be >= 1 (got %d)", max_q_len);
  if (!q_off || (total_q > 0 && !Qr)) return fail(MSA_ERR_INVALID_ARG, "null query pointer");
  if (h_r < 1 || h_r > 16) return fail(MSA_ERR_UNSUPPORTED, "h_r %d not in [1, 16]", h_r);
  if (!head_dim_ok(d)) return fail(MSA_ERR_UNSUPPORTED, "head dim %d not in {32, 64, 128}", d);
  if (n_docs < 1) return fail(MSA_ERR_INVALID_ARG, "n_docs must be >= 1 (got %d)", n_docs);
  if (n_chunks < n_docs) return fail(MSA_ERR_INVALID_ARG, "n_chunks (%lld) < n_docs (%d)", (long long)n_chunks, n_docs);
  if (!chunk_off || !Krbar) return fail(MSA_ERR_INVALID_ARG, "null bank pointer");
  return MSA_OK;
}

// check_route, then (MSA_DEBUG_VALIDATE=1) the device offsets
msa_status check_route_all(msa_dtype dtype, int32_t n_queries, int64_t total_q, const int32_t* q_off,
                           int32_t max_q_len, const void* Qr, int32_t h_r, int32_t d, int32_t n_docs,
                           int64_t n_chunks, const int64_t* chunk_off, const void* Krbar, msa_stream_t stream) {
  const msa_status st = check_route(dtype, n_queries, total_q, q_off, max_q_len, Qr, h_r, d, n_docs, n_chunks,
                                    chunk_off, Krbar);
  if (st != MSA_OK || !msa::debug_validate_enabled()) return st;
  return msa::debug_validate_route(n_queries, total_q, q_off, max_q_len, n_docs, n_chunks, chunk_off,
                                   (hipStream_t)stream);
}

msa_status check_topk(int32_t n_queries, int32_t n_docs, int32_t k, const int32_t* ids, const float* sc) {
  if (n_queries < 1 || n_queries > 65535) return fail(MSA_ERR_INVALID_ARG, "n_queries %d not in [1, 65535]", n_queries);
  if (n_docs < 1) return fail(MSA_ERR_INVALID_ARG, "n_docs must be >= 1 (got %d)", n_docs);
  if (k < 1) return fail(MSA_ERR_INVALID_ARG, "k must be >= 1 (got %d)", k);
  if (k > 1024) return fail(MSA_ERR_UNSUPPORTED, "k %d > 1024", k);
  if (!ids || !sc) return fail(MSA_ERR_INVALID_ARG, "null output pointer");
  return MSA_OK;
}

}  // namespace

msa_status msa_route_scan(msa_dtype dtype, int32_t n_queries, int64_t total_q, const int32_t* q_off,
                          int32_t max_q_len, const void* Qr, int32_t h_r, int32_t d, int32_t n_docs,
                          int64_t n_chunks, const int64_t* chunk_off, const void* Krbar,
                          float* doc_scores, float* row_scores, int32_t* row_arg,
                          msa_stream_t stream) {
  g_last_error.clear();
  msa_status st = check_route_all(dtype, n_queries, total_q, q_off, max_q_len, Qr, h_r, d, n_docs,
                                  n_chunks, chunk_off, Krbar, stream);
  if (st != MSA_OK) return st;
  if (!doc_scores) return fail(MSA_ERR_INVALID_ARG, "null doc_scores");
  if ((row_scores == nullptr) != (row_arg == nullptr))
    return fail(MSA_ERR_INVALID_ARG, "row_scores and row_arg go together (both or neither)");
  msa::RouteArgs r{(int)dtype, n_queries, total_q, q_off, max_q_len, Qr, h_r, d, n_docs, n_chunks,
                   chunk_off, Krbar, doc_scores, route_path_override()};
  r.row_scores = row_scores;
  r.row_arg = row_arg;
  return hip_status(msa::launch_route_scan(r, (hipStream_t)stream), "msa_route_scan launch");
}

msa_status msa_topk(int32_t n_queries, int32_t n_docs, const float* doc_scores, int32_t k,
                    int32_t* topk_ids, float* topk_scores, void* workspace,
                    size_t workspace_bytes, msa_stream_t stream) {
  g_last_error.clear();
  msa_status st = check_topk(n_queries, n_docs, k, topk_ids, topk_scores);
  if (st != MSA_OK) return st;
  if (!doc_scores) return fail(MSA_ERR_INVALID_ARG, "null doc_scores");
  const size_t need = msa_topk_workspace(n_queries, n_docs, k);
  if (need && (!workspace || workspace_bytes < need)) return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
  if (need && ((uintptr_t)workspace & 255u) != 0) return fail(MSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  msa::TopkArgs t{n_queries, n_docs, k, doc_scores, topk_ids, topk_scores};
  return hip_status(msa::launch_topk(t, workspace, (hipStream_t)stream), "msa_topk launch");
}

}  // extern "C"

namespace {

// msa_route_topk after validation, with a workspace of at least route_topk_need() bytes.
msa_status route_topk_run(msa_dtype dtype, int32_t n_queries, int64_t total_q, const int32_t* q_off,
                          int32_t max_q_len, const void* Qr, int32_t h_r, int32_t d, int32_t n_docs,
                          int64_t n_chunks, const int64_t* chunk_off, const void* Krbar, int32_t k,
                          int32_t* topk_ids, float* topk_scores, float* doc_scores, void* workspace,
                          msa_stream_t stream) {
  // workspace: [document scores when doc_scores is NULL][top-k candidates]
  const size_t score_bytes = doc_scores ? 0 : msa::align256((size_t)n_queries * n_docs * sizeof(float));
  float* scores = doc_scores ? doc_scores : (float*)workspace;
  void* topk_ws = msa::topk_workspace_bytes(n_queries, n_docs, k) ? (void*)((char*)workspace + score_bytes) : nullptr;
  hipStream_t s = (hipStream_t)stream;
  msa::RouteArgs r{(int)dtype, n_queries, total_q, q_off, max_q_len, Qr, h_r, d, n_docs, n_chunks,
                   chunk_off, Krbar, scores, route_path_override()};
  msa_status st = hip_status(msa::launch_route_scan(r, s), "msa_route_topk scan launch");
  if (st != MSA_OK) return st;
  msa::TopkArgs t{n_queries, n_docs, k, scores, topk_ids, topk_scores};
  return hip_status(msa::launch_topk(t, topk_ws, s), "msa_route_topk top-k launch");
}

size_t route_topk_need(int32_t n_queries, int32_t n_docs, int32_t k, const float* doc_scores) {
  const size_t score_bytes = doc_scores ? 0 : msa::align256((size_t)n_queries * n_docs * sizeof(float));
  return score_bytes + msa::topk_workspace_bytes(n_queries, n_docs, k);
}

}  // namespace

extern "C" {

msa_status msa_route_topk(msa_dtype dtype, int32_t n_queries, int64_t total_q,
                          const int32_t* q_off, int32_t max_q_len, const void* Qr, int32_t h_r,
                          int32_t d, int32_t n_docs, int64_t n_chunks, const int64_t* chunk_off,
                          const void* Krbar, int32_t k, int32_t* topk_ids, float* topk_scores,
                          float* doc_scores, void* workspace, size_t workspace_bytes,
                          msa_stream_t stream) {
  g_last_error.clear();
  msa_status st = check_route_all(dtype, n_queries, total_q, q_off, max_q_len, Qr, h_r, d, n_docs,
                                  n_chunks, chunk_off, Krbar, stream);
  if (st != MSA_OK) return st;
  st = check_topk(n_queries, n_docs, k, topk_ids, topk_scores);
  if (st != MSA_OK) return st;
  const size_t need = route_topk_need(n_queries, n_docs, k, doc_scores);
  if (need && (!workspace || workspace_bytes < need)) return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
  if (need && ((uintptr_t)workspace & 255u) != 0) return fail(MSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return route_topk_run(dtype, n_queries, total_q, q_off, max_q_len, Qr, h_r, d, n_docs, n_chunks, chunk_off, Krbar,
                        k, topk_ids, topk_scores, doc_scores, need ? workspace : nullptr, stream);
}

}  // extern "C"

// ---- the router without allocation -----------------------------------------------------
// msa_route_topk_noalloc keeps its scratch (document scores when the caller passes none, and
// the top-k candidates) in a file-scope device array instead of a caller workspace.  Each
// device holds its own copy of the array for the life of the process; in host code the
// array's name is only a handle, so its device address is looked up once per device and
// kept.  Calls that overlap on one device share the array and race.
namespace {

constexpr size_t NOALLOC_SCRATCH_BYTES = MSA_ROUTE_TOPK_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The current device's scratch address (looked up with that device current, on its first use).
msa_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return fail(MSA_ERR_UNSUPPORTED, "device %d: the library tracks devices 0..%d", dev, MAX_DEVICES - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress of the scratch array");
    if (!p) return fail(MSA_ERR_HIP, "hipGetSymbolAddress returned no address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

}  // namespace

extern "C" {

msa_status msa_route_topk_noalloc(msa_dtype dtype, int32_t n_queries, int64_t total_q,
                                  const int32_t* q_off, int32_t max_q_len, const void* Qr, int32_t h_r,
                                  int32_t d, int32_t n_docs, int64_t n_chunks, const int64_t* chunk_off,
                                  const void* Krbar, int32_t k, int32_t* topk_ids, float* topk_scores,
                                  float* doc_scores, msa_stream_t stream) {
  g_last_error.clear();
  // host checks only: the opt-in debug validation copies offsets into host buffers
  msa_status st = check_route(dtype, n_queries, total_q, q_off, max_q_len, Qr, h_r, d, n_docs, n_chunks, chunk_off,
                              Krbar);
  if (st != MSA_OK) return st;
  st = check_topk(n_queries, n_docs, k, topk_ids, topk_scores);
  if (st != MSA_OK) return st;
  const size_t need = route_topk_need(n_queries, n_docs, k, doc_scores);
  if (need > NOALLOC_SCRATCH_BYTES)
    return fail(MSA_ERR_WORKSPACE,
                "%d queries x %d documents need %zu bytes of scratch, more than the %zu this entry point holds "
                "(pass doc_scores, or call msa_route_topk with a workspace)",
                n_queries, n_docs, need, NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need) {
    st = scratch_address(&ws);
    if (st != MSA_OK) return st;
  }
  return route_topk_run(dtype, n_queries, total_q, q_off, max_q_len, Qr, h_r, d, n_docs, n_chunks, chunk_off, Krbar,
                        k, topk_ids, topk_scores, doc_scores, ws, stream);
}

size_t msa_route_backward_workspace(int32_t n_queries, int32_t n_docs, int64_t n_chunks, int32_t h_r) {
  if (n_queries < 1 || n_docs < 1 || n_chunks < n_docs || h_r < 1 || h_r > 16) return 0;
  return msa::route_bwd_workspace_bytes(n_queries, n_docs, n_chunks, h_r);
}

msa_status msa_route_backward(msa_dtype dtype, int32_t n_queries, int64_t total_q,
                              const int32_t* q_off, int32_t max_q_len, const void* Qr, int32_t h_r,
                              int32_t d, int32_t n_docs, int64_t n_chunks, const int64_t* chunk_off,
                              const void* Krbar, const float* dD, const float* row_scores,
                              const int32_t* row_arg, float* dQr, float* dKrbar, void* workspace,
                              size_t workspace_bytes, msa_stream_t stream) {
  g_last_error.clear();
  msa_status st = check_route_all(dtype, n_queries, total_q, q_off, max_q_len, Qr, h_r, d, n_docs,
                                  n_chunks, chunk_off, Krbar, stream);
  if (st != MSA_OK) return st;
  if (!dD || !dKrbar || (total_q > 0 && !dQr)) return fail(MSA_ERR_INVALID_ARG, "null gradient pointer");
  if ((row_scores == nullptr) != (row_arg == nullptr))
    return fail(MSA_ERR_INVALID_ARG, "row_scores and row_arg go together (both or neither)");
  const size_t need = msa_route_backward_workspace(n_queries, n_docs, n_chunks, h_r);
  if (!workspace || workspace_bytes < need) return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
  if (((uintptr_t)workspace & 255u) != 0) return fail(MSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  msa::RouteBwdArgs r{(int)dtype, n_queries, total_q, q_off, max_q_len, Qr, h_r, d, n_docs, n_chunks,
                      chunk_off, Krbar, dD, dQr, dKrbar, workspace};
  r.row_scores = row_scores;
  r.row_arg = row_arg;
  return hip_status(msa::launch_route_backward(r, (hipStream_t)stream), "msa_route_backward launch");
}

msa_status msa_route_aux_loss(int32_t kind, int32_t n_queries, int32_t n_docs, const float* doc_scores,
                              const float* labels, float temperature, float* loss, float* dD,
                              msa_stream_t stream) {
  g_last_error.clear();
  if (kind != MSA_AUX_BCE && kind != MSA_AUX_INFONCE) return fail(MSA_ERR_UNSUPPORTED, "unknown loss kind %d", kind);
  if (n_queries < 1 || n_docs < 1) return fail(MSA_ERR_INVALID_ARG, "need n_queries >= 1 and n_docs >= 1 (got %d, %d)", n_queries, n_docs);
  if (!(temperature > 0.f && isfinite(temperature))) return fail(MSA_ERR_INVALID_ARG, "temperature must be finite and > 0");
  if (!doc_scores || !labels || !loss || !dD) return fail(MSA_ERR_INVALID_ARG, "null pointer");
  msa::AuxArgs a{kind, n_queries, n_docs, doc_scores, labels, temperature, loss, dD};
  return hip_status(msa::launch_aux_loss(a, (hipStream_t)stream), "msa_route_aux_loss launch");
}

// The bank's content rows live in page-locked host memory: the device-side aliases.
static msa_status host_bank_alias(const void* Kbar, const void* Vbar, const void** kb, const void** vb) {
  const void* host[2] = {Kbar, Vbar};
  const void* dev[2] = {nullptr, nullptr};
  for (int i = 0; i < 2; ++i) {
    hipPointerAttribute_t attr;
    hipError_t e = hipPointerGetAttributes(&attr, host[i]);
    if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
      (void)hipGetLastError();
      return fail(MSA_ERR_INVALID_ARG, "kv_source=1 needs page-locked host memory for %s", i ? "Vbar" : "Kbar");
    }
    void* p = nullptr;
    e = hipHostGetDevicePointer(&p, const_cast<void*>(host[i]), 0);
    if (e != hipSuccess) return hip_status(e, "hipHostGetDevicePointer");
    dev[i] = p;
  }
  *kb = dev[0];
  *vb = dev[1];
  return MSA_OK;
}

size_t msa_sparse_attn_workspace(msa_dtype dtype, int32_t n_queries, int64_t total_q,
                                 int64_t total_kv, int32_t max_q_len, int32_t hq, int32_t h_kv,
                                 int32_t d) {
  if ((dtype != MSA_F32 && dtype != MSA_BF16) || n_queries < 1 || total_q < 0 || total_kv < 0 ||
      max_q_len < 1 || hq < 1 || h_kv < 1 || hq % h_kv || !head_dim_ok(d))
    return 0;
  return msa::attn_workspace_bytes((int)dtype, n_queries, total_q, total_kv, max_q_len, hq, h_kv, d);
}

msa_status msa_sparse_attn(msa_dtype dtype, int32_t n_queries, int64_t total_q, int64_t total_kv,
                           const int32_t* q_off, const int32_t* kv_off, int32_t max_q_len,
                           const void* Q, const void* Kloc, const void* Vloc, int32_t hq,
                           int32_t h_kv, int32_t d, float rope_base, float scale, int32_t k,
                           const int32_t* topk_ids, int32_t n_docs, int64_t n_chunks,
                           const int64_t* chunk_off, const void* Kbar, const void* Vbar,
                           int32_t kv_source, void* O, float* lse, void* workspace,
                           size_t workspace_bytes, msa_stream_t stream) {
  g_last_error.clear();
  if (dtype != MSA_F32 && dtype != MSA_BF16) return fail(MSA_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (n_queries < 1 || n_queries > 65535) return fail(MSA_ERR_INVALID_ARG, "n_queries %d not in [1, 65535]", n_queries);
  if (total_q < 0 || total_q > INT32_MAX || total_kv < total_q || total_kv > INT32_MAX)
    return fail(MSA_ERR_INVALID_ARG, "need 0 <= total_q <= total_kv < 2^31 (got %lld, %lld)", (long long)total_q, (long long)total_kv);
  if (max_q_len < 1) return fail(MSA_ERR_INVALID_ARG, "max_q_len must be >= 1 (got %d)", max_q_len);
  if (!q_off || !kv_off) return fail(MSA_ERR_INVALID_ARG, "null offset array");
  if (total_q > 0 && (!Q || !O)) return fail(MSA_ERR_INVALID_ARG, "null query/output pointer");
  if (total_kv > 0 && (!Kloc || !Vloc)) return fail(MSA_ERR_INVALID_ARG, "null local K/V pointer");
  if (hq < 1 || h_kv < 1) return fail(MSA_ERR_INVALID_ARG, "head counts must be >= 1 (got %d, %d)", hq, h_kv);
  if (hq % h_kv) return fail(MSA_ERR_INVALID_ARG, "hq (%d) is not a multiple of h_kv (%d)", hq, h_kv);
  if (!head_dim_ok(d)) return fail(MSA_ERR_UNSUPPORTED, "head dim %d not in {32, 64, 128}", d);
  if (!(rope_base > 0.f && isfinite(rope_base))) return fail(MSA_ERR_INVALID_ARG, "rope_base must be finite and > 0");
  if (!isfinite(scale) || scale < 0.f) return fail(MSA_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if (k < 1) return fail(MSA_ERR_INVALID_ARG, "k must be >= 1 (got %d)", k);
  if (k > 1024) return fail(MSA_ERR_UNSUPPORTED, "k %d > 1024", k);
  if (!topk_ids) return fail(MSA_ERR_INVALID_ARG, "null topk_ids");
  if (n_docs < 1 || n_chunks < n_docs) return fail(MSA_ERR_INVALID_ARG, "need n_docs >= 1 and n_chunks >= n_docs");
  if (!chunk_off || !Kbar || !Vbar) return fail(MSA_ERR_INVALID_ARG, "null bank pointer");
  if (kv_source != 0 && kv_source != 1) return fail(MSA_ERR_INVALID_ARG, "kv_source must be 0 (device) or 1 (pinned host)");
  const size_t need = msa_sparse_attn_workspace(dtype, n_queries, total_q, total_kv, max_q_len, hq, h_kv, d);
  if (!workspace || workspace_bytes < need) return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
  if (((uintptr_t)workspace & 255u) != 0) return fail(MSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

  const void* kb = Kbar;
  const void* vb = Vbar;
  if (kv_source == 1) {
    const msa_status st = host_bank_alias(Kbar, Vbar, &kb, &vb);
    if (st != MSA_OK) return st;
  }
  if (msa::debug_validate_enabled()) {
    const msa_status v = msa::debug_validate_attn(n_queries, total_q, total_kv, q_off, kv_off, max_q_len, k,
                                                  topk_ids, n_docs, n_chunks, chunk_off, (hipStream_t)stream);
    if (v != MSA_OK) return v;
  }
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
  msa::AttnArgs a{(int)dtype, n_queries, total_q, total_kv, q_off, kv_off, max_q_len, Q, Kloc, Vloc,
                  hq, h_kv, d, rope_base, sc, k, topk_ids, n_docs, n_chunks, chunk_off, kb, vb, O,
                  lse, workspace};
  return hip_status(msa::launch_sparse_attn(a, (hipStream_t)stream), "msa_sparse_attn launch");
}

size_t msa_sparse_attn_backward_workspace(int64_t total_q, int64_t total_kv, int32_t hq, int32_t h_kv,
                                          int32_t d) {
  if (total_q < 0 || total_kv < 0 || hq < 1 || h_kv < 1 || hq % h_kv || (d != 64 && d != 128)) return 0;
  return msa::attn_bwd_workspace_bytes(total_q, total_kv, hq, h_kv, d);
}

msa_status msa_sparse_attn_backward(msa_dtype dtype, int32_t n_queries, int64_t total_q, int64_t total_kv,
                                    const int32_t* q_off, const int32_t* kv_off, int32_t max_q_len,
                                    const void* Q, const void* Kloc, const void* Vloc, int32_t hq,
                                    int32_t h_kv, int32_t d, float rope_base, float scale, int32_t k,
                                    const int32_t* topk_ids, int32_t n_docs, int64_t n_chunks,
                                    const int64_t* chunk_off, const void* Kbar, const void* Vbar,
                                    int32_t kv_source, const void* O, const float* lse,
                                    const void* dO, float* dQ,
                                    float* dKloc, float* dVloc, float* dKbar, float* dVbar,
                                    void* workspace, size_t workspace_bytes, msa_stream_t stream) {
  g_last_error.clear();
  if (dtype != MSA_BF16) return fail(MSA_ERR_UNSUPPORTED, "the backward supports bf16 only (dtype %d)", (int)dtype);
  if (n_queries < 1 || n_queries > 65535) return fail(MSA_ERR_INVALID_ARG, "n_queries %d not in [1, 65535]", n_queries);
  if (total_q < 0 || total_q > INT32_MAX || total_kv < total_q || total_kv > INT32_MAX)
    return fail(MSA_ERR_INVALID_ARG, "need 0 <= total_q <= total_kv < 2^31 (got %lld, %lld)", (long long)total_q, (long long)total_kv);
  if (max_q_len < 1) return fail(MSA_ERR_INVALID_ARG, "max_q_len must be >= 1 (got %d)", max_q_len);
  if (!q_off || !kv_off) return fail(MSA_ERR_INVALID_ARG, "null offset array");
  if (total_q > 0 && (!Q || !O || !dO || !dQ)) return fail(MSA_ERR_INVALID_ARG, "null query-side pointer");
  if (total_kv > 0 && (!Kloc || !Vloc || !dKloc || !dVloc)) return fail(MSA_ERR_INVALID_ARG, "null local K/V pointer");
  if (hq < 1 || h_kv < 1) return fail(MSA_ERR_INVALID_ARG, "head counts must be >= 1 (got %d, %d)", hq, h_kv);
  if (hq % h_kv) return fail(MSA_ERR_INVALID_ARG, "hq (%d) is not a multiple of h_kv (%d)", hq, h_kv);
  if (d != 64 && d != 128) return fail(MSA_ERR_UNSUPPORTED, "the backward supports head dim 64 or 128 (got %d)", d);
  if (!(rope_base > 0.f && isfinite(rope_base))) return fail(MSA_ERR_INVALID_ARG, "rope_base must be finite and > 0");
  if (!isfinite(scale) || scale < 0.f) return fail(MSA_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if (k < 1) return fail(MSA_ERR_INVALID_ARG, "k must be >= 1 (got %d)", k);
  if (k > 1024) return fail(MSA_ERR_UNSUPPORTED, "k %d > 1024", k);
  if (!topk_ids) return fail(MSA_ERR_INVALID_ARG, "null topk_ids");
  if (n_docs < 1 || n_chunks < n_docs) return fail(MSA_ERR_INVALID_ARG, "need n_docs >= 1 and n_chunks >= n_docs");
  if (!chunk_off || !Kbar || !Vbar || !dKbar || !dVbar) return fail(MSA_ERR_INVALID_ARG, "null bank pointer");
  if (kv_source != 0 && kv_source != 1) return fail(MSA_ERR_INVALID_ARG, "kv_source must be 0 (device) or 1 (pinned host)");
  const size_t need = msa_sparse_attn_backward_workspace(total_q, total_kv, hq, h_kv, d);
  if (!workspace || workspace_bytes < need) return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
  if (((uintptr_t)workspace & 255u) != 0) return fail(MSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const void* kb = Kbar;
  const void* vb = Vbar;
  if (kv_source == 1) {
    const msa_status st = host_bank_alias(Kbar, Vbar, &kb, &vb);
    if (st != MSA_OK) return st;
  }
  if (msa::debug_validate_enabled()) {
    const msa_status v = msa::debug_validate_attn(n_queries, total_q, total_kv, q_off, kv_off, max_q_len, k,
                                                  topk_ids, n_docs, n_chunks, chunk_off, (hipStream_t)stream);
    if (v != MSA_OK) return v;
  }
  msa::AttnBwdArgs a{};
  a.f = msa::AttnArgs{(int)dtype, n_queries, total_q, total_kv, q_off, kv_off, max_q_len, Q, Kloc, Vloc,
                      hq, h_kv, d, rope_base, scale, k, topk_ids, n_docs, n_chunks, chunk_off, kb, vb,
                      nullptr, nullptr, workspace};
  a.O = O;
  a.lse = lse;
  a.dO = dO;
  a.dQ = dQ;
  a.dKloc = dKloc;
  a.dVloc = dVloc;
  a.dKbar = dKbar;
  a.dVbar = dVbar;
  a.workspace = workspace;
  return hip_status(msa::launch_sparse_attn_backward(a, (hipStream_t)stream), "msa_sparse_attn_backward launch");
}

}  // extern "C"
