// Opt-in validation of the device-resident index arrays (MSA_DEBUG_VALIDATE=1).
//
// The kernels take the offset arrays and selected ids as preconditions and never read them
// on the host.  With the environment variable MSA_DEBUG_VALIDATE set to 1, every entry point
// first copies the arrays it is given to the host (synchronising `stream`), checks them,
// and returns MSA_ERR_INVALID_ARG with a message naming the first offending entry, before
// any kernel is launched.  Host code only.
#include <stdlib.h>

#include <vector>

#include "launch.hpp"
#include "status.hpp"

namespace msa {

bool debug_validate_enabled() {
  const char* v = getenv("MSA_DEBUG_VALIDATE");
  return v != nullptr && v[0] == '1' && v[1] == '\0';
}

namespace {

template <typename T>
msa_status fetch(const T* dev, size_t n, std::vector<T>& out, hipStream_t s, const char* what) {
  out.resize(n);
  if (n == 0) return MSA_OK;
  hipError_t e = hipMemcpyAsync(out.data(), dev, n * sizeof(T), hipMemcpyDefault, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(MSA_ERR_HIP, "validation copy of %s: %s", what, hipGetErrorString(e));
  return MSA_OK;
}

// off[0] == first (any first >= 0 when first < 0), off[n] == off[0] + total, and each entry
// at least `min_len` past the previous one.
template <typename T>
msa_status check_offsets(const std::vector<T>& off, int64_t total, int64_t min_len, const char* what,
                         int64_t first = 0) {
  const size_t n = off.size() - 1;
  if (first >= 0 && (int64_t)off[0] != first)
    return fail(MSA_ERR_INVALID_ARG, "%s[0] is %lld, not %lld", what, (long long)off[0], (long long)first);
  if (off[0] < 0) return fail(MSA_ERR_INVALID_ARG, "%s[0] is %lld, negative", what, (long long)off[0]);
  total += (int64_t)off[0];
  for (size_t i = 0; i < n; ++i)
    if ((int64_t)off[i + 1] - (int64_t)off[i] < min_len)
      return fail(MSA_ERR_INVALID_ARG, "%s[%zu] = %lld after %lld: entries must grow by at least %lld", what,
                  i + 1, (long long)off[i + 1], (long long)off[i], (long long)min_len);
  if ((int64_t)off[n] != total)
    return fail(MSA_ERR_INVALID_ARG, "%s[%zu] is %lld, not %lld", what, n, (long long)off[n], (long long)total);
  return MSA_OK;
}

// first = -1: the offsets may start past row 0 (pooling after the rows a bank holds)
msa_status check_chunk_off(const int64_t* chunk_off, int32_t n_docs, int64_t n_chunks, hipStream_t s,
                           std::vector<int64_t>& co, int64_t first = 0) {
  msa_status st = fetch(chunk_off, (size_t)n_docs + 1, co, s, "chunk_off");
  if (st != MSA_OK) return st;
  return check_offsets(co, n_chunks, 1, "chunk_off", first);  // every document has >= 1 row
}

msa_status check_queries(const int32_t* q_off, int32_t n_queries, int64_t total_q, int32_t max_q_len,
                         hipStream_t s, std::vector<int32_t>& qo) {
  msa_status st = fetch(q_off, (size_t)n_queries + 1, qo, s, "q_off");
  if (st == MSA_OK) st = check_offsets(qo, total_q, 0, "q_off");
  if (st != MSA_OK) return st;
  for (int32_t b = 0; b < n_queries; ++b)
    if (qo[b + 1] - qo[b] > max_q_len)
      return fail(MSA_ERR_INVALID_ARG, "query %d has %d tokens, more than max_q_len %d", b, qo[b + 1] - qo[b],
                  max_q_len);
  return MSA_OK;
}

}  // namespace

msa_status debug_validate_pool(int32_t n_docs, int64_t n_tokens, int64_t n_chunks, int32_t chunk,
                               const int64_t* doc_tok_off, const int64_t* chunk_off, hipStream_t s) {
  std::vector<int64_t> to, co;
  msa_status st = fetch(doc_tok_off, (size_t)n_docs + 1, to, s, "doc_tok_off");
  if (st == MSA_OK) st = check_offsets(to, n_tokens, 1, "doc_tok_off");  // every document has >= 1 token
  if (st == MSA_OK) st = check_chunk_off(chunk_off, n_docs, n_chunks, s, co, -1);
  if (st != MSA_OK) return st;
  for (int32_t d = 0; d < n_docs; ++d) {
    const int64_t want = (to[d + 1] - to[d] + chunk - 1) / chunk;
    if (co[d + 1] - co[d] != want)
      return fail(MSA_ERR_INVALID_ARG, "document %d: %lld tokens need %lld rows of %d, chunk_off gives %lld", d,
                  (long long)(to[d + 1] - to[d]), (long long)want, chunk, (long long)(co[d + 1] - co[d]));
  }
  return MSA_OK;
}

msa_status debug_validate_route(int32_t n_queries, int64_t total_q, const int32_t* q_off, int32_t max_q_len,
                                int32_t n_docs, int64_t n_chunks, const int64_t* chunk_off, hipStream_t s) {
  std::vector<int32_t> qo;
  std::vector<int64_t> co;
  msa_status st = check_queries(q_off, n_queries, total_q, max_q_len, s, qo);
  if (st == MSA_OK) st = check_chunk_off(chunk_off, n_docs, n_chunks, s, co);
  return st;
}

msa_status debug_validate_attn(int32_t n_queries, int64_t total_q, int64_t total_kv, const int32_t* q_off,
                               const int32_t* kv_off, int32_t max_q_len, int32_t k, const int32_t* ids,
                               int32_t n_docs, int64_t n_chunks, const int64_t* chunk_off, hipStream_t s) {
  std::vector<int32_t> qo, ko, id;
  std::vector<int64_t> co;
  msa_status st = check_queries(q_off, n_queries, total_q, max_q_len, s, qo);
  if (st == MSA_OK) st = fetch(kv_off, (size_t)n_queries + 1, ko, s, "kv_off");
  if (st == MSA_OK) st = check_offsets(ko, total_kv, 0, "kv_off");
  if (st == MSA_OK) st = check_chunk_off(chunk_off, n_docs, n_chunks, s, co);
  if (st == MSA_OK) st = fetch(ids, (size_t)n_queries * k, id, s, "topk_ids");
  if (st != MSA_OK) return st;
  for (int32_t b = 0; b < n_queries; ++b) {
    if (ko[b + 1] - ko[b] < qo[b + 1] - qo[b])
      return fail(MSA_ERR_INVALID_ARG, "query %d: %d local tokens, fewer than its %d query tokens", b,
                  ko[b + 1] - ko[b], qo[b + 1] - qo[b]);
    for (int32_t r = 0; r < k; ++r) {
      const int32_t v = id[(size_t)b * k + r];
      if (v < -1 || v >= n_docs)
        return fail(MSA_ERR_INVALID_ARG, "topk_ids[%d][%d] = %d is not a document id in [0, %d) or -1", b, r, v,
                    n_docs);
    }
  }
  return MSA_OK;
}

}  // namespace msa
