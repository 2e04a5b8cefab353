// Error reporting shared by the C-ABI translation units: a status code plus a
// thread-local message that msa_last_error() returns.
#pragma once

#include <hip/hip_runtime.h>

#include <string>

#include "../../include/msa.h"

extern thread_local std::string g_last_error;

// Sets the thread's last-error message (printf format) and returns s.
msa_status fail(msa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

namespace msa {
// Opt-in checks of the device index arrays (environment MSA_DEBUG_VALIDATE=1): copy them to
// the host, synchronising the stream, and return MSA_ERR_INVALID_ARG on the first bad entry.
bool debug_validate_enabled();
msa_status debug_validate_pool(int32_t n_docs, int64_t n_tokens, int64_t n_chunks, int32_t chunk,
                               const int64_t* doc_tok_off, const int64_t* chunk_off, hipStream_t s);
msa_status debug_validate_route(int32_t n_queries, int64_t total_q, const int32_t* q_off, int32_t max_q_len,
                                int32_t n_docs, int64_t n_chunks, const int64_t* chunk_off, hipStream_t s);
msa_status debug_validate_attn(int32_t n_queries, int64_t total_q, int64_t total_kv, const int32_t* q_off,
                               const int32_t* kv_off, int32_t max_q_len, int32_t k, const int32_t* ids,
                               int32_t n_docs, int64_t n_chunks, const int64_t* chunk_off, hipStream_t s);
}  // namespace msa
