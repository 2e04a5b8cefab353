/*
 * msa.h -- C ABI of the MI355X (gfx950) Memory Sparse Attention hot path.
 *
 * The library implements, for one upper attention layer, the four steps of MSA's
 * inference path:
 *   A. msa_pool        offline memory encoding: document-wise RoPE, then chunk-mean
 *                      pooling of token-level K, V, Kr into bank rows K-bar, V-bar, Kr-bar;
 *   B+C. msa_route_topk the router: cosine of the query's Qr against every Kr-bar row,
 *                      mean over heads, max over query tokens, max over each document's
 *                      rows, then the top-k documents;
 *   D. msa_sparse_attn context assembly (selected documents' K-bar/V-bar followed by the
 *                      query's local K/V under global RoPE) and GQA softmax attention.
 *
 * Sources: hysenlabs.com "EverMind-AI/MSA: routing top-k compressed documents inside
 * attention, and where the 100M-token claim stops" (sections "Routing happens inside
 * attention ...", "Document-wise RoPE resets every document to position zero", "Memory
 * must be encoded offline ...", "The 100M-token setup depends on host memory ...");
 * yeyulingfeng.com "深度分析MSA：把超长文档组织成可检索内部记忆的工程路径" (section 三,
 * chunk compression; section 五, inference).
 *
 * Conventions for every call:
 *  - Tensors are caller-owned, contiguous, row-major, and device-accessible unless a
 *    parameter says "host".  Element type is given by `dtype` (MSA_F32 or MSA_BF16);
 *    bf16 is the upper half of an IEEE float32.  Offsets are device arrays unless noted.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream).  The
 *    library allocates no memory and keeps no state between calls: scratch space comes
 *    from the caller's `workspace`.
 *  - Arguments are validated on the host before any HIP call; a bad argument returns
 *    MSA_ERR_INVALID_ARG or MSA_ERR_UNSUPPORTED at once, with a message in
 *    msa_last_error().  A failed launch returns MSA_ERR_HIP.  Nothing is printed and no
 *    exception or abort crosses the ABI.
 *  - Device-resident offset arrays and selected ids are a caller precondition (offsets
 *    start at 0, never decrease and end at the stated totals, every document has >= 1
 *    token and >= 1 bank row, every query has <= max_q_len tokens and at least as many
 *    local tokens, ids lie in [-1, n_docs)); they are not read on the host.  With the
 *    environment variable MSA_DEBUG_VALIDATE=1, every entry point copies them to the host
 *    first (synchronising `stream`) and returns MSA_ERR_INVALID_ARG, naming the first bad
 *    entry, before any kernel runs.
 *  - Results are deterministic: the same inputs give the same bits.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* msa_stream_t; /* same type as hipStream_t */

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = 1, /* null pointer, bad size, inconsistent shapes           */
  MSA_ERR_UNSUPPORTED = 2, /* valid but not implemented (head dim, dtype, k > 1024) */
  MSA_ERR_WORKSPACE = 3,   /* workspace smaller than the matching *_workspace() size */
  MSA_ERR_HIP = 4,         /* a HIP call or kernel launch failed                     */
  MSA_ERR_IO = 5           /* a bank file could not be written, read or verified     */
} msa_status;

/* Element type of the tensors.  The type is a plain 32-bit integer rather than an enum so
 * that any value a caller passes is well defined in C++ and reaches argument validation,
 * which rejects values other than these two with MSA_ERR_UNSUPPORTED. */
enum { MSA_F32 = 0, MSA_BF16 = 1 };
typedef int32_t msa_dtype;

/* Which tensors msa_pool rotates with document-wise RoPE.  The default reading rotates
 * K only (keys carry positions; V and the routing keys Kr are left as they are). */
enum { MSA_ROPE_K = 1u, MSA_ROPE_V = 2u, MSA_ROPE_KR = 4u };

/*
 * Routing-key bank layout (hysenlabs.com "The 100M-token setup depends on host memory as
 * well as two GPUs": the routing keys stay resident in GPU memory and every query scores
 * all of them, so they are stored the way the scan reads them).  Every Krbar argument of
 * this library uses this layout:
 *  - MSA_BF16: rows in tiles of 16.  Tile T holds bank rows 16T..16T+15 as h_r * (d/32)
 *    blocks of 512 elements, in (head h, 32-dimension slice s) order.  In block (h, s),
 *    element (row 16T + r, head h, dim 32s + 8g + j), r < 16, g < 4, j < 8, sits at
 *    position (16g + r) * 8 + j: each block is the B operand of a 16x16x32 matrix-core
 *    product, one contiguous 1 KB load.  A bank of C rows occupies ceil(C/16) whole tiles;
 *    the rows past C in the last tile are padding: they are read but no result depends on
 *    their contents (msa_krbar_pack writes them as zero, msa_pool leaves them alone).
 *  - MSA_F32: row-major [C, h_r, d].
 * The gradient dKrbar of msa_route_backward is float32 row-major [C, h_r, d] in every case.
 */

/* Elements of Krbar storage for a bank of n_chunks rows: 16 * ceil(n_chunks/16) * h_r * d
 * for MSA_BF16, n_chunks * h_r * d for MSA_F32; -1 on a bad argument (d in {32, 64, 128},
 * h_r in [1, 64], n_chunks >= 0). */
int64_t msa_krbar_elems(msa_dtype dtype, int64_t n_chunks, int32_t h_r, int32_t d);

/* Row-major routing keys `rows` [n_chunks, h_r, d] (device) -> the bank layout `Krbar`
 * (device, msa_krbar_elems() elements, padding rows written as zero).  The buffers must not
 * overlap.  Asynchronous on `stream`. */
msa_status msa_krbar_pack(msa_dtype dtype, int64_t n_chunks, int32_t h_r, int32_t d,
                          const void* rows, void* Krbar, msa_stream_t stream);

/* The bank layout `Krbar` -> row-major `rows` [n_chunks, h_r, d] (both device, not
 * overlapping).  Asynchronous on `stream`. */
msa_status msa_krbar_unpack(msa_dtype dtype, int64_t n_chunks, int32_t h_r, int32_t d,
                            const void* Krbar, void* rows, msa_stream_t stream);

/* Library version, major*10000 + minor*100 + patch. */
int32_t msa_version(void);

/* Text for a status code (static storage). */
const char* msa_status_string(msa_status s);

/* Detail of the last error raised on the calling thread ("" if none). */
const char* msa_last_error(void);

/*
 * msa_chunk_offsets -- host-side chunk layout of a bank (yeyulingfeng.com section 三,
 * chunk compression: one chunk per `chunk` tokens; its worked example maps 180 tokens to
 * 3 chunks, so a partial last chunk counts).
 *   doc_tok_off  host [n_docs+1] token offsets of the documents, non-decreasing, with
 *                doc_tok_off[0] == 0 and every document holding >= 1 token.
 *   chunk_off    host [n_docs+1] output: document d owns bank rows
 *                [chunk_off[d], chunk_off[d+1]), ceil(L_d / chunk) of them.
 * Returns the total number of bank rows, or -1 on a bad argument (see msa_last_error).
 */
int64_t msa_chunk_offsets(const int64_t* doc_tok_off, int32_t n_docs, int32_t chunk,
                          int64_t* chunk_off);

/*
 * msa_pool -- step A, offline memory encoding (hysenlabs.com "Memory must be encoded
 * offline ...": one pass over the corpus caches chunk-pooled K, V and Kr; yeyulingfeng.com
 * section 三: mean pooling per chunk; hysenlabs.com "Document-wise RoPE resets every
 * document to position zero").
 *   K, V       [n_tokens, h_kv, d]; Kr [n_tokens, h_r, d]; documents concatenated.
 *   doc_tok_off device [n_docs+1], starting at 0.
 *   chunk_off  device [n_docs+1]: document d's first bank row, with the row counts of
 *              msa_chunk_offsets.  It may start past row 0: the documents are then written
 *              after the rows a bank already holds (a bank grown by appending documents
 *              holds the same bits as one pooled at once).
 *   n_chunks   rows written, chunk_off[n_docs] - chunk_off[0].
 *   rope_mask  MSA_ROPE_* bits: tensors rotated at their in-document position p
 *              (restarting at 0 per document), angle p * rope_base^(-2i/d) on the pair
 *              (i, i + d/2).
 *   Kbar, Vbar [rows, h_kv, d] row-major; Krbar in the routing-key bank layout (above),
 *              outputs holding at least chunk_off[n_docs] rows.  Row chunk_off[doc] + j is
 *              the mean of tokens [j*chunk, min((j+1)*chunk, L)) of the document, after
 *              rotation; means are accumulated in float32 and rounded once to dtype.  Only
 *              rows chunk_off[0] .. chunk_off[n_docs] - 1 are written.
 *   Supported: d in {32, 64, 128}; 1 <= chunk <= 128; h_kv, h_r in [1, 64].
 */
msa_status msa_pool(msa_dtype dtype, int32_t n_docs, int64_t n_tokens, int64_t n_chunks,
                    const int64_t* doc_tok_off, const int64_t* chunk_off,
                    int32_t h_kv, int32_t h_r, int32_t d, int32_t chunk, float rope_base,
                    uint32_t rope_mask, const void* K, const void* V, const void* Kr,
                    void* Kbar, void* Vbar, void* Krbar, msa_stream_t stream);

/*
 * msa_route_scan -- step B alone: every document's router score.
 *   Same inputs and score definition as msa_route_topk below;
 *   doc_scores device float [n_queries, n_docs] output (written in full).
 *   A query with no tokens scores -inf for every document.
 *   row_scores, row_arg  optional (both or neither; NULL: not written), for training:
 *              device float / int32 [n_queries, n_chunks].  row_scores[b, c] is bank row
 *              c's largest token score for query b (-inf for a query with no tokens), and
 *              row_arg[b, c] the first token (index within the query) reaching it, defined
 *              where row_scores is finite.  A document's score is the largest of its rows'.
 *              msa_route_backward takes them to skip its own scan.
 */
msa_status msa_route_scan(msa_dtype dtype, int32_t n_queries, int64_t total_q,
                          const int32_t* q_off, int32_t max_q_len, const void* Qr,
                          int32_t h_r, int32_t d, int32_t n_docs, int64_t n_chunks,
                          const int64_t* chunk_off, const void* Krbar, float* doc_scores,
                          float* row_scores, int32_t* row_arg, msa_stream_t stream);

/* Bytes of workspace msa_topk needs (0 when none; else a 256-byte aligned buffer). */
size_t msa_topk_workspace(int32_t n_queries, int32_t n_docs, int32_t k);

/*
 * msa_topk -- step C alone (github-wiki.com project 250, section 6 item 1: top-k document
 * selection; yeyulingfeng.com section 五 step 2).
 *   doc_scores device float [n_queries, n_docs]; finite or -inf (NaN is undefined).
 *   topk_ids   device int32 [n_queries, k]: the min(k, n_docs) best documents by (score
 *              descending, id ascending; -0.0 equals +0.0); remaining slots -1.
 *   topk_scores device float [n_queries, k]: their scores; -inf in unused slots.
 *   workspace  msa_topk_workspace() bytes (may be NULL when that is 0): candidates of
 *              document slices, reduced in parallel before a final merge.
 *   Supported: 1 <= k <= 1024.
 */
msa_status msa_topk(int32_t n_queries, int32_t n_docs, const float* doc_scores, int32_t k,
                    int32_t* topk_ids, float* topk_scores, void* workspace,
                    size_t workspace_bytes, msa_stream_t stream);

/* Bytes of workspace msa_route_topk needs when doc_scores is NULL (256-byte aligned);
 * with doc_scores given it needs msa_topk_workspace() bytes. */
size_t msa_route_topk_workspace(int32_t n_queries, int32_t n_docs, int32_t k);

/*
 * msa_route_topk -- steps B and C, the router (hysenlabs.com "Routing happens inside
 * attention ...": cosine similarity of the query's routing vectors with the pooled routing
 * keys, averaged over heads, then the maximum over the query's tokens, then top-k
 * documents; yeyulingfeng.com section 五 step 2).
 *   Qr         [total_q, h_r, d]; query b owns rows [q_off[b], q_off[b+1]).
 *   q_off      device int32 [n_queries+1].
 *   max_q_len  host-side upper bound of every query's length; it picks the kernel tile
 *              (rows are still read from q_off, so a loose bound is only slower).
 *   Krbar      n_chunks rows of h_r heads, in the routing-key bank layout (above);
 *              chunk_off device [n_docs+1], starting at 0.
 *   Scores: s(t,c) = (1/h_r) sum_h cos(Qr[t,h], Krbar[c,h]) (cos = 0 if a norm is 0),
 *           chunk score = max_t s(t,c), document score = max over its rows.
 *   topk_ids   device int32 [n_queries, k]: the min(k, n_docs) best documents by (score
 *              descending, id ascending); remaining slots -1.
 *   topk_scores device float [n_queries, k]: their scores; -inf in unused slots.
 *   doc_scores device float [n_queries, n_docs] or NULL: every document's score; when
 *              NULL the scores are kept in `workspace` instead.
 *   Supported: d in {32, 64, 128}; h_r in [1, 16]; 1 <= k <= 1024.  bf16 inputs with
 *   h_r <= 8 run on matrix-core tiles (exact bf16 products, float32 sums); other bf16
 *   inputs sum in float32 and float32 inputs in double.
 */
msa_status msa_route_topk(msa_dtype dtype, int32_t n_queries, int64_t total_q,
                          const int32_t* q_off, int32_t max_q_len, const void* Qr,
                          int32_t h_r, int32_t d, int32_t n_docs, int64_t n_chunks,
                          const int64_t* chunk_off, const void* Krbar, int32_t k,
                          int32_t* topk_ids, float* topk_scores, float* doc_scores,
                          void* workspace, size_t workspace_bytes, msa_stream_t stream);

/* Scratch that msa_route_topk_noalloc holds per device (16 MiB). */
#define MSA_ROUTE_TOPK_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * msa_route_topk_noalloc -- msa_route_topk for callers that cannot allocate (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments and results, without a workspace.  Its scratch (the document scores when
 * doc_scores is NULL, and the top-k candidates; msa_route_topk_workspace() bytes, or
 * msa_topk_workspace() bytes with doc_scores given) lives in a device array of
 * MSA_ROUTE_TOPK_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on
 * until the process ends; larger inputs return MSA_ERR_WORKSPACE.  Nothing is allocated
 * (no hipMalloc/hipFree); the array's device address is looked up on the first call on a
 * device.  Every call on a device shares that device's array and leaves its contents
 * behind: calls that overlap on one device (other streams or threads) race.  The debug
 * validation of MSA_DEBUG_VALIDATE is not run here (it copies offsets into host buffers).
 */
msa_status msa_route_topk_noalloc(msa_dtype dtype, int32_t n_queries, int64_t total_q,
                                  const int32_t* q_off, int32_t max_q_len, const void* Qr,
                                  int32_t h_r, int32_t d, int32_t n_docs, int64_t n_chunks,
                                  const int64_t* chunk_off, const void* Krbar, int32_t k,
                                  int32_t* topk_ids, float* topk_scores, float* doc_scores,
                                  msa_stream_t stream);

/* Bytes of workspace msa_route_backward needs for these sizes (0 if unsupported). */
size_t msa_route_backward_workspace(int32_t n_queries, int32_t n_docs, int64_t n_chunks,
                                    int32_t h_r);

/*
 * msa_route_backward -- gradient of the router for training (yeyulingfeng.com section 四:
 * an auxiliary routing loss on the document scores, whose gradient reaches the routing
 * projections through Qr and the pooled routing keys Krbar).  For L = sum(dD * S), S the
 * document scores msa_route_scan returns for the same arguments:
 *   The first 12 arguments are those of msa_route_scan (same meaning, same layout).
 *   dD         device float [n_queries, n_docs]: dL/dS (0 entries cost nothing).
 *   row_scores, row_arg  optional (both or neither): msa_route_scan's row outputs for the
 *              same arguments; NULL runs that scan again (into the workspace).
 *   dQr        device float [total_q, h_r, d], overwritten: dL/dQr.
 *   dKrbar     device float [n_chunks, h_r, d] row-major, ADDED TO (the caller zeroes it
 *              once).
 *   A document score is one maximum, so its gradient reaches one (token, row) pair: the
 *   first row of the document (in bank order) with the largest row score, then the first
 *   token (in query order) with the largest score on that row.  For that pair and each
 *   head h with nonzero vectors q, k and cosine c:
 *     dQr[t,h] += g/h_r * (k/|k| - c q/|q|) / |q|,  dKrbar[row,h] += g/h_r * (q/|q| - c k/|k|) / |k|.
 *   Heads with a zero vector get nothing; a query with no tokens gets nothing.  When two
 *   pairs tie the choice follows the forward kernel's float32 scores, so a near-tie can
 *   resolve differently from a float64 computation.  Row gradients shared by several
 *   queries are summed in a fixed order for bf16 banks of 4 or 8 heads of dim 128, and
 *   added atomically otherwise (their last bits can then vary from run to run).
 *   workspace  msa_route_backward_workspace() bytes, 256-byte aligned: the scan's document
 *              and row scores plus one record per (query, document); with 4 or 8 routing
 *              heads each record also keeps its maximising bank row (h_r * 256 bytes).
 *   Supported: as msa_route_scan (d in {32, 64, 128}; h_r in [1, 16]).
 */
msa_status msa_route_backward(msa_dtype dtype, int32_t n_queries, int64_t total_q,
                              const int32_t* q_off, int32_t max_q_len, const void* Qr,
                              int32_t h_r, int32_t d, int32_t n_docs, int64_t n_chunks,
                              const int64_t* chunk_off, const void* Krbar, const float* dD,
                              const float* row_scores, const int32_t* row_arg, float* dQr,
                              float* dKrbar, void* workspace, size_t workspace_bytes,
                              msa_stream_t stream);

/* Loss forms of msa_route_aux_loss. */
enum { MSA_AUX_BCE = 0, MSA_AUX_INFONCE = 1 };

/*
 * msa_route_aux_loss -- the routing auxiliary loss (yeyulingfeng.com section 四: the document
 * scores are supervised directly, commonly with BCE or InfoNCE, to train retrieval), with
 * its gradient, ready for msa_route_backward.  With z = doc_scores[b] / temperature:
 *   MSA_AUX_BCE:     loss[b] = mean over documents of softplus(z) - y z  (y in [0, 1])
 *   MSA_AUX_INFONCE: loss[b] = log sum_d e^z_d - log sum_d y_d e^z_d     (y >= 0; a single
 *                    positive label gives the usual cross-entropy)
 *   doc_scores, labels  device float [n_queries, n_docs] (scores as msa_route_scan writes).
 *   loss       device float [n_queries]: the per-query losses (the total is their mean).
 *   dD         device float [n_queries, n_docs]: d(mean of loss)/d(doc_scores).
 *   A query with a non-finite score (a query without tokens) or, for InfoNCE, without a
 *   positive label gets loss 0 and a zero gradient row.  Sums run in double in a fixed
 *   order; each log-sum-exp is shifted by its own maximum.
 */
msa_status msa_route_aux_loss(int32_t kind, int32_t n_queries, int32_t n_docs,
                              const float* doc_scores, const float* labels, float temperature,
                              float* loss, float* dD, msa_stream_t stream);

/*
 * Bank persistence (hysenlabs.com "Memory must be encoded offline before a query can reach
 * it": the corpus is encoded once and later queries read the result; yeyulingfeng.com
 * section 三 part 3: the bank holds K-bar / V-bar / Kr-bar for every layer).  A bank file
 * stores the document and row offsets and, for each routed layer, Kr-bar, K-bar and V-bar,
 * each section with a checksum.  All pointers are host memory (pageable or pinned); the
 * caller copies to and from the device.  Failures return MSA_ERR_IO (open, write or read
 * error, not a bank file, truncated, checksum mismatch) or MSA_ERR_INVALID_ARG.
 */
typedef struct {
  int32_t dtype;      /* msa_dtype of the tensors */
  int32_t n_layers;   /* routed layers, one Kr-bar / K-bar / V-bar each */
  int32_t n_docs;
  int32_t h_kv, h_r, d;
  int32_t chunk;      /* tokens per bank row, as given to msa_chunk_offsets / msa_pool */
  uint32_t rope_mask; /* as given to msa_pool (recorded, not interpreted) */
  float rope_base;    /* as given to msa_pool (recorded, not interpreted) */
  int32_t reserved;   /* 0 */
  int64_t n_tokens;   /* doc_tok_off[n_docs] */
  int64_t n_chunks;   /* chunk_off[n_docs] = C */
} msa_bank_info;

/* Writes a bank: doc_tok_off / chunk_off [n_docs+1] (chunk_off must follow the chunking
 * rule of msa_chunk_offsets for info->chunk), and for layer l the arrays Krbar[l]
 * (msa_krbar_elems() elements in the routing-key bank layout), Kbar[l] and Vbar[l]
 * [C, h_kv, d] of info->dtype.  Overwrites `path`. */
msa_status msa_bank_save(const char* path, const msa_bank_info* info, const int64_t* doc_tok_off,
                         const int64_t* chunk_off, const void* const* Krbar,
                         const void* const* Kbar, const void* const* Vbar);

/* Reads a bank file's header, to size the buffers of msa_bank_load. */
msa_status msa_bank_read_info(const char* path, msa_bank_info* info);

/* Reads a bank into caller buffers sized for `expect` (the file must describe the same
 * bank: dtype, layers, documents, heads, head dim, chunk and sizes), verifying every
 * section's checksum and the offsets' chunking rule.  On failure the buffers' contents
 * are unspecified. */
msa_status msa_bank_load(const char* path, const msa_bank_info* expect, int64_t* doc_tok_off,
                         int64_t* chunk_off, void* const* Krbar, void* const* Kbar,
                         void* const* Vbar);

/* Bytes of workspace msa_sparse_attn needs for these sizes. */
size_t msa_sparse_attn_workspace(msa_dtype dtype, int32_t n_queries, int64_t total_q,
                                 int64_t total_kv, int32_t max_q_len, int32_t hq,
                                 int32_t h_kv, int32_t d);

/*
 * msa_sparse_attn -- step D, context assembly and sparse attention (hysenlabs.com
 * "Routing happens inside attention ...": the selected documents' compressed K/V are
 * joined with the query's local K/V; "Document-wise RoPE ..." second paragraph: global
 * RoPE over the active context with the query's start shifted by the number of retrieved
 * blocks, causal order memory -> query -> generation; "The 100M-token setup ...": content
 * K/V may stay in host memory and be fetched when selected).
 *   Q          [total_q, hq, d]; query b owns rows [q_off[b], q_off[b+1]).
 *   Kloc, Vloc [total_kv, h_kv, d]; query b owns rows [kv_off[b], kv_off[b+1]) with
 *              Lkv_b >= Lq_b; its Lq_b query tokens are the last Lq_b local tokens.
 *              Not rotated: the call applies global RoPE itself.
 *   topk_ids   device int32 [n_queries, k] as written by msa_route_topk (-1 = unused).
 *   Kbar, Vbar [n_chunks, h_kv, d] bank rows, used as stored (no second rotation).
 *   kv_source  0: Kbar/Vbar are device memory; 1: they are page-locked host memory
 *              (hipHostMalloc / pinned) read over the host link by the kernel.
 *   Let k_eff = number of valid ids.  Memory = rows of the selected documents in rank
 *   order.  Local token j is rotated at global position k_eff + j; query token t is local
 *   token Lkv - Lq + t and attends to every memory row and to local tokens <= its own.
 *   Query head hq reads kv head hq / (hq_count / h_kv).  scale 0 means 1/sqrt(d).
 *   O          [total_q, hq, d] output.
 *   lse        optional (NULL: not written) device float [total_q, hq], output: the natural
 *              log of each row's softmax normaliser, ln sum_j exp(scale * q . k_j) over the
 *              keys the row sees.  msa_sparse_attn_backward takes it to skip recomputing it.
 *   Supported: d in {32, 64, 128}; hq % h_kv == 0; 1 <= k <= 1024.
 */
msa_status msa_sparse_attn(msa_dtype dtype, int32_t n_queries, int64_t total_q,
                           int64_t total_kv, const int32_t* q_off, const int32_t* kv_off,
                           int32_t max_q_len, const void* Q, const void* Kloc,
                           const void* Vloc, int32_t hq, int32_t h_kv, int32_t d,
                           float rope_base, float scale, int32_t k, const int32_t* topk_ids,
                           int32_t n_docs, int64_t n_chunks, const int64_t* chunk_off,
                           const void* Kbar, const void* Vbar, int32_t kv_source, void* O,
                           float* lse, void* workspace, size_t workspace_bytes,
                           msa_stream_t stream);

/* Bytes of workspace msa_sparse_attn_backward needs for these sizes (0 if unsupported). */
size_t msa_sparse_attn_backward_workspace(int64_t total_q, int64_t total_kv, int32_t hq,
                                          int32_t h_kv, int32_t d);

/*
 * msa_sparse_attn_backward -- gradients of step D for training (yeyulingfeng.com section
 * 四: the language-model loss reaches Q, K/V and the routing keys through the selected
 * memory; github-wiki.com project 250, section 6 item 1: the layer stays differentiable end
 * to end).  For L = sum(dO * O), O = msa_sparse_attn(...) with the same arguments:
 *   The first 23 arguments are those of msa_sparse_attn (same meaning, same layout).
 *   O          [total_q, hq, d]: the forward output for these inputs.
 *   lse        optional [total_q, hq]: the forward's lse output for these inputs; NULL
 *              recomputes it (one more pass over the keys).
 *   dO         [total_q, hq, d]: dL/dO.
 *   dQ         device float [total_q, hq, d], overwritten: dL/dQ (the un-rotated input).
 *   dKloc      device float [total_kv, h_kv, d], overwritten: dL/dKloc (un-rotated input).
 *   dVloc      device float [total_kv, h_kv, d], overwritten: dL/dVloc.
 *   dKbar, dVbar device float [n_chunks, h_kv, d], ADDED TO: the gradients of the selected
 *              documents' bank rows (rows nobody selected are left as they are); the caller
 *              zeroes them once.  A row selected by several queries receives the sum of
 *              their shares; those additions are atomic, so their order (and the last bits
 *              of such rows) can vary from run to run.  Every other output is deterministic.
 *   Supported: dtype MSA_BF16; d in {64, 128}; 1 <= k <= 1024.  Products in bf16 on MFMA,
 *   sums and softmax statistics in float32.  Kbar/Vbar may be pinned host memory
 *   (kv_source 1); the gradient arrays are device memory.
 *   Streams: with lse given, the key-side gradients run on a second stream that the library
 *   keeps per device (created on the first such call made outside graph capture), forked
 *   from `stream` and joined back to it with events, so the call still completes in order
 *   on `stream` and can be captured in a graph.
 */
msa_status msa_sparse_attn_backward(msa_dtype dtype, int32_t n_queries, int64_t total_q,
                                    int64_t total_kv, const int32_t* q_off, const int32_t* kv_off,
                                    int32_t max_q_len, const void* Q, const void* Kloc,
                                    const void* Vloc, int32_t hq, int32_t h_kv, int32_t d,
                                    float rope_base, float scale, int32_t k,
                                    const int32_t* topk_ids, int32_t n_docs, int64_t n_chunks,
                                    const int64_t* chunk_off, const void* Kbar, const void* Vbar,
                                    int32_t kv_source, const void* O, const float* lse,
                                    const void* dO, float* dQ,
                                    float* dKloc, float* dVloc, float* dKbar, float* dVbar,
                                    void* workspace, size_t workspace_bytes, msa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
