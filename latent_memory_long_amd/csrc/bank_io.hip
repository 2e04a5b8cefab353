// Bank persistence: a layer-stacked memory bank written to and read from one file.
//
// hysenlabs.com "EverMind-AI/MSA: routing top-k compressed documents inside attention ...",
// section "Memory must be encoded offline before a query can reach it": the corpus is
// encoded once into pooled K, V and Kr, which later queries read; yeyulingfeng.com
// "深度分析MSA ..." section 三 part 3: the memory bank holds K-bar / V-bar / Kr-bar for every
// layer.  Keeping the encoded bank on disk lets a serving process start from it instead of
// encoding the corpus again, and an extended bank (new documents pooled after the existing
// rows) be saved as a whole.
//
// File layout (little-endian):
//   "MSABANK1" | FileHeader (64 bytes) | doc_tok_off int64[N+1] | chunk_off int64[N+1] |
//   for each layer: Kr-bar in the routing-key bank layout (msa_krbar_elems elements: 16-row
//   tiles for bf16, row-major for float32), K-bar [C, h_kv, d], V-bar [C, h_kv, d] (dtype) |
//   checksums uint64[2 + 3 L] (one per section above, in order) | "MSABEND1"
// The checksum of a section is FNV-1a over its 64-bit little-endian words in four
// interleaved lanes (word i goes to lane i mod 4; a zero-padded tail word), the lanes then
// folded in order with the same step; it detects corruption and truncation, not tampering.
// Host code only: the caller moves tensors between host and device memory.
#include <stdio.h>
#include <string.h>

#include <vector>

#include "../../include/msa.h"
#include "status.hpp"

namespace {

constexpr char MAGIC[8] = {'M', 'S', 'A', 'B', 'A', 'N', 'K', '1'};
constexpr char END_MAGIC[8] = {'M', 'S', 'A', 'B', 'E', 'N', 'D', '1'};
constexpr uint32_t FORMAT_VERSION = 2;  // 2: bf16 Kr-bar in tiles of 16 rows
constexpr size_t IO_BLOCK = size_t(16) << 20;

struct FileHeader {
  uint32_t header_bytes, version;
  int32_t dtype, n_layers, n_docs, h_kv, h_r, d, chunk;
  uint32_t rope_mask;
  float rope_base;
  int32_t reserved;
  int64_t n_tokens, n_chunks;
};
static_assert(sizeof(FileHeader) == 64, "file header layout");

constexpr uint64_t FNV_OFFSET = 0xcbf29ce484222325ull;
constexpr uint64_t FNV_PRIME = 0x100000001b3ull;

struct Checksum {
  uint64_t lane[4] = {FNV_OFFSET, FNV_OFFSET, FNV_OFFSET, FNV_OFFSET};
  uint64_t words = 0;
  unsigned char tail[8];
  int tail_n = 0;

  void word(uint64_t w) {
    uint64_t& h = lane[words & 3];
    h = (h ^ w) * FNV_PRIME;
    ++words;
  }
  void update(const void* p, size_t n) {
    const unsigned char* b = static_cast<const unsigned char*>(p);
    while (n && tail_n) {  // complete a pending partial word
      tail[tail_n++] = *b++;
      --n;
      if (tail_n == 8) {
        uint64_t w;
        memcpy(&w, tail, 8);
        word(w);
        tail_n = 0;
      }
    }
    for (; n >= 8; n -= 8, b += 8) {
      uint64_t w;
      memcpy(&w, b, 8);
      word(w);
    }
    while (n--) tail[tail_n++] = *b++;
  }
  uint64_t finish() {
    if (tail_n) {
      memset(tail + tail_n, 0, 8 - tail_n);
      uint64_t w;
      memcpy(&w, tail, 8);
      word(w);
      tail_n = 0;
    }
    uint64_t h = FNV_OFFSET;
    for (int i = 0; i < 4; ++i) h = (h ^ lane[i]) * FNV_PRIME;
    return h;
  }
};

size_t elem_bytes(int32_t dtype) { return dtype == MSA_F32 ? 4 : 2; }

msa_status check_info(const msa_bank_info* in) {
  if (!in) return fail(MSA_ERR_INVALID_ARG, "null bank info");
  if (in->dtype != MSA_F32 && in->dtype != MSA_BF16) return fail(MSA_ERR_UNSUPPORTED, "unknown dtype %d", in->dtype);
  if (in->n_layers < 1 || in->n_layers > 1024) return fail(MSA_ERR_INVALID_ARG, "n_layers %d not in [1, 1024]", in->n_layers);
  if (in->n_docs < 1) return fail(MSA_ERR_INVALID_ARG, "n_docs must be >= 1 (got %d)", in->n_docs);
  if (in->h_kv < 1 || in->h_kv > 64 || in->h_r < 1 || in->h_r > 64)
    return fail(MSA_ERR_INVALID_ARG, "head counts must lie in [1, 64] (got %d, %d)", in->h_kv, in->h_r);
  if (in->d != 32 && in->d != 64 && in->d != 128) return fail(MSA_ERR_UNSUPPORTED, "head dim %d not in {32, 64, 128}", in->d);
  if (in->chunk < 1) return fail(MSA_ERR_INVALID_ARG, "chunk must be >= 1 (got %d)", in->chunk);
  if (in->n_chunks < in->n_docs || in->n_tokens < in->n_chunks)
    return fail(MSA_ERR_INVALID_ARG, "need n_docs <= n_chunks <= n_tokens (got %d, %lld, %lld)", in->n_docs,
                (long long)in->n_chunks, (long long)in->n_tokens);
  return MSA_OK;
}

// The offsets must describe the bank: documents of >= 1 token, ceil(L / chunk) rows each.
msa_status check_offsets(const msa_bank_info* in, const int64_t* doc_tok_off, const int64_t* chunk_off) {
  if (doc_tok_off[0] != 0 || chunk_off[0] != 0) return fail(MSA_ERR_INVALID_ARG, "offsets must start at 0");
  for (int32_t d = 0; d < in->n_docs; ++d) {
    const int64_t len = doc_tok_off[d + 1] - doc_tok_off[d];
    if (len < 1) return fail(MSA_ERR_INVALID_ARG, "document %d has %lld tokens", d, (long long)len);
    if (chunk_off[d + 1] - chunk_off[d] != (len + in->chunk - 1) / in->chunk)
      return fail(MSA_ERR_INVALID_ARG, "document %d: %lld rows for %lld tokens at chunk %d", d,
                  (long long)(chunk_off[d + 1] - chunk_off[d]), (long long)len, in->chunk);
  }
  if (doc_tok_off[in->n_docs] != in->n_tokens || chunk_off[in->n_docs] != in->n_chunks)
    return fail(MSA_ERR_INVALID_ARG, "offsets end at %lld tokens / %lld rows, info says %lld / %lld",
                (long long)doc_tok_off[in->n_docs], (long long)chunk_off[in->n_docs], (long long)in->n_tokens,
                (long long)in->n_chunks);
  return MSA_OK;
}

struct File {
  FILE* f = nullptr;
  ~File() {
    if (f) fclose(f);
  }
};

bool write_section(FILE* f, const void* p, size_t n, uint64_t* sum) {
  Checksum c;
  const char* b = static_cast<const char*>(p);
  for (size_t done = 0; done < n;) {
    const size_t m = n - done < IO_BLOCK ? n - done : IO_BLOCK;
    c.update(b + done, m);
    if (fwrite(b + done, 1, m, f) != m) return false;
    done += m;
  }
  *sum = c.finish();
  return true;
}

bool read_section(FILE* f, void* p, size_t n, uint64_t* sum) {
  Checksum c;
  char* b = static_cast<char*>(p);
  for (size_t done = 0; done < n;) {
    const size_t m = n - done < IO_BLOCK ? n - done : IO_BLOCK;
    if (fread(b + done, 1, m, f) != m) return false;
    c.update(b + done, m);
    done += m;
  }
  *sum = c.finish();
  return true;
}

msa_status read_header(FILE* f, const char* path, msa_bank_info* info) {
  char magic[8];
  FileHeader h;
  if (fread(magic, 1, 8, f) != 8 || memcmp(magic, MAGIC, 8) != 0) return fail(MSA_ERR_IO, "%s: not a bank file", path);
  if (fread(&h, 1, sizeof h, f) != sizeof h) return fail(MSA_ERR_IO, "%s: truncated header", path);
  if (h.header_bytes != sizeof h || h.version != FORMAT_VERSION)
    return fail(MSA_ERR_IO, "%s: header of %u bytes, version %u (expected %zu, %u)", path, h.header_bytes, h.version,
                sizeof h, FORMAT_VERSION);
  *info = msa_bank_info{h.dtype, h.n_layers, h.n_docs, h.h_kv, h.h_r, h.d, h.chunk, h.rope_mask, h.rope_base,
                        0, h.n_tokens, h.n_chunks};
  const msa_status st = check_info(info);
  if (st != MSA_OK) return fail(MSA_ERR_IO, "%s: bad header (%s)", path, g_last_error.c_str());
  return MSA_OK;
}

}  // namespace

extern "C" {

msa_status msa_bank_save(const char* path, const msa_bank_info* info, const int64_t* doc_tok_off,
                         const int64_t* chunk_off, const void* const* Krbar, const void* const* Kbar,
                         const void* const* Vbar) {
  g_last_error.clear();
  if (!path || !doc_tok_off || !chunk_off || !Krbar || !Kbar || !Vbar) return fail(MSA_ERR_INVALID_ARG, "null pointer");
  msa_status st = check_info(info);
  if (st != MSA_OK) return st;
  st = check_offsets(info, doc_tok_off, chunk_off);
  if (st != MSA_OK) return st;
  for (int32_t l = 0; l < info->n_layers; ++l)
    if (!Krbar[l] || !Kbar[l] || !Vbar[l]) return fail(MSA_ERR_INVALID_ARG, "null tensor for layer %d", l);
  const size_t esz = elem_bytes(info->dtype);
  const size_t C = (size_t)info->n_chunks;
  const size_t kr_bytes = (size_t)msa_krbar_elems((msa_dtype)info->dtype, info->n_chunks, info->h_r, info->d) * esz;
  const size_t kv_bytes = C * info->h_kv * info->d * esz;
  const size_t off_bytes = ((size_t)info->n_docs + 1) * sizeof(int64_t);
  File out;
  out.f = fopen(path, "wb");
  if (!out.f) return fail(MSA_ERR_IO, "%s: cannot open for writing", path);
  FileHeader h{(uint32_t)sizeof(FileHeader), FORMAT_VERSION, info->dtype, info->n_layers, info->n_docs, info->h_kv,
               info->h_r, info->d, info->chunk, info->rope_mask, info->rope_base, 0, info->n_tokens,
               info->n_chunks};
  std::vector<uint64_t> sums(2 + 3 * (size_t)info->n_layers);
  bool ok = fwrite(MAGIC, 1, 8, out.f) == 8 && fwrite(&h, 1, sizeof h, out.f) == sizeof h &&
            write_section(out.f, doc_tok_off, off_bytes, &sums[0]) &&
            write_section(out.f, chunk_off, off_bytes, &sums[1]);
  for (int32_t l = 0; ok && l < info->n_layers; ++l)
    ok = write_section(out.f, Krbar[l], kr_bytes, &sums[2 + 3 * l]) &&
         write_section(out.f, Kbar[l], kv_bytes, &sums[3 + 3 * l]) &&
         write_section(out.f, Vbar[l], kv_bytes, &sums[4 + 3 * l]);
  ok = ok && fwrite(sums.data(), sizeof(uint64_t), sums.size(), out.f) == sums.size() &&
       fwrite(END_MAGIC, 1, 8, out.f) == 8;
  const bool closed = fclose(out.f) == 0;
  out.f = nullptr;
  if (!ok || !closed) return fail(MSA_ERR_IO, "%s: write failed", path);
  return MSA_OK;
}

msa_status msa_bank_read_info(const char* path, msa_bank_info* info) {
  g_last_error.clear();
  if (!path || !info) return fail(MSA_ERR_INVALID_ARG, "null pointer");
  File in;
  in.f = fopen(path, "rb");
  if (!in.f) return fail(MSA_ERR_IO, "%s: cannot open for reading", path);
  return read_header(in.f, path, info);
}

msa_status msa_bank_load(const char* path, const msa_bank_info* expect, int64_t* doc_tok_off, int64_t* chunk_off,
                         void* const* Krbar, void* const* Kbar, void* const* Vbar) {
  g_last_error.clear();
  if (!path || !expect || !doc_tok_off || !chunk_off || !Krbar || !Kbar || !Vbar)
    return fail(MSA_ERR_INVALID_ARG, "null pointer");
  File in;
  in.f = fopen(path, "rb");
  if (!in.f) return fail(MSA_ERR_IO, "%s: cannot open for reading", path);
  msa_bank_info info;
  msa_status st = read_header(in.f, path, &info);
  if (st != MSA_OK) return st;
  const bool same = info.dtype == expect->dtype && info.n_layers == expect->n_layers &&
                    info.n_docs == expect->n_docs && info.h_kv == expect->h_kv && info.h_r == expect->h_r &&
                    info.d == expect->d && info.chunk == expect->chunk && info.n_tokens == expect->n_tokens &&
                    info.n_chunks == expect->n_chunks;
  if (!same) return fail(MSA_ERR_INVALID_ARG, "%s: the file's bank differs from the one the buffers were sized for", path);
  for (int32_t l = 0; l < info.n_layers; ++l)
    if (!Krbar[l] || !Kbar[l] || !Vbar[l]) return fail(MSA_ERR_INVALID_ARG, "null tensor for layer %d", l);
  const size_t esz = elem_bytes(info.dtype);
  const size_t C = (size_t)info.n_chunks;
  const size_t kr_bytes = (size_t)msa_krbar_elems((msa_dtype)info.dtype, info.n_chunks, info.h_r, info.d) * esz;
  const size_t kv_bytes = C * info.h_kv * info.d * esz;
  const size_t off_bytes = ((size_t)info.n_docs + 1) * sizeof(int64_t);
  std::vector<uint64_t> got(2 + 3 * (size_t)info.n_layers), want(got.size());
  bool ok = read_section(in.f, doc_tok_off, off_bytes, &got[0]) && read_section(in.f, chunk_off, off_bytes, &got[1]);
  for (int32_t l = 0; ok && l < info.n_layers; ++l)
    ok = read_section(in.f, Krbar[l], kr_bytes, &got[2 + 3 * l]) &&
         read_section(in.f, Kbar[l], kv_bytes, &got[3 + 3 * l]) &&
         read_section(in.f, Vbar[l], kv_bytes, &got[4 + 3 * l]);
  char end[8];
  ok = ok && fread(want.data(), sizeof(uint64_t), want.size(), in.f) == want.size() && fread(end, 1, 8, in.f) == 8 &&
       memcmp(end, END_MAGIC, 8) == 0 && fgetc(in.f) == EOF;
  if (!ok) return fail(MSA_ERR_IO, "%s: truncated or malformed file", path);
  static const char* const names[3] = {"Kr-bar", "K-bar", "V-bar"};
  for (size_t i = 0; i < got.size(); ++i) {
    if (got[i] == want[i]) continue;
    if (i < 2) return fail(MSA_ERR_IO, "%s: checksum mismatch in %s", path, i ? "chunk_off" : "doc_tok_off");
    return fail(MSA_ERR_IO, "%s: checksum mismatch in layer %zu %s", path, (i - 2) / 3, names[(i - 2) % 3]);
  }
  st = check_offsets(&info, doc_tok_off, chunk_off);
  if (st != MSA_OK) return fail(MSA_ERR_IO, "%s: %s", path, g_last_error.c_str());
  return MSA_OK;
}

}  // extern "C"
