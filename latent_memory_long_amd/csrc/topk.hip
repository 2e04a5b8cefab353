// Step C -- top-k document selection.
//
// github-wiki.com project 250, section 6 item 1 (the layer fuses top-k document selection
// with sparse attention); yeyulingfeng.com "深度分析MSA ..." section 五 step 2 (score ->
// top-k memory); hysenlabs.com "... Routing happens inside attention ...".
// Order: score descending, ties to the lower document id; k_eff = min(k, N).
//
// One workgroup (1024 threads) per query, working on order-preserving uint32 keys of the
// float document scores (the key order is the float order, with -0.0 folded into +0.0):
//  1. Radix select, most significant digit first (11 + 11 + 10 bits): an LDS histogram of
//     the keys that share the digits chosen so far finds, digit by digit, the exact key T
//     of the k_eff-th largest score and how many of the winners must be taken among keys
//     equal to T.
//  2. One compaction pass in id order: keys > T are all taken; keys == T are taken in id
//     order through a block-wide prefix count until the quota is filled.
//  3. The <= 1024 winners are sorted in LDS by (key descending, id ascending) with a
//     bitonic network on 64-bit composites key << 32 | ~id.
// The work per query is latency-bound (a few hundred KB at most).  Two kernels:
//  * topk_reg: each thread keeps up to 8 keys in registers, so the scores are read once;
//    banks of more than 8192 documents are cut into slices whose local top-k are found in
//    parallel and merged by topk_merge (the k best of all are among the slices' k best).  The radix digits start below the leading bits that every key shares
//    (scores of one query usually share sign and exponent bits), which spreads the
//    histogram; the id-ordered pass over equal keys runs only when an exact tie straddles
//    the k-th place; up to 64 winners are sorted in one wave with lane shuffles.
//  * topk_kernel (more candidates than one merge can sort): the same steps reading the
//    scores from memory on every pass.
#include "common.hpp"
#include "launch.hpp"

namespace msa {
namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int SLICE_KPT = 8;                       // keys per thread of one slice
constexpr int SLICE = SLICE_KPT * TK_THREADS;      // documents per slice
constexpr int MERGE_MAX = 4096;                    // candidates one merge can sort

// Exclusive prefix sum over the workgroup in thread order; *total gets the sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  if (w == 0) {
    uint32_t s = (lane < TK_WAVES) ? wsum[lane] : 0u;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(s, o);
      if (lane >= o) s += y;
    }
    if (lane < TK_WAVES) wsum[lane] = s;  // inclusive per-wave totals
  }
  __syncthreads();
  const uint32_t before = (w > 0) ? wsum[w - 1] : 0u;
  *total = wsum[TK_WAVES - 1];
  __syncthreads();  // wsum is reused by the next call
  return before + x - v;
}

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(TopkArgs a) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wsum[TK_WAVES];
  __shared__ unsigned long long sel[1024];
  __shared__ uint32_t sh_digit, sh_above, sh_cnt;

  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int N = a.n_docs;
  const int keff = min(a.k, N);
  const float* sb = a.doc_scores + (int64_t)b * N;

  uint32_t prefix = 0, pmask = 0;
  uint32_t remaining = (uint32_t)keff;
  const int shifts[3] = {21, 10, 0};
  const int bitsv[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass], bits = bitsv[pass];
    const uint32_t nb = 1u << bits, dmask = nb - 1u;
    for (uint32_t i = tid; i < 2048; i += TK_THREADS) hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < N; i += TK_THREADS) {
      const uint32_t key = score_key(sb[i]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    // thread t owns bins (descending) nb-1-2t and nb-2-2t (those that exist)
    const int per = (int)nb / TK_THREADS;  // 2 or 1
    const int j0 = (int)nb - 1 - per * tid;
    const uint32_t h0 = hist[j0];
    const uint32_t h1 = (per == 2) ? hist[j0 - 1] : 0u;
    uint32_t tot;
    const uint32_t excl = block_excl_scan(h0 + h1, wsum, &tot);
    if (excl < remaining && excl + h0 + h1 >= remaining) {
      if (excl + h0 >= remaining) { sh_digit = (uint32_t)j0; sh_above = excl; }
      else { sh_digit = (uint32_t)(j0 - 1); sh_above = excl + h0; }
    }
    __syncthreads();
    remaining -= sh_above;
    prefix |= sh_digit << shift;
    pmask |= dmask << shift;
    __syncthreads();
  }
  const uint32_t T = prefix;  // key of the k_eff-th best document

  if (tid == 0) sh_cnt = 0u;
  __syncthreads();
  uint32_t eq_base = 0;
  for (int base = 0; base < N; base += TK_THREADS) {
    const int i = base + tid;
    const uint32_t key = (i < N) ? score_key(sb[i]) : 0u;
    const bool gt = (i < N) && key > T;
    const bool eq = (i < N) && key == T;
    if (gt) {
      const uint32_t pos = atomicAdd(&sh_cnt, 1u);
      sel[pos] = ((unsigned long long)key << 32) | (uint32_t)(~(uint32_t)i);
    }
    uint32_t tot;
    const uint32_t rank = block_excl_scan(eq ? 1u : 0u, wsum, &tot);
    if (eq && eq_base + rank < remaining) {
      const uint32_t pos = atomicAdd(&sh_cnt, 1u);
      sel[pos] = ((unsigned long long)key << 32) | (uint32_t)(~(uint32_t)i);
    }
    eq_base += tot;
  }
  __syncthreads();

  int n2 = 1;
  while (n2 < keff) n2 <<= 1;
  for (int i = tid; i < n2; i += TK_THREADS)
    if (i >= keff) sel[i] = 0ull;
  __syncthreads();
  for (int k2 = 2; k2 <= n2; k2 <<= 1) {
    for (int j = k2 >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < n2; i += TK_THREADS) {
        const int p = i ^ j;
        if (p > i) {
          const unsigned long long x = sel[i], y = sel[p];
          const bool desc = (i & k2) == 0;
          if (desc ? (x < y) : (x > y)) { sel[i] = y; sel[p] = x; }
        }
      }
      __syncthreads();
    }
  }
  for (int r = tid; r < a.k; r += TK_THREADS) {
    if (r < keff) {
      const unsigned long long v = sel[r];
      a.ids[(int64_t)b * a.k + r] = (int32_t)(~(uint32_t)(v & 0xffffffffull));
      a.scores[(int64_t)b * a.k + r] = key_score((uint32_t)(v >> 32));
    } else {
      a.ids[(int64_t)b * a.k + r] = -1;
      a.scores[(int64_t)b * a.k + r] = -INFINITY;
    }
  }
}

// ---- register-resident variant ---------------------------------------------------------
__device__ __forceinline__ uint32_t block_and_or(uint32_t v, bool is_and, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t y = __shfl_xor(v, o);
    v = is_and ? (v & y) : (v | y);
  }
  if (lane == 0) wsum[w] = v;
  __syncthreads();
  uint32_t r = wsum[0];
  for (int i = 1; i < TK_WAVES; ++i) r = is_and ? (r & wsum[i]) : (r | wsum[i]);
  __syncthreads();
  return r;
}

// Sort up to 64 composites (key << 32 | ~id) descending inside one wave (lane i holds one).
__device__ __forceinline__ unsigned long long wave_bitonic_desc(unsigned long long x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k2 = 2; k2 <= 64; k2 <<= 1) {
#pragma unroll
    for (int j = k2 >> 1; j > 0; j >>= 1) {
      const unsigned long long y = __shfl_xor(x, j);
      const bool lower = (lane & j) == 0;        // this lane keeps the larger of the pair
      const bool desc = (lane & k2) == 0;        // direction of this bitonic sequence
      const bool keep_max = (lower == desc);
      x = keep_max ? (x > y ? x : y) : (x < y ? x : y);
    }
  }
  return x;
}

// Top-k of documents [blockIdx.x * SLICE, ...) of query blockIdx.y.  With cand == null the
// slice is the whole query and the result goes to ids / scores; otherwise the slice's
// best min(k, slice) composites (key << 32 | ~id, zero-padded to k) go to cand.
// Exclusive prefix sum over the workgroup in thread order with one barrier: each thread adds
// the totals of the waves before its own.  *total gets the sum.  wsum is written before the
// barrier and read after it, so callers alternate two buffers between successive calls.
__device__ __forceinline__ uint32_t block_excl_scan1(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < TK_WAVES; ++i) {
    const uint32_t t = wsum[i];
    before += i < w ? t : 0u;
    all += t;
  }
  *total = all;
  return before + x - v;
}

template <int KPT>
__global__ __launch_bounds__(TK_THREADS) void topk_reg(TopkArgs a, unsigned long long* cand) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wsum[TK_WAVES];
  __shared__ uint32_t wsc[2][TK_WAVES];  // the radix passes' scans, alternating by pass
  __shared__ uint32_t wao[2][TK_WAVES];  // the AND / OR of each wave's keys
  __shared__ unsigned long long sel[1024];
  __shared__ uint32_t sh_digit[2], sh_above[2], sh_bucket[2], sh_cnt;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int b = blockIdx.y;
  const int id0 = blockIdx.x * KPT * TK_THREADS;  // first document of the slice
  const int N = min(a.n_docs - id0, KPT * TK_THREADS);
  const int keff = min(a.k, N);
  const float* sb = a.doc_scores + (int64_t)b * a.n_docs + id0;

  uint32_t key[KPT];
  uint32_t kand = 0xffffffffu, kor = 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = tid + j * TK_THREADS;
    key[j] = (i < N) ? score_key(sb[i]) : 0u;
    if (i < N) { kand &= key[j]; kor |= key[j]; }
  }
  // The AND and OR of all keys, the histogram cleared and the selection counter reset,
  // behind one barrier.
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kand &= __shfl_xor(kand, o);
    kor |= __shfl_xor(kor, o);
  }
  if (lane == 0) {
    wao[0][w] = kand;
    wao[1][w] = kor;
  }
  hist[2 * tid] = 0u;
  hist[2 * tid + 1] = 0u;
  if (tid == 0) sh_cnt = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TK_WAVES; ++i) {
    kand &= wao[0][i];
    kor |= wao[1][i];
  }
  const uint32_t diff = kand ^ kor;
  int hi_bit = diff ? 31 - __clz(diff) : -1;      // highest bit on which keys differ
  uint32_t pmask = hi_bit >= 31 ? 0u : ~((2u << hi_bit) - 1u);
  if (hi_bit < 0) pmask = 0xffffffffu;
  uint32_t prefix = kand & pmask;                 // bits shared by every key
  uint32_t remaining = (uint32_t)keff;
  uint32_t bucket = (uint32_t)N;                  // keys whose determined bits equal prefix
  // Each pass: histogram of the next digit (barrier), a one-barrier scan of it, the digit
  // holding the k-th key published (barrier).  A thread reads only its own two bins and
  // clears them for the next pass right after, and the published digit alternates between
  // two slots, so three barriers a pass suffice.
  int pass = 0;
  while (hi_bit >= 0 && bucket != remaining) {
    const int bits = min(11, hi_bit + 1);
    const int shift = hi_bit + 1 - bits;
    const uint32_t nb = 1u << bits, dmask = nb - 1u;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int i = tid + j * TK_THREADS;
      if (i < N && (key[j] & pmask) == prefix) atomicAdd(&hist[(key[j] >> shift) & dmask], 1u);
    }
    __syncthreads();
    // thread t owns bins (descending) nb-1-2t and nb-2-2t, where they exist
    const int j0 = (int)nb - 1 - 2 * tid;
    const uint32_t h0 = (j0 >= 0) ? hist[j0] : 0u;
    const uint32_t h1 = (j0 >= 1) ? hist[j0 - 1] : 0u;
    if (j0 >= 0) hist[j0] = 0u;
    if (j0 >= 1) hist[j0 - 1] = 0u;
    const int ps = pass & 1;
    uint32_t tot;
    const uint32_t excl = block_excl_scan1(h0 + h1, wsc[ps], &tot);
    if (excl < remaining && excl + h0 + h1 >= remaining) {
      if (excl + h0 >= remaining) { sh_digit[ps] = (uint32_t)j0; sh_above[ps] = excl; sh_bucket[ps] = h0; }
      else { sh_digit[ps] = (uint32_t)(j0 - 1); sh_above[ps] = excl + h0; sh_bucket[ps] = h1; }
    }
    __syncthreads();
    remaining -= sh_above[ps];
    bucket = sh_bucket[ps];
    prefix |= sh_digit[ps] << shift;
    pmask |= dmask << shift;
    hi_bit = shift - 1;
    ++pass;
  }
  // Selected: keys whose determined bits exceed prefix, plus `remaining` keys equal to it
  // on those bits (all of them when bucket == remaining, else the lowest ids).
  const bool take_all = bucket == remaining;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = tid + j * TK_THREADS;
    const uint32_t m = key[j] & pmask;
    if (i < N && (m > prefix || (take_all && m == prefix))) {
      const uint32_t pos = atomicAdd(&sh_cnt, 1u);
      sel[pos] = ((unsigned long long)key[j] << 32) | (uint32_t)(~(uint32_t)(id0 + i));
    }
  }
  if (!take_all) {  // exact tie across the k-th place: lowest ids first (ids j*1024 + t)
    uint32_t base = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {  // unrolled: key[] must stay in registers
      const int i = tid + j * TK_THREADS;
      const bool eq = i < N && key[j] == prefix;
      uint32_t tot;
      const uint32_t rank = block_excl_scan(eq ? 1u : 0u, wsum, &tot);
      if (eq && base + rank < remaining) {
        const uint32_t pos = atomicAdd(&sh_cnt, 1u);
        sel[pos] = ((unsigned long long)key[j] << 32) | (uint32_t)(~(uint32_t)(id0 + i));
      }
      base += tot;
    }
  }
  __syncthreads();

  if (keff <= 64) {
    if (tid < 64) {
      unsigned long long x = (tid < keff) ? sel[tid] : 0ull;
      x = wave_bitonic_desc(x);
      if (tid < keff) sel[tid] = x;
    }
    __syncthreads();
  } else {
    int n2 = 1;
    while (n2 < keff) n2 <<= 1;
    for (int i = tid; i < n2; i += TK_THREADS)
      if (i >= keff) sel[i] = 0ull;
    __syncthreads();
    for (int k2 = 2; k2 <= n2; k2 <<= 1) {
      for (int j = k2 >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < n2; i += TK_THREADS) {
          const int p = i ^ j;
          if (p > i) {
            const unsigned long long x = sel[i], y = sel[p];
            const bool desc = (i & k2) == 0;
            if (desc ? (x < y) : (x > y)) { sel[i] = y; sel[p] = x; }
          }
        }
        __syncthreads();
      }
    }
  }
  if (cand) {
    unsigned long long* c = cand + ((int64_t)b * gridDim.x + blockIdx.x) * a.k;
    for (int r = tid; r < a.k; r += TK_THREADS) c[r] = (r < keff) ? sel[r] : 0ull;
    return;
  }
  for (int r = tid; r < a.k; r += TK_THREADS) {
    if (r < keff) {
      const unsigned long long v = sel[r];
      a.ids[(int64_t)b * a.k + r] = (int32_t)(~(uint32_t)(v & 0xffffffffull));
      a.scores[(int64_t)b * a.k + r] = key_score((uint32_t)(v >> 32));
    } else {
      a.ids[(int64_t)b * a.k + r] = -1;
      a.scores[(int64_t)b * a.k + r] = -INFINITY;
    }
  }
}

// Merge of the slices' candidates: the k best composites of n_slices * k, sorted.  The
// composites of distinct documents are distinct, so up to RANK_MAX candidates are placed by
// rank (the number of larger candidates) after one barrier; more go through a bitonic sort.
// Every valid document's composite is nonzero and at least min(k, n_docs) of them are
// candidates, so the zero padding of short slices only takes ranks past the valid ones.
constexpr int RANK_MAX = 512;
__global__ __launch_bounds__(TK_THREADS) void topk_merge(TopkArgs a, int n_slices,
                                                         const unsigned long long* cand) {
  __shared__ unsigned long long buf[MERGE_MAX];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int total = n_slices * a.k;
  const int keff = min(a.k, a.n_docs);
  const unsigned long long* c = cand + (int64_t)b * total;
  int32_t* ids = a.ids + (int64_t)b * a.k;
  float* scores = a.scores + (int64_t)b * a.k;
  if (total <= RANK_MAX) {
    for (int i = tid; i < total; i += TK_THREADS) buf[i] = c[i];
    __syncthreads();
    for (int i = tid; i < total; i += TK_THREADS) {
      const unsigned long long x = buf[i];
      int r = 0;
      for (int j = 0; j < total; ++j) r += buf[j] > x;
      if (r < keff) {
        ids[r] = (int32_t)(~(uint32_t)(x & 0xffffffffull));
        scores[r] = key_score((uint32_t)(x >> 32));
      }
    }
    for (int r = keff + tid; r < a.k; r += TK_THREADS) {
      ids[r] = -1;
      scores[r] = -INFINITY;
    }
    return;
  }
  int n2 = 1;
  while (n2 < total) n2 <<= 1;
  for (int i = tid; i < n2; i += TK_THREADS) buf[i] = (i < total) ? c[i] : 0ull;
  __syncthreads();
  for (int k2 = 2; k2 <= n2; k2 <<= 1) {
    for (int j = k2 >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < n2; i += TK_THREADS) {
        const int p = i ^ j;
        if (p > i) {
          const unsigned long long x = buf[i], y = buf[p];
          const bool desc = (i & k2) == 0;
          if (desc ? (x < y) : (x > y)) { buf[i] = y; buf[p] = x; }
        }
      }
      __syncthreads();
    }
  }
  for (int r = tid; r < a.k; r += TK_THREADS) {
    if (r < keff) {
      const unsigned long long v = buf[r];
      ids[r] = (int32_t)(~(uint32_t)(v & 0xffffffffull));
      scores[r] = key_score((uint32_t)(v >> 32));
    } else {
      ids[r] = -1;
      scores[r] = -INFINITY;
    }
  }
}

}  // namespace

size_t topk_workspace_bytes(int n_queries, int n_docs, int k) {
  const int64_t n_slices = ((int64_t)n_docs + SLICE - 1) / SLICE;
  if (n_slices <= 1 || n_slices * k > MERGE_MAX) return 0;
  return align256((size_t)n_queries * n_slices * k * sizeof(unsigned long long));
}

hipError_t launch_topk(const TopkArgs& a, void* workspace, hipStream_t s) {
  const dim3 block(TK_THREADS);
  const int64_t n_slices = ((int64_t)a.n_docs + SLICE - 1) / SLICE;
  if (n_slices <= 1) {
    const int kpt = (a.n_docs + TK_THREADS - 1) / TK_THREADS;
    const dim3 grid(1, a.n_queries);
    if (kpt <= 4) hipLaunchKernelGGL(topk_reg<4>, grid, block, 0, s, a, nullptr);
    else hipLaunchKernelGGL(topk_reg<8>, grid, block, 0, s, a, nullptr);
    return hipGetLastError();
  }
  if (n_slices * a.k > MERGE_MAX) {  // too many candidates for one merge: passes over memory
    hipLaunchKernelGGL(topk_kernel, dim3(a.n_queries), block, 0, s, a);
    return hipGetLastError();
  }
  unsigned long long* cand = (unsigned long long*)workspace;
  hipLaunchKernelGGL(topk_reg<SLICE_KPT>, dim3((unsigned)n_slices, a.n_queries), block, 0, s, a, cand);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_merge, dim3(a.n_queries), block, 0, s, a, (int)n_slices, (const unsigned long long*)cand);
  return hipGetLastError();
}

}  // namespace msa
