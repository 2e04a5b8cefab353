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
// The work per query is a few reads of 4 * N bytes that stay in L2; it is latency-bound.
#include "common.hpp"
#include "launch.hpp"

namespace msa {
namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;

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

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3(a.n_queries), dim3(TK_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace msa
