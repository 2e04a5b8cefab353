// Step D -- context assembly and sparse attention.
//
// hysenlabs.com "EverMind-AI/MSA: routing top-k compressed documents inside attention ...":
//  * "Routing happens inside attention ...": the selected documents' compressed K/V are
//    concatenated with the query's local K/V for decoding;
//  * "Document-wise RoPE resets ..." (second paragraph): positions over the active context
//    are global; local tokens sit at positions k_eff + j, after the k_eff selected
//    documents, and every key is visible in the order memory, query, generated tokens;
//  * "The 100M-token setup depends on host memory ...": content K/V may stay in host
//    DRAM and be fetched only when selected.
// yeyulingfeng.com "深度分析MSA ..." section 五 step 3: generation sees only the query's
// local states and the top-k memory.
//
// Kernels:
//  * rope_local (float32): rotates Q and the local K at their global positions (k_eff +
//    local index) into the workspace, angles in double precision, once per row.
//  * rope_prep (bf16): in one launch, the cos / sin table of every position a row or local
//    key can take (double-precision angles) and the local K rotated the same way;
//    attn_mfma rotates Q with the table while loading its operands.
//  * attn_mfma (bf16): one workgroup per (query, kv head, block of query rows, key split);
//    each wave holds one or two 16-row tiles of query rows, so each staged K/V tile serves
//    every row of the block.  The key sequence is [rows of the selected documents in rank
//    order ; local keys]; a branch-free table in LDS maps each key to its source row (bank
//    row of a selected document, read from HBM or over the host link from pinned memory, or
//    a local row).  K and V are staged in LDS row-major, double-buffered, with the gathers
//    of the next tiles in flight during the current tile's math.  The softmax runs in
//    float32 with a lazily moved reference maximum.
//    S^T = K * Q^T on v_mfma_f32_16x16x32_bf16 leaves each lane with 8 scores of one
//    query row, which are exactly the P^T operand of O^T = V^T * P^T, so probabilities
//    never leave registers; V^T comes from the row-major tile through gfx950's
//    transposing LDS load, and each K / V operand read serves both row tiles of a wave.
//  * attn_valu (float32): one wave per (query token, kv head, up to 4 query heads), 16 lanes
//    per head, online softmax in float32.
//  * attn_combine: merges the per-split (max, sum, unnormalised output) triples.
#include <math.h>

#include "attn_shared.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace msa {
namespace {

// Maximum over the four lanes cl, cl + 16, cl + 32, cl + 48 (the 16-lane rows of a wave):
// gfx950's permlane swaps exchange odd and even rows, then the two halves, so each lane
// holds its own value in one result and its partner's in the other.
__device__ __forceinline__ float row_max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <int D, int NW, int MTW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void attn_mfma(AttnK a, int nsub) {
  constexpr int KK = D / 32;
  constexpr int MD = D / 16;
  constexpr int KSTR = D + 16;  // bf16 per K / V row in LDS: 32 bytes of padding keep the
                                // row reads and the transposed reads conflict-free
  constexpr int THREADS = 64 * NW;
  constexpr int UPK = (KT * (D / 8) + THREADS - 1) / THREADS;  // 16-byte units per thread per tile
  constexpr int RING = UPK == 1 ? 4 : 2;                       // tiles in flight
  constexpr int ROWS = NW * MTW * 16;  // query rows per workgroup (MTW 16-row tiles per wave)
  // Lazy rescaling: a row's reference maximum moves only when a score exceeds it by more
  // than LAZY in the base-2 exponent, so probabilities stay below 2^LAZY (far inside the
  // float32 and bf16 ranges) and most tiles rescale nothing.
  constexpr float LAZY = 8.f;
  __shared__ __align__(16) bf16_t Ks[2][KT * KSTR];
  __shared__ __align__(16) bf16_t Vs[2][KT * KSTR];
  __shared__ int64_t mstart[1025], mpre[1025];
  __shared__ __align__(16) bf16_t sink[8];
  __shared__ int64_t tabk[2 * TCH], tabv[2 * TCH];
  __shared__ int sh_keff;
  __shared__ int64_t sh_M;

  int pair, sub;
  if (!place_pair(a.n_queries * a.h_kv, nsub, pair, sub)) return;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int cl = lane & 15, g4 = lane >> 4;
  const int b = pair / a.h_kv, g = pair % a.h_kv;
  const int split = sub % a.splits;
  const int G = a.hq / a.h_kv;
  const int hq_n = a.hq;
  const int q0 = a.q_off[b], Lq = a.q_off[b + 1] - q0;
  const int kv0 = a.kv_off[b], Lkv = a.kv_off[b + 1] - kv0;
  const int nrows = Lq * G;
  const int rb = (sub / a.splits) * ROWS;
  if (rb >= nrows) return;

  if (w == 0) {
    MemMap mm = build_memmap(a.ids + (int64_t)b * a.k, a.k, a.chunk_off, mstart, mpre);
    if (lane == 0) { sh_keff = mm.keff; sh_M = mm.M; }
  }
  __syncthreads();
  const int keff = sh_keff;
  const int64_t M = sh_M;
  const int64_t NK = M + Lkv;
  int64_t k_lo = NK * split / a.splits, k_hi = NK * (split + 1) / a.splits;
  // keys past the last local position any row of this block may see are never needed
  const int t_max = min(Lq - 1, (rb + ROWS - 1) / G);
  k_hi = min(k_hi, M + (int64_t)(Lkv - Lq + t_max + 1));
  const float sc = a.scale_log2;

  // this wave's rows: MTW 16-row tiles from wr0; a wave with none skips the math
  const int wr0 = rb + w * MTW * 16;
  const bool wave_rows = wr0 < nrows;
  // Keys relative to k_lo (int: fewer than 2^31 keys).  Every key up to lim_w is visible to
  // every row of the wave; lim_r[m] is the lane's row's last visible key.
  const int n_keys = (int)max(k_hi - k_lo, (int64_t)0);
  const int lim_w = (int)(M + (Lkv - Lq) + min(wr0, nrows - 1) / G - k_lo);

  // this lane's query rows (one per row tile; B operands of S^T) and causal limits.  Q is
  // rotated here to its global position keff + (Lkv - Lq) + t: each lane also loads the
  // pair partners (d +- D/2) of its 8 elements and takes cos / sin from the table.
  int t_of[MTW], hq_of[MTW];
  bool row_ok[MTW];
  int lim_r[MTW];
  bf16x8_t Qf[MTW][KK];
#pragma unroll
  for (int m = 0; m < MTW; ++m) {
    const int row = wr0 + m * 16 + cl;
    row_ok[m] = row < nrows;
    t_of[m] = row_ok[m] ? row / G : 0;
    hq_of[m] = g * G + (row_ok[m] ? row % G : 0);
    lim_r[m] = (int)(M + (Lkv - Lq) + t_of[m] - k_lo);
    const bf16_t* qp = (const bf16_t*)a.Q + ((int64_t)(q0 + t_of[m]) * hq_n + hq_of[m]) * D;
    const int64_t pos = (int64_t)keff + (Lkv - Lq) + t_of[m];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const uint4 w = rope_load8<D>(qp, kk * 32 + g4 * 8, pos, a.rtab, a.n_pos);
      Qf[m][kk] = __builtin_bit_cast(bf16x8_t, row_ok[m] ? w : make_uint4(0, 0, 0, 0));
    }
  }

  f32x4_t acc[MTW][MD];
  // Row sums of the probabilities come from the matrix cores: a ones operand in place of V^T
  // gives every lane of a row the sum over the tile's keys of the same rounded values that
  // weight V, accumulated in float32 (so the output is a weighted mean whatever the
  // rounding; with a stale reference maximum no weight is exactly 1).
  f32x4_t lsum[MTW];
  // reference maximum (raw score), its scaled value, and the rescale threshold
  float m_ref[MTW], mb[MTW], thr[MTW];
#pragma unroll
  for (int m = 0; m < MTW; ++m) {
    m_ref[m] = -INFINITY;
    mb[m] = 0.f;
    thr[m] = -INFINITY;
    lsum[m] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int md = 0; md < MD; ++md) acc[m][md] = {0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
  const float lazy_raw = LAZY / sc;  // the threshold in raw score units (sc > 0)

  auto tile_math = [&](int buf, int rel) __attribute__((always_inline)) {
    // ---- S^T = K Q^T: each K operand read once for all of the wave's row tiles ----
    f32x4_t s[MTW][2];
#pragma unroll
    for (int m = 0; m < MTW; ++m) s[m][0] = s[m][1] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const bf16x8_t kw =
            __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&Ks[buf][(n * 16 + cl) * KSTR + kk * 32 + g4 * 8]));
#pragma unroll
        for (int m = 0; m < MTW; ++m) s[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kw, Qf[m][kk], s[m][n], 0, 0, 0);
      }
    // lane holds S[row cl of tile m][key rel + n*16 + g4*4 + i]; keys relative to k_lo.
    // At most two uniform branches per tile, both rare (the masks near the end of the range
    // and the moves of the reference maximum), so that the exponentials of one row tile and
    // the products of the other share one block the scheduler can interleave.
    if (rel + KT > n_keys || rel + KT - 1 > lim_w) {  // uniform
#pragma unroll
      for (int m = 0; m < MTW; ++m) {
        // key visible: below the range end and at most the row's causal limit
        const int lim = min(n_keys - 1, lim_r[m]) - rel - g4 * 4;
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[m][n][i] = n * 16 + i <= lim ? s[m][n][i] : -INFINITY;
      }
    }
    // Does any score pass its row's threshold (also the first visible key of a row)?  Only
    // then are the rows' maxima (over their 4 lanes) formed and the references moved.
    bool over = false;
#pragma unroll
    for (int m = 0; m < MTW; ++m) {
      const float t = thr[m];
      over |= (s[m][0][0] > t) | (s[m][0][1] > t) | (s[m][0][2] > t) | (s[m][0][3] > t) |
              (s[m][1][0] > t) | (s[m][1][1] > t) | (s[m][1][2] > t) | (s[m][1][3] > t);
    }
    if (__ballot(over) != 0) {
#pragma unroll
      for (int m = 0; m < MTW; ++m) {
        const float mx = fmaxf(fmaxf(fmaxf(s[m][0][0], s[m][0][1]), fmaxf(s[m][0][2], s[m][0][3])),
                               fmaxf(fmaxf(s[m][1][0], s[m][1][1]), fmaxf(s[m][1][2], s[m][1][3])));
        const float rmx = row_max4(mx);
        const float m_new = fmaxf(m_ref[m], rmx);
        const float alpha = m_ref[m] == -INFINITY ? 0.f : exp2_hw(m_ref[m] * sc - m_new * sc);
        m_ref[m] = m_new;
        mb[m] = m_new == -INFINITY ? 0.f : m_new * sc;
        thr[m] = m_new + lazy_raw;
#pragma unroll
        for (int i = 0; i < 4; ++i) lsum[m][i] *= alpha;
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[m][md][i] *= alpha;
      }
    }
    bf16x8_t Pf[MTW];
#pragma unroll
    for (int m = 0; m < MTW; ++m) {
      float p[2][4];
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[n][i] = exp2_hw(fmaf(s[m][n][i], sc, -mb[m]));
      // P^T operand: k-slot g4*8 + j  <->  key g4*4 + j (j < 4), 16 + g4*4 + (j-4) (j >= 4)
      uint4 pw;
      pw.x = f32x2_to_bf16x2(p[0][0], p[0][1]);
      pw.y = f32x2_to_bf16x2(p[0][2], p[0][3]);
      pw.z = f32x2_to_bf16x2(p[1][0], p[1][1]);
      pw.w = f32x2_to_bf16x2(p[1][2], p[1][3]);
      Pf[m] = __builtin_bit_cast(bf16x8_t, pw);
      lsum[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, Pf[m], lsum[m], 0, 0, 0);
    }
    // ---- O^T += V^T P^T: each V^T operand read once for all row tiles ----
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      // A operand V^T: element md*16 + cl over keys g4*4 .. +3 and 16 + g4*4 .. +3
      const bf16_t* vr = &Vs[buf][(g4 * 4 + (cl >> 2)) * KSTR + md * 16 + (cl & 3) * 4];
      const uint2 v0 = lds_read_tr16(vr);
      const uint2 v1 = lds_read_tr16(vr + 16 * KSTR);
      const bf16x8_t Vf = __builtin_bit_cast(bf16x8_t, make_uint4(v0.x, v0.y, v1.x, v1.y));
#pragma unroll
      for (int m = 0; m < MTW; ++m) acc[m][md] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Vf, Pf[m], acc[m][md], 0, 0, 0);
    }
  };

  // ---- the key loop (an empty key split still writes its empty partial rows) ----
  key_loop<RING, D, THREADS, KSTR, true>(a, g, tid, k_lo, n_keys, mstart, mpre, keff, M, kv0, tabk, tabv, Ks[0], Ks[1],
                                         Vs[0], Vs[1], sink, [&](int buf, int rel) __attribute__((always_inline)) {
                                           if (wave_rows) tile_math(buf, rel);
                                         });

#pragma unroll
  for (int m = 0; m < MTW; ++m) {
    const float l_row = lsum[m][0];  // every lane of a row holds the row's total
    if (!row_ok[m]) continue;
    const int64_t orow = (int64_t)(q0 + t_of[m]) * hq_n + hq_of[m];
    if (a.splits == 1) {
      if (a.lse != nullptr && g4 == 0)
        a.lse[orow] = l_row > 0.f ? (m_ref[m] * sc + log2f(l_row)) * LN2 : -INFINITY;
      const float inv = l_row > 0.f ? 1.0f / l_row : 0.f;
      bf16_t* o = (bf16_t*)a.O + orow * D + g4 * 4;
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        float f[4] = {acc[m][md][0] * inv, acc[m][md][1] * inv, acc[m][md][2] * inv, acc[m][md][3] * inv};
        Elem<bf16_t>::store4(o + md * 16, f);
      }
    } else {
      const int64_t prow = (int64_t)split * a.total_q * hq_n + orow;
      float* po = a.part_o + prow * D + g4 * 4;
#pragma unroll
      for (int md = 0; md < MD; ++md)
        *reinterpret_cast<float4*>(po + md * 16) =
            make_float4(acc[m][md][0], acc[m][md][1], acc[m][md][2], acc[m][md][3]);
      if (g4 == 0) {
        a.part_ml[prow * 2] = m_ref[m] == -INFINITY ? -INFINITY : m_ref[m] * sc;  // scaled maxima
        a.part_ml[prow * 2 + 1] = l_row;
      }
    }
  }
}

// ---- float32 path: one thread per (query row, head) ----------------------------------
// float32 inputs: one wave per (query token, kv head, block of up to 4 of the group's query
// heads).  16 lanes per query head hold D/16 elements of its rotated row and of its output;
// every key row is read once per wave (the four 16-lane groups read the same addresses),
// each dot product is reduced across its 16 lanes, and the online softmax runs in float32,
// replicated on the 16 lanes of a head.
template <typename T, int D>
__global__ __launch_bounds__(64) void attn_valu(AttnK a, int hblocks) {
  constexpr int E = D / 16;  // elements per lane
  const int b = blockIdx.y;
  const int q0 = a.q_off[b], Lq = a.q_off[b + 1] - q0;
  const int kv0 = a.kv_off[b], Lkv = a.kv_off[b + 1] - kv0;
  const int G = a.hq / a.h_kv;
  const int x = blockIdx.x;
  const int hb = x % hblocks, g = (x / hblocks) % a.h_kv, t = x / (hblocks * a.h_kv);
  if (t >= Lq) return;  // uniform
  const int lane = threadIdx.x, li = lane & 15;
  const int j = hb * 4 + (lane >> 4);  // query head within the group
  const bool row_ok = j < G;
  const int hq = g * G + (row_ok ? j : 0);
  const int e0 = li * E;
  const T* Qr = (const T*)a.Qrot + ((int64_t)(q0 + t) * a.hq + hq) * D + e0;
  float q[E], acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = row_ok ? (float)Qr[e] : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  auto visit = [&](const T* kp, const T* vp) __attribute__((always_inline)) {
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) dot = fmaf(q[e], (float)kp[e0 + e], dot);
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) dot += __shfl_xor(dot, o, 16);
    const float s = dot * a.scale_log2;
    const float mn = fmaxf(m, s);
    const float al = exp2f(m - mn), p = exp2f(s - mn);
    l = l * al + p;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(acc[e], al, p * (float)vp[e0 + e]);
    m = mn;
  };
  const int32_t* ids = a.ids + (int64_t)b * a.k;
  const T* Kb = (const T*)a.Kbar;
  const T* Vb = (const T*)a.Vbar;
  for (int rr = 0; rr < a.k; ++rr) {
    const int id = ids[rr];
    if (id < 0) continue;
    for (int64_t c = a.chunk_off[id]; c < a.chunk_off[id + 1]; ++c)
      visit(Kb + (c * a.h_kv + g) * D, Vb + (c * a.h_kv + g) * D);
  }
  const T* Kr = (const T*)a.Krot;
  const T* Vl = (const T*)a.Vloc;
  for (int jj = 0; jj <= Lkv - Lq + t; ++jj)
    visit(Kr + ((int64_t)(kv0 + jj) * a.h_kv + g) * D, Vl + ((int64_t)(kv0 + jj) * a.h_kv + g) * D);
  if (!row_ok) return;
  const int64_t orow = (int64_t)(q0 + t) * a.hq + hq;
  if (a.lse != nullptr && li == 0) a.lse[orow] = l > 0.f ? (m + log2f(l)) * LN2 : -INFINITY;
  const float inv = 1.0f / l;
  T* o = (T*)a.O + orow * D + e0;
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = (T)(acc[e] * inv);
}

// ---- merge of key splits -------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_combine(AttnK a) {
  // one wave per output row; lane covers D/64 elements (at least one)
  const int64_t row = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / 64;
  const int lane = threadIdx.x & 63;
  const int64_t rows = a.total_q * a.hq;
  if (row >= rows) return;
  float mstar = -INFINITY;
  for (int s = 0; s < a.splits; ++s)
    mstar = fmaxf(mstar, a.part_ml[((int64_t)s * rows + row) * 2]);
  float L = 0.f;
  constexpr int PER = (D + 63) / 64;
  float o[PER];
#pragma unroll
  for (int x = 0; x < PER; ++x) o[x] = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const int64_t pr = (int64_t)s * rows + row;
    const float ms = a.part_ml[pr * 2];
    if (ms == -INFINITY) continue;
    const float wgt = exp2f(ms - mstar);
    L += wgt * a.part_ml[pr * 2 + 1];
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int e = lane + 64 * x;
      if (e < D) o[x] += wgt * a.part_o[pr * D + e];
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  if (a.lse != nullptr && lane == 0) a.lse[row] = L > 0.f ? (mstar + log2f(L)) * LN2 : -INFINITY;
  bf16_t* out = (bf16_t*)a.O + row * D;
#pragma unroll
  for (int x = 0; x < PER; ++x) {
    const int e = lane + 64 * x;
    if (e < D) out[e] = (bf16_t)f32_to_bf16(o[x] * inv);
  }
}

template <typename T, int D>
hipError_t launch_attn_t(const AttnArgs& r, AttnK& k, bool host, hipStream_t s) {
  if (r.total_q == 0) return hipSuccess;  // no rows: nothing reads the rotated local K
  // float32: Q and the local K rotated into the workspace; bf16: the cos / sin table, then
  // the local K rotated with it (the attention kernel rotates Q with it as it loads it)
  const int nq_blocks = sizeof(T) == 4 ? (int)((r.total_q + RPW - 1) / RPW) : 0;
  const int nk_blocks = (int)((r.total_kv + RPW - 1) / RPW);
  if constexpr (sizeof(T) == 2) {
    hipError_t e = launch_rope_setup<D>(k, 0, nk_blocks, s);
    if (e != hipSuccess) return e;
  } else if (nq_blocks + nk_blocks > 0) {
    hipLaunchKernelGGL((rope_local<T, D>), dim3(nq_blocks + nk_blocks), dim3(256), 0, s, k, nq_blocks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if constexpr (sizeof(T) == 4) {
    k.splits = 1;
    const int G = r.hq / r.h_kv, hblocks = (G + 3) / 4;
    dim3 grid((unsigned)((int64_t)r.max_q_len * r.h_kv * hblocks), (unsigned)r.n_queries);
    hipLaunchKernelGGL((attn_valu<T, D>), grid, dim3(64), 0, s, k, hblocks);
    return hipGetLastError();
  } else {
    const int G = r.hq / r.h_kv;
    const int brows = attn_fwd_rows(r.max_q_len, G, host);
    const int rblocks = (r.max_q_len * G + brows - 1) / brows;
    const int nsub = rblocks * k.splits;
    const int n_pairs = r.n_queries * r.h_kv;
    const dim3 grid((unsigned)(((n_pairs + 7) / 8) * 8 * nsub));
    // 16-row tiles: two per wave (each K / V operand serves both) from 128 rows; below, fewer
    // threads would each stage more of a tile, and the registers would not fit
    switch (brows) {
      case 16: hipLaunchKernelGGL((attn_mfma<D, 1, 1>), grid, dim3(64), 0, s, k, nsub); break;
      case 32: hipLaunchKernelGGL((attn_mfma<D, 2, 1>), grid, dim3(128), 0, s, k, nsub); break;
      case 64: hipLaunchKernelGGL((attn_mfma<D, 4, 1>), grid, dim3(256), 0, s, k, nsub); break;
      case 128: hipLaunchKernelGGL((attn_mfma<D, 4, 2>), grid, dim3(256), 0, s, k, nsub); break;
      default: hipLaunchKernelGGL((attn_mfma<D, 8, 2>), grid, dim3(512), 0, s, k, nsub); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || k.splits == 1) return e;
    const int64_t rows = r.total_q * r.hq;
    hipLaunchKernelGGL((attn_combine<D>), dim3((unsigned)((rows * 64 + 255) / 256)), dim3(256), 0, s, k);
    return hipGetLastError();
  }
}

}  // namespace

// Query rows per attention workgroup: every row of one (query, kv head) up to 256, so that
// a staged K/V tile serves all the rows that need it (16 rows per wave up to 8 waves, then
// two 16-row tiles per wave).
int attn_rows_per_block(int max_q_len, int G) {
  const int need = max_q_len * G;
  int rows = 16;
  while (rows < need && rows < 256) rows <<= 1;
  return rows;
}

// Query rows per forward workgroup.  With K-bar / V-bar in device memory, up to 128 (4 waves
// of two 16-row tiles), so that two workgroups share a CU and the barriers of one overlap
// the math of the other; the row blocks of one (query, kv head) run on one XCD, whose L2
// serves the second block the rows the first read from HBM.  Over the host link every row
// is read once: one block holds all the rows of a (query, kv head), up to 256.
int attn_fwd_rows(int max_q_len, int G, bool host) {
  const int rows = attn_rows_per_block(max_q_len, G);
  return host || rows < 128 ? rows : 128;
}

// Key splits per (query, kv head): enough workgroups in flight to keep the host link or HBM
// busy (about 32), bounded so the partial results stay small.  Counted on row blocks of up
// to 256 rows whatever the placement, so that a bank in host memory and one in HBM split
// the keys alike and give the same bits (waves hold the same 32 rows in both).
int attn_splits(int n_queries, int max_q_len, int hq, int h_kv) {
  const int G = hq / h_kv;
  const int rows = attn_rows_per_block(max_q_len, G);
  const int rblocks = (max_q_len * G + rows - 1) / rows;
  const long base = (long)n_queries * h_kv * (rblocks > 0 ? rblocks : 1);
  // more splits only add partials to merge (on the 100M bank with pinned-host K/V, 4 splits
  // per pair attend in 86 us against 95 us with 8 and 107 us with 16)
  long s = (32 + base - 1) / base;
  if (s < 1) s = 1;
  if (s > 16) s = 16;
  return (int)s;
}

// Positions a query's rows and local keys can take: below keff + Lkv <= 1024 + total_kv.
static int64_t attn_max_positions(int64_t total_kv, int k) { return (int64_t)k + total_kv; }

// Workspace: float32 [rotated Q][rotated local K]; bf16 [rotated local K][cos / sin table]
// [per-split partial outputs][per-split (max, sum)].
size_t attn_workspace_bytes(int dtype, int n_queries, int64_t total_q, int64_t total_kv,
                            int max_q_len, int hq, int h_kv, int d) {
  const size_t esz = dtype == 0 ? 4 : 2;
  size_t bytes = align256((size_t)total_kv * h_kv * d * esz);
  if (dtype == 0) bytes += align256((size_t)total_q * hq * d * esz);
  if (dtype == 1) {
    bytes += align256((size_t)attn_max_positions(total_kv, 1024) * d * 4);
    const int s = attn_splits(n_queries, max_q_len, hq, h_kv);
    if (s > 1) {
      bytes += align256((size_t)s * total_q * hq * d * 4);
      bytes += align256((size_t)s * total_q * hq * 2 * 4);
    }
  }
  return bytes;
}

hipError_t launch_sparse_attn(const AttnArgs& r, hipStream_t s) {
  AttnK k{};
  k.n_queries = r.n_queries;
  k.total_q = r.total_q;
  k.total_kv = r.total_kv;
  k.q_off = r.q_off;
  k.kv_off = r.kv_off;
  k.Q = r.Q;
  k.Kloc = r.Kloc;
  k.Vloc = r.Vloc;
  k.hq = r.hq;
  k.h_kv = r.h_kv;
  k.rope_base = r.rope_base;
  k.scale_log2 = r.scale * LOG2E;
  k.k = r.k;
  k.ids = r.ids;
  k.chunk_off = r.chunk_off;
  k.Kbar = r.Kbar;
  k.Vbar = r.Vbar;
  k.O = r.O;
  k.lse = r.lse;
  const size_t esz = r.dtype == 0 ? 4 : 2;
  char* ws = (char*)r.workspace;
  k.Krot = ws;
  ws += align256((size_t)r.total_kv * r.h_kv * r.d * esz);
  if (r.dtype == 0) {
    k.Qrot = ws;
    ws += align256((size_t)r.total_q * r.hq * r.d * esz);
  } else {
    k.n_pos = attn_max_positions(r.total_kv, r.k);
    k.rtab = (const float*)ws;
    ws += align256((size_t)attn_max_positions(r.total_kv, 1024) * r.d * 4);
  }
  // K-bar / V-bar in host memory (pinned): read over the host link, once per row
  bool host = false;
  if (r.dtype == 1) {
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, r.Kbar) == hipSuccess) host = at.type == hipMemoryTypeHost;
    else (void)hipGetLastError();  // not a HIP allocation: nothing to record
  }
  k.splits = r.dtype == 1 ? attn_splits(r.n_queries, r.max_q_len, r.hq, r.h_kv) : 1;
  if (k.splits > 1) {
    k.part_o = (float*)ws;
    ws += align256((size_t)k.splits * r.total_q * r.hq * r.d * 4);
    k.part_ml = (float*)ws;
  }
  if (r.dtype == 0) {
    switch (r.d) {
      case 32: return launch_attn_t<float, 32>(r, k, host, s);
      case 64: return launch_attn_t<float, 64>(r, k, host, s);
      default: return launch_attn_t<float, 128>(r, k, host, s);
    }
  }
  switch (r.d) {
    case 32: return launch_attn_t<bf16_t, 32>(r, k, host, s);
    case 64: return launch_attn_t<bf16_t, 64>(r, k, host, s);
    default: return launch_attn_t<bf16_t, 128>(r, k, host, s);
  }
}

}  // namespace msa
