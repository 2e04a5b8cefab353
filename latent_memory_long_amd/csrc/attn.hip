// Step D -- context assembly and sparse attention.
//
// hysenlabs.com "EverMind-AI/MSA: routing top-k compressed documents inside attention ...":
//  * "Routing happens inside attention ...": the selected documents' compressed K/V are
//    concatenated with the query's local K/V for decoding;
//  * "Document-wise RoPE resets ..." (second paragraph): global RoPE over the active
//    context; the query's start index is offset by k, the number of retrieved blocks, so
//    the causal order is memory, then query, then generation;
//  * "The 100M-token setup depends on host memory ...": content K/V may stay in host
//    DRAM and be fetched only when selected.
// yeyulingfeng.com "深度分析MSA ..." section 五 step 3: generation sees only the query's
// local states and the top-k memory.
//
// Kernels:
//  * rope_local: rotates Q and the local K at their global positions (k_eff + local
//    index) into the workspace, angles in double precision, once per row.
//  * attn_mfma (bf16): one workgroup per (query, kv head, block of up to 256 query rows,
//    key split), with one 16-row wave per row slice, so each staged K/V tile serves every
//    query row of the kv head and every byte read over the host link is read once.  The
//    key sequence is [rows of the selected documents in rank order ; local keys]; the
//    workgroup maps each key of a 32-key tile to its source row (bank row of a selected
//    document, read from HBM or over the host link from pinned memory, or a local row),
//    stages K and V in LDS row-major (double-buffered, the gathers of the next tiles in
//    flight during the current tile's math: tile_pipeline), and runs an online softmax in
//    float32.
//    S^T = K * Q^T on v_mfma_f32_16x16x32_bf16 leaves each lane with 8 scores of one
//    query row, which are exactly the P^T operand of O^T = V^T * P^T, so probabilities
//    never leave registers; V^T comes from the row-major tile through gfx950's
//    transposing LDS load.
//  * attn_valu (float32): one thread per (query row, head), plain online softmax.
//  * attn_combine: merges the per-split (max, sum, unnormalised output) triples.
#include <math.h>

#include "attn_shared.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace msa {
namespace {

template <int D, int NW, int MTW>
__global__ __launch_bounds__(64 * NW) void attn_mfma(AttnK a) {
  constexpr int KK = D / 32;
  constexpr int MD = D / 16;
  constexpr int KSTR = D + 16;  // bf16 per K / V row in LDS: 32 bytes of padding keep the
                                // row reads and the transposed reads conflict-free
  constexpr int THREADS = 64 * NW;
  constexpr int UPT = 2 * tile_upk<D, THREADS>();
  constexpr int ROWS = NW * MTW * 16;  // query rows per workgroup (MTW 16-row tiles per wave)
  __shared__ __align__(16) bf16_t Ks[2][KT * KSTR];
  __shared__ __align__(16) bf16_t Vs[2][KT * KSTR];
  __shared__ int64_t mstart[1025], mpre[1025];
  __shared__ int sh_keff;
  __shared__ int64_t sh_M;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int cl = lane & 15, g4 = lane >> 4;
  const int b = blockIdx.z;
  const int g = blockIdx.y % a.h_kv;
  const int split = blockIdx.y / a.h_kv;
  const int G = a.hq / a.h_kv;
  const int hq_n = a.hq;
  const int q0 = a.q_off[b], Lq = a.q_off[b + 1] - q0;
  const int kv0 = a.kv_off[b], Lkv = a.kv_off[b + 1] - kv0;
  const int nrows = Lq * G;
  const int rb = blockIdx.x * ROWS;
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
  const float scale_log2 = a.scale_log2;

  // this lane's query rows (one per row tile; B operands of S^T) and causal limits
  bool row_ok[MTW];
  int t_of[MTW], hq_of[MTW];
  int64_t key_lim[MTW];
  bf16x8_t Qf[MTW][KK];
#pragma unroll
  for (int m = 0; m < MTW; ++m) {
    const int row = rb + (w * MTW + m) * 16 + cl;
    row_ok[m] = row < nrows;
    t_of[m] = row_ok[m] ? row / G : 0;
    hq_of[m] = g * G + (row_ok[m] ? row % G : 0);
    key_lim[m] = M + (int64_t)(Lkv - Lq + t_of[m]);  // last visible key index
    const bf16_t* qp = (const bf16_t*)a.Qrot + ((int64_t)(q0 + t_of[m]) * hq_n + hq_of[m]) * D + g4 * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      Qf[m][kk] = row_ok[m] ? __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qp + kk * 32))
                            : __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
  }

  f32x4_t acc[MTW][MD];
  float m_run[MTW], l_run[MTW];
#pragma unroll
  for (int m = 0; m < MTW; ++m) {
    m_run[m] = -INFINITY;
    l_run[m] = 0.f;
#pragma unroll
    for (int md = 0; md < MD; ++md) acc[m][md] = {0.f, 0.f, 0.f, 0.f};
  }

  // the smallest causal limit over the block's rows (its first row's)
  const int64_t key_lim_min = M + (int64_t)(Lkv - Lq + rb / G);

  TileSrc ts;
  ts.Kb = (const bf16_t*)a.Kbar;
  ts.Vb = (const bf16_t*)a.Vbar;
  ts.Kr = (const bf16_t*)a.Krot;
  ts.Vl = (const bf16_t*)a.Vloc;
  ts.mstart = mstart;
  ts.mpre = mpre;
  ts.keff = keff;
  ts.hkv = a.h_kv;
  ts.g = g;
  ts.kv0 = kv0;
  ts.M = M;
  ts.k_hi = k_hi;
  // The gathers run TILE_RING tiles ahead of the math (tile_pipeline; two when a stage
  // takes many registers per thread).
  auto tile_math = [&](int buf, int64_t kt) __attribute__((always_inline)) {
    // every key of the tile is visible to every row of the block: no masking needed
    const bool full_tile = kt + KT <= k_hi && kt + KT - 1 <= key_lim_min && rb + ROWS <= nrows;
#pragma unroll
    for (int m = 0; m < MTW; ++m) {
      // ---- S^T = K Q^T for two 16-key halves ----
      f32x4_t s[2];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        s[n] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const uint4 kw = *reinterpret_cast<const uint4*>(&Ks[buf][(n * 16 + cl) * KSTR + kk * 32 + g4 * 8]);
          s[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kw), Qf[m][kk], s[n], 0, 0, 0);
        }
      }
      // lane holds S[row cl of tile m][key kt + n*16 + g4*4 + i]; the running max is kept
      // on the raw scores (scale_log2 > 0 keeps their order), scaled inside the exponent
      float mx = -INFINITY;
      if (full_tile) {
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[n][i]);
      } else {
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t key = kt + n * 16 + g4 * 4 + i;
            const bool vis = row_ok[m] && key < k_hi && key <= key_lim[m];
            s[n][i] = vis ? s[n][i] : -INFINITY;
            mx = fmaxf(mx, s[n][i]);
          }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[m], mx);
      float alpha = 1.f;
      float p[2][4];
      if (m_new == -INFINITY) {
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) p[n][i] = 0.f;
      } else {
        const float mb = m_new * scale_log2;
        alpha = exp2_hw(m_run[m] * scale_log2 - mb);
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) p[n][i] = exp2_hw(fmaf(s[n][i], scale_log2, -mb));
      }
      m_run[m] = m_new;
      float ps = 0.f;
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) ps += p[n][i];
      l_run[m] = l_run[m] * alpha + ps;
      // P^T operand: k-slot g4*8 + j  <->  key g4*4 + j (j < 4), 16 + g4*4 + (j-4) (j >= 4)
      uint4 pw;
      pw.x = f32x2_to_bf16x2(p[0][0], p[0][1]);
      pw.y = f32x2_to_bf16x2(p[0][2], p[0][3]);
      pw.z = f32x2_to_bf16x2(p[1][0], p[1][1]);
      pw.w = f32x2_to_bf16x2(p[1][2], p[1][3]);
      const bf16x8_t Pf = __builtin_bit_cast(bf16x8_t, pw);
      // the output columns are rescaled only when some row's maximum moved (alpha != 1)
      const bool rescale = __ballot(alpha != 1.f) != 0;
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        // A operand V^T: element md*16 + cl over keys g4*4 .. +3 and 16 + g4*4 .. +3
        const bf16_t* vr = &Vs[buf][(g4 * 4 + (cl >> 2)) * KSTR + md * 16 + (cl & 3) * 4];
        const uint2 v0 = lds_read_tr16(vr);
        const uint2 v1 = lds_read_tr16(vr + 16 * KSTR);
        const bf16x8_t Vf = __builtin_bit_cast(bf16x8_t, make_uint4(v0.x, v0.y, v1.x, v1.y));
        if (rescale) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[m][md][i] *= alpha;
        }
        acc[m][md] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Vf, Pf, acc[m][md], 0, 0, 0);
      }
    }
  };
  tile_pipeline<(UPT <= 4 ? TILE_RING : 2), D, THREADS, UPT, KSTR, true>(ts, tid, k_lo, k_hi, Ks[0], Ks[1], Vs[0], Vs[1], tile_math);

#pragma unroll
  for (int m = 0; m < MTW; ++m) {
    // row totals: the 4 lane groups of a row hold partial sums
    float l_row = l_run[m] + __shfl_xor(l_run[m], 16);
    l_row += __shfl_xor(l_row, 32);
    if (!row_ok[m]) continue;
    const int64_t orow = (int64_t)(q0 + t_of[m]) * hq_n + hq_of[m];
    if (a.splits == 1) {
      if (a.lse != nullptr && g4 == 0)
        a.lse[orow] = l_row > 0.f ? (m_run[m] * scale_log2 + log2f(l_row)) * LN2 : -INFINITY;
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
        a.part_ml[prow * 2] = m_run[m] * scale_log2;  // the combine works on scaled maxima
        a.part_ml[prow * 2 + 1] = l_row;
      }
    }
  }
}

// ---- float32 path: one thread per (query row, head) ----------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void attn_valu(AttnK a) {
  const int b = blockIdx.y;
  const int q0 = a.q_off[b], Lq = a.q_off[b + 1] - q0;
  const int kv0 = a.kv_off[b], Lkv = a.kv_off[b + 1] - kv0;
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= Lq * a.hq) return;
  const int t = r / a.hq, hq = r % a.hq;
  const int g = hq / (a.hq / a.h_kv);
  const T* Qr = (const T*)a.Qrot + ((int64_t)(q0 + t) * a.hq + hq) * D;
  float q[D], acc[D];
#pragma unroll
  for (int e = 0; e < D; e += 8) Elem<T>::load8(Qr + e, q + e);
#pragma unroll
  for (int e = 0; e < D; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;
  auto visit = [&](const T* kp, const T* vp) {
    float kv[8], dot = 0.f;
#pragma unroll
    for (int e = 0; e < D; e += 8) {
      Elem<T>::load8(kp + e, kv);
#pragma unroll
      for (int x = 0; x < 8; ++x) dot += q[e + x] * kv[x];
    }
    const float s = dot * a.scale_log2;
    const float mn = fmaxf(m, s);
    const float al = exp2f(m - mn), p = exp2f(s - mn);
    l = l * al + p;
#pragma unroll
    for (int e = 0; e < D; e += 8) {
      Elem<T>::load8(vp + e, kv);
#pragma unroll
      for (int x = 0; x < 8; ++x) acc[e + x] = acc[e + x] * al + p * kv[x];
    }
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
  for (int j = 0; j <= Lkv - Lq + t; ++j)
    visit(Kr + ((int64_t)(kv0 + j) * a.h_kv + g) * D, Vl + ((int64_t)(kv0 + j) * a.h_kv + g) * D);
  T* o = (T*)a.O + ((int64_t)(q0 + t) * a.hq + hq) * D;
  if (a.lse != nullptr) a.lse[(int64_t)(q0 + t) * a.hq + hq] = l > 0.f ? (m + log2f(l)) * LN2 : -INFINITY;
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < D; e += 8) {
    float f[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) f[x] = acc[e + x] * inv;
    Elem<T>::store8(o + e, f);
  }
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
hipError_t launch_attn_t(const AttnArgs& r, AttnK& k, hipStream_t s) {
  const int nq_blocks = (int)((r.total_q + RPW - 1) / RPW);
  const int nk_blocks = (int)((r.total_kv + RPW - 1) / RPW);
  if (nq_blocks + nk_blocks > 0) {
    hipLaunchKernelGGL((rope_local<T, D>), dim3(nq_blocks + nk_blocks), dim3(256), 0, s, k, nq_blocks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (r.total_q == 0) return hipSuccess;
  if constexpr (sizeof(T) == 4) {
    k.splits = 1;
    dim3 grid((unsigned)((r.max_q_len * r.hq + 63) / 64), (unsigned)r.n_queries);
    hipLaunchKernelGGL((attn_valu<T, D>), grid, dim3(64), 0, s, k);
    return hipGetLastError();
  } else {
    const int G = r.hq / r.h_kv;
    const int brows = attn_rows_per_block(r.max_q_len, G);
    const int rblocks = (r.max_q_len * G + brows - 1) / brows;
    dim3 grid((unsigned)rblocks, (unsigned)(r.h_kv * k.splits), (unsigned)r.n_queries);
    switch (brows) {
      case 16: hipLaunchKernelGGL((attn_mfma<D, 1, 1>), grid, dim3(64), 0, s, k); break;
      case 32: hipLaunchKernelGGL((attn_mfma<D, 2, 1>), grid, dim3(128), 0, s, k); break;
      case 64: hipLaunchKernelGGL((attn_mfma<D, 4, 1>), grid, dim3(256), 0, s, k); break;
      case 128: hipLaunchKernelGGL((attn_mfma<D, 8, 1>), grid, dim3(512), 0, s, k); break;
      default: hipLaunchKernelGGL((attn_mfma<D, 8, 2>), grid, dim3(512), 0, s, k); break;
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

// Key splits per (query, kv head): enough workgroups in flight to keep the host link or HBM
// busy (about 64), bounded so the partial results stay small.
int attn_splits(int n_queries, int max_q_len, int hq, int h_kv) {
  const int G = hq / h_kv;
  const int rows = attn_rows_per_block(max_q_len, G);
  const int rblocks = (max_q_len * G + rows - 1) / rows;
  const long base = (long)n_queries * h_kv * (rblocks > 0 ? rblocks : 1);
  long s = (64 + base - 1) / base;
  if (s < 1) s = 1;
  if (s > 16) s = 16;
  return (int)s;
}

size_t attn_workspace_bytes(int dtype, int n_queries, int64_t total_q, int64_t total_kv,
                            int max_q_len, int hq, int h_kv, int d) {
  const size_t esz = dtype == 0 ? 4 : 2;
  size_t bytes = align256((size_t)total_q * hq * d * esz) + align256((size_t)total_kv * h_kv * d * esz);
  if (dtype == 1) {
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
  k.Qrot = ws;
  ws += align256((size_t)r.total_q * r.hq * r.d * esz);
  k.Krot = ws;
  ws += align256((size_t)r.total_kv * r.h_kv * r.d * esz);
  k.splits = r.dtype == 1 ? attn_splits(r.n_queries, r.max_q_len, r.hq, r.h_kv) : 1;
  if (k.splits > 1) {
    k.part_o = (float*)ws;
    ws += align256((size_t)k.splits * r.total_q * r.hq * r.d * 4);
    k.part_ml = (float*)ws;
  }
  if (r.dtype == 0) {
    switch (r.d) {
      case 32: return launch_attn_t<float, 32>(r, k, s);
      case 64: return launch_attn_t<float, 64>(r, k, s);
      default: return launch_attn_t<float, 128>(r, k, s);
    }
  }
  switch (r.d) {
    case 32: return launch_attn_t<bf16_t, 32>(r, k, s);
    case 64: return launch_attn_t<bf16_t, 64>(r, k, s);
    default: return launch_attn_t<bf16_t, 128>(r, k, s);
  }
}

}  // namespace msa
