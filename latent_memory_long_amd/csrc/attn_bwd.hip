// Backward of step D -- gradients of the sparse attention for training.
//
// yeyulingfeng.com "深度分析MSA ..." section 四 (training): the language-model loss reaches
// Q, K/V and the routing vectors through the selected memory; github-wiki.com project 250,
// section 6 item 1: the layer is differentiable end to end.  For L = sum(dO * O):
//   P = softmax(scale * Q~ K^T) (causal on the local keys), O = P V,
//   dV = P^T dO,  dP = dO V^T,  dS = P (dP - rowsum(dO O)),
//   dQ~ = scale dS K,  dK = scale dS^T Q~,
// with Q~ and the local K rotated at their global positions; the gradients of the
// un-rotated Q and local K are the rotated-domain gradients turned back by the same angles.
// Memory rows are the selected documents' bank rows, so their gradients are added into
// bank-shaped arrays (a row chosen by several queries collects every query's share).
//
// Kernels (bf16 inputs, float32 gradients, MFMA with float32 accumulation):
//  * rope_local (shared with the forward): rotated Q and local K into the workspace.
//  * bwd_dq: one workgroup per (query, kv head, block of query rows), like the forward.
//    Unless the forward's per-row log-sum-exp is passed in, a first pass over the key tiles
//    recomputes it; the second computes S^T = K Q~^T, P^T, dP^T = V dO^T and dS^T in
//    registers and accumulates dQ~^T = K^T dS^T, reading K^T straight from the row-major
//    key tile with gfx950's transposing LDS load.  It stores the rows' log-sum-exp and
//    rowsum(dO O) for bwd_dkv.
//  * bwd_dkv: workgroups over blocks of keys of a (query, kv head); each wave keeps one
//    16-key tile of K and V in registers and walks all query rows of the kv head in 32-row
//    stages (Q~ and dO staged in LDS one stage ahead through registers).  S = Q~ K^T leaves
//    every lane with probabilities of one key over 4 rows of each 16-row half, which are the
//    A operand of the 16x16x32 products dV += P^T dO and dK += dS^T Q~; their B operands are
//    read transposed from the row-major stage.
//  * rope_unrotate: turns dQ and the local dK back to the un-rotated inputs, in place.
#include <math.h>

#include "attn_shared.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace msa {
namespace {

struct BwdK {
  AttnK f;         // forward arguments; f.Qrot / f.Krot are the rotated copies
  const void* O;   // forward output [total_q, hq, D]
  const void* dO;  // [total_q, hq, D]
  float* dQ;       // [total_q, hq, D]
  float* dKl;      // [total_kv, h_kv, D]
  float* dVl;      // [total_kv, h_kv, D]
  float* dKb;      // [n_chunks, h_kv, D], accumulated
  float* dVb;      // [n_chunks, h_kv, D], accumulated
  float* lse;      // [total_q * hq]: log2 of sum_k 2^(s * scale_log2)
  float* drow;     // [total_q * hq]: rowsum(dO * O)
  const float* lse_in;  // optional: the forward's per-row log-sum-exp (natural log)
  float scale;     // softmax scale (natural)
  int kblocks;     // bwd_dkv workgroups per (query, kv head)
};

// ---- dQ and the row statistics -----------------------------------------------------
// K and V tiles are staged row-major (A operands of S^T and dP^T); dQ^T reads K transposed.

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32x2_to_bf16x2(lo, hi);
}

template <int D, int NW, int MTW>
__global__ __launch_bounds__(64 * NW) void bwd_dq(BwdK bk) {
  const AttnK& a = bk.f;
  constexpr int KK = D / 32;
  constexpr int MD = D / 16;
  constexpr int KSTR = D + 16;  // 32 bytes of padding: row and transposed reads are conflict-free
  constexpr int THREADS = 64 * NW;
  constexpr int UPT = 2 * tile_upk<D, THREADS>();
  constexpr int ROWS = NW * MTW * 16;
  __shared__ __align__(16) bf16_t Ks[2][KT * KSTR];
  __shared__ __align__(16) bf16_t Vs[2][KT * KSTR];
  __shared__ int64_t mstart[1025], mpre[1025];
  __shared__ int sh_keff;
  __shared__ int64_t sh_M;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int cl = lane & 15, g4 = lane >> 4;
  const int b = blockIdx.z, g = blockIdx.y;
  const int G = a.hq / a.h_kv;
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
  const int t_max = min(Lq - 1, (rb + ROWS - 1) / G);
  const int64_t k_hi = M + (int64_t)(Lkv - Lq + t_max + 1);
  const float sl2 = a.scale_log2;

  bool row_ok[MTW];
  int t_of[MTW], hq_of[MTW];
  int64_t key_lim[MTW];
  bf16x8_t Qf[MTW][KK], dOf[MTW][KK];
  float drow[MTW];
#pragma unroll
  for (int m = 0; m < MTW; ++m) {
    const int row = rb + (w * MTW + m) * 16 + cl;
    row_ok[m] = row < nrows;
    t_of[m] = row_ok[m] ? row / G : 0;
    hq_of[m] = g * G + (row_ok[m] ? row % G : 0);
    key_lim[m] = M + (int64_t)(Lkv - Lq + t_of[m]);
    const int64_t ro = ((int64_t)(q0 + t_of[m]) * a.hq + hq_of[m]) * D + g4 * 8;
    const bf16_t* qp = (const bf16_t*)a.Qrot + ro;
    const bf16_t* dp = (const bf16_t*)bk.dO + ro;
    const bf16_t* op = (const bf16_t*)bk.O + ro;
    float dsum = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint4 qv = make_uint4(0, 0, 0, 0), dv = qv, ov = qv;
      if (row_ok[m]) {
        qv = *reinterpret_cast<const uint4*>(qp + kk * 32);
        dv = *reinterpret_cast<const uint4*>(dp + kk * 32);
        ov = *reinterpret_cast<const uint4*>(op + kk * 32);
      }
      Qf[m][kk] = __builtin_bit_cast(bf16x8_t, qv);
      dOf[m][kk] = __builtin_bit_cast(bf16x8_t, dv);
      float x[8], y[8];
      unpack8(dv, x);
      unpack8(ov, y);
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum += x[e] * y[e];
    }
    dsum += __shfl_xor(dsum, 16);
    dsum += __shfl_xor(dsum, 32);
    drow[m] = dsum;
  }

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

  // the smallest causal limit over the block's rows (its first row's)
  const int64_t key_lim_min = M + (int64_t)(Lkv - Lq + rb / G);

  // S^T for row tile m and key tile kt from Ks: s[n][i] = logit (log2 units) of key
  // kt + n*16 + g4*4 + i for row cl, -inf where not visible.  A tile whose keys every row
  // of the block sees skips the masks.
  auto logits = [&](const bf16_t* ks, int m, int64_t kt, float (&s)[2][4]) __attribute__((always_inline)) {
    const bool full = kt + KT <= k_hi && kt + KT - 1 <= key_lim_min && rb + ROWS <= nrows;
    // limits relative to kt, clamped into int range: visible iff rel < hi_rel && rel <= lim_rel
    const int hi_rel = (int)(k_hi - kt < KT ? k_hi - kt : KT);
    const int64_t lr = key_lim[m] - kt;
    const int lim_rel = row_ok[m] ? (int)(lr < -1 ? -1 : (lr > KT ? KT : lr)) : -1;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint4 kw = *reinterpret_cast<const uint4*>(&ks[(n * 16 + cl) * KSTR + kk * 32 + g4 * 8]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kw), Qf[m][kk], acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rel = n * 16 + g4 * 4 + i;
        s[n][i] = (full || (rel < hi_rel && rel <= lim_rel)) ? acc[i] * sl2 : -INFINITY;
      }
    }
  };

  // ---- pass 1: log-sum-exp of every row (log2 units), unless the forward's is given ----
  float lse[MTW];
  if (bk.lse_in == nullptr) {
    float m_run[MTW], l_run[MTW];
#pragma unroll
    for (int m = 0; m < MTW; ++m) { m_run[m] = -INFINITY; l_run[m] = 0.f; }
    auto lse_math = [&](int buf, int64_t kt) __attribute__((always_inline)) {
#pragma unroll
      for (int m = 0; m < MTW; ++m) {
        float s[2][4];
        logits(Ks[buf], m, kt, s);
        float mx = -INFINITY;
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[n][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[m], mx);
        if (m_new != -INFINITY) {
          float ps = 0.f;
#pragma unroll
          for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) ps += exp2_hw(s[n][i] - m_new);
          l_run[m] = l_run[m] * exp2_hw(m_run[m] - m_new) + ps;
          m_run[m] = m_new;
        }
      }
    };
    tile_pipeline<(UPT <= 4 ? TILE_RING : 2), D, THREADS, UPT, KSTR, false>(ts, tid, 0, k_hi, Ks[0], Ks[1], Vs[0], Vs[1], lse_math);
#pragma unroll
    for (int m = 0; m < MTW; ++m) {
      float l = l_run[m] + __shfl_xor(l_run[m], 16);
      l += __shfl_xor(l, 32);
      lse[m] = (l > 0.f) ? m_run[m] + log2f(l) : INFINITY;  // a row with no visible key: P = 0
    }
    __syncthreads();  // the stage buffers are reused
  } else {
#pragma unroll
    for (int m = 0; m < MTW; ++m) {
      const float v = row_ok[m] ? bk.lse_in[(int64_t)(q0 + t_of[m]) * a.hq + hq_of[m]] : -INFINITY;
      lse[m] = v > -INFINITY ? v * LOG2E : INFINITY;
    }
  }
#pragma unroll
  for (int m = 0; m < MTW; ++m) {
    if (row_ok[m] && g4 == 0) {
      const int64_t orow = (int64_t)(q0 + t_of[m]) * a.hq + hq_of[m];
      bk.lse[orow] = lse[m];
      bk.drow[orow] = drow[m];
    }
  }

  // ---- pass 2: dQ~^T = K^T dS^T ----
  f32x4_t acc[MTW][MD];
#pragma unroll
  for (int m = 0; m < MTW; ++m)
#pragma unroll
    for (int md = 0; md < MD; ++md) acc[m][md] = {0.f, 0.f, 0.f, 0.f};
  auto dq_math = [&](int buf, int64_t kt) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < MTW; ++m) {
      float s[2][4];
      logits(Ks[buf], m, kt, s);
      float ds[2][4];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        f32x4_t dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const uint4 vw = *reinterpret_cast<const uint4*>(&Vs[buf][(n * 16 + cl) * KSTR + kk * 32 + g4 * 8]);
          dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vw), dOf[m][kk], dp, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = exp2_hw(s[n][i] - lse[m]);  // 0 where not visible (s = -inf)
          ds[n][i] = p * (dp[i] - drow[m]);
        }
      }
      // dS^T operand: k-slot g4*8 + j <-> key g4*4 + j (j < 4), 16 + g4*4 + (j-4) (j >= 4)
      uint4 pw;
      pw.x = pack_bf16x2(ds[0][0], ds[0][1]);
      pw.y = pack_bf16x2(ds[0][2], ds[0][3]);
      pw.z = pack_bf16x2(ds[1][0], ds[1][1]);
      pw.w = pack_bf16x2(ds[1][2], ds[1][3]);
      const bf16x8_t dSf = __builtin_bit_cast(bf16x8_t, pw);
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        // A operand K^T: element md*16 + cl over keys g4*4 .. +3 and 16 + g4*4 .. +3
        const bf16_t* kr = &Ks[buf][(g4 * 4 + (cl >> 2)) * KSTR + md * 16 + (cl & 3) * 4];
        const uint2 k0 = lds_read_tr16(kr);
        const uint2 k1 = lds_read_tr16(kr + 16 * KSTR);
        const bf16x8_t Kf = __builtin_bit_cast(bf16x8_t, make_uint4(k0.x, k0.y, k1.x, k1.y));
        acc[m][md] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Kf, dSf, acc[m][md], 0, 0, 0);
      }
    }
  };
  tile_pipeline<(UPT <= 4 ? TILE_RING : 2), D, THREADS, UPT, KSTR, true>(ts, tid, 0, k_hi, Ks[0], Ks[1], Vs[0], Vs[1], dq_math);

  // lane holds dQ~^T[d = md*16 + g4*4 + i][row cl]; natural-scale gradient = scale * acc
#pragma unroll
  for (int m = 0; m < MTW; ++m) {
    if (!row_ok[m]) continue;
    float* o = bk.dQ + ((int64_t)(q0 + t_of[m]) * a.hq + hq_of[m]) * D + g4 * 4;
#pragma unroll
    for (int md = 0; md < MD; ++md)
      *reinterpret_cast<float4*>(o + md * 16) = make_float4(acc[m][md][0] * bk.scale, acc[m][md][1] * bk.scale,
                                                           acc[m][md][2] * bk.scale, acc[m][md][3] * bk.scale);
  }
}

// ---- dK and dV --------------------------------------------------------------------------
constexpr int DKV_NW = 4;   // waves per workgroup
constexpr int DKV_NT = 1;   // 16-key tiles per wave
constexpr int DKV_RS = 32;  // query rows per LDS stage (two 16-row tiles)

template <int D>
__global__ __launch_bounds__(64 * DKV_NW) void bwd_dkv(BwdK bk) {
  const AttnK& a = bk.f;
  constexpr int KK = D / 32;
  constexpr int MD = D / 16;
  constexpr int STR = D + 16;  // bf16 per staged row: 32 bytes of padding keep the reads conflict-free
  constexpr int UPR = D / 8;   // 16-byte units per row
  constexpr int THREADS = 64 * DKV_NW;
  constexpr int UNITS = DKV_RS * UPR;  // 16-byte units per array per stage
  constexpr int UPT = (UNITS + THREADS - 1) / THREADS;
  constexpr int KEYS = DKV_NW * DKV_NT * 16;  // keys per workgroup round
  __shared__ __align__(16) bf16_t Qs[2][DKV_RS * STR], dOs[2][DKV_RS * STR];
  __shared__ __align__(16) float lse_s[2][DKV_RS], drow_s[2][DKV_RS];
  __shared__ int64_t mstart[1025], mpre[1025];
  __shared__ int sh_keff;
  __shared__ int64_t sh_M;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int cl = lane & 15, g4 = lane >> 4;
  const int b = blockIdx.z, g = blockIdx.y;
  const int G = a.hq / a.h_kv;
  const int q0 = a.q_off[b], Lq = a.q_off[b + 1] - q0;
  const int kv0 = a.kv_off[b], Lkv = a.kv_off[b + 1] - kv0;
  const int nrows = Lq * G;
  const int nst = (nrows + DKV_RS - 1) / DKV_RS;

  if (w == 0) {
    MemMap mm = build_memmap(a.ids + (int64_t)b * a.k, a.k, a.chunk_off, mstart, mpre);
    if (lane == 0) { sh_keff = mm.keff; sh_M = mm.M; }
  }
  __syncthreads();
  const int keff = sh_keff;
  const int64_t M = sh_M;
  const int64_t NK = M + Lkv;
  const int64_t nchunk = (NK + KEYS - 1) / KEYS;
  const int64_t c0 = nchunk * blockIdx.x / bk.kblocks, c1 = nchunk * (blockIdx.x + 1) / bk.kblocks;
  const float sl2 = a.scale_log2;
  const bf16_t* Kb = (const bf16_t*)a.Kbar;
  const bf16_t* Vb = (const bf16_t*)a.Vbar;
  const bf16_t* Kr = (const bf16_t*)a.Krot;
  const bf16_t* Vl = (const bf16_t*)a.Vloc;
  const bf16_t* Qg = (const bf16_t*)a.Qrot;
  const bf16_t* dOg = (const bf16_t*)bk.dO;

  // Stage `st` (query rows st*32 .. +31, row = t*G + j for token t and query head g*G + j)
  // is read into registers one stage ahead and written to LDS buffer st & 1.
  uint4 pq[UPT], pd[UPT];
  float pl = INFINITY, pr = 0.f;
  auto fetch = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = tid + j * THREADS;
      const int rr = u / UPR, e0 = (u % UPR) * 8;
      const int row = st * DKV_RS + rr;
      pq[j] = pd[j] = make_uint4(0, 0, 0, 0);
      if ((UNITS % THREADS == 0 || u < UNITS) && row < nrows) {
        const int64_t ro = ((int64_t)(q0 + row / G) * a.hq + g * G + row % G) * D + e0;
        pq[j] = *reinterpret_cast<const uint4*>(Qg + ro);
        pd[j] = *reinterpret_cast<const uint4*>(dOg + ro);
      }
    }
    if (tid < DKV_RS) {
      const int row = st * DKV_RS + tid;
      pl = INFINITY;  // rows past the end: P = 0
      pr = 0.f;
      if (row < nrows) {
        const int64_t orow = (int64_t)(q0 + row / G) * a.hq + g * G + row % G;
        pl = bk.lse[orow];
        pr = bk.drow[orow];
      }
    }
  };
  auto commit = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = tid + j * THREADS;
      const int rr = u / UPR, e0 = (u % UPR) * 8;
      if (UNITS % THREADS != 0 && u >= UNITS) break;
      *reinterpret_cast<uint4*>(&Qs[buf][rr * STR + e0]) = pq[j];
      *reinterpret_cast<uint4*>(&dOs[buf][rr * STR + e0]) = pd[j];
    }
    if (tid < DKV_RS) {
      lse_s[buf][tid] = pl;
      drow_s[buf][tid] = pr;
    }
  };

  for (int64_t c = c0; c < c1; ++c) {
    // this wave's keys: c*KEYS + (w*NT + nt)*16 + 0..15.  B operands of S = Q~ K^T and
    // dP = dO V^T: lane (cl, g4) holds key base + cl, elements kk*32 + g4*8 .. +8.
    bf16x8_t Kf[DKV_NT][KK], Vf[DKV_NT][KK];
    int rowmin[DKV_NT];  // key base + cl is visible to rows >= rowmin (causal on local keys)
#pragma unroll
    for (int nt = 0; nt < DKV_NT; ++nt) {
      const int64_t key = c * KEYS + (w * DKV_NT + nt) * 16 + cl;
      uint4 kz[KK], vz[KK];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kz[kk] = vz[kk] = make_uint4(0, 0, 0, 0);
      rowmin[nt] = 0;
      if (key < NK) {
        bool bank;
        int64_t row;
        const int64_t off = key_row(mstart, mpre, keff, M, key, kv0, a.h_kv, g, D, bank, row);
        const bf16_t* kp = (bank ? Kb : Kr) + off + g4 * 8;
        const bf16_t* vp = (bank ? Vb : Vl) + off + g4 * 8;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          kz[kk] = *reinterpret_cast<const uint4*>(kp + kk * 32);
          vz[kk] = *reinterpret_cast<const uint4*>(vp + kk * 32);
        }
        // local key i = key - M is visible to token t when i <= Lkv - Lq + t
        if (!bank) {
          const int64_t tmin = (key - M) - (Lkv - Lq);
          rowmin[nt] = tmin > 0 ? (int)tmin * G : 0;
        }
      }
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        Kf[nt][kk] = __builtin_bit_cast(bf16x8_t, kz[kk]);
        Vf[nt][kk] = __builtin_bit_cast(bf16x8_t, vz[kk]);
      }
    }
    f32x4_t dK[DKV_NT][MD], dV[DKV_NT][MD];
#pragma unroll
    for (int nt = 0; nt < DKV_NT; ++nt)
#pragma unroll
      for (int md = 0; md < MD; ++md) dK[nt][md] = dV[nt][md] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    if (nst > 0) fetch(0);
    for (int st = 0; st < nst; ++st) {
      const int buf = st & 1;
      commit(buf);
      __syncthreads();  // stage st is visible, and every wave is done with stage st-2 (this buffer)
      if (st + 1 < nst) fetch(st + 1);
      const bf16_t* qs = Qs[buf];
      const bf16_t* ds_ = dOs[buf];
      // P and dS of this wave's keys over the stage's 32 rows, packed as the A operands
      // (key cl, k-slot g4*8 + j) of the 16x16x32 products; k-slot g4*8 + j is row
      // g4*4 + j for j < 4 and 16 + g4*4 + (j - 4) for j >= 4.
      uint32_t pw[DKV_NT][4], sw[DKV_NT][4];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        f32x4_t sacc[DKV_NT], dpacc[DKV_NT];
#pragma unroll
        for (int nt = 0; nt < DKV_NT; ++nt) sacc[nt] = dpacc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const uint4 qa = *reinterpret_cast<const uint4*>(&qs[(sub * 16 + cl) * STR + kk * 32 + g4 * 8]);
          const uint4 da = *reinterpret_cast<const uint4*>(&ds_[(sub * 16 + cl) * STR + kk * 32 + g4 * 8]);
#pragma unroll
          for (int nt = 0; nt < DKV_NT; ++nt) {
            sacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa), Kf[nt][kk], sacc[nt], 0, 0, 0);
            dpacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, da), Vf[nt][kk], dpacc[nt], 0, 0, 0);
          }
        }
        // lane holds rows sub*16 + g4*4 + i of key cl
        const float4 L4 = *reinterpret_cast<const float4*>(&lse_s[buf][sub * 16 + g4 * 4]);
        const float4 R4 = *reinterpret_cast<const float4*>(&drow_s[buf][sub * 16 + g4 * 4]);
        const float Lr[4] = {L4.x, L4.y, L4.z, L4.w}, Rr[4] = {R4.x, R4.y, R4.z, R4.w};
        const int row0 = st * DKV_RS + sub * 16 + g4 * 4;
#pragma unroll
        for (int nt = 0; nt < DKV_NT; ++nt) {
          float p[4], dsv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[i] = row0 + i >= rowmin[nt] ? exp2_hw(fmaf(sacc[nt][i], sl2, -Lr[i])) : 0.f;
            dsv[i] = p[i] * (dpacc[nt][i] - Rr[i]);
          }
          pw[nt][sub * 2] = pack_bf16x2(p[0], p[1]);
          pw[nt][sub * 2 + 1] = pack_bf16x2(p[2], p[3]);
          sw[nt][sub * 2] = pack_bf16x2(dsv[0], dsv[1]);
          sw[nt][sub * 2 + 1] = pack_bf16x2(dsv[2], dsv[3]);
        }
      }
      // dV += P^T dO and dK += dS^T Q~: B operand (element md*16 + cl, k-slots g4*8 .. +8)
      // read transposed from the row-major stage, rows g4*4 .. +3 and 16 + g4*4 .. +3
      const int trow = g4 * 4 + (cl >> 2), tcol = (cl & 3) * 4;
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const uint2 d0 = lds_read_tr16(&ds_[trow * STR + md * 16 + tcol]);
        const uint2 d1 = lds_read_tr16(&ds_[(16 + trow) * STR + md * 16 + tcol]);
        const uint2 q0v = lds_read_tr16(&qs[trow * STR + md * 16 + tcol]);
        const uint2 q1v = lds_read_tr16(&qs[(16 + trow) * STR + md * 16 + tcol]);
        const bf16x8_t dOb = __builtin_bit_cast(bf16x8_t, make_uint4(d0.x, d0.y, d1.x, d1.y));
        const bf16x8_t Qb = __builtin_bit_cast(bf16x8_t, make_uint4(q0v.x, q0v.y, q1v.x, q1v.y));
#pragma unroll
        for (int nt = 0; nt < DKV_NT; ++nt) {
          const bf16x8_t Pa = __builtin_bit_cast(bf16x8_t, make_uint4(pw[nt][0], pw[nt][1], pw[nt][2], pw[nt][3]));
          const bf16x8_t Sa = __builtin_bit_cast(bf16x8_t, make_uint4(sw[nt][0], sw[nt][1], sw[nt][2], sw[nt][3]));
          dV[nt][md] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Pa, dOb, dV[nt][md], 0, 0, 0);
          dK[nt][md] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Sa, Qb, dK[nt][md], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // the stage buffers are free for the next round
    // lane holds dK / dV of key base + g4*4 + i at element md*16 + cl
#pragma unroll
    for (int nt = 0; nt < DKV_NT; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t key = c * KEYS + (w * DKV_NT + nt) * 16 + g4 * 4 + i;
        if (key >= NK) continue;
        bool bank;
        int64_t row;
        const int64_t off = key_row(mstart, mpre, keff, M, key, kv0, a.h_kv, g, D, bank, row) + cl;
#pragma unroll
        for (int md = 0; md < MD; ++md) {
          const float gk = dK[nt][md][i] * bk.scale, gv = dV[nt][md][i];
          if (bank) {
            atomicAdd(bk.dKb + off + md * 16, gk);
            atomicAdd(bk.dVb + off + md * 16, gv);
          } else {
            bk.dKl[off + md * 16] = gk;
            bk.dVl[off + md * 16] = gv;
          }
        }
      }
    }
  }
}

// ---- turning the gradients of the rotated Q and local K back, in place ---------------
template <int D>
__global__ __launch_bounds__(256) void rope_unrotate(AttnK a, float* dQ, float* dKl, int nq_blocks) {
  __shared__ float cs_tab[RPW][D / 2], sn_tab[RPW][D / 2];
  __shared__ int64_t row_pos[RPW];
  const bool is_q = blockIdx.x < (unsigned)nq_blocks;
  const int64_t r0 = (int64_t)(is_q ? blockIdx.x : blockIdx.x - nq_blocks) * RPW;
  const int64_t total = is_q ? a.total_q : a.total_kv;
  const int heads = is_q ? a.hq : a.h_kv;
  float* x = is_q ? dQ : dKl;
  const int32_t* off = is_q ? a.q_off : a.kv_off;
  const int tid = threadIdx.x;
  if (tid < RPW) {
    const int64_t r = r0 + tid;
    int64_t pos = -1;
    if (r < total) {
      const int b = find_query(off, a.n_queries, r);
      const int keff = count_valid_ids(a.ids + (int64_t)b * a.k, a.k);
      const int64_t Lq = a.q_off[b + 1] - a.q_off[b];
      const int64_t Lkv = a.kv_off[b + 1] - a.kv_off[b];
      pos = is_q ? keff + (Lkv - Lq) + (r - off[b]) : keff + (r - off[b]);
    }
    row_pos[tid] = pos;
  }
  __syncthreads();
  for (int e = tid; e < RPW * (D / 2); e += blockDim.x) {
    const int rr = e / (D / 2), i = e % (D / 2);
    const double th = pow((double)a.rope_base, -2.0 * (double)i / (double)D);
    double sn = 0.0, cs = 1.0;
    if (row_pos[rr] >= 0) sincos((double)row_pos[rr] * th, &sn, &cs);
    cs_tab[rr][i] = (float)cs;
    sn_tab[rr][i] = (float)sn;
  }
  __syncthreads();
  const int units = RPW * heads * (D / 8);
  for (int u = tid; u < units; u += blockDim.x) {
    const int rr = u / (heads * (D / 8));
    const int rem = u % (heads * (D / 8));
    const int h = rem / (D / 8), i0 = (rem % (D / 8)) * 4;
    const int64_t r = r0 + rr;
    if (r >= total) continue;
    float* p = x + (r * heads + h) * D;
    const float4 lo = *reinterpret_cast<const float4*>(p + i0);
    const float4 hi = *reinterpret_cast<const float4*>(p + i0 + D / 2);
    const float l[4] = {lo.x, lo.y, lo.z, lo.w}, hh[4] = {hi.x, hi.y, hi.z, hi.w};
    float ol[4], oh[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // rotation by the negative angle
      const float c = cs_tab[rr][i0 + q], s = sn_tab[rr][i0 + q];
      ol[q] = l[q] * c + hh[q] * s;
      oh[q] = hh[q] * c - l[q] * s;
    }
    *reinterpret_cast<float4*>(p + i0) = make_float4(ol[0], ol[1], ol[2], ol[3]);
    *reinterpret_cast<float4*>(p + i0 + D / 2) = make_float4(oh[0], oh[1], oh[2], oh[3]);
  }
}

template <int D>
hipError_t launch_bwd_t(const AttnBwdArgs& r, hipStream_t s) {
  const AttnArgs& f = r.f;
  BwdK k{};
  k.f.n_queries = f.n_queries;
  k.f.total_q = f.total_q;
  k.f.total_kv = f.total_kv;
  k.f.q_off = f.q_off;
  k.f.kv_off = f.kv_off;
  k.f.Q = f.Q;
  k.f.Kloc = f.Kloc;
  k.f.Vloc = f.Vloc;
  k.f.hq = f.hq;
  k.f.h_kv = f.h_kv;
  k.f.rope_base = f.rope_base;
  const float scale = f.scale > 0.f ? f.scale : 1.0f / sqrtf((float)D);
  k.f.scale_log2 = scale * LOG2E;
  k.f.k = f.k;
  k.f.ids = f.ids;
  k.f.chunk_off = f.chunk_off;
  k.f.Kbar = f.Kbar;
  k.f.Vbar = f.Vbar;
  char* ws = (char*)r.workspace;
  k.f.Qrot = ws;
  ws += align256((size_t)f.total_q * f.hq * D * 2);
  k.f.Krot = ws;
  ws += align256((size_t)f.total_kv * f.h_kv * D * 2);
  k.lse = (float*)ws;
  ws += align256((size_t)f.total_q * f.hq * 4);
  k.drow = (float*)ws;
  k.O = r.O;
  k.lse_in = r.lse;
  k.dO = r.dO;
  k.dQ = r.dQ;
  k.dKl = r.dKloc;
  k.dVl = r.dVloc;
  k.dKb = r.dKbar;
  k.dVb = r.dVbar;
  k.scale = scale;
  k.kblocks = 16;

  const int nq_blocks = (int)((f.total_q + RPW - 1) / RPW);
  const int nk_blocks = (int)((f.total_kv + RPW - 1) / RPW);
  if (nq_blocks + nk_blocks > 0)
    hipLaunchKernelGGL((rope_local<bf16_t, D>), dim3(nq_blocks + nk_blocks), dim3(256), 0, s, k.f, nq_blocks);
  const int G = f.hq / f.h_kv;
  const int rows = min(attn_rows_per_block(f.max_q_len, G), 128);
  const int rblocks = (f.max_q_len * G + rows - 1) / rows;
  if (rblocks > 0) {
    dim3 grid((unsigned)rblocks, (unsigned)f.h_kv, (unsigned)f.n_queries);
    switch (rows) {
      case 16: hipLaunchKernelGGL((bwd_dq<D, 1, 1>), grid, dim3(64), 0, s, k); break;
      case 32: hipLaunchKernelGGL((bwd_dq<D, 2, 1>), grid, dim3(128), 0, s, k); break;
      case 64: hipLaunchKernelGGL((bwd_dq<D, 4, 1>), grid, dim3(256), 0, s, k); break;
      default: hipLaunchKernelGGL((bwd_dq<D, 8, 1>), grid, dim3(512), 0, s, k); break;
    }
  }
  dim3 gkv((unsigned)k.kblocks, (unsigned)f.h_kv, (unsigned)f.n_queries);
  hipLaunchKernelGGL((bwd_dkv<D>), gkv, dim3(64 * DKV_NW), 0, s, k);
  if (nq_blocks + nk_blocks > 0)
    hipLaunchKernelGGL((rope_unrotate<D>), dim3(nq_blocks + nk_blocks), dim3(256), 0, s, k.f, r.dQ, r.dKloc,
                       nq_blocks);
  return hipGetLastError();
}

}  // namespace

size_t attn_bwd_workspace_bytes(int64_t total_q, int64_t total_kv, int hq, int h_kv, int d) {
  return align256((size_t)total_q * hq * d * 2) + align256((size_t)total_kv * h_kv * d * 2) +
         2 * align256((size_t)total_q * hq * 4);
}

hipError_t launch_sparse_attn_backward(const AttnBwdArgs& r, hipStream_t s) {
  return r.f.d == 64 ? launch_bwd_t<64>(r, s) : launch_bwd_t<128>(r, s);
}

}  // namespace msa
