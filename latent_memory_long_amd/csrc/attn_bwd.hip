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
//  * bwd_dq: one workgroup per (query, kv head, block of query rows), like the forward.  A
//    first pass over the key tiles recomputes each row's log-sum-exp; a second computes
//    S^T = K Q~^T, P^T, dP^T = V dO^T and dS^T in registers and accumulates
//    dQ~^T = K^T dS^T.  It stores the rows' log-sum-exp and rowsum(dO O) for bwd_dkv.
//  * bwd_dkv: workgroups over blocks of keys of a (query, kv head); each wave owns a
//    16-key tile and walks all query rows of the kv head in 16-row tiles staged in LDS.
//    S = Q~ K^T leaves every lane with 4 probabilities of one key, which are exactly the
//    A operand of the 16x16x16 products dV += P^T dO and dK += dS^T Q~, so nothing is
//    transposed in registers.
//  * rope_unrotate: turns dQ and the local dK back to the un-rotated inputs, in place.
#include <math.h>

#include "attn_shared.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace msa {
namespace {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

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
  float scale;     // softmax scale (natural)
  int kblocks;     // bwd_dkv workgroups per (query, kv head)
};

// Source row of key `key` of a query: a bank row of the document of rank r (mpre[r] <=
// key < mpre[r+1]) while key < M, else local row key - M.  Returns the row's element
// offset for kv head g and whether it is a bank row.
__device__ __forceinline__ int64_t key_row(const int64_t* mstart, const int64_t* mpre, int keff, int64_t M,
                                           int64_t key, int kv0, int hkv, int g, int D, bool& bank,
                                           int64_t& row) {
  if (key < M) {
    int lo = 0, hi = keff;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (mpre[mid] <= key) lo = mid; else hi = mid;
    }
    row = mstart[lo] + (key - mpre[lo]);
    bank = true;
  } else {
    row = kv0 + (key - M);
    bank = false;
  }
  return (row * hkv + g) * D;
}

// ---- dQ and the row statistics -----------------------------------------------------
// Tile staging: K row-major (A of S^T), K transposed (A of dQ^T), V row-major (A of dP^T).
template <int D, int THREADS, int UPT, bool WITHV>
__device__ __forceinline__ void bwd_fetch(const TileSrc ts, int tid, int64_t kt, uint4 (&stage)[UPT]) {
  constexpr int UPR = D / 8;
  constexpr int UNITS = (WITHV ? 2 : 1) * KT * UPR;
#pragma unroll
  for (int j = 0; j < UPT; ++j) {
    const int u = tid + j * THREADS;
    uint4 wv = make_uint4(0, 0, 0, 0);
    if (u < UNITS) {
      const bool isv = u >= KT * UPR;
      const int uu = isv ? u - KT * UPR : u;
      const int kr = uu / UPR, e0 = (uu % UPR) * 8;
      const int64_t key = kt + kr;
      if (key < ts.k_hi) {
        bool bank;
        int64_t row;
        const int64_t off = key_row(ts.mstart, ts.mpre, ts.keff, ts.M, key, ts.kv0, ts.hkv, ts.g, D, bank, row);
        const bf16_t* p = bank ? (isv ? ts.Vb : ts.Kb) : (isv ? ts.Vl : ts.Kr);
        wv = *reinterpret_cast<const uint4*>(p + off + e0);
      }
    }
    stage[j] = wv;
  }
}

template <int D, int THREADS, int UPT, int KSTR, int TSTR, bool WITHV>
__device__ __forceinline__ void bwd_commit(int tid, const uint4 (&stage)[UPT], bf16_t* Ks, bf16_t* Kt, bf16_t* Vs) {
  constexpr int UPR = D / 8;
  constexpr int UNITS = (WITHV ? 2 : 1) * KT * UPR;
#pragma unroll
  for (int j = 0; j < UPT; ++j) {
    const int u = tid + j * THREADS;
    if (u < UNITS) {
      const bool isv = u >= KT * UPR;
      const int uu = isv ? u - KT * UPR : u;
      const int kr = uu / UPR, e0 = (uu % UPR) * 8;
      if (isv) {
        *reinterpret_cast<uint4*>(&Vs[kr * KSTR + e0]) = stage[j];
      } else {
        *reinterpret_cast<uint4*>(&Ks[kr * KSTR + e0]) = stage[j];
        if (WITHV) {
          const uint32_t w[4] = {stage[j].x, stage[j].y, stage[j].z, stage[j].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            Kt[(e0 + 2 * q) * TSTR + kr] = (bf16_t)(w[q] & 0xffffu);
            Kt[(e0 + 2 * q + 1) * TSTR + kr] = (bf16_t)(w[q] >> 16);
          }
        }
      }
    }
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32x2_to_bf16x2(lo, hi);
}

template <int D, int NW, int MTW>
__global__ __launch_bounds__(64 * NW) void bwd_dq(BwdK bk) {
  const AttnK& a = bk.f;
  constexpr int KK = D / 32;
  constexpr int MD = D / 16;
  constexpr int KSTR = D + 8;
  constexpr int TSTR = KT + 8;
  constexpr int THREADS = 64 * NW;
  constexpr int UPT = (2 * KT * (D / 8) + THREADS - 1) / THREADS;
  constexpr int ROWS = NW * MTW * 16;
  __shared__ __align__(16) bf16_t Ks[2][KT * KSTR];
  __shared__ __align__(16) bf16_t Vs[2][KT * KSTR];
  __shared__ __align__(16) bf16_t Kt[2][D * TSTR];
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
  uint4 stage[UPT];

  // S^T for row tile m and key tile kt from Ks: s[n][i] = logit (log2 units) of key
  // kt + n*16 + g4*4 + i for row cl, -inf where not visible
  auto logits = [&](const bf16_t* ks, int m, int64_t kt, float (&s)[2][4]) __attribute__((always_inline)) {
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
        const int64_t key = kt + n * 16 + g4 * 4 + i;
        s[n][i] = (row_ok[m] && key < k_hi && key <= key_lim[m]) ? acc[i] * sl2 : -INFINITY;
      }
    }
  };

  // ---- pass 1: log-sum-exp of every row ----
  float m_run[MTW], l_run[MTW];
#pragma unroll
  for (int m = 0; m < MTW; ++m) { m_run[m] = -INFINITY; l_run[m] = 0.f; }
  if (0 < k_hi) bwd_fetch<D, THREADS, UPT, false>(ts, tid, 0, stage);
  int it = 0;
  for (int64_t kt = 0; kt < k_hi; kt += KT, ++it) {
    const int buf = it & 1;
    bwd_commit<D, THREADS, UPT, KSTR, TSTR, false>(tid, stage, Ks[buf], Kt[buf], Vs[buf]);
    __syncthreads();
    if (kt + KT < k_hi) bwd_fetch<D, THREADS, UPT, false>(ts, tid, kt + KT, stage);
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
          for (int i = 0; i < 4; ++i) ps += exp2f(s[n][i] - m_new);
        l_run[m] = l_run[m] * exp2f(m_run[m] - m_new) + ps;
        m_run[m] = m_new;
      }
    }
  }
  float lse[MTW];
#pragma unroll
  for (int m = 0; m < MTW; ++m) {
    float l = l_run[m] + __shfl_xor(l_run[m], 16);
    l += __shfl_xor(l, 32);
    lse[m] = (l > 0.f) ? m_run[m] + log2f(l) : INFINITY;  // a row with no visible key: P = 0
    if (row_ok[m] && g4 == 0) {
      const int64_t orow = (int64_t)(q0 + t_of[m]) * a.hq + hq_of[m];
      bk.lse[orow] = lse[m];
      bk.drow[orow] = drow[m];
    }
  }
  __syncthreads();  // the stage buffers are reused

  // ---- pass 2: dQ~^T = K^T dS^T ----
  f32x4_t acc[MTW][MD];
#pragma unroll
  for (int m = 0; m < MTW; ++m)
#pragma unroll
    for (int md = 0; md < MD; ++md) acc[m][md] = {0.f, 0.f, 0.f, 0.f};
  if (0 < k_hi) bwd_fetch<D, THREADS, UPT, true>(ts, tid, 0, stage);
  it = 0;
  for (int64_t kt = 0; kt < k_hi; kt += KT, ++it) {
    const int buf = it & 1;
    bwd_commit<D, THREADS, UPT, KSTR, TSTR, true>(tid, stage, Ks[buf], Kt[buf], Vs[buf]);
    __syncthreads();
    if (kt + KT < k_hi) bwd_fetch<D, THREADS, UPT, true>(ts, tid, kt + KT, stage);
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
          const float p = exp2f(s[n][i] - lse[m]);  // 0 where not visible (s = -inf)
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
        const bf16_t* kr = &Kt[buf][(md * 16 + cl) * TSTR];
        const uint2 k0 = *reinterpret_cast<const uint2*>(kr + g4 * 4);
        const uint2 k1 = *reinterpret_cast<const uint2*>(kr + 16 + g4 * 4);
        const bf16x8_t Kf = __builtin_bit_cast(bf16x8_t, make_uint4(k0.x, k0.y, k1.x, k1.y));
        acc[m][md] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Kf, dSf, acc[m][md], 0, 0, 0);
      }
    }
  }

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
constexpr int DKV_NW = 4;  // waves per workgroup, one 16-key tile each per round

template <int D>
__global__ __launch_bounds__(64 * DKV_NW) void bwd_dkv(BwdK bk) {
  const AttnK& a = bk.f;
  constexpr int KK = D / 32;
  constexpr int MD = D / 16;
  constexpr int QSTR = D + 8;   // bf16 per staged row (row-major)
  constexpr int RSTR = 16 + 8;  // bf16 per staged column (transposed)
  __shared__ __align__(16) bf16_t Qs[16 * QSTR], dOs[16 * QSTR];
  __shared__ __align__(16) bf16_t Qt[D * RSTR], dOt[D * RSTR];
  __shared__ float lse_s[16], drow_s[16];
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
  const int nrt = (nrows + 15) / 16;

  if (w == 0) {
    MemMap mm = build_memmap(a.ids + (int64_t)b * a.k, a.k, a.chunk_off, mstart, mpre);
    if (lane == 0) { sh_keff = mm.keff; sh_M = mm.M; }
  }
  __syncthreads();
  const int keff = sh_keff;
  const int64_t M = sh_M;
  const int64_t NK = M + Lkv;
  const int64_t ntile = (NK + 15) / 16;
  const int64_t tile0 = ntile * blockIdx.x / bk.kblocks, tile1 = ntile * (blockIdx.x + 1) / bk.kblocks;
  const float sl2 = a.scale_log2;
  const bf16_t* Kb = (const bf16_t*)a.Kbar;
  const bf16_t* Vb = (const bf16_t*)a.Vbar;
  const bf16_t* Kr = (const bf16_t*)a.Krot;
  const bf16_t* Vl = (const bf16_t*)a.Vloc;

  for (int64_t r0 = tile0; r0 < tile1; r0 += DKV_NW) {
    const int64_t tile = r0 + w;  // this wave's key tile in this round
    const bool active = tile < tile1;
    // B operands of S = Q~ K^T and dP = dO V^T: lane (cl, g4) holds key tile*16 + cl,
    // elements kk*32 + g4*8 .. + 8
    bf16x8_t Kf[KK], Vf[KK];
    const int64_t mykey = tile * 16 + cl;
    bool mybank = false;
    int64_t myrow = 0;
    {
      uint4 kz[KK], vz[KK];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kz[kk] = vz[kk] = make_uint4(0, 0, 0, 0);
      if (active && mykey < NK) {
        const int64_t off = key_row(mstart, mpre, keff, M, mykey, kv0, a.h_kv, g, D, mybank, myrow);
        const bf16_t* kp = (mybank ? Kb : Kr) + off + g4 * 8;
        const bf16_t* vp = (mybank ? Vb : Vl) + off + g4 * 8;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          kz[kk] = *reinterpret_cast<const uint4*>(kp + kk * 32);
          vz[kk] = *reinterpret_cast<const uint4*>(vp + kk * 32);
        }
      }
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        Kf[kk] = __builtin_bit_cast(bf16x8_t, kz[kk]);
        Vf[kk] = __builtin_bit_cast(bf16x8_t, vz[kk]);
      }
    }
    f32x4_t dK[MD], dV[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) dK[md] = dV[md] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // the local index past which this tile's keys are invisible to row t: key - M <= Lkv - Lq + t
    for (int rt = 0; rt < nrt; ++rt) {
      __syncthreads();  // the previous row tile's readers are done
      // stage rows rt*16 .. +15 (row = t * G + j: token t, query head g*G + j)
      for (int u = tid; u < 16 * (D / 8); u += 64 * DKV_NW) {
        const int rr = u / (D / 8), e0 = (u % (D / 8)) * 8;
        const int row = rt * 16 + rr;
        uint4 qv = make_uint4(0, 0, 0, 0), dv = qv;
        if (row < nrows) {
          const int64_t ro = ((int64_t)(q0 + row / G) * a.hq + g * G + row % G) * D + e0;
          qv = *reinterpret_cast<const uint4*>((const bf16_t*)a.Qrot + ro);
          dv = *reinterpret_cast<const uint4*>((const bf16_t*)bk.dO + ro);
        }
        *reinterpret_cast<uint4*>(&Qs[rr * QSTR + e0]) = qv;
        *reinterpret_cast<uint4*>(&dOs[rr * QSTR + e0]) = dv;
        const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w}, dw[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          Qt[(e0 + 2 * q) * RSTR + rr] = (bf16_t)(qw[q] & 0xffffu);
          Qt[(e0 + 2 * q + 1) * RSTR + rr] = (bf16_t)(qw[q] >> 16);
          dOt[(e0 + 2 * q) * RSTR + rr] = (bf16_t)(dw[q] & 0xffffu);
          dOt[(e0 + 2 * q + 1) * RSTR + rr] = (bf16_t)(dw[q] >> 16);
        }
      }
      if (tid < 16) {
        const int row = rt * 16 + tid;
        float l = INFINITY, d = 0.f;
        if (row < nrows) {
          const int64_t orow = (int64_t)(q0 + row / G) * a.hq + g * G + row % G;
          l = bk.lse[orow];
          d = bk.drow[orow];
        }
        lse_s[tid] = l;
        drow_s[tid] = d;
      }
      __syncthreads();
      if (!active) continue;
      // S = Q~ K^T and dP = dO V^T: lane holds rows g4*4 + i of key cl
      f32x4_t s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint4 qw = *reinterpret_cast<const uint4*>(&Qs[cl * QSTR + kk * 32 + g4 * 8]);
        const uint4 dw = *reinterpret_cast<const uint4*>(&dOs[cl * QSTR + kk * 32 + g4 * 8]);
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qw), Kf[kk], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, dw), Vf[kk], dp, 0, 0, 0);
      }
      float p[4], ds[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = g4 * 4 + i;
        const int row = rt * 16 + rr;
        const int t = row / G;
        const bool vis = row < nrows && mykey < NK && (mykey < M || mykey - M <= (int64_t)(Lkv - Lq + t));
        p[i] = vis ? exp2f(s[i] * sl2 - lse_s[rr]) : 0.f;
        ds[i] = p[i] * (dp[i] - drow_s[rr]);
      }
      // A operands: P^T and dS^T of this lane's key cl over rows g4*4 .. +3
      const bf16x4_t Pa = __builtin_bit_cast(bf16x4_t, make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])));
      const bf16x4_t Sa = __builtin_bit_cast(bf16x4_t, make_uint2(pack_bf16x2(ds[0], ds[1]), pack_bf16x2(ds[2], ds[3])));
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        // B operands: dO and Q~ at element md*16 + cl over rows g4*4 .. +3
        const bf16x4_t dOb = __builtin_bit_cast(bf16x4_t, *reinterpret_cast<const uint2*>(&dOt[(md * 16 + cl) * RSTR + g4 * 4]));
        const bf16x4_t Qb = __builtin_bit_cast(bf16x4_t, *reinterpret_cast<const uint2*>(&Qt[(md * 16 + cl) * RSTR + g4 * 4]));
        dV[md] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(Pa, dOb, dV[md], 0, 0, 0);
        dK[md] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(Sa, Qb, dK[md], 0, 0, 0);
      }
    }
    if (!active) continue;
    // lane holds dK / dV of key tile*16 + g4*4 + i at element md*16 + cl
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t key = tile * 16 + g4 * 4 + i;
      if (key >= NK) continue;
      bool bank;
      int64_t row;
      const int64_t off = key_row(mstart, mpre, keff, M, key, kv0, a.h_kv, g, D, bank, row) + cl;
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const float gk = dK[md][i] * bk.scale, gv = dV[md][i];
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
  k.f.scale_log2 = scale * 1.4426950408889634f;
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
