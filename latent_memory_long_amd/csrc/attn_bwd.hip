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
//  * rope_table (shared with the forward): the cos / sin table of every position in use.
//  * bwd_prep: in one launch, Q and the local K rotated with the table into the workspace
//    (rope_local's blocks) and, in the other blocks, every row's rowsum(dO O) and its
//    log-sum-exp in log2 units (the row statistics, below).
//  * bwd_dq: one workgroup per (query, kv head, block of query rows), with the forward's key
//    loop (attn_shared.hpp's key_loop).
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
//  The gradients of the un-rotated Q and local K are turned back by the same angles in the
//  epilogues of bwd_dq and bwd_dkv, where each lane holds both elements of every rotation
//  pair it writes.
#include <math.h>

#include <mutex>

#include "attn_shared.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace msa {
namespace {

struct BwdK {
  AttnK f;         // forward arguments; f.Qrot / f.Krot are the rotated copies, f.rtab the cos / sin table
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
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq(BwdK bk, int nsub) {
  const AttnK& a = bk.f;
  constexpr int KK = D / 32;
  constexpr int MD = D / 16;
  constexpr int KSTR = D + 16;  // 32 bytes of padding: row and transposed reads are conflict-free
  constexpr int THREADS = 64 * NW;
  constexpr int UPK = (KT * (D / 8) + THREADS - 1) / THREADS;  // 16-byte units per thread per tile
  constexpr int RING = UPK == 1 ? 4 : 2;                       // tiles in flight
  constexpr int ROWS = NW * MTW * 16;
  __shared__ __align__(16) bf16_t Ks[2][KT * KSTR];
  __shared__ __align__(16) bf16_t Vs[2][KT * KSTR];
  __shared__ int64_t mstart[1025], mpre[1025];
  __shared__ int64_t tabk[2 * TCH], tabv[2 * TCH];
  __shared__ __align__(16) bf16_t sink[8];
  __shared__ int sh_keff;
  __shared__ int64_t sh_M;

  int pair, sub;
  if (!place_pair(a.n_queries * a.h_kv, nsub, pair, sub)) return;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int cl = lane & 15, g4 = lane >> 4;
  const int b = pair / a.h_kv, g = pair % a.h_kv;
  const int G = a.hq / a.h_kv;
  const int q0 = a.q_off[b], Lq = a.q_off[b + 1] - q0;
  const int kv0 = a.kv_off[b], Lkv = a.kv_off[b + 1] - kv0;
  const int nrows = Lq * G;
  const int rb = sub * ROWS;
  if (rb >= nrows) return;
  // this wave's rows: MTW 16-row tiles; a wave with none skips the math
  const bool wave_rows = rb + w * MTW * 16 < nrows;

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
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint4 qv = make_uint4(0, 0, 0, 0), dv = qv;
      if (row_ok[m]) {
        qv = *reinterpret_cast<const uint4*>(qp + kk * 32);
        dv = *reinterpret_cast<const uint4*>(dp + kk * 32);
      }
      Qf[m][kk] = __builtin_bit_cast(bf16x8_t, qv);
      dOf[m][kk] = __builtin_bit_cast(bf16x8_t, dv);
    }
    // rowsum(dO * O), from bwd_prep's row statistics
    drow[m] = row_ok[m] ? bk.drow[(int64_t)(q0 + t_of[m]) * a.hq + hq_of[m]] : 0.f;
  }


  // the smallest causal limit over the block's rows (its first row's)
  const int64_t key_lim_min = M + (int64_t)(Lkv - Lq + rb / G);

  // S^T of key tile kt for every row tile of the wave (each K operand read once for all):
  // s[m][n][i] = logit (log2 units) of key kt + n*16 + g4*4 + i for row cl of tile m, -inf
  // where not visible.  A tile whose keys every row of the block sees skips the masks.
  auto logits = [&](const bf16_t* ks, int kt, float (&s)[MTW][2][4]) __attribute__((always_inline)) {
    f32x4_t acc[MTW][2];
#pragma unroll
    for (int m = 0; m < MTW; ++m) acc[m][0] = acc[m][1] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const bf16x8_t kw =
            __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&ks[(n * 16 + cl) * KSTR + kk * 32 + g4 * 8]));
#pragma unroll
        for (int m = 0; m < MTW; ++m) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kw, Qf[m][kk], acc[m][n], 0, 0, 0);
      }
    const bool full = kt + KT <= k_hi && kt + KT - 1 <= key_lim_min && rb + ROWS <= nrows;
    // limits relative to kt, clamped into int range: visible iff rel < hi_rel && rel <= lim_rel
    const int hi_rel = (int)(k_hi - kt < KT ? k_hi - kt : KT);
#pragma unroll
    for (int m = 0; m < MTW; ++m) {
      const int64_t lr = key_lim[m] - kt;
      const int lim_rel = row_ok[m] ? (int)(lr < -1 ? -1 : (lr > KT ? KT : lr)) : -1;
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rel = n * 16 + g4 * 4 + i;
          s[m][n][i] = (full || (rel < hi_rel && rel <= lim_rel)) ? acc[m][n][i] * sl2 : -INFINITY;
        }
    }
  };

  // ---- pass 1: log-sum-exp of every row (log2 units), unless the forward's is given ----
  float lse[MTW];
  if (bk.lse_in == nullptr) {
    float m_run[MTW], l_run[MTW];
#pragma unroll
    for (int m = 0; m < MTW; ++m) { m_run[m] = -INFINITY; l_run[m] = 0.f; }
    auto lse_math = [&](int buf, int kt) __attribute__((always_inline)) {
      if (!wave_rows) return;
      float s[MTW][2][4];
      logits(Ks[buf], kt, s);
#pragma unroll
      for (int m = 0; m < MTW; ++m) {
        float mx = -INFINITY;
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[m][n][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[m], mx);
        if (m_new != -INFINITY) {
          float ps = 0.f;
#pragma unroll
          for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) ps += exp2_hw(s[m][n][i] - m_new);
          l_run[m] = l_run[m] * exp2_hw(m_run[m] - m_new) + ps;
          m_run[m] = m_new;
        }
      }
    };
    key_loop<RING, D, THREADS, KSTR, false>(a, g, tid, 0, (int)k_hi, mstart, mpre, keff, M, kv0, tabk, tabv, Ks[0],
                                            Ks[1], Vs[0], Vs[1], sink, lse_math);
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
  if (bk.lse_in == nullptr) {  // else bwd_prep has written the log2-unit copy for bwd_dkv
#pragma unroll
    for (int m = 0; m < MTW; ++m) {
      if (row_ok[m] && g4 == 0) bk.lse[(int64_t)(q0 + t_of[m]) * a.hq + hq_of[m]] = lse[m];
    }
  }

  // ---- pass 2: dQ~^T = K^T dS^T (K, V and K^T operands read once for all row tiles) ----
  f32x4_t acc[MTW][MD];
#pragma unroll
  for (int m = 0; m < MTW; ++m)
#pragma unroll
    for (int md = 0; md < MD; ++md) acc[m][md] = {0.f, 0.f, 0.f, 0.f};
  auto dq_math = [&](int buf, int kt) __attribute__((always_inline)) {
    if (!wave_rows) return;
    float s[MTW][2][4];
    logits(Ks[buf], kt, s);
    f32x4_t dp[MTW][2];
#pragma unroll
    for (int m = 0; m < MTW; ++m) dp[m][0] = dp[m][1] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const bf16x8_t vw =
            __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&Vs[buf][(n * 16 + cl) * KSTR + kk * 32 + g4 * 8]));
#pragma unroll
        for (int m = 0; m < MTW; ++m) dp[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vw, dOf[m][kk], dp[m][n], 0, 0, 0);
      }
    bf16x8_t dSf[MTW];
#pragma unroll
    for (int m = 0; m < MTW; ++m) {
      float ds[2][4];
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = exp2_hw(s[m][n][i] - lse[m]);  // 0 where not visible (s = -inf)
          ds[n][i] = p * (dp[m][n][i] - drow[m]);
        }
      // dS^T operand: k-slot g4*8 + j <-> key g4*4 + j (j < 4), 16 + g4*4 + (j-4) (j >= 4)
      uint4 pw;
      pw.x = pack_bf16x2(ds[0][0], ds[0][1]);
      pw.y = pack_bf16x2(ds[0][2], ds[0][3]);
      pw.z = pack_bf16x2(ds[1][0], ds[1][1]);
      pw.w = pack_bf16x2(ds[1][2], ds[1][3]);
      dSf[m] = __builtin_bit_cast(bf16x8_t, pw);
    }
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      // A operand K^T: element md*16 + cl over keys g4*4 .. +3 and 16 + g4*4 .. +3
      const bf16_t* kr = &Ks[buf][(g4 * 4 + (cl >> 2)) * KSTR + md * 16 + (cl & 3) * 4];
      const uint2 k0 = lds_read_tr16(kr);
      const uint2 k1 = lds_read_tr16(kr + 16 * KSTR);
      const bf16x8_t Kf = __builtin_bit_cast(bf16x8_t, make_uint4(k0.x, k0.y, k1.x, k1.y));
#pragma unroll
      for (int m = 0; m < MTW; ++m) acc[m][md] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Kf, dSf[m], acc[m][md], 0, 0, 0);
    }
  };
  key_loop<RING, D, THREADS, KSTR, true>(a, g, tid, 0, (int)k_hi, mstart, mpre, keff, M, kv0, tabk, tabv, Ks[0], Ks[1],
                                         Vs[0], Vs[1], sink, dq_math);

  // lane holds dQ~^T[d = md*16 + g4*4 + i][row cl] for every md, so both elements of each
  // rotation pair (d, d + D/2); the gradient of the un-rotated Q is the natural-scale
  // gradient scale * acc turned back by the row's angle
#pragma unroll
  for (int m = 0; m < MTW; ++m) {
    if (!row_ok[m]) continue;
    const int64_t pos = (int64_t)keff + (Lkv - Lq) + t_of[m];
    float* o = bk.dQ + ((int64_t)(q0 + t_of[m]) * a.hq + hq_of[m]) * D + g4 * 4;
#pragma unroll
    for (int md = 0; md < MD / 2; ++md) {
      const int i0 = md * 16 + g4 * 4;  // pair index of the lane's first element
      const float4 c4 = *reinterpret_cast<const float4*>(a.rtab + pos * (D / 2) + i0);
      const float4 s4 = *reinterpret_cast<const float4*>(a.rtab + (a.n_pos + pos) * (D / 2) + i0);
      const float c[4] = {c4.x, c4.y, c4.z, c4.w}, sn[4] = {s4.x, s4.y, s4.z, s4.w};
      float lo[4], hi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // rotation by the negative angle
        const float x = acc[m][md][i] * bk.scale, y = acc[m][md + MD / 2][i] * bk.scale;
        lo[i] = rot_lo(x, y, c[i], -sn[i]);
        hi[i] = rot_hi(x, y, c[i], -sn[i]);
      }
      *reinterpret_cast<float4*>(o + md * 16) = make_float4(lo[0], lo[1], lo[2], lo[3]);
      *reinterpret_cast<float4*>(o + (md + MD / 2) * 16) = make_float4(hi[0], hi[1], hi[2], hi[3]);
      // a compiler-only fence: the next pair group's table loads are not hoisted above it,
      // so their registers are taken only as the accumulators above are freed
      __asm__ volatile("" ::: "memory");
    }
  }
}

// ---- row statistics ahead of both gradient kernels ------------------------------------
// rowsum(dO * O) of every (token, query head) row and, when the forward's log-sum-exp is
// given, its copy in log2 units: after them bwd_dq and bwd_dkv depend on nothing of each
// other.  Block blk covers rows blk*64 .. +63.  Lane (cl, g4) of a wave sums elements kk*32 + g4*8 .. +7 of row cl, then the
// four lanes of the row are added (the order the values were first summed in).
template <int D>
__device__ __forceinline__ void bwd_rows_block(const BwdK& bk, int64_t n_rows, int64_t blk) {
  constexpr int KK = D / 32;
  const int lane = threadIdx.x & 63, cl = lane & 15, g4 = lane >> 4;
  const int64_t orow = (blk * 4 + (threadIdx.x >> 6)) * 16 + cl;
  const bool ok = orow < n_rows;
  const int64_t ro = (ok ? orow : 0) * D + g4 * 8;
  const bf16_t* dp = (const bf16_t*)bk.dO + ro;
  const bf16_t* op = (const bf16_t*)bk.O + ro;
  float dsum = 0.f;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    uint4 dv = make_uint4(0, 0, 0, 0), ov = dv;
    if (ok) {
      dv = *reinterpret_cast<const uint4*>(dp + kk * 32);
      ov = *reinterpret_cast<const uint4*>(op + kk * 32);
    }
    float x[8], y[8];
    unpack8(dv, x);
    unpack8(ov, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) dsum += x[e] * y[e];
  }
  dsum += __shfl_xor(dsum, 16);
  dsum += __shfl_xor(dsum, 32);
  if (ok && g4 == 0) {
    bk.drow[orow] = dsum;
    if (bk.lse_in != nullptr) {
      const float v = bk.lse_in[orow];
      bk.lse[orow] = v > -INFINITY ? v * LOG2E : INFINITY;
    }
  }
}

// The backward's set-up in one launch (the cos / sin table already written): blocks below
// n_rot rotate Q and the local K as rope_local does, the others compute the row statistics.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep(BwdK bk, int nq_blocks, int n_rot, int64_t n_rows) {
  if ((int)blockIdx.x < n_rot) {  // uniform over the block
    rope_local_rows<bf16_t, D>(bk.f, nq_blocks, blockIdx.x);
    return;
  }
  bwd_rows_block<D>(bk, n_rows, (int64_t)blockIdx.x - n_rot);
}

// A second stream per device, for running bwd_dkv beside bwd_dq: created once (default
// priority, non-blocking), with the two events that fork it from and join it to the
// caller's stream.  The fork / join sequence is enqueued under a lock, so that calls from
// several host threads do not interleave their uses of the events.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int MAX_DEVICES = 64;
SideStream g_side[MAX_DEVICES];
std::mutex g_side_mu;

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

  int pair, kblock;
  if (!place_pair(a.n_queries * a.h_kv, bk.kblocks, pair, kblock)) return;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int cl = lane & 15, g4 = lane >> 4;
  const int b = pair / a.h_kv, g = pair % a.h_kv;
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
  const int64_t c0 = nchunk * kblock / bk.kblocks, c1 = nchunk * (kblock + 1) / bk.kblocks;
  const float sl2 = a.scale_log2;
  const bf16_t* Kb = (const bf16_t*)a.Kbar;
  const bf16_t* Vb = (const bf16_t*)a.Vbar;
  const bf16_t* Kr = (const bf16_t*)a.Krot;
  const bf16_t* Vl = (const bf16_t*)a.Vloc;
  const bf16_t* Qg = (const bf16_t*)a.Qrot;
  const bf16_t* dOg = (const bf16_t*)bk.dO;

  // Stage `st` (query rows st*32 .. +31, row = t*G + j for token t and query head g*G + j)
  // is read into registers one stage ahead and written to LDS buffer st & 1.  A thread's
  // rows advance by DKV_RS from stage to stage, so their (t, j) = (row / G, row % G) are
  // stepped rather than divided out: fq / fr for the next stage, slot UPT for the row of
  // the log-sum-exp and rowsum(dO O) (threads below DKV_RS), reset for every key chunk.
  const int step_q = DKV_RS / G, step_r = DKV_RS % G;
  int fq0[UPT + 1], fr0[UPT + 1], fq[UPT + 1], fr[UPT + 1];
#pragma unroll
  for (int j = 0; j <= UPT; ++j) {
    const int rr = j < UPT ? (tid + j * THREADS) / UPR : tid;
    fq0[j] = rr / G;
    fr0[j] = rr % G;
  }
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
        const int64_t ro = (int64_t)((q0 + fq[j]) * a.hq + g * G + fr[j]) * D + e0;
        pq[j] = *reinterpret_cast<const uint4*>(Qg + ro);
        pd[j] = *reinterpret_cast<const uint4*>(dOg + ro);
      }
    }
    if (tid < DKV_RS) {
      const int row = st * DKV_RS + tid;
      pl = INFINITY;  // rows past the end: P = 0
      pr = 0.f;
      if (row < nrows) {
        const int64_t orow = (int64_t)(q0 + fq[UPT]) * a.hq + g * G + fr[UPT];
        pl = bk.lse[orow];
        pr = bk.drow[orow];
      }
    }
#pragma unroll
    for (int j = 0; j <= UPT; ++j) {
      fq[j] += step_q;
      fr[j] += step_r;
      if (fr[j] >= G) {
        fr[j] -= G;
        ++fq[j];
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

    // Stages before the one holding the chunk's first visible row are skipped: a local key i
    // is hidden from the rows of tokens below i - (Lkv - Lq), and the chunk's first key has
    // the smallest such bound (bank keys see every row).  The thread's row indices start
    // at that stage.
    int st_first = 0;
    {
      const int64_t tmin0 = (c * KEYS - M) - (Lkv - Lq);
      if (c * KEYS >= M && tmin0 > 0) st_first = (int)min((int64_t)nst, tmin0 * G / DKV_RS);
    }
#pragma unroll
    for (int j = 0; j <= UPT; ++j) {
      if (st_first == 0) {
        fq[j] = fq0[j];
        fr[j] = fr0[j];
      } else {
        const int rr = j < UPT ? (tid + j * THREADS) / UPR : tid;
        fq[j] = (st_first * DKV_RS + rr) / G;
        fr[j] = (st_first * DKV_RS + rr) % G;
      }
    }
    if (st_first < nst) fetch(st_first);
    for (int st = st_first; st < nst; ++st) {
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
          const int vis = rowmin[nt] - row0;  // element i is visible when i >= vis
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[i] = i >= vis ? exp2_hw(fmaf(sacc[nt][i], sl2, -Lr[i])) : 0.f;
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
        if (bank) {
#pragma unroll
          for (int md = 0; md < MD; ++md) {
            atomicAdd(bk.dKb + off + md * 16, dK[nt][md][i] * bk.scale);
            atomicAdd(bk.dVb + off + md * 16, dV[nt][md][i]);
          }
        } else {
          // a local key: the lane holds both elements of each rotation pair (md, md + MD/2);
          // the un-rotated gradient turns back by the key's angle (position keff + index)
          const int64_t pos = (int64_t)keff + (key - M);
#pragma unroll
          for (int md = 0; md < MD / 2; ++md) {
            const float c = a.rtab[pos * (D / 2) + md * 16 + cl];
            const float sn = a.rtab[(a.n_pos + pos) * (D / 2) + md * 16 + cl];
            const float x = dK[nt][md][i] * bk.scale, y = dK[nt][md + MD / 2][i] * bk.scale;
            bk.dKl[off + md * 16] = rot_lo(x, y, c, -sn);
            bk.dKl[off + (md + MD / 2) * 16] = rot_hi(x, y, c, -sn);
          }
#pragma unroll
          for (int md = 0; md < MD; ++md) bk.dVl[off + md * 16] = dV[nt][md][i];
        }
      }
    }
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
  // cos / sin of every position a row or local key can take (< k + total_kv)
  k.f.n_pos = (int64_t)f.k + f.total_kv;
  k.f.rtab = (const float*)ws;
  ws += align256((size_t)(1024 + f.total_kv) * D * 4);
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

  // Q and the local K rotated once per row, and the table written, in one launch: bwd_dkv
  // reads every query row once per key block, so rotating them in the kernels would repeat
  // the work many times
  {
    const int nq_blocks = (int)((f.total_q + RPW - 1) / RPW);
    const int nk_blocks = (int)((f.total_kv + RPW - 1) / RPW);
    const int64_t n_rows = f.total_q * f.hq;
    const int tab_blocks = (int)((k.f.n_pos * (D / 2) + 255) / 256);
    hipLaunchKernelGGL((rope_table<D>), dim3((unsigned)tab_blocks), dim3(256), 0, s, (float*)k.f.rtab, k.f.n_pos,
                       k.f.rope_base);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t blocks = nq_blocks + nk_blocks + (n_rows + 63) / 64;
    if (blocks > 0)
      hipLaunchKernelGGL((bwd_prep<D>), dim3((unsigned)blocks), dim3(256), 0, s, k, nq_blocks, nq_blocks + nk_blocks,
                         n_rows);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int G = f.hq / f.h_kv;
  const int rows = min(attn_rows_per_block(f.max_q_len, G), 128);
  const int rblocks = (f.max_q_len * G + rows - 1) / rows;
  const int n_pairs = f.n_queries * f.h_kv;
  auto launch_dq = [&](hipStream_t st) {
    if (rblocks <= 0) return;
    // the row blocks of a (query, kv head) on one XCD (place_pair); two 16-row tiles per
    // wave at 128 rows, so each K / V operand read serves both
    const dim3 grid((unsigned)(((n_pairs + 7) / 8) * 8 * rblocks));
    switch (rows) {
      case 16: hipLaunchKernelGGL((bwd_dq<D, 1, 1>), grid, dim3(64), 0, st, k, rblocks); break;
      case 32: hipLaunchKernelGGL((bwd_dq<D, 2, 1>), grid, dim3(128), 0, st, k, rblocks); break;
      case 64: hipLaunchKernelGGL((bwd_dq<D, 4, 1>), grid, dim3(256), 0, st, k, rblocks); break;
      default: hipLaunchKernelGGL((bwd_dq<D, 4, 2>), grid, dim3(256), 0, st, k, rblocks); break;
    }
  };
  auto launch_dkv = [&](hipStream_t st) {
    // the key blocks of a (query, kv head) on one XCD (place_pair): they all stream the
    // pair's query rows, which that XCD's L2 then holds
    const dim3 gkv((unsigned)(((n_pairs + 7) / 8) * 8 * k.kblocks));
    hipLaunchKernelGGL((bwd_dkv<D>), gkv, dim3(64 * DKV_NW), 0, st, k);
  };
  // With the forward's log-sum-exp the two gradient kernels are independent: bwd_dkv runs
  // on the side stream beside bwd_dq, whose workgroups then fill each other's idle issue
  // slots and tails.  Without it bwd_dq computes the log-sum-exp that bwd_dkv reads.
  int dev = -1;
  SideStream* side = nullptr;
  if (r.lse != nullptr && hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < MAX_DEVICES) side = &g_side[dev];
  if (side != nullptr) {
    std::lock_guard<std::mutex> lock(g_side_mu);
    // created outside any graph capture only (a first call under capture runs in order)
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (side->s == nullptr && hipStreamIsCapturing(s, &cap) == hipSuccess && cap == hipStreamCaptureStatusNone) {
      hipStream_t st;
      hipEvent_t e0, e1;
      if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) == hipSuccess) {
        if (hipEventCreateWithFlags(&e0, hipEventDisableTiming) == hipSuccess) {
          if (hipEventCreateWithFlags(&e1, hipEventDisableTiming) == hipSuccess) {
            side->s = st;
            side->fork = e0;
            side->join = e1;
          } else {
            (void)hipEventDestroy(e0);
            (void)hipStreamDestroy(st);
          }
        } else {
          (void)hipStreamDestroy(st);
        }
      }
      (void)hipGetLastError();
    }
    if (side->s != nullptr) {
      hipError_t e = hipEventRecord(side->fork, s);
      if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
      if (e != hipSuccess) return e;
      launch_dkv(side->s);
      launch_dq(s);
      e = hipEventRecord(side->join, side->s);
      if (e == hipSuccess) e = hipStreamWaitEvent(s, side->join, 0);
      if (e != hipSuccess) return e;
      return hipGetLastError();
    }
  }
  launch_dq(s);
  launch_dkv(s);
  return hipGetLastError();
}

}  // namespace

size_t attn_bwd_workspace_bytes(int64_t total_q, int64_t total_kv, int hq, int h_kv, int d) {
  // rotated Q and local K, the cos / sin table (k <= 1024), per-row log-sum-exp and rowsum(dO O)
  return align256((size_t)total_q * hq * d * 2) + align256((size_t)total_kv * h_kv * d * 2) +
         align256((size_t)(1024 + total_kv) * d * 4) + 2 * align256((size_t)total_q * hq * 4);
}

hipError_t launch_sparse_attn_backward(const AttnBwdArgs& r, hipStream_t s) {
  return r.f.d == 64 ? launch_bwd_t<64>(r, s) : launch_bwd_t<128>(r, s);
}

}  // namespace msa
