// Pieces shared by the sparse-attention forward (attn.hip) and backward (attn_bwd.hip):
// the kernel argument block, the global RoPE of the local context, the memory map of a
// query's selected documents and the staging of 32-key tiles.
#pragma once

#include <math.h>

#include "common.hpp"

namespace msa {
namespace {

constexpr int RPW = 4;          // rows per workgroup in rope_local
constexpr int KT = 32;          // keys per tile

struct AttnK {
  int n_queries;
  int64_t total_q, total_kv;
  const int32_t *q_off, *kv_off;
  const void *Q, *Kloc, *Vloc;
  int hq, h_kv;
  float rope_base, scale_log2;
  int k;
  const int32_t* ids;
  const int64_t* chunk_off;
  const void *Kbar, *Vbar;
  void* O;
  void* Qrot;
  void* Krot;
  float* part_o;
  float* part_ml;
  int splits;
  float* lse;  // optional per-row log-sum-exp output (natural log)
  const float* rtab;  // rope_table of n_pos positions, or null (bf16 forward: Q is rotated in
                      // the attention kernel, local K by rope_local, both from this table)
  int64_t n_pos;
};

__device__ __forceinline__ int find_query(const int32_t* off, int n, int64_t row) {
  int lo = 0, hi = n;  // largest b with off[b] <= row
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= row) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ int count_valid_ids(const int32_t* ids, int k) {
  int n = 0;
  for (int r = 0; r < k; ++r) n += ids[r] >= 0;
  return n;
}

// ---- global RoPE of the local context --------------------------------------------------
// One rotation pair (x_i, x_{i+d/2}) by the angle with cosine c and sine s, with the
// roundings written out, so that every kernel that rotates gets the same bits.
__device__ __forceinline__ float rot_lo(float lo, float hi, float c, float s) { return fmaf(lo, c, -(hi * s)); }
__device__ __forceinline__ float rot_hi(float lo, float hi, float c, float s) { return fmaf(hi, c, lo * s); }

// cos and sin of p * theta_i for positions p < n_pos and pairs i < D/2, the angles in double
// precision (theta_i = base^(-2i/D)), rounded to float: cos at [p][i], sin at
// [n_pos + p][i].
template <int D>
__global__ __launch_bounds__(256) void rope_table(float* tab, int64_t n_pos, float rope_base) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n_pos * (D / 2)) return;
  const int64_t p = e / (D / 2);
  const int i = (int)(e % (D / 2));
  const double th = pow((double)rope_base, -2.0 * (double)i / (double)D);
  double sn, cs;
  sincos((double)p * th, &sn, &cs);
  tab[e] = (float)cs;
  tab[n_pos * (D / 2) + e] = (float)sn;
}
template <typename T, int D>
__global__ __launch_bounds__(256) void rope_local(AttnK a, int nq_blocks) {
  __shared__ float cs_tab[RPW][D / 2], sn_tab[RPW][D / 2];
  __shared__ int row_q[RPW];
  __shared__ int64_t row_pos[RPW];
  const bool is_q = blockIdx.x < (unsigned)nq_blocks;
  const int64_t r0 = (int64_t)(is_q ? blockIdx.x : blockIdx.x - nq_blocks) * RPW;
  const int64_t total = is_q ? a.total_q : a.total_kv;
  const int heads = is_q ? a.hq : a.h_kv;
  const T* src = (const T*)(is_q ? a.Q : a.Kloc);
  T* dst = (T*)(is_q ? a.Qrot : a.Krot);
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
      row_q[tid] = b;
    }
    row_pos[tid] = pos;
  }
  __syncthreads();
  for (int e = tid; e < RPW * (D / 2); e += blockDim.x) {
    const int rr = e / (D / 2), i = e % (D / 2);
    if (a.rtab != nullptr) {  // the values of rope_table, already computed
      const int64_t p = row_pos[rr] >= 0 ? row_pos[rr] : 0;
      cs_tab[rr][i] = a.rtab[p * (D / 2) + i];
      sn_tab[rr][i] = a.rtab[(a.n_pos + p) * (D / 2) + i];
      continue;
    }
    const double th = pow((double)a.rope_base, -2.0 * (double)i / (double)D);
    double sn = 0.0, cs = 1.0;
    if (row_pos[rr] >= 0) sincos((double)row_pos[rr] * th, &sn, &cs);
    cs_tab[rr][i] = (float)cs;
    sn_tab[rr][i] = (float)sn;
  }
  __syncthreads();
  const int units = RPW * heads * (D / 8);  // unit = 4 rotation pairs
  for (int u = tid; u < units; u += blockDim.x) {
    const int rr = u / (heads * (D / 8));
    const int rem = u % (heads * (D / 8));
    const int h = rem / (D / 8), i0 = (rem % (D / 8)) * 4;
    const int64_t r = r0 + rr;
    if (r >= total) continue;
    const T* p = src + (r * heads + h) * D;
    float lo[4], hi[4], o_lo[4], o_hi[4];
    Elem<T>::load4(p + i0, lo);
    Elem<T>::load4(p + i0 + D / 2, hi);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float c = cs_tab[rr][i0 + q], s = sn_tab[rr][i0 + q];
      o_lo[q] = rot_lo(lo[q], hi[q], c, s);
      o_hi[q] = rot_hi(lo[q], hi[q], c, s);
    }
    T* o = dst + (r * heads + h) * D;
    Elem<T>::store4(o + i0, o_lo);
    Elem<T>::store4(o + i0 + D / 2, o_hi);
  }
}

// Memory layout of one query: the selected documents' bank rows in rank order.
struct MemMap {
  int keff;
  int64_t M;
};

// Fills mstart[r] (first bank row of the r-th valid document) and mpre[r] (its first key
// index); mpre[keff] = M.  Runs on wave 0; k <= 1024.
__device__ __forceinline__ MemMap build_memmap(const int32_t* ids, int k, const int64_t* chunk_off,
                                               int64_t* mstart, int64_t* mpre) {
  const int lane = threadIdx.x & 63;
  int64_t run = 0;
  int keff = 0;
  for (int r0 = 0; r0 < k; r0 += 64) {
    const int r = r0 + lane;
    const int id = (r < k) ? ids[r] : -1;
    const bool ok = id >= 0;
    int64_t cnt = 0, st = 0;
    if (ok) { st = chunk_off[id]; cnt = chunk_off[id + 1] - st; }
    // exclusive scans of cnt and of ok over the wave
    int64_t x = cnt;
    int y = ok ? 1 : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t xo = __shfl_up(x, o);
      const int yo = __shfl_up(y, o);
      if (lane >= o) { x += xo; y += yo; }
    }
    if (ok) {
      const int slot = keff + y - 1;
      mstart[slot] = st;
      mpre[slot] = run + x - cnt;
    }
    run += __shfl(x, 63);
    keff += __shfl(y, 63);
  }
  if (lane == 0) mpre[keff] = run;
  return {keff, run};
}

// Staging of one 32-key tile, K and V row-major.  Key index -> source row: a bank row of
// the selected document of rank r (mpre[r] <= key < mpre[r+1]) while key < M, else local
// row key - M.
struct TileSrc {
  const bf16_t *Kb, *Vb, *Kr, *Vl;
  const int64_t *mstart, *mpre;
  int keff, hkv, g, kv0;
  int64_t M, k_hi;
};

// Source row of key `key` of a query; returns the row's element offset for kv head g and
// whether it is a bank row.
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

// 16-byte K units of a tile per thread; stage slot j < UPK holds K unit tid + j*THREADS,
// slot UPK + j the V unit of the same key and elements, so each key's row is located once.
template <int D, int THREADS>
constexpr int tile_upk() { return (KT * (D / 8) + THREADS - 1) / THREADS; }

template <int D, int THREADS, int UPT, bool WITHV>
__device__ __forceinline__ void tile_fetch(const TileSrc ts, int tid, int64_t kt, uint4 (&stage)[UPT]) {
  constexpr int UPR = D / 8;
  constexpr int UPK = tile_upk<D, THREADS>();
  static_assert(UPT >= (WITHV ? 2 : 1) * UPK, "stage too small");
#pragma unroll
  for (int j = 0; j < UPK; ++j) {
    const int u = tid + j * THREADS;
    uint4 kv = make_uint4(0, 0, 0, 0), vv = kv;
    if (u < KT * UPR) {
      const int kr = u / UPR, e0 = (u % UPR) * 8;
      const int64_t key = kt + kr;
      if (key < ts.k_hi) {
        bool bank;
        int64_t row;
        const int64_t off = key_row(ts.mstart, ts.mpre, ts.keff, ts.M, key, ts.kv0, ts.hkv, ts.g, D, bank, row) + e0;
        kv = *reinterpret_cast<const uint4*>((bank ? ts.Kb : ts.Kr) + off);
        if (WITHV) vv = *reinterpret_cast<const uint4*>((bank ? ts.Vb : ts.Vl) + off);
      }
    }
    stage[j] = kv;
    if (WITHV) stage[UPK + j] = vv;
  }
}

template <int D, int THREADS, int UPT, int KSTR, bool WITHV>
__device__ __forceinline__ void tile_commit(int tid, const uint4 (&stage)[UPT], bf16_t* Ks, bf16_t* Vs) {
  constexpr int UPR = D / 8;
  constexpr int UPK = tile_upk<D, THREADS>();
#pragma unroll
  for (int j = 0; j < UPK; ++j) {
    const int u = tid + j * THREADS;
    if (u < KT * UPR) {
      const int kr = u / UPR, e0 = (u % UPR) * 8;
      *reinterpret_cast<uint4*>(&Ks[kr * KSTR + e0]) = stage[j];
      if (WITHV) *reinterpret_cast<uint4*>(&Vs[kr * KSTR + e0]) = stage[UPK + j];
    }
  }
}

// The key loop of the attention kernels: tiles k_lo, k_lo + KT, ... below k_hi are gathered
// into a ring of RING register stages, RING tiles ahead of their use, and written to the LDS
// buffer of their parity just before their math (RING even: a tile's buffer alternates).
// One barrier per tile: a wave writes tile i's buffer only after every wave has passed tile
// i-1's barrier, hence finished tile i-2's math on that buffer.  (The barrier waits for the
// LDS traffic only; the gathers of the tiles ahead stay in flight across it.)
constexpr int TILE_RING = 4;

template <int RING, int D, int THREADS, int UPT, int KSTR, bool WITHV, typename F>
__device__ __forceinline__ void tile_pipeline(const TileSrc& ts, int tid, int64_t k_lo, int64_t k_hi,
                                              bf16_t* Ks0, bf16_t* Ks1, bf16_t* Vs0, bf16_t* Vs1, F&& math) {
  static_assert(RING % 2 == 0, "tiles alternate between two LDS buffers");
  uint4 st[RING][UPT];
#pragma unroll
  for (int r = 0; r < RING; ++r)
    if (k_lo + r * KT < k_hi) tile_fetch<D, THREADS, UPT, WITHV>(ts, tid, k_lo + r * KT, st[r]);
  for (int64_t k0 = k_lo; k0 < k_hi; k0 += RING * KT) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      const int64_t kt = k0 + r * KT;
      if (kt >= k_hi) break;  // uniform
      tile_commit<D, THREADS, UPT, KSTR, WITHV>(tid, st[r], (r & 1) ? Ks1 : Ks0, (r & 1) ? Vs1 : Vs0);
      __syncthreads();
      if (kt + RING * KT < k_hi) tile_fetch<D, THREADS, UPT, WITHV>(ts, tid, kt + RING * KT, st[r]);
      math(r & 1, kt);
    }
  }
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16 lanes, lane L
// names 4 consecutive 16-bit elements E[L][0..3]; lane i receives E[i/4 + 4j][i%4] for
// j = 0..3.  Pointing lane L at row r0 + L/4, column c0 + 4*(L%4) of a row-major tile thus
// hands lane i the column c0 + i over rows r0 .. r0+3: the k-contiguous operand of a
// product that sums over the tile's rows.
__device__ __forceinline__ uint2 lds_read_tr16(const bf16_t* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  return __builtin_bit_cast(uint2, v);
}

}  // namespace
}  // namespace msa
