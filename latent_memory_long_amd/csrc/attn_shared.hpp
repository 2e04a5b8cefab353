// Pieces shared by the sparse-attention forward (attn.hip) and backward (attn_bwd.hip):
// the kernel argument block, the global RoPE of the local context, the memory map of a
// query's selected documents and the key loop that stages 32-key tiles.
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

// ---- global RoPE of the local context --------------------------------------------------
// One rotation pair (x_i, x_{i+d/2}) by the angle with cosine c and sine s, with the
// roundings written out, so that every kernel that rotates gets the same bits.
__device__ __forceinline__ float rot_lo(float lo, float hi, float c, float s) { return fmaf(lo, c, -(hi * s)); }
__device__ __forceinline__ float rot_hi(float lo, float hi, float c, float s) { return fmaf(hi, c, lo * s); }

// cos and sin of p * theta_i for positions p < n_pos and pairs i < D/2, the angles in double
// precision (theta_i = base^(-2i/D)), rounded to float: cos at [p][i], sin at
// [n_pos + p][i].
template <int D>
__device__ __forceinline__ void rope_table_entry(float* tab, int64_t n_pos, float rope_base, int64_t e) {
  if (e >= n_pos * (D / 2)) return;
  const int64_t p = e / (D / 2);
  const int i = (int)(e % (D / 2));
  const double th = pow((double)rope_base, -2.0 * (double)i / (double)D);
  double sn, cs;
  sincos((double)p * th, &sn, &cs);
  tab[e] = (float)cs;
  tab[n_pos * (D / 2) + e] = (float)sn;
}
template <int D>
__global__ __launch_bounds__(256) void rope_table(float* tab, int64_t n_pos, float rope_base) {
  rope_table_entry<D>(tab, n_pos, rope_base, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}


// Elements d0 .. d0+7 of a bf16 row rotated to position pos with the rope_table values,
// as one bf16 MFMA operand: the lane also loads the pair partners (d +- D/2) of its 8
// elements.  The same roundings as rope_local (rot_lo / rot_hi), then one rounding to bf16.
template <int D>
__device__ __forceinline__ uint4 rope_load8(const bf16_t* row, int d0, int64_t pos, const float* tab, int64_t n_pos) {
  const bool low = d0 < D / 2;           // x_i (else x_{i+D/2})
  const int i0 = low ? d0 : d0 - D / 2;  // first pair index
  float x[8], y[8], o[8];
  Elem<bf16_t>::load8(row + d0, x);
  Elem<bf16_t>::load8(row + (low ? d0 + D / 2 : i0), y);
  const float* cp = tab + pos * (D / 2) + i0;
  const float* sp = cp + n_pos * (D / 2);
  const float4 c0 = *reinterpret_cast<const float4*>(cp), c1 = *reinterpret_cast<const float4*>(cp + 4);
  const float4 s0 = *reinterpret_cast<const float4*>(sp), s1 = *reinterpret_cast<const float4*>(sp + 4);
  const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = low ? rot_lo(x[j], y[j], c[j], sn[j]) : rot_hi(y[j], x[j], c[j], sn[j]);
  uint4 w;
  w.x = f32x2_to_bf16x2(o[0], o[1]);
  w.y = f32x2_to_bf16x2(o[2], o[3]);
  w.z = f32x2_to_bf16x2(o[4], o[5]);
  w.w = f32x2_to_bf16x2(o[6], o[7]);
  return w;
}
// Block blk of rope_local: RPW rows of Q (blk < nq_blocks) or of the local K.
template <typename T, int D>
__device__ __forceinline__ void rope_local_rows(const AttnK& a, int nq_blocks, int blk) {
  __shared__ float cs_tab[RPW][D / 2], sn_tab[RPW][D / 2];
  __shared__ int64_t row_pos[RPW];
  const bool is_q = blk < nq_blocks;
  const int64_t r0 = (int64_t)(is_q ? blk : blk - nq_blocks) * RPW;
  const int64_t total = is_q ? a.total_q : a.total_kv;
  const int heads = is_q ? a.hq : a.h_kv;
  const T* src = (const T*)(is_q ? a.Q : a.Kloc);
  T* dst = (T*)(is_q ? a.Qrot : a.Krot);
  const int32_t* off = is_q ? a.q_off : a.kv_off;
  const int tid = threadIdx.x;
  // Wave 0 finds each row's query and position: the 16 lanes of group rr = lane / 16 serve
  // row r0 + rr, and count the valid ids of its query in parallel (every workgroup has its
  // own rows to set up, so a serial walk over the k ids would hold all of them up).
  static_assert(RPW == 4, "one 16-lane group per row");
  if (tid < 64) {
    const int rr = tid >> 4, sl = tid & 15;
    const int64_t r = r0 + rr;
    int64_t pos = -1;
    int b = 0;
    if (r < total) {
      b = find_query(off, a.n_queries, r);
      const int32_t* ids = a.ids + (int64_t)b * a.k;
      int cnt = 0;
#pragma unroll 4
      for (int j = sl; j < a.k; j += 16) cnt += ids[j] >= 0;
      cnt += __shfl_xor(cnt, 1, 16);
      cnt += __shfl_xor(cnt, 2, 16);
      cnt += __shfl_xor(cnt, 4, 16);
      cnt += __shfl_xor(cnt, 8, 16);
      const int64_t Lq = a.q_off[b + 1] - a.q_off[b];
      const int64_t Lkv = a.kv_off[b + 1] - a.kv_off[b];
      pos = is_q ? cnt + (Lkv - Lq) + (r - off[b]) : cnt + (r - off[b]);
    }
    if (sl == 0) row_pos[rr] = pos;
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
template <typename T, int D>
__global__ __launch_bounds__(256) void rope_local(AttnK a, int nq_blocks) {
  rope_local_rows<T, D>(a, nq_blocks, blockIdx.x);
}

// The bf16 RoPE set-up in one launch: blocks below n_rot rotate rows as rope_local does
// (a.rtab must be null: they take their own angles, the same double-precision values the
// table holds), the others write the cos / sin table of a.n_pos positions into tab.
template <int D>
__global__ __launch_bounds__(256) void rope_prep(AttnK a, int nq_blocks, int n_rot, float* tab) {
  if ((int)blockIdx.x < n_rot) {  // uniform over the block
    rope_local_rows<bf16_t, D>(a, nq_blocks, blockIdx.x);
    return;
  }
  rope_table_entry<D>(tab, a.n_pos, a.rope_base, (int64_t)(blockIdx.x - n_rot) * blockDim.x + threadIdx.x);
}

// The bf16 RoPE set-up: the cos / sin table of k.n_pos positions into k.rtab, and the rows
// of nq_blocks blocks of Q and then of the local K rotated (n_rot blocks in all).  Few rows
// (a decode step, one short query): one rope_prep launch, whose row blocks take their own
// double-precision angles.  Many rows: the table first, then rope_local reading it, the same
// float values, so that the angles are evaluated once per position rather than once per row
// (the 4,617-row batch: 11.4 us in one launch for 22 MB of rows).
constexpr int ROPE_ONE_LAUNCH_BLOCKS = 64;
template <int D>
hipError_t launch_rope_setup(const AttnK& k, int nq_blocks, int n_rot, hipStream_t s) {
  const int tab_blocks = (int)((k.n_pos * (D / 2) + 255) / 256);
  if (n_rot <= ROPE_ONE_LAUNCH_BLOCKS) {
    AttnK kp = k;
    kp.rtab = nullptr;
    hipLaunchKernelGGL((rope_prep<D>), dim3((unsigned)(n_rot + tab_blocks)), dim3(256), 0, s, kp, nq_blocks, n_rot,
                       (float*)k.rtab);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((rope_table<D>), dim3((unsigned)tab_blocks), dim3(256), 0, s, (float*)k.rtab, k.n_pos,
                     k.rope_base);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((rope_local<bf16_t, D>), dim3((unsigned)n_rot), dim3(256), 0, s, k, nq_blocks);
  return hipGetLastError();
}

// Workgroup -> (kv pair, sub-block) of a 1-D grid of ceil(n_pairs / 8) * 8 * nsub
// workgroups.  Workgroups reach the eight XCDs round-robin in linear order; the nsub
// sub-blocks (row blocks, key splits) of one (query, kv head) pair are placed on one XCD
// back to back, so the selected K-bar / V-bar rows that all of them gather come from HBM
// once and from that XCD's L2 after.  False for the padding workgroups.
__device__ __forceinline__ bool place_pair(int n_pairs, int nsub, int& pair, int& sub) {
  const int L = (int)blockIdx.x;
  pair = (L >> 3) / nsub * 8 + (L & 7);
  sub = (L >> 3) % nsub;
  return pair < n_pairs;
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

// Key -> source of a query's keys [rows of the selected documents in rank order ; local
// rows], as tables in LDS for TCH consecutive keys of a workgroup's range (a chunk): the
// element offset of the key's row of kv head g from K-bar and from V-bar (a local row's
// offset reaches the rotated local K / the local V through the distance between the two
// allocations).  Two chunk slots alternate.  Lookups are branch-free (binary lifting over
// the document starts, keff <= 1024), so no control flow sits between the loads in flight.
constexpr int TCH = 16 * KT;

// 16 bytes as a native vector (a struct copy such as HIP's uint4 would go through memory)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int D, int THREADS>
__device__ __forceinline__ void build_key_chunk(int64_t* tk, int64_t* tv, int tid, int64_t key0,
                                                const int64_t* mstart, const int64_t* mpre, int keff, int64_t M,
                                                int kv0, const AttnK& a, int g) {
  // local K / V relative to K-bar / V-bar, in elements (all are 2-byte aligned)
  const int64_t dk = ((int64_t)(uintptr_t)a.Krot - (int64_t)(uintptr_t)a.Kbar) / 2;
  const int64_t dv = ((int64_t)(uintptr_t)a.Vloc - (int64_t)(uintptr_t)a.Vbar) / 2;
  for (int i = tid; i < TCH; i += THREADS) {
    const int64_t key = key0 + i;
    int lo = 0;  // largest rank t <= keff with mpre[t] <= key (mpre[keff] = M)
#pragma unroll
    for (int step = 1024; step > 0; step >>= 1) {
      const int t = min(lo + step, keff);
      lo = mpre[t] <= key ? t : lo;
    }
    const bool bank = lo < keff;
    const int64_t row = bank ? mstart[lo] + (key - mpre[lo]) : kv0 + (key - M);
    const int64_t off = (row * a.h_kv + g) * D;
    tk[i] = bank ? off : dk + off;
    tv[i] = bank ? off : dv + off;
  }
}

// The key loop of the attention kernels over keys [k_lo, k_lo + n_keys) of one (query, kv
// head): 32-key tiles of K (and V) gathered into a ring of RING register stages, RING tiles
// ahead of their use, written to the LDS buffers of their parity, then math(buf, rel) for
// each tile (rel: the tile's first key relative to k_lo; called by every wave).  One
// barrier per tile: a wave writes tile i's buffer only after every wave has passed tile
// i-1's barrier, hence finished tile i-2's math on that buffer.  The loads are
// unconditional -- keys past the range re-read its last key (V zeroed when the tile is
// written to LDS) -- and the ring runs in whole groups with no exit inside one, so the
// wait for the oldest tile can count the younger tiles' loads as still in flight.  The
// offset tables are rebuilt a chunk ahead: entering chunk c, chunk c+1 replaces chunk
// c-1, whose last lookup came before that tile's barrier.
template <int RING, int D, int THREADS, int KSTR, bool WITHV, typename F>
__device__ __forceinline__ void key_loop(const AttnK& a, int g, int tid, int64_t k_lo, int n_keys,
                                         const int64_t* mstart, const int64_t* mpre, int keff, int64_t M, int kv0,
                                         int64_t* tabk, int64_t* tabv, bf16_t* Ks0, bf16_t* Ks1, bf16_t* Vs0,
                                         bf16_t* Vs1, bf16_t* sink, F&& math) {
  static_assert(RING % 2 == 0, "tiles alternate between two LDS buffers");
  constexpr int UPR = D / 8;                                // 16-byte units per key row
  constexpr int UPK = (KT * UPR + THREADS - 1) / THREADS;  // units per thread per tile
  constexpr int NS = WITHV ? 2 * UPK : UPK;
  if (n_keys <= 0) return;  // uniform
  // this thread's units of a tile: key kr[j] of the tile, elements e0[j] .. + 7; units past
  // the tile go to a sink (no branch: one here would make the compiler drain the ring)
  int kr[UPK], e0[UPK], ko[UPK];
  bool unit[UPK];
#pragma unroll
  for (int j = 0; j < UPK; ++j) {
    const int u = min(tid + j * THREADS, KT * UPR - 1);  // threads past the tile repeat its last unit
    kr[j] = u / UPR;
    e0[j] = (u % UPR) * 8;
    ko[j] = kr[j] * KSTR + e0[j];
    unit[j] = (KT * UPR) % THREADS == 0 || tid + j * THREADS < KT * UPR;
  }
  const bf16_t* kb = (const bf16_t*)a.Kbar;
  const bf16_t* vb = (const bf16_t*)a.Vbar;
  auto fetch = [&](int rel, u32x4 (&st)[NS]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < UPK; ++j) {
      const int kc = min(rel + kr[j], n_keys - 1);
      const int e = kc & (2 * TCH - 1);  // chunk slot (kc / TCH) & 1, entry kc % TCH
      st[j] = *reinterpret_cast<const u32x4*>(kb + (tabk[e] + e0[j]));
      if (WITHV) st[UPK + j] = *reinterpret_cast<const u32x4*>(vb + (tabv[e] + e0[j]));
    }
  };
  build_key_chunk<D, THREADS>(tabk, tabv, tid, k_lo, mstart, mpre, keff, M, kv0, a, g);
  __syncthreads();
  u32x4 st[RING][NS];
#pragma unroll
  for (int r = 0; r < RING; ++r) fetch(r * KT, st[r]);
  // chunk 1 goes to the other slot; its first use comes many barriers later
  build_key_chunk<D, THREADS>(tabk + TCH, tabv + TCH, tid, k_lo + TCH, mstart, mpre, keff, M, kv0, a, g);
  for (int t0 = 0; t0 < n_keys; t0 += RING * KT) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      const int rel = t0 + r * KT;  // this tile's first key, relative to k_lo
      bf16_t* Kd = (r & 1) ? Ks1 : Ks0;
      bf16_t* Vd = (r & 1) ? Vs1 : Vs0;
#pragma unroll
      for (int j = 0; j < UPK; ++j) {
        *reinterpret_cast<u32x4*>(unit[j] ? Kd + ko[j] : sink) = st[r][j];
        if (WITHV) {  // V of keys past the range: zeros (probability 0 times V must stay 0)
          const uint32_t in = rel + kr[j] < n_keys ? ~0u : 0u;
          *reinterpret_cast<u32x4*>(unit[j] ? Vd + ko[j] : sink) = st[r][UPK + j] & in;
        }
      }
      __syncthreads();
      const int relf = rel + RING * KT;  // the tile fetched now
      fetch(relf, st[r]);
      if (relf % TCH == 0 && relf + TCH < n_keys) {  // uniform branch, LDS only
        const int slot = ((relf / TCH + 1) & 1) * TCH;
        build_key_chunk<D, THREADS>(tabk + slot, tabv + slot, tid, k_lo + relf + TCH, mstart, mpre, keff, M, kv0, a,
                                    g);
      }
      if (rel < n_keys) math(r & 1, rel);  // tiles past the range only skip the math
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
