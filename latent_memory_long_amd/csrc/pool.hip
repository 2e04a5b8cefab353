// Step A -- offline memory encoding: document-wise RoPE + chunk-mean pooling.
//
// hysenlabs.com "EverMind-AI/MSA: routing top-k compressed documents inside attention ...",
// sections "Memory must be encoded offline before a query can reach it" (one pass over the
// corpus caches chunk-pooled K, V, Kr) and "Document-wise RoPE resets every document to
// position zero"; yeyulingfeng.com "深度分析MSA ..." section 三 (mean pooling of each
// 64-token chunk into K-bar / V-bar / Kr-bar; a partial last chunk still counts).
//
// Design (HBM-bound streaming read, ~6 KB per token for the Qwen3-4B-like layer):
//  * Persistent workgroups each own a contiguous range of bank rows; every row reads its
//    chunk's tokens once, coalesced (each token row of K, V and Kr is read by consecutive
//    threads in 16-byte pieces).
//  * One thread owns an 8-element "unit" of a token row: 8 consecutive elements, or for a
//    rotated tensor 4 rotation pairs (i..i+3 together with i+d/2..i+d/2+3).  It sums its
//    unit over the chunk's tokens in float32 registers.
//  * Rotation by in-document position p = s + r (s = first position of the chunk) is split
//    as R(s) * R(r): the token loop applies R(r) from a per-workgroup LDS table
//    (cos/sin of r*theta_i, r < chunk, evaluated in double precision), and R(s) is applied
//    once to the chunk sum with double-precision angles.  Both are exact rotations, so the
//    result is the same mean up to float32 rounding.
//  * The mean divides by the number of real tokens with an IEEE division (a constant chunk
//    pools to itself bit for bit), then rounds once to the storage type.
#include "common.hpp"
#include "launch.hpp"

namespace msa {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(512) void pool_kernel(PoolArgs a) {
  extern __shared__ float rope_tab[];  // [chunk][D/2] cos, then [chunk][D/2] sin
  const int tid = threadIdx.x;
  const int units_per_head = D / 8;
  const int n_units = (2 * a.h_kv + a.h_r) * units_per_head;
  const int u = blockIdx.y * blockDim.x + tid;
  const int half = D / 2;

  // Which tensor / head / piece this thread owns.
  int tensor = 0, head = 0, piece = 0, heads = a.h_kv;
  const T* src = nullptr;
  T* dst = nullptr;
  bool valid = u < n_units;
  if (valid) {
    int v = u;
    if (v < a.h_kv * units_per_head) {
      tensor = 0; heads = a.h_kv; src = (const T*)a.K; dst = (T*)a.Kbar;
    } else if ((v -= a.h_kv * units_per_head) < a.h_kv * units_per_head) {
      tensor = 1; heads = a.h_kv; src = (const T*)a.V; dst = (T*)a.Vbar;
    } else {
      v -= a.h_kv * units_per_head;
      tensor = 2; heads = a.h_r; src = (const T*)a.Kr; dst = (T*)a.Krbar;
    }
    head = v / units_per_head;
    piece = v % units_per_head;
  }
  const bool rotate = valid && ((a.rope_mask >> tensor) & 1u);
  // Element offsets of the unit inside one token row of its tensor.
  const int e_lo = head * D + (rotate ? piece * 4 : piece * 8);
  const int e_hi = e_lo + half;  // second half of the rotation pairs
  const int i0 = piece * 4;      // first pair index when rotating
  const int row_elems = heads * D;

  // Per-workgroup table of R(r): angles r * theta_i, r < chunk, in double precision.
  if (a.rope_mask) {
    for (int e = tid; e < a.chunk * half; e += blockDim.x) {
      const int r = e / half, i = e % half;
      const double th = pow((double)a.rope_base, -2.0 * (double)i / (double)D);
      double sn, cs;
      sincos((double)r * th, &sn, &cs);
      rope_tab[e] = (float)cs;
      rope_tab[a.chunk * half + e] = (float)sn;
    }
  }
  __syncthreads();

  const int64_t c_begin = a.n_chunks * (int64_t)blockIdx.x / gridDim.x;
  const int64_t c_end = a.n_chunks * ((int64_t)blockIdx.x + 1) / gridDim.x;
  if (c_begin >= c_end) return;
  // Every lane of every wave takes part in the search (it votes across the wave).
  int doc = find_doc_wave(a.chunk_off, a.n_docs, c_begin);
  if (!valid) return;

  double theta[4];
  if (rotate) {
#pragma unroll
    for (int q = 0; q < 4; ++q) theta[q] = pow((double)a.rope_base, -2.0 * (double)(i0 + q) / (double)D);
  }

  int64_t doc_c0 = a.chunk_off[doc], doc_c1 = a.chunk_off[doc + 1];
  int64_t doc_t0 = a.doc_tok_off[doc], doc_t1 = a.doc_tok_off[doc + 1];

  for (int64_t c = c_begin; c < c_end; ++c) {
    while (c >= doc_c1) {  // advance to the document owning row c
      ++doc;
      doc_c0 = doc_c1;
      doc_c1 = a.chunk_off[doc + 1];
      doc_t0 = doc_t1;
      doc_t1 = a.doc_tok_off[doc + 1];
    }
    const int64_t j = c - doc_c0;                     // chunk index inside the document
    const int64_t tok0 = doc_t0 + j * a.chunk;
    const int n = (int)min((int64_t)a.chunk, doc_t1 - tok0);
    const T* base = src + tok0 * row_elems;

    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;

    for (int r0 = 0; r0 < n; r0 += 8) {
      float v[8][8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (r0 + t < n) {
          const T* p = base + (int64_t)(r0 + t) * row_elems;
          if (rotate) {
            Elem<T>::load4(p + e_lo, v[t]);
            Elem<T>::load4(p + e_hi, v[t] + 4);
          } else {
            Elem<T>::load8(p + e_lo, v[t]);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (r0 + t < n) {
          if (rotate) {
            const float* cs = rope_tab + (r0 + t) * half + i0;
            const float* sn = rope_tab + a.chunk * half + (r0 + t) * half + i0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float x = v[t][q], y = v[t][4 + q];
              acc[q] += x * cs[q] - y * sn[q];
              acc[4 + q] += y * cs[q] + x * sn[q];
            }
          } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] += v[t][q];
          }
        }
      }
    }

    if (rotate && j > 0) {  // R(s), s = first in-document position of the chunk
      const double s = (double)(j * a.chunk);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        double sn, cs;
        sincos(s * theta[q], &sn, &cs);
        const float c32 = (float)cs, s32 = (float)sn;
        const float x = acc[q], y = acc[4 + q];
        acc[q] = x * c32 - y * s32;
        acc[4 + q] = y * c32 + x * s32;
      }
    }
    const float fn = (float)n;
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = acc[q] / fn;

    T* out = dst + c * row_elems;
    if (rotate) {
      Elem<T>::store4(out + e_lo, acc);
      Elem<T>::store4(out + e_hi, acc + 4);
    } else {
      Elem<T>::store8(out + e_lo, acc);
    }
  }
}

template <typename T, int D>
hipError_t launch_pool_t(const PoolArgs& a, hipStream_t s) {
  const int n_units = (2 * a.h_kv + a.h_r) * (D / 8);
  int threads = ((n_units + 63) / 64) * 64;
  if (threads > 512) threads = 512;
  const int ygroups = (n_units + threads - 1) / threads;
  // Enough workgroups to fill 256 CUs several times over, never more than one per row.
  int64_t wgs = 1024 / ygroups;
  if (wgs < 256) wgs = 256;
  if (wgs > a.n_chunks) wgs = a.n_chunks;
  const size_t lds = a.rope_mask ? (size_t)a.chunk * D * sizeof(float) : 0;
  dim3 grid((unsigned)wgs, (unsigned)ygroups);
  hipLaunchKernelGGL((pool_kernel<T, D>), grid, dim3(threads), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const PoolArgs& a, hipStream_t s) {
  if (a.n_chunks == 0) return hipSuccess;
  if (a.dtype == 0) {
    switch (a.d) {
      case 32: return launch_pool_t<float, 32>(a, s);
      case 64: return launch_pool_t<float, 64>(a, s);
      default: return launch_pool_t<float, 128>(a, s);
    }
  }
  switch (a.d) {
    case 32: return launch_pool_t<bf16_t, 32>(a, s);
    case 64: return launch_pool_t<bf16_t, 64>(a, s);
    default: return launch_pool_t<bf16_t, 128>(a, s);
  }
}

}  // namespace msa
