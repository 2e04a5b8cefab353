// Routing-key bank layout conversions.
//
// hysenlabs.com "EverMind-AI/MSA: routing top-k compressed documents inside attention ...",
// section "The 100M-token setup depends on host memory as well as two GPUs": the routing
// keys stay resident in GPU memory and every query scans all of them, so they are stored
// the way the scan reads them.  A bf16 bank is kept in 16-row tiles whose 1 KB blocks are
// MFMA B operands (the layout is spelled out in common.hpp); float32 banks are row-major.
// These kernels convert between that layout and row-major [C, h_r, d], for callers that
// hold or need plain rows.  One thread moves one 16-byte unit (8 elements of one head).
#include "common.hpp"
#include "launch.hpp"

namespace msa {
namespace {

template <int D, bool PACK>
__global__ __launch_bounds__(256) void krbar_convert(const bf16_t* src, bf16_t* dst, int64_t n_chunks, int H) {
  const int units_per_row = H * D / 8;
  const int64_t rows = PACK ? kr_tiles(n_chunks) * 16 : n_chunks;  // pack also fills the padding
  const int64_t n = rows * units_per_row;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n; u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = u / units_per_row;
    const int i = (int)(u - c * units_per_row) * 8;
    const int64_t tiled = kr_tiled<D>(c, i, H), plain = c * (H * D) + i;
    if (PACK) {
      const uint4 v = c < n_chunks ? *reinterpret_cast<const uint4*>(src + plain) : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(dst + tiled) = v;
    } else {
      *reinterpret_cast<uint4*>(dst + plain) = *reinterpret_cast<const uint4*>(src + tiled);
    }
  }
}

__global__ __launch_bounds__(256) void copy_words(const uint4* src, uint4* dst, int64_t n) {
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n; u += (int64_t)gridDim.x * blockDim.x)
    dst[u] = src[u];
}

unsigned grid_for(int64_t n) {
  const int64_t g = (n + 255) / 256;
  return (unsigned)(g < 8192 ? (g > 0 ? g : 1) : 8192);
}

template <bool PACK>
hipError_t convert(int dtype, int64_t n_chunks, int h_r, int d, const void* src, void* dst, hipStream_t s) {
  if (dtype == 0) {  // float32: row-major either way, a copy (a kernel, so it can be captured)
    const int64_t n = n_chunks * h_r * d / 4;  // d is a multiple of 32: whole 16-byte words
    hipLaunchKernelGGL(copy_words, dim3(grid_for(n)), dim3(256), 0, s, (const uint4*)src, (uint4*)dst, n);
    return hipGetLastError();
  }
  const int64_t units = (PACK ? kr_tiles(n_chunks) * 16 : n_chunks) * h_r * d / 8;
  const dim3 g(grid_for(units));
  const bf16_t* a = (const bf16_t*)src;
  bf16_t* b = (bf16_t*)dst;
  switch (d) {
    case 32: hipLaunchKernelGGL((krbar_convert<32, PACK>), g, dim3(256), 0, s, a, b, n_chunks, h_r); break;
    case 64: hipLaunchKernelGGL((krbar_convert<64, PACK>), g, dim3(256), 0, s, a, b, n_chunks, h_r); break;
    default: hipLaunchKernelGGL((krbar_convert<128, PACK>), g, dim3(256), 0, s, a, b, n_chunks, h_r); break;
  }
  return hipGetLastError();
}

}  // namespace

int64_t krbar_elems(int dtype, int64_t n_chunks, int h_r, int d) {
  return (dtype == 0 ? n_chunks : kr_tiles(n_chunks) * 16) * h_r * d;
}

hipError_t launch_krbar_pack(int dtype, int64_t n_chunks, int h_r, int d, const void* rows, void* krbar,
                             hipStream_t s) {
  return convert<true>(dtype, n_chunks, h_r, d, rows, krbar, s);
}

hipError_t launch_krbar_unpack(int dtype, int64_t n_chunks, int h_r, int d, const void* krbar, void* rows,
                               hipStream_t s) {
  return convert<false>(dtype, n_chunks, h_r, d, krbar, rows, s);
}

}  // namespace msa
