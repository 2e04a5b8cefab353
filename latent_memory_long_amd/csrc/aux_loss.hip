// The routing auxiliary loss: supervision of the router's document scores.
//
// yeyulingfeng.com "深度分析MSA ..." section 四 (training): besides the language-model loss, an
// auxiliary loss on the document scores trains the router; the common forms are BCE and
// InfoNCE.  With z = S / temperature for one query's scores S over the N documents and
// labels y (L = mean over queries of the per-query loss l):
//   BCE:     l = (1/N) sum_d [softplus(z_d) - y_d z_d],  dl/dz_d = (sigmoid(z_d) - y_d) / N
//   InfoNCE: l = log sum_d e^z_d - log sum_d y_d e^z_d,  dl/dz_d = p_d - y_d e^z_d / sum y e^z
// where p = softmax(z).  Each log-sum-exp is shifted by its own maximum.  A query with a
// non-finite score (a query without tokens scores -inf), or for InfoNCE without a positive
// label, contributes nothing.
//
// One workgroup per query, three passes over its row (maxima, sums, gradient); sums run in
// double with a fixed reduction order, so results do not depend on scheduling.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace msa {
namespace {

constexpr int AUX_THREADS = 256;
constexpr int AUX_WAVES = AUX_THREADS / 64;

struct AuxRed {
  double v[AUX_WAVES][3];
};

// Sum (op 0) or max (op 1) of three values over the workgroup, same order on every run.
template <int OP>
__device__ __forceinline__ void block_reduce3(double (&x)[3], AuxRed& r) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double y = __shfl_xor(x[i], o, 64);
      x[i] = OP ? fmax(x[i], y) : x[i] + y;
    }
  }
  __syncthreads();  // r is free
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < 3; ++i) r.v[w][i] = x[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    double t = r.v[0][i];
#pragma unroll
    for (int k = 1; k < AUX_WAVES; ++k) t = OP ? fmax(t, r.v[k][i]) : t + r.v[k][i];
    x[i] = t;
  }
}

__device__ __forceinline__ double softplus(double z) { return fmax(z, 0.0) + log1p(exp(-fabs(z))); }
__device__ __forceinline__ double sigmoid(double z) {
  const double e = exp(-fabs(z));
  return z >= 0 ? 1.0 / (1.0 + e) : e / (1.0 + e);
}

template <int KIND>
__global__ __launch_bounds__(AUX_THREADS) void aux_loss_kernel(AuxArgs a) {
  __shared__ AuxRed red;
  const int b = blockIdx.x;
  const int N = a.n_docs;
  const float* S = a.scores + (int64_t)b * N;
  const float* Y = a.labels + (int64_t)b * N;
  float* G = a.dD + (int64_t)b * N;
  const double tau = (double)a.temperature;
  // pass 1: finiteness, max logit, max logit over positives
  double x[3] = {0.0, -INFINITY, -INFINITY};  // non-finite count, max z, max positive z
  for (int d = threadIdx.x; d < N; d += AUX_THREADS) {
    const float v = S[d];
    if (!isfinite(v)) x[0] = 1.0;
    const double z = (double)v / tau;
    x[1] = fmax(x[1], z);
    if (Y[d] > 0.f) x[2] = fmax(x[2], z);
  }
  block_reduce3<1>(x, red);
  if (x[0] != 0.0 || (KIND == AUX_INFONCE && !(x[2] > -INFINITY))) {
    for (int d = threadIdx.x; d < N; d += AUX_THREADS) G[d] = 0.f;
    if (threadIdx.x == 0) a.loss[b] = 0.f;
    return;
  }
  const double m = x[1], mp = x[2];
  // pass 2: the sums
  double s[3] = {0.0, 0.0, 0.0};
  for (int d = threadIdx.x; d < N; d += AUX_THREADS) {
    const double z = (double)S[d] / tau, y = (double)Y[d];
    if (KIND == AUX_BCE) {
      s[0] += softplus(z) - y * z;
    } else {
      s[0] += exp(z - m);
      if (y > 0.0) s[1] += y * exp(z - mp);
    }
  }
  block_reduce3<0>(s, red);
  const double scale = 1.0 / (tau * (double)a.n_queries);
  if (threadIdx.x == 0)
    a.loss[b] = KIND == AUX_BCE ? (float)(s[0] / N) : (float)((m + log(s[0])) - (mp + log(s[1])));
  // pass 3: the gradient of the mean over queries
  for (int d = threadIdx.x; d < N; d += AUX_THREADS) {
    const double z = (double)S[d] / tau, y = (double)Y[d];
    double g;
    if (KIND == AUX_BCE) {
      g = (sigmoid(z) - y) / N;
    } else {
      g = exp(z - m) / s[0];
      if (y > 0.0) g -= y * exp(z - mp) / s[1];
    }
    G[d] = (float)(g * scale);
  }
}

}  // namespace

hipError_t launch_aux_loss(const AuxArgs& a, hipStream_t s) {
  if (a.kind == AUX_BCE)
    hipLaunchKernelGGL((aux_loss_kernel<AUX_BCE>), dim3(a.n_queries), dim3(AUX_THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((aux_loss_kernel<AUX_INFONCE>), dim3(a.n_queries), dim3(AUX_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace msa
