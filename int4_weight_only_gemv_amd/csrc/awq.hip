// AWQ helpers around the W4A16 path: calibration statistic, smoothing scale,
// and the fold of diag(s)^-1 into the activations' producer (Axe Corsa model
// card, "Stage 1: Activation-Aware Weight Scaling").  These run once per
// model at calibration time; the fold makes the rescaling free at inference.

#include "common.h"

namespace w4a16 {
namespace {

// importance[k] = (1/T) sum_t |X[t,k]|, float64 sum in token order.
__global__ __launch_bounds__(256) void importance_kernel(const uint16_t* __restrict__ X, int64_t T,
                                                         int64_t K, int64_t ldx,
                                                         float* __restrict__ out) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  double acc = 0.0;
  for (int64_t t = 0; t < T; ++t) acc += fabs((double)bf16_to_f32(X[t * ldx + k]));
  out[k] = (float)(acc / (double)T);
}

// s[k] = importance[k] ** alpha in float64, rounded to float32.
__global__ __launch_bounds__(256) void scale_kernel(const float* __restrict__ imp, int64_t K,
                                                    double alpha, float* __restrict__ s) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  s[k] = (float)pow((double)imp[k], alpha);
}

// gamma[k] = bf16_rne(gamma[k] / s[k]) (and beta likewise).
__global__ __launch_bounds__(256) void fold_kernel(const float* __restrict__ s, int64_t K,
                                                   uint16_t* __restrict__ gamma,
                                                   uint16_t* __restrict__ beta) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= K) return;
  const float sk = s[k];
  gamma[k] = f32_to_bf16_rne(__fdiv_rn(bf16_to_f32(gamma[k]), sk));
  if (beta) beta[k] = f32_to_bf16_rne(__fdiv_rn(bf16_to_f32(beta[k]), sk));
}

// Xout[m,k] = bf16_rne(X[m,k] * gamma[k]).
__global__ __launch_bounds__(256) void scale_channels_kernel(const uint16_t* __restrict__ X,
                                                             int64_t M, int64_t K, int64_t ldx,
                                                             const uint16_t* __restrict__ gamma,
                                                             uint16_t* Xout, int64_t ldo) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M * K) return;
  const int64_t m = i / K, k = i - m * K;
  Xout[m * ldo + k] = f32_to_bf16_rne(__fmul_rn(bf16_to_f32(X[m * ldx + k]), bf16_to_f32(gamma[k])));
}

// err[0] = sqrt(sum (Y - R)^2 / sum R^2) over an M x N output pair, the
// objective of AWQ's exponent search.  One workgroup: each thread sums a
// fixed strided share in float64, then a fixed-order tree in LDS, so the
// result does not depend on timing.
constexpr int kErrThreads = 1024;
__global__ __launch_bounds__(kErrThreads) void rel_l2_kernel(const uint16_t* __restrict__ Y, int64_t ldy,
                                                             const uint16_t* __restrict__ R, int64_t ldr,
                                                             int64_t M, int64_t N, double* __restrict__ err) {
  __shared__ double num[kErrThreads], den[kErrThreads];
  double a = 0.0, b = 0.0;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = threadIdx.x; n < N; n += kErrThreads) {
      const double r = (double)bf16_to_f32(R[m * ldr + n]);
      const double d = (double)bf16_to_f32(Y[m * ldy + n]) - r;
      a += d * d;
      b += r * r;
    }
  num[threadIdx.x] = a;
  den[threadIdx.x] = b;
  __syncthreads();
  for (int h = kErrThreads / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) {
      num[threadIdx.x] += num[threadIdx.x + h];
      den[threadIdx.x] += den[threadIdx.x + h];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) err[0] = sqrt(num[0] / den[0]);
}

unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

int launch_awq_importance(const uint16_t* X, int64_t T, int64_t K, int64_t ldx, float* out,
                          hipStream_t stream) {
  hipLaunchKernelGGL(importance_kernel, dim3(blocks_for(K)), dim3(256), 0, stream, X, T, K, ldx, out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int launch_awq_scale(const float* imp, int64_t K, float alpha, float* s, hipStream_t stream) {
  hipLaunchKernelGGL(scale_kernel, dim3(blocks_for(K)), dim3(256), 0, stream, imp, K,
                     (double)alpha, s);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int launch_awq_fold(const float* s, int64_t K, uint16_t* gamma, uint16_t* beta,
                    hipStream_t stream) {
  hipLaunchKernelGGL(fold_kernel, dim3(blocks_for(K)), dim3(256), 0, stream, s, K, gamma, beta);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int launch_scale_channels(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                          const uint16_t* gamma, uint16_t* Xout, int64_t ldo, hipStream_t stream) {
  hipLaunchKernelGGL(scale_channels_kernel, dim3(blocks_for(M * K)), dim3(256), 0, stream, X, M, K,
                     ldx, gamma, Xout, ldo);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int launch_rel_l2(const uint16_t* Y, int64_t ldy, const uint16_t* R, int64_t ldr, int64_t M, int64_t N,
                  double* err, hipStream_t stream) {
  hipLaunchKernelGGL(rel_l2_kernel, dim3(1), dim3(kErrThreads), 0, stream, Y, ldy, R, ldr, M, N, err);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace w4a16
