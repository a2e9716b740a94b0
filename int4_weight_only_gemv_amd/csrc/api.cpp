// C ABI of the W4A16 library: synchronous argument checks, then one launch
// on the caller's stream.  See include/w4a16.h for the contract.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstring>

#include "w4a16.h"

namespace w4a16 {
int launch_pack(const uint16_t*, int64_t, int64_t, int64_t, const float*, int, uint32_t*,
                uint16_t*, int32_t*, bool, bool, hipStream_t);
int launch_gemv_int8(const uint16_t*, int64_t, int64_t, const uint32_t*, const uint16_t*,
                     const int32_t*, int64_t, int64_t, uint16_t*, int64_t, hipStream_t);
int launch_gemm_int8(const uint16_t*, int64_t, int64_t, const uint32_t*, const uint16_t*,
                     const int32_t*, int64_t, int64_t, uint16_t*, int64_t, hipStream_t);
int launch_gemv(const uint16_t*, int64_t, int64_t, const uint32_t*, const uint16_t*,
                const int32_t*, int64_t, int64_t, int, uint16_t*, int64_t, hipStream_t);
int launch_gemm(const uint16_t*, int64_t, int64_t, const uint32_t*, const uint16_t*,
                const int32_t*, int64_t, int64_t, int, uint16_t*, int64_t, hipStream_t);
int launch_awq_importance(const uint16_t*, int64_t, int64_t, int64_t, float*, hipStream_t);
int launch_awq_scale(const float*, int64_t, float, float*, hipStream_t);
int launch_awq_fold(const float*, int64_t, uint16_t*, uint16_t*, hipStream_t);
int launch_rel_l2(const uint16_t*, int64_t, const uint16_t*, int64_t, int64_t, int64_t, double*,
                  hipStream_t);
int launch_hbm_read_probe(const void*, int64_t, uint32_t*, hipStream_t);
int launch_scale_channels(const uint16_t*, int64_t, int64_t, int64_t, const uint16_t*, uint16_t*,
                          int64_t, hipStream_t);
int launch_dequant_bf16(const uint32_t*, const uint16_t*, const int32_t*, int64_t, int64_t,
                        uint16_t*, int64_t, hipStream_t);
int launch_dense_gemv(const uint16_t*, int64_t, int64_t, const uint16_t*, int64_t, int64_t, int64_t,
                      uint16_t*, int64_t, hipStream_t);
int launch_dense_gemm(const uint16_t*, int64_t, int64_t, const uint16_t*, int64_t, int64_t, int64_t,
                      uint16_t*, int64_t, hipStream_t);
}  // namespace w4a16

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 30;  // N, K, M each below 2^30

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// The kernels are built for gfx950 only: the current HIP device must be one
// (checked once per device, then cached; no device counts as unsupported).
int device_check() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> state[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();   // leave no sticky error for the caller's next call
    return W4A16_ERR_UNSUPPORTED;
  }
  int st = state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    st = 2;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess && std::strncmp(prop.gcnArchName, "gfx950", 6) == 0)
      st = 1;
    else
      (void)hipGetLastError();
    state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? W4A16_OK : W4A16_ERR_UNSUPPORTED;
}

// The matrix-core GEMM addresses a tile's rows of X, codes and metadata with
// 32-bit byte offsets from a per-tile base, and numbers its tiles with 31
// bits (tiles of at least 64 x 128).
int check_gemm_limits(int64_t M, int64_t N, int64_t K, int64_t ldx) {
  if (ldx >= W4A16_GEMM_MAX_LD || K >= W4A16_GEMM_MAX_K) return W4A16_ERR_UNSUPPORTED;
  if (((M + 63) / 64) * ((N + 127) / 128) >= ((int64_t)1 << 31)) return W4A16_ERR_UNSUPPORTED;
  return W4A16_OK;
}

bool group_ok(int64_t group) { return group == 32 || group == 64 || group == 128; }

// Checks shared by gemv and gemm (any group size; smaller groups need
// 16-byte aligned scales and zero points).
int check_matmul(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                 const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K,
                 const uint16_t* Y, int64_t ldy, int64_t group = W4A16_GROUP) {
  if (!X || !codes || !scales || !zeros || !Y || !group_ok(group)) return W4A16_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < W4A16_GROUP || K % W4A16_GROUP) return W4A16_ERR_INVALID_ARG;
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return W4A16_ERR_UNSUPPORTED;
  if (ldx < K || ldy < N) return W4A16_ERR_INVALID_ARG;
  if (!aligned(X, 16) || ldx % 8 || !aligned(codes, 16) || !aligned(scales, 2) ||
      !aligned(zeros, 4) || !aligned(Y, 2))
    return W4A16_ERR_MISALIGNED;
  if (group != W4A16_GROUP && (!aligned(scales, 16) || !aligned(zeros, 16))) return W4A16_ERR_MISALIGNED;
  return W4A16_OK;
}

// Checks shared by the dense comparisons.
int check_dense(const uint16_t* X, int64_t M, int64_t ldx, const uint16_t* W, int64_t ldw,
                int64_t N, int64_t K, const uint16_t* Y, int64_t ldy) {
  if (!X || !W || !Y) return W4A16_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < W4A16_GROUP || K % W4A16_GROUP) return W4A16_ERR_INVALID_ARG;
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return W4A16_ERR_UNSUPPORTED;
  if (ldx < K || ldw < K || ldy < N) return W4A16_ERR_INVALID_ARG;
  if (!aligned(X, 16) || ldx % 8 || !aligned(W, 16) || ldw % 8 || !aligned(Y, 2))
    return W4A16_ERR_MISALIGNED;
  return W4A16_OK;
}

}  // namespace

extern "C" {

int w4a16_abi_version(void) { return W4A16_ABI_VERSION; }

const char* w4a16_strerror(int status) {
  switch (status) {
    case W4A16_OK: return "ok";
    case W4A16_ERR_INVALID_ARG: return "invalid argument (null pointer, size or leading dimension)";
    case W4A16_ERR_MISALIGNED: return "misaligned pointer or leading dimension";
    case W4A16_ERR_UNSUPPORTED: return "unsupported size or device";
    case W4A16_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

namespace {
int pack_checked(const uint16_t* W, int64_t N, int64_t K, int64_t ldw, const float* awq_s,
                 int64_t group, uint32_t* codes, uint16_t* scales, int32_t* zeros, bool symmetric,
                 void* stream, bool int8 = false) {
  if (!W || !codes || !scales || !zeros || !group_ok(group)) return W4A16_ERR_INVALID_ARG;
  if (N < 1 || K < W4A16_GROUP || K % W4A16_GROUP || ldw < K) return W4A16_ERR_INVALID_ARG;
  if (N >= kMaxDim || K >= kMaxDim || N * (K / 8) >= ((int64_t)1 << 38)) return W4A16_ERR_UNSUPPORTED;
  if (!aligned(W, 2) || !aligned(codes, 16) || !aligned(scales, 2) || !aligned(zeros, 4) ||
      (awq_s && !aligned(awq_s, 4)))
    return W4A16_ERR_MISALIGNED;
  if (int dc = device_check()) return dc;
  return w4a16::launch_pack(W, N, K, ldw, awq_s, (int)group, codes, scales, zeros, symmetric,
                            int8, (hipStream_t)stream);
}
}  // namespace

int w4a16_pack(const uint16_t* W, int64_t N, int64_t K, int64_t ldw, const float* awq_s,
               uint32_t* codes, uint16_t* scales, int32_t* zeros, void* stream) {
  return pack_checked(W, N, K, ldw, awq_s, W4A16_GROUP, codes, scales, zeros, false, stream);
}

int w4a16_pack_int8(const uint16_t* W, int64_t N, int64_t K, int64_t ldw, const float* awq_s,
                    uint32_t* codes, uint16_t* scales, int32_t* zeros, void* stream) {
  return pack_checked(W, N, K, ldw, awq_s, W4A16_GROUP, codes, scales, zeros, false, stream, true);
}

int w4a16_gemv_int8(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                    const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K, uint16_t* Y,
                    int64_t ldy, void* stream) {
  int st = check_matmul(X, M, ldx, codes, scales, zeros, N, K, Y, ldy);
  if (st != W4A16_OK) return st;
  if (M > W4A16_INT8_GEMV_MAX_M) return W4A16_ERR_INVALID_ARG;
  if (K > W4A16_INT8_GEMV_MAX_K) return W4A16_ERR_UNSUPPORTED;
  if (int dc = device_check()) return dc;
  return w4a16::launch_gemv_int8(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, (hipStream_t)stream);
}

int w4a16_gemm_int8(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                    const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K, uint16_t* Y,
                    int64_t ldy, void* stream) {
  int st = check_matmul(X, M, ldx, codes, scales, zeros, N, K, Y, ldy);
  if (st != W4A16_OK) return st;
  st = check_gemm_limits(M, N, K, ldx);
  if (st != W4A16_OK) return st;
  if (int dc = device_check()) return dc;
  return w4a16::launch_gemm_int8(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, (hipStream_t)stream);
}

int w4a16_pack_grouped(const uint16_t* W, int64_t N, int64_t K, int64_t ldw, const float* awq_s,
                       int64_t group, uint32_t* codes, uint16_t* scales, int32_t* zeros,
                       void* stream) {
  return pack_checked(W, N, K, ldw, awq_s, group, codes, scales, zeros, false, stream);
}

int w4a16_pack_symmetric(const uint16_t* W, int64_t N, int64_t K, int64_t ldw, const float* awq_s,
                         uint32_t* codes, uint16_t* scales, int32_t* zeros, void* stream) {
  return pack_checked(W, N, K, ldw, awq_s, W4A16_GROUP, codes, scales, zeros, true, stream);
}

int w4a16_gemv(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
               const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K, uint16_t* Y,
               int64_t ldy, void* stream) {
  int st = check_matmul(X, M, ldx, codes, scales, zeros, N, K, Y, ldy);
  if (st != W4A16_OK) return st;
  if (M > W4A16_GEMV_MAX_M) return W4A16_ERR_INVALID_ARG;
  if (int dc = device_check()) return dc;
  return w4a16::launch_gemv(X, M, ldx, codes, scales, zeros, N, K, W4A16_GROUP, Y, ldy,
                            (hipStream_t)stream);
}

int w4a16_gemv_grouped(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                       const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K,
                       int64_t group, uint16_t* Y, int64_t ldy, void* stream) {
  int st = check_matmul(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, group);
  if (st != W4A16_OK) return st;
  if (M > W4A16_GEMV_MAX_M) return W4A16_ERR_INVALID_ARG;
  if (M > 8 && (st = check_gemm_limits(M, N, K, ldx)) != W4A16_OK) return st;   // the GEMM runs M > 8
  if (int dc = device_check()) return dc;
  return w4a16::launch_gemv(X, M, ldx, codes, scales, zeros, N, K, (int)group, Y, ldy,
                            (hipStream_t)stream);
}

int w4a16_gemm(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
               const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K, uint16_t* Y,
               int64_t ldy, void* stream) {
  int st = check_matmul(X, M, ldx, codes, scales, zeros, N, K, Y, ldy);
  if (st != W4A16_OK) return st;
  st = check_gemm_limits(M, N, K, ldx);
  if (st != W4A16_OK) return st;
  if (int dc = device_check()) return dc;
  return w4a16::launch_gemm(X, M, ldx, codes, scales, zeros, N, K, W4A16_GROUP, Y, ldy,
                            (hipStream_t)stream);
}

int w4a16_gemm_grouped(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                       const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K,
                       int64_t group, uint16_t* Y, int64_t ldy, void* stream) {
  int st = check_matmul(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, group);
  if (st != W4A16_OK) return st;
  st = check_gemm_limits(M, N, K, ldx);
  if (st != W4A16_OK) return st;
  if (int dc = device_check()) return dc;
  return w4a16::launch_gemm(X, M, ldx, codes, scales, zeros, N, K, (int)group, Y, ldy,
                            (hipStream_t)stream);
}

int w4a16_awq_importance(const uint16_t* Xcal, int64_t T, int64_t K, int64_t ldx,
                         float* importance, void* stream) {
  if (!Xcal || !importance || T < 1 || K < 1 || ldx < K) return W4A16_ERR_INVALID_ARG;
  if (T >= kMaxDim || K >= kMaxDim) return W4A16_ERR_UNSUPPORTED;
  if (!aligned(Xcal, 2) || !aligned(importance, 4)) return W4A16_ERR_MISALIGNED;
  if (int dc = device_check()) return dc;
  return w4a16::launch_awq_importance(Xcal, T, K, ldx, importance, (hipStream_t)stream);
}

int w4a16_awq_scale(const float* importance, int64_t K, float alpha, float* s, void* stream) {
  if (!importance || !s || K < 1 || !(alpha >= 0.0f && alpha <= 1.0f)) return W4A16_ERR_INVALID_ARG;
  if (K >= kMaxDim) return W4A16_ERR_UNSUPPORTED;
  if (!aligned(importance, 4) || !aligned(s, 4)) return W4A16_ERR_MISALIGNED;
  if (int dc = device_check()) return dc;
  return w4a16::launch_awq_scale(importance, K, alpha, s, (hipStream_t)stream);
}

int w4a16_awq_fold(const float* s, int64_t K, uint16_t* gamma, uint16_t* beta, void* stream) {
  if (!s || !gamma || K < 1) return W4A16_ERR_INVALID_ARG;
  if (K >= kMaxDim) return W4A16_ERR_UNSUPPORTED;
  if (!aligned(s, 4) || !aligned(gamma, 2) || (beta && !aligned(beta, 2))) return W4A16_ERR_MISALIGNED;
  if (int dc = device_check()) return dc;
  return w4a16::launch_awq_fold(s, K, gamma, beta, (hipStream_t)stream);
}

int w4a16_scale_channels(const uint16_t* X, int64_t M, int64_t K, int64_t ldx,
                         const uint16_t* gamma, uint16_t* Xout, int64_t ldo, void* stream) {
  if (!X || !gamma || !Xout || M < 1 || K < 1 || ldx < K || ldo < K) return W4A16_ERR_INVALID_ARG;
  if (M >= kMaxDim || K >= kMaxDim || M * K >= ((int64_t)1 << 38)) return W4A16_ERR_UNSUPPORTED;
  if (!aligned(X, 2) || !aligned(gamma, 2) || !aligned(Xout, 2)) return W4A16_ERR_MISALIGNED;
  if (int dc = device_check()) return dc;
  return w4a16::launch_scale_channels(X, M, K, ldx, gamma, Xout, ldo, (hipStream_t)stream);
}

int w4a16_awq_search_error(const uint16_t* Y, int64_t ldy, const uint16_t* Yref, int64_t ldr,
                           int64_t M, int64_t N, double* err, void* stream) {
  if (!Y || !Yref || !err || M < 1 || N < 1 || ldy < N || ldr < N) return W4A16_ERR_INVALID_ARG;
  if (M >= kMaxDim || N >= kMaxDim) return W4A16_ERR_UNSUPPORTED;
  if (!aligned(Y, 2) || !aligned(Yref, 2) || !aligned(err, 8)) return W4A16_ERR_MISALIGNED;
  if (int dc = device_check()) return dc;
  return w4a16::launch_rel_l2(Y, ldy, Yref, ldr, M, N, err, (hipStream_t)stream);
}

int w4a16_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16) return W4A16_ERR_INVALID_ARG;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return W4A16_ERR_MISALIGNED;
  if (int dc = device_check()) return dc;
  return w4a16::launch_hbm_read_probe(buf, bytes, sink, (hipStream_t)stream);
}

int w4a16_dequantize_bf16(const uint32_t* codes, const uint16_t* scales, const int32_t* zeros,
                          int64_t N, int64_t K, uint16_t* W, int64_t ldw, void* stream) {
  if (!codes || !scales || !zeros || !W) return W4A16_ERR_INVALID_ARG;
  if (N < 1 || K < W4A16_GROUP || K % W4A16_GROUP || ldw < K) return W4A16_ERR_INVALID_ARG;
  if (N >= kMaxDim || K >= kMaxDim || N * (K / 8) >= ((int64_t)1 << 38)) return W4A16_ERR_UNSUPPORTED;
  if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(zeros, 4) || !aligned(W, 16) || ldw % 8)
    return W4A16_ERR_MISALIGNED;
  if (int dc = device_check()) return dc;
  return w4a16::launch_dequant_bf16(codes, scales, zeros, N, K, W, ldw, (hipStream_t)stream);
}

int w4a16_dense_gemv(const uint16_t* X, int64_t M, int64_t ldx, const uint16_t* W, int64_t ldw,
                     int64_t N, int64_t K, uint16_t* Y, int64_t ldy, void* stream) {
  int st = check_dense(X, M, ldx, W, ldw, N, K, Y, ldy);
  if (st != W4A16_OK) return st;
  if (M > W4A16_DENSE_GEMV_MAX_M) return W4A16_ERR_INVALID_ARG;
  if (int dc = device_check()) return dc;
  return w4a16::launch_dense_gemv(X, M, ldx, W, ldw, N, K, Y, ldy, (hipStream_t)stream);
}

int w4a16_dense_gemm(const uint16_t* X, int64_t M, int64_t ldx, const uint16_t* W, int64_t ldw,
                     int64_t N, int64_t K, uint16_t* Y, int64_t ldy, void* stream) {
  int st = check_dense(X, M, ldx, W, ldw, N, K, Y, ldy);
  if (st != W4A16_OK) return st;
  if (ldx >= W4A16_GEMM_MAX_LD || ldw >= W4A16_GEMM_MAX_LD ||
      ((M + 255) / 256) * ((N + 255) / 256) >= ((int64_t)1 << 31))
    return W4A16_ERR_UNSUPPORTED;
  if (int dc = device_check()) return dc;
  return w4a16::launch_dense_gemm(X, M, ldx, W, ldw, N, K, Y, ldy, (hipStream_t)stream);
}

}  // extern "C"
