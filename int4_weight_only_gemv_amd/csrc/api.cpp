// C ABI of the W4A16 library: synchronous argument checks, then the call's
// launches on the caller's stream.  See include/w4a16.h for the contract.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <vector>

#include "chain.h"
#include "common.h"
#include "w4a16.h"

namespace w4a16 {
int launch_pack(const uint16_t*, int64_t, int64_t, int64_t, const float*, int, uint32_t*,
                uint16_t*, int32_t*, bool, bool, hipStream_t);
int launch_gemv_int8(const uint16_t*, int64_t, int64_t, const uint32_t*, const uint16_t*,
                     const int32_t*, int64_t, int64_t, uint16_t*, int64_t, hipStream_t);
int launch_gemm_int8(const uint16_t*, int64_t, int64_t, const uint32_t*, const uint16_t*,
                     const int32_t*, int64_t, int64_t, uint16_t*, int64_t, hipStream_t);
int launch_gemv(const uint16_t*, int64_t, int64_t, const uint32_t*, const uint16_t*,
                const int32_t*, int64_t, int64_t, int, uint16_t*, int64_t, void*, int64_t, hipStream_t);
int64_t gemv_workspace_bytes(int64_t, int64_t, int64_t, int);
int launch_gemm(const uint16_t*, int64_t, int64_t, const uint32_t*, const uint16_t*,
                const int32_t*, int64_t, int64_t, int, uint16_t*, int64_t, hipStream_t, void* = nullptr,
                int64_t = 0);
int64_t gemm_workspace_bytes(int64_t, int64_t, int64_t);
int launch_awq_importance(const uint16_t*, int64_t, int64_t, int64_t, float*, hipStream_t);
int launch_awq_scale(const float*, int64_t, float, float*, hipStream_t);
int launch_awq_fold(const float*, int64_t, uint16_t*, uint16_t*, hipStream_t);
int launch_rel_l2(const uint16_t*, int64_t, const uint16_t*, int64_t, int64_t, int64_t, double*,
                  hipStream_t);
int launch_hbm_read_probe(const void*, int64_t, uint32_t*, hipStream_t);
int launch_chain(const void*, int, int, const uint16_t*, int64_t, unsigned*, int, int, int, int, size_t,
                 hipStream_t);
int launch_chain_noalloc(const ChainDesc*, int, int, const uint16_t*, int64_t, int, int, int, size_t, int*,
                         hipStream_t);
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

bool ranges_overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + (uintptr_t)bbytes && y < x + (uintptr_t)abytes;
}

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
  return w4a16::launch_gemv(X, M, ldx, codes, scales, zeros, N, K, W4A16_GROUP, Y, ldy, nullptr, 0,
                            (hipStream_t)stream);
}

int w4a16_gemv_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t* bytes) {
  if (!bytes) return W4A16_ERR_INVALID_ARG;
  *bytes = 0;
  if (M < 1 || M > W4A16_GEMV_MAX_M || N < 1 || K < W4A16_GROUP || K % W4A16_GROUP)
    return W4A16_ERR_INVALID_ARG;
  if (N >= kMaxDim || K >= kMaxDim) return W4A16_ERR_UNSUPPORTED;
  if (int dc = device_check()) return dc;   // the plan depends on the device's CU count
  *bytes = w4a16::gemv_workspace_bytes(M, N, K, W4A16_GROUP);
  return W4A16_OK;
}

int w4a16_gemv_ws(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                  const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K, uint16_t* Y,
                  int64_t ldy, void* workspace, int64_t workspace_bytes, void* stream) {
  int st = check_matmul(X, M, ldx, codes, scales, zeros, N, K, Y, ldy);
  if (st != W4A16_OK) return st;
  if (M > W4A16_GEMV_MAX_M || workspace_bytes < 0 || (workspace_bytes > 0 && !workspace))
    return W4A16_ERR_INVALID_ARG;
  if (workspace && !aligned(workspace, 64)) return W4A16_ERR_MISALIGNED;
  if (workspace && workspace_bytes > 0) {
    const int64_t G = K / W4A16_GROUP;
    if (ranges_overlap(workspace, workspace_bytes, X, ((M - 1) * ldx + K) * 2) ||
        ranges_overlap(workspace, workspace_bytes, Y, ((M - 1) * ldy + N) * 2) ||
        ranges_overlap(workspace, workspace_bytes, codes, N * (K / 2)) ||
        ranges_overlap(workspace, workspace_bytes, scales, N * G * 2) ||
        ranges_overlap(workspace, workspace_bytes, zeros, N * G * 4))
      return W4A16_ERR_INVALID_ARG;
  }
  if (int dc = device_check()) return dc;
  return w4a16::launch_gemv(X, M, ldx, codes, scales, zeros, N, K, W4A16_GROUP, Y, ldy, workspace,
                            workspace_bytes, (hipStream_t)stream);
}

int w4a16_gemv_grouped(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                       const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K,
                       int64_t group, uint16_t* Y, int64_t ldy, void* stream) {
  int st = check_matmul(X, M, ldx, codes, scales, zeros, N, K, Y, ldy, group);
  if (st != W4A16_OK) return st;
  if (M > W4A16_GEMV_MAX_M) return W4A16_ERR_INVALID_ARG;
  if (M > 8 && (st = check_gemm_limits(M, N, K, ldx)) != W4A16_OK) return st;   // the GEMM runs M > 8
  if (int dc = device_check()) return dc;
  return w4a16::launch_gemv(X, M, ldx, codes, scales, zeros, N, K, (int)group, Y, ldy, nullptr, 0,
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

int w4a16_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t* bytes) {
  if (!bytes) return W4A16_ERR_INVALID_ARG;
  *bytes = 0;
  if (M < 1 || N < 1 || K < W4A16_GROUP || K % W4A16_GROUP) return W4A16_ERR_INVALID_ARG;
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return W4A16_ERR_UNSUPPORTED;
  if (int dc = device_check()) return dc;   // the plan depends on the device's CU count
  *bytes = w4a16::gemm_workspace_bytes(M, N, K);
  return W4A16_OK;
}

int w4a16_gemm_ws(const uint16_t* X, int64_t M, int64_t ldx, const uint32_t* codes,
                  const uint16_t* scales, const int32_t* zeros, int64_t N, int64_t K, uint16_t* Y,
                  int64_t ldy, void* workspace, int64_t workspace_bytes, void* stream) {
  int st = check_matmul(X, M, ldx, codes, scales, zeros, N, K, Y, ldy);
  if (st != W4A16_OK) return st;
  st = check_gemm_limits(M, N, K, ldx);
  if (st != W4A16_OK) return st;
  if (workspace_bytes < 0 || (workspace_bytes > 0 && !workspace)) return W4A16_ERR_INVALID_ARG;
  if (workspace && !aligned(workspace, 16)) return W4A16_ERR_MISALIGNED;
  if (workspace && workspace_bytes > 0) {
    const int64_t G = K / W4A16_GROUP;
    if (ranges_overlap(workspace, workspace_bytes, X, ((M - 1) * ldx + K) * 2) ||
        ranges_overlap(workspace, workspace_bytes, Y, ((M - 1) * ldy + N) * 2) ||
        ranges_overlap(workspace, workspace_bytes, codes, N * (K / 2)) ||
        ranges_overlap(workspace, workspace_bytes, scales, N * G * 2) ||
        ranges_overlap(workspace, workspace_bytes, zeros, N * G * 4))
      return W4A16_ERR_INVALID_ARG;
  }
  if (int dc = device_check()) return dc;
  return w4a16::launch_gemm(X, M, ldx, codes, scales, zeros, N, K, W4A16_GROUP, Y, ldy, (hipStream_t)stream,
                            workspace_bytes > 0 ? workspace : nullptr, workspace_bytes);
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

namespace {
constexpr int64_t kChainHeader = w4a16::kChainHeaderBytes;   // barrier state and status word
constexpr int64_t kChainMaxLds = 160 * 1024;
constexpr int kChainSliceK = 2048;

}  // namespace

int w4a16_chain_workspace_bytes(int n_linears, int64_t* bytes) {
  if (!bytes || n_linears < 1 || n_linears > W4A16_CHAIN_MAX_LINEARS) return W4A16_ERR_INVALID_ARG;
  *bytes = w4a16::kChainDescOffset + (int64_t)n_linears * (int64_t)sizeof(w4a16::ChainDesc);
  return W4A16_OK;
}

namespace {
// Checks of a chain (host array) shared by w4a16_chain_prepare and
// w4a16_chain_run_noalloc.
int chain_check(const w4a16_chain_linear* L, int n, int64_t M) {
  if (!L || n < 1 || n > W4A16_CHAIN_MAX_LINEARS) return W4A16_ERR_INVALID_ARG;
  if (M < 1 || M > W4A16_CHAIN_MAX_M) return W4A16_ERR_INVALID_ARG;
  for (int l = 0; l < n; ++l) {
    const w4a16_chain_linear& a = L[l];
    if (!a.codes || !a.scales || !a.zeros || !a.Y) return W4A16_ERR_INVALID_ARG;
    if (a.N < 1 || a.K < W4A16_GROUP || a.K % W4A16_GROUP || a.ldy < a.N) return W4A16_ERR_INVALID_ARG;
    if (a.N >= kMaxDim || a.K > W4A16_CHAIN_MAX_K) return W4A16_ERR_UNSUPPORTED;
    if (!aligned(a.codes, 16) || !aligned(a.scales, 2) || !aligned(a.zeros, 4) || !aligned(a.Y, 16) ||
        a.ldy % 8 || (a.gamma && !aligned(a.gamma, 16)))
      return W4A16_ERR_MISALIGNED;
    if (a.input < W4A16_CHAIN_X0 || a.input > W4A16_CHAIN_ATTN1) return W4A16_ERR_INVALID_ARG;
    if (l == 0 && a.input != W4A16_CHAIN_X0) return W4A16_ERR_INVALID_ARG;
    if (l > 0) {
      const int64_t pn = L[l - 1].N;
      if (a.input == W4A16_CHAIN_PREV && a.K > pn) return W4A16_ERR_INVALID_ARG;
      if (a.input == W4A16_CHAIN_SWIGLU && 2 * a.K > pn) return W4A16_ERR_INVALID_ARG;
      if (a.input == W4A16_CHAIN_ATTN1) {
        if (a.head_dim < 1 || a.group < 1 || a.v_offset < 0 || a.K % a.head_dim) return W4A16_ERR_INVALID_ARG;
        const int64_t kv_heads = (a.K / a.head_dim - 1) / a.group + 1;
        if (a.v_offset + kv_heads * a.head_dim > pn) return W4A16_ERR_INVALID_ARG;
      }
    }
    // an output may not overlap the matrix, metadata or producer weight it
    // is computed from, nor the output its own input is formed from
    const int64_t ybytes = ((M - 1) * a.ldy + a.N) * 2;
    if (ranges_overlap(a.Y, ybytes, a.codes, a.N * (a.K / 2)) ||
        ranges_overlap(a.Y, ybytes, a.scales, a.N * (a.K / W4A16_GROUP) * 2) ||
        ranges_overlap(a.Y, ybytes, a.zeros, a.N * (a.K / W4A16_GROUP) * 4) ||
        (a.gamma && ranges_overlap(a.Y, ybytes, a.gamma, a.K * 2)) ||
        (l > 0 && ranges_overlap(a.Y, ybytes, L[l - 1].Y, ((M - 1) * L[l - 1].ldy + L[l - 1].N) * 2)))
      return W4A16_ERR_INVALID_ARG;
  }
  return W4A16_OK;
}

// Descriptors (d[0 .. n)) and launch parameters of a checked chain.
int chain_build(const w4a16_chain_linear* L, int n, int64_t M, w4a16::ChainDesc* d, w4a16_chain_plan* plan) {
  const int grid = w4a16::device_cu_count();
  int64_t max_k = 0, max_rows = 0, max_slices = 0, kx = 0;
  for (int l = 0; l < n; ++l) {
    const w4a16_chain_linear& a = L[l];
    w4a16::ChainDesc& e = d[l];
    e.codes = a.codes; e.scales = a.scales; e.zeros = a.zeros; e.gamma = a.gamma; e.y = a.Y; e.ldy = a.ldy;
    e.N = (int32_t)a.N; e.K = (int32_t)a.K; e.input = a.input;
    e.v_offset = a.v_offset; e.head_dim = a.head_dim; e.group = a.group;
    // a producer of exactly [gate | up] for a SwiGLU consumer pairs its rows
    // (gate k and up pair + k in one block) and forms that input once
    const bool paired = l + 1 < n && L[l + 1].input == W4A16_CHAIN_SWIGLU && a.N == 2 * L[l + 1].K;
    e.pair = paired ? (int32_t)L[l + 1].K : 0;
    e.glued = (l > 0 && a.input == W4A16_CHAIN_SWIGLU && L[l - 1].N == 2 * a.K) ? 1 : 0;
    const int64_t batches = paired ? L[l + 1].K / 4 : (a.N + 3) / 4;
    e.batches_per_block = (int32_t)(batches / grid);
    e.batches_rem = (int32_t)(batches % grid);
    e.slices = (int32_t)((a.K + kChainSliceK - 1) / kChainSliceK);
    e.pad = 0;
    max_k = std::max<int64_t>(max_k, a.K);
    max_rows = std::max<int64_t>(max_rows, (paired ? 8 : 4) * (e.batches_per_block + (e.batches_rem ? 1 : 0)));
    max_slices = std::max<int64_t>(max_slices, e.slices);
    if (a.input == W4A16_CHAIN_X0) kx = std::max<int64_t>(kx, a.K);   // the widest read of X0
  }
  const int64_t lds = M * (max_k / kChainSliceK + 1) * 4096 + M * (max_k / 32) * 4 + max_slices * max_rows * M * 4;
  if (lds > kChainMaxLds) return W4A16_ERR_UNSUPPORTED;
  plan->n_linears = n;
  plan->M = (int32_t)M;
  plan->grid = grid;
  plan->max_k = (int32_t)max_k;
  plan->max_rows = (int32_t)max_rows;
  plan->k0 = (int32_t)kx;
  plan->spin_limit = W4A16_CHAIN_SPIN_LIMIT;
  plan->reserved = 0;
  plan->lds_bytes = lds;
  return W4A16_OK;
}
}  // namespace

int w4a16_chain_prepare(const w4a16_chain_linear* L, int n, int64_t M, void* workspace, int64_t ws_bytes,
                        w4a16_chain_plan* plan, void* stream) {
  int64_t need = 0;
  if (!L || !plan || !workspace) return W4A16_ERR_INVALID_ARG;
  if (w4a16_chain_workspace_bytes(n, &need) != W4A16_OK || ws_bytes < need) return W4A16_ERR_INVALID_ARG;
  if (!aligned(workspace, 256)) return W4A16_ERR_MISALIGNED;
  if (int st = chain_check(L, n, M)) return st;
  if (int dc = device_check()) return dc;
  std::vector<w4a16::ChainDesc> d((size_t)n);
  w4a16_chain_plan p{};
  if (int st = chain_build(L, n, M, d.data(), &p)) return st;
  hipStream_t s = (hipStream_t)stream;
  char* ws = static_cast<char*>(workspace);
  if (hipMemsetAsync(ws, 0, kChainHeader, s) != hipSuccess ||
      hipMemcpyAsync(ws + w4a16::kChainDescOffset, d.data(), d.size() * sizeof(w4a16::ChainDesc), hipMemcpyHostToDevice, s) !=
          hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return W4A16_ERR_HIP;
  p.workspace = workspace;
  *plan = p;
  return W4A16_OK;
}

int w4a16_chain_run_noalloc(const w4a16_chain_linear* L, int n, int64_t M, const uint16_t* X0, int64_t ldx,
                            int* status, void* stream) {
  if (!X0) return W4A16_ERR_INVALID_ARG;
  if (n > W4A16_CHAIN_NOALLOC_MAX_LINEARS) return W4A16_ERR_UNSUPPORTED;
  if (int st = chain_check(L, n, M)) return st;
  if (!aligned(X0, 16) || ldx % 8) return W4A16_ERR_MISALIGNED;
  if (int dc = device_check()) return dc;
  w4a16::ChainDesc d[W4A16_CHAIN_NOALLOC_MAX_LINEARS];   // host staging on the stack: nothing allocated
  w4a16_chain_plan p{};
  if (int st = chain_build(L, n, M, d, &p)) return st;
  if (ldx < p.k0) return W4A16_ERR_INVALID_ARG;
  return w4a16::launch_chain_noalloc(d, n, (int)M, X0, ldx, p.max_k, p.max_rows, p.grid, (size_t)p.lds_bytes,
                                     status, (hipStream_t)stream);
}

int w4a16_chain_run(const w4a16_chain_plan* plan, const uint16_t* X0, int64_t ldx, void* stream) {
  if (!plan || !plan->workspace || !X0) return W4A16_ERR_INVALID_ARG;
  if (plan->n_linears < 1 || plan->n_linears > W4A16_CHAIN_MAX_LINEARS || plan->M < 1 ||
      plan->M > W4A16_CHAIN_MAX_M || plan->grid < 1 || plan->max_k < W4A16_GROUP ||
      plan->max_k > W4A16_CHAIN_MAX_K || plan->max_rows < 4 || plan->lds_bytes < 1 ||
      plan->lds_bytes > kChainMaxLds || plan->spin_limit < 0 || ldx < plan->k0)
    return W4A16_ERR_INVALID_ARG;
  if (!aligned(X0, 16) || ldx % 8 || !aligned(plan->workspace, 256)) return W4A16_ERR_MISALIGNED;
  if (int dc = device_check()) return dc;
  char* ws = static_cast<char*>(plan->workspace);
  return w4a16::launch_chain(ws + w4a16::kChainDescOffset, plan->n_linears, plan->M, X0, ldx,
                             reinterpret_cast<unsigned*>(ws), plan->spin_limit, plan->max_k, plan->max_rows,
                             plan->grid, (size_t)plan->lds_bytes, (hipStream_t)stream);
}

int w4a16_chain_status(const w4a16_chain_plan* plan, int* status, void* stream) {
  if (!plan || !plan->workspace || !status) return W4A16_ERR_INVALID_ARG;
  if (int dc = device_check()) return dc;
  hipStream_t s = (hipStream_t)stream;
  // after a timeout the barrier count may be left mid-way: the whole barrier
  // state is cleared (runs read the generation they start from)
  char* header = static_cast<char*>(plan->workspace);
  unsigned v = 0;
  if (hipStreamSynchronize(s) != hipSuccess ||
      hipMemcpy(&v, header + w4a16::kChainStatusWord * 4, 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemset(header, 0, kChainHeader) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
    return W4A16_ERR_HIP;
  *status = (int)v;
  return W4A16_OK;
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
