// The backward's two gradient GEMMs: dX = dY + [dQ dK dV] theta and
// dtheta (+)= [dQ dK dV]^T X (the outer-loop projections of "One-Minute Video
// Generation with Test-Time Training", paper-notes page, key designs
// "TTT-MLP layer": theta_K, theta_V, theta_Q learned through the layer).  They
// are plain fp32 GEMMs, so they run on rocBLAS (rocblas_gemm_ex_64, fp32
// operands, fp32 accumulation, its fp32 matrix-core kernels).  bf16 operands
// (X, X' and theta when the io dtype is bf16) are widened exactly to fp32 in the
// caller's workspace first.
//
// rocBLAS takes column-major matrices; a row-major [R, C] matrix is the
// column-major [C, R] one, so row-major C = A B is computed as C^T = B^T A^T.
//
// Each device gets two handles, created on first use: one for the caller's
// stream and one for the library's side stream (a bidirectional backward runs
// the reversed pass's dtheta GEMM there beside other work), each pointed at its
// own slice of the caller's workspace on every call, so that rocBLAS allocates
// nothing on a call.
#include <rocblas/rocblas.h>

#include <map>
#include <mutex>

#include "internal.h"

namespace ttt {
namespace {

__global__ void widen_bf16_kernel(const uint16_t* in, float* out, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = __uint_as_float((uint32_t)in[i] << 16);
}

struct Handles {
  rocblas_handle h[2] = {nullptr, nullptr};
};
std::mutex g_mu;  // held while a call configures a handle and enqueues on it
std::map<int, Handles> g_handles;

const char* status_text(rocblas_status st) { return rocblas_status_to_string(st); }

// The handle `slot` of the current device (created on first use), set to `s` and
// to the workspace slice [ws, ws + ws_bytes); call with g_mu held.
rocblas_status handle_for(int slot, hipStream_t s, void* ws, size_t ws_bytes, rocblas_handle* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return rocblas_status_internal_error;
  Handles& hs = g_handles[dev];
  if (!hs.h[slot]) {
    rocblas_status st = rocblas_create_handle(&hs.h[slot]);
    if (st != rocblas_status_success) {
      hs.h[slot] = nullptr;
      return st;
    }
  }
  rocblas_status st = rocblas_set_stream(hs.h[slot], s);
  if (st == rocblas_status_success) st = rocblas_set_workspace(hs.h[slot], ws, ws_bytes);
  *out = hs.h[slot];
  return st;
}

}  // namespace

size_t grad_gemm_workspace_bytes() { return (size_t)256 << 20; }

hipError_t widen_bf16(const uint16_t* in, float* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(widen_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, in, out, n);
  return hipGetLastError();
}

// dX [BT, D] = dY [BT, D] + dQKV [BT, 3D] theta [3D, D], row-major, fp32.
const char* grad_gemm_dx(int slot, const float* dqkv, const float* theta32, const float* dy, float* dx, int64_t BT,
                         int64_t D, void* ws, size_t ws_bytes, hipStream_t s) {
  if (BT == 0 || D == 0) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  rocblas_handle h = nullptr;
  rocblas_status st = handle_for(slot, s, ws, ws_bytes, &h);
  const float one = 1.0f;
  // column-major: dX^T [D, BT] = theta^T [D, 3D] dQKV^T [3D, BT] + dY^T
  if (st == rocblas_status_success)
    st = rocblas_gemm_ex_64(h, rocblas_operation_none, rocblas_operation_none, D, BT, 3 * D, &one, theta32,
                            rocblas_datatype_f32_r, D, dqkv, rocblas_datatype_f32_r, 3 * D, &one, dy,
                            rocblas_datatype_f32_r, D, dx, rocblas_datatype_f32_r, D, rocblas_datatype_f32_r,
                            rocblas_gemm_algo_standard, 0, 0);
  return st == rocblas_status_success ? nullptr : status_text(st);
}

// dtheta [3D, D] = (accumulate ? dtheta : 0) + dQKV^T [3D, BT] X [BT, D], row-major, fp32.
const char* grad_gemm_dtheta(int slot, const float* dqkv, const float* x32, float* dtheta, int64_t BT, int64_t D,
                             int accumulate, void* ws, size_t ws_bytes, hipStream_t s) {
  if (D == 0) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  rocblas_handle h = nullptr;
  rocblas_status st = handle_for(slot, s, ws, ws_bytes, &h);
  const float one = 1.0f, beta = accumulate ? 1.0f : 0.0f;
  // column-major: dtheta^T [D, 3D] = X^T [D, BT] (dQKV^T)^T, dQKV^T stored as the column-major [3D, BT]
  if (st == rocblas_status_success)
    st = rocblas_gemm_ex_64(h, rocblas_operation_none, rocblas_operation_transpose, D, 3 * D, BT, &one, x32,
                            rocblas_datatype_f32_r, D, dqkv, rocblas_datatype_f32_r, 3 * D, &beta, dtheta,
                            rocblas_datatype_f32_r, D, dtheta, rocblas_datatype_f32_r, D, rocblas_datatype_f32_r,
                            rocblas_gemm_algo_standard, 0, 0);
  return st == rocblas_status_success ? nullptr : status_text(st);
}

}  // namespace ttt
