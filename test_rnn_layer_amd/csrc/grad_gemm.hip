// The backward's two gradient GEMMs: dX = dY + [dQ dK dV] theta and
// dtheta (+)= [dQ dK dV]^T X (the outer-loop projections of "One-Minute Video
// Generation with Test-Time Training", paper-notes page, key designs
// "TTT-MLP layer": theta_K, theta_V, theta_Q learned through the layer).  They
// are plain GEMMs, so they run on rocBLAS (rocblas_gemm_ex_64, fp32 accumulation).
//
// With fp32 io all operands are fp32 and the GEMMs run on rocBLAS's fp32
// matrix-core kernels.  With bf16 io, X, X' and theta are exact bf16 numbers and
// only dQKV is fp32.  Then dQKV is split exactly into three bf16 parts,
// x = h + m + l (h: x with its low 16 bits cleared, m: the same of x - h, l: the
// rest, which has at most 8 significant bits, so the split is exact for
// |x| >= 2^-103), and the GEMMs run on the bf16 matrix cores with fp32
// accumulation: every product of two bf16 numbers is exact in fp32, so the
// result has the accuracy of an fp32 GEMM at a third of the bf16 rate, about
// five times the fp32 matrix-core rate.  dX takes the three parts as one
// contraction of length 9D against theta stacked three times; dtheta is one
// product over the 9D columns of the parts, whose three blocks are then added
// smallest first.
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

// x -> (h, m, l), bf16 bit patterns with h + m + l = x; Inf and NaN go to h alone
// (NaN as a quiet NaN), their m and l are zero.
__device__ inline void split3(float x, uint32_t& h, uint32_t& m, uint32_t& l) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7F800000u) == 0x7F800000u) {
    h = (u & 0x007FFFFFu) ? 0x7FC0u : u >> 16;
    m = l = 0;
    return;
  }
  h = u >> 16;
  const float r = x - __uint_as_float(h << 16);  // exact: the low 16 bits of x
  m = __float_as_uint(r) >> 16;
  const float q = r - __uint_as_float(m << 16);  // exact, at most 8 significant bits
  l = __float_as_uint(q) >> 16;
}

// in: row-major [rows, cols] fp32, cols % 4 == 0; out: row-major [rows, 3 cols] bf16,
// row r = [h | m | l] of in's row r.  Block x covers 256 float4 columns of a row.
// (in2, when given: [rows, add4 float4] added first to the row's first add4 float4 of in)
__global__ void split_bf16x3_kernel(const float4* __restrict__ in, const float4* __restrict__ in2,
                                    uint2* __restrict__ out, int64_t rows, int64_t cols4, int64_t add4) {
  const int64_t c4 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c4 >= cols4) return;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    float4 v = in[r * cols4 + c4];
    if (in2 && c4 < add4) {
      const float4 w = in2[r * add4 + c4];
      v = make_float4(v.x + w.x, v.y + w.y, v.z + w.z, v.w + w.w);
    }
    uint32_t h[4], m[4], l[4];
    split3(v.x, h[0], m[0], l[0]);
    split3(v.y, h[1], m[1], l[1]);
    split3(v.z, h[2], m[2], l[2]);
    split3(v.w, h[3], m[3], l[3]);
    uint2* o = out + r * 3 * cols4 + c4;
    o[0] = make_uint2(h[0] | h[1] << 16, h[2] | h[3] << 16);
    o[cols4] = make_uint2(m[0] | m[1] << 16, m[2] | m[3] << 16);
    o[2 * cols4] = make_uint2(l[0] | l[1] << 16, l[2] | l[3] << 16);
  }
}

// out[i] = (((accumulate ? out[i] : 0) + p[2 n + i]) + p[n + i]) + p[i]: the three parts' products
// added smallest first (p: [3][n] fp32)
__global__ void sum3_kernel(const float* __restrict__ p, float* __restrict__ out, int64_t n, int accumulate) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float base = accumulate ? out[i] : 0.0f;
    out[i] = ((base + p[2 * n + i]) + p[n + i]) + p[i];
  }
}

// out[j n + i] = in[i] for j < 3 (n 16-bit elements)
__global__ void stack3_u16_kernel(const uint16_t* __restrict__ in, uint16_t* __restrict__ out, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint16_t v = in[i];
    out[i] = v;
    out[n + i] = v;
    out[2 * n + i] = v;
  }
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

hipError_t split_bf16x3(const float* in, const float* in2, int64_t cols2, uint16_t* out, int64_t rows, int64_t cols,
                        hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (cols % 4 != 0 || (in2 && (cols2 % 4 != 0 || cols2 > cols))) return hipErrorInvalidValue;
  const int64_t cols4 = cols / 4;
  const dim3 grid((unsigned)((cols4 + 255) / 256), (unsigned)std::min<int64_t>(rows, 8192));
  hipLaunchKernelGGL(split_bf16x3_kernel, grid, dim3(256), 0, s, (const float4*)in, (const float4*)in2, (uint2*)out,
                     rows, cols4, in2 ? cols2 / 4 : (int64_t)0);
  return hipGetLastError();
}

hipError_t stack3_u16(const uint16_t* in, uint16_t* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(stack3_u16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, in, out, n);
  return hipGetLastError();
}

// dX [BT, D] = dY [BT, D] + S [BT, 9D] theta3 [9D, D], row-major; S = [h | m | l] of dQKV
// (bf16), theta3 = theta stacked three times (bf16), fp32 accumulation and output.
const char* grad_gemm_dx_split(int slot, const uint16_t* sp, const uint16_t* theta3, const float* dy, float* dx,
                               int64_t BT, int64_t D, void* ws, size_t ws_bytes, hipStream_t s) {
  if (BT == 0 || D == 0) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  rocblas_handle h = nullptr;
  rocblas_status st = handle_for(slot, s, ws, ws_bytes, &h);
  const float one = 1.0f;
  // column-major: dX^T [D, BT] = theta3^T [D, 9D] S^T [9D, BT] + dY^T
  if (st == rocblas_status_success)
    st = rocblas_gemm_ex_64(h, rocblas_operation_none, rocblas_operation_none, D, BT, 9 * D, &one, theta3,
                            rocblas_datatype_bf16_r, D, sp, rocblas_datatype_bf16_r, 9 * D, &one, dy,
                            rocblas_datatype_f32_r, D, dx, rocblas_datatype_f32_r, D, rocblas_datatype_f32_r,
                            rocblas_gemm_algo_standard, 0, 0);
  return st == rocblas_status_success ? nullptr : status_text(st);
}

// dtheta [3D, D] = (accumulate ? dtheta : 0) + l^T X + m^T X + h^T X, with h, m, l the column
// blocks of S [BT, 9D] (bf16) and X [BT, D] bf16; fp32 accumulation and output.  One GEMM writes
// the three products S^T X into p3 ([9D, D] fp32; one product over the 9D columns keeps every CU
// busy, where three of 3D columns each left a third of the tiles' last round empty), then they
// are added smallest first.
const char* grad_gemm_dtheta_split(int slot, const uint16_t* sp, const uint16_t* x16, float* dtheta, float* p3,
                                   int64_t BT, int64_t D, int accumulate, void* ws, size_t ws_bytes, hipStream_t s) {
  if (D == 0) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  rocblas_handle h = nullptr;
  rocblas_status st = handle_for(slot, s, ws, ws_bytes, &h);
  const float one = 1.0f, zero = 0.0f;
  // column-major: p3^T [D, 9D] = X^T [D, BT] (S^T)^T, S^T the column-major [9D, BT]
  if (st == rocblas_status_success)
    st = rocblas_gemm_ex_64(h, rocblas_operation_none, rocblas_operation_transpose, D, 9 * D, BT, &one, x16,
                            rocblas_datatype_bf16_r, D, sp, rocblas_datatype_bf16_r, 9 * D, &zero, p3,
                            rocblas_datatype_f32_r, D, p3, rocblas_datatype_f32_r, D, rocblas_datatype_f32_r,
                            rocblas_gemm_algo_standard, 0, 0);
  if (st != rocblas_status_success) return status_text(st);
  const int64_t n = 3 * D * D, blocks = std::min<int64_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(sum3_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p3, dtheta, n, accumulate);
  return hipGetLastError() == hipSuccess ? nullptr : "sum3 launch failed";
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
