// Generic kernels: an fp32-accumulating projection GEMM with fp32 output and
// an fp32 VALU scan that supports every shape whose mini-batch working set
// fits in LDS.  They serve the fp32 configurations and act as the plain
// reference for the MFMA path.
//
// The scan computes one direction of the TTT-MLP layer ("One-Minute Video
// Generation with Test-Time Training", paper-notes page, key designs,
// "TTT-MLP layer" and "gate + bidirectional") in the mini-batch dual form:
// for a mini-batch of n tokens starting at state (W1, W2),
//   A  = K W1,  Hk = GELU(A),  G2 = c (Hk W2 - V),  G1 = (G2 W2^T) * GELU'(A)
//   Aq = Q W1 - eta tril(Q K^T) G1,   Hq = GELU(Aq)
//   Z  = Hq W2 - eta tril(Hq Hk^T) G2
//   W1 -= eta K^T G1,   W2 -= eta Hk^T G2
// which equals reading out each token with the state after the summed
// gradient steps of the tokens up to and including it (tril keeps the
// diagonal).  Then y = x + tanh(alpha) * z per channel.
#include "internal.h"

namespace ttt {
namespace {

__device__ inline float load_io(const void* p, int64_t i, int bf16) {
  if (bf16) return __uint_as_float((uint32_t)(((const uint16_t*)p)[i]) << 16);
  return ((const float*)p)[i];
}

__device__ inline uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // keep NaN a NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ inline void store_io(void* p, int64_t i, float v, int bf16) {
  if (bf16)
    ((uint16_t*)p)[i] = bf16_rne(v);
  else
    ((float*)p)[i] = v;
}

// GELU and its derivative.  erf form: GELU(a) = a Phi(a), GELU'(a) = Phi(a) + a phi(a).
__device__ inline float gelu_f(float a, int tanh_form) {
  if (tanh_form) {
    const float u = 0.7978845608028654f * (a + 0.044715f * a * a * a);
    return 0.5f * a * (1.0f + tanhf(u));
  }
  return 0.5f * a * (1.0f + erff(a * 0.7071067811865476f));
}

__device__ inline void gelu_and_grad(float a, int tanh_form, float* g, float* dg) {
  if (tanh_form) {
    const float u = 0.7978845608028654f * (a + 0.044715f * a * a * a);
    const float th = tanhf(u);
    const float du = 0.7978845608028654f * (1.0f + 3.0f * 0.044715f * a * a);
    *g = 0.5f * a * (1.0f + th);
    *dg = 0.5f * (1.0f + th) + 0.5f * a * (1.0f - th * th) * du;
    return;
  }
  const float cdf = 0.5f * (1.0f + erff(a * 0.7071067811865476f));
  *g = a * cdf;
  *dg = cdf + a * 0.3989422804014327f * expf(-0.5f * a * a);
}

// ---------------------------------------------------------------------------
// projection: out[p, s, h, t, j] = sum_i X[s, t, i] theta[p, h*d + j, i]
// ---------------------------------------------------------------------------
constexpr int PT_M = 64, PT_N = 64, PT_K = 16;

__global__ __launch_bounds__(256) void project_f32out_kernel(ProjArgs a) {
  __shared__ float As[PT_K][PT_M + 4];
  __shared__ float Bs[PT_K][PT_N + 4];
  const int D = a.H * a.d;
  const int64_t M = a.B * a.T;
  const int N = 3 * D;
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  const int64_t m0 = (int64_t)blockIdx.x * PT_M;
  const int n0 = blockIdx.y * PT_N;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < D; k0 += PT_K) {
    for (int i = tid; i < PT_M * PT_K; i += 256) {
      const int r = i / PT_K, c = i % PT_K;
      const int64_t gr = m0 + r;
      const int gc = k0 + c;
      As[c][r] = (gr < M && gc < D) ? load_io(a.X, gr * D + gc, a.bf16) : 0.0f;
      const int gn = n0 + r;
      Bs[c][r] = (gn < N && gc < D) ? load_io(a.theta, (int64_t)gn * D + gc, a.bf16) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PT_K; ++k) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* out = (float*)a.out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t gr = m0 + ty * 4 + i;
    if (gr >= M) continue;
    const int64_t s = gr / a.T, t = gr % a.T;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tx * 4 + j;
      if (gn >= N) continue;
      const int p = gn / D, rem = gn % D, h = rem / a.d, jj = rem % a.d;
      out[((((int64_t)p * a.B + s) * a.H + h) * a.T + t) * a.d + jj] = acc[i][j];
    }
  }
}

// ---------------------------------------------------------------------------
// generic scan: one workgroup per (sequence, head)
// ---------------------------------------------------------------------------
constexpr int GS_THREADS = 256;

__global__ __launch_bounds__(GS_THREADS) void scan_generic_kernel(ScanArgs a) {
  extern __shared__ float lds[];
  const int d = a.d, m = a.m, b = a.b, tid = threadIdx.x;
  const int64_t T = a.T;
  const int s = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int D = a.H * d;
  const float eta = a.eta;

  float* Ks = lds;          // [b, d]
  float* Qs = Ks + b * d;   // [b, d]
  float* Vs = Qs + b * d;   // [b, d]; becomes G2
  float* Hk = Vs + b * d;   // [b, m]
  float* Dg = Hk + b * m;   // [b, m] GELU'(A); becomes G1
  float* Hq = Dg + b * m;   // [b, m]
  float* S = Hq + b * m;    // [b, b] tril(Q K^T)
  float* P = S + b * b;     // [b, b] tril(Hq Hk^T)

  float* W1 = a.wstate + ((int64_t)s * a.H + h) * (2LL * d * m);
  float* W2 = W1 + (int64_t)d * m;
  const float* w10 = a.w1_0 + (int64_t)h * d * m;
  const float* w20 = a.w2_0 + (int64_t)h * m * d;
  for (int i = tid; i < d * m; i += GS_THREADS) {
    W1[i] = w10[i];
    W2[i] = w20[i];
  }
  __syncthreads();

  const int64_t plane = a.B * a.H * T * d;
  const float* qb = a.qkv + ((int64_t)s * a.H + h) * T * d;
  const float* kb = qb + plane;
  const float* vb = kb + plane;

  for (int64_t n0 = 0; n0 < T; n0 += b) {
    const int n = (int)((T - n0) < b ? (T - n0) : b);
    for (int i = tid; i < n * d; i += GS_THREADS) {
      const int r = i / d, j = i % d;
      const int64_t t = a.reverse ? T - 1 - (n0 + r) : n0 + r;
      Ks[r * d + j] = kb[t * d + j];
      Qs[r * d + j] = qb[t * d + j];
      Vs[r * d + j] = vb[t * d + j];
    }
    __syncthreads();
    // A = K W1 -> Hk, GELU'(A)
    for (int i = tid; i < n * m; i += GS_THREADS) {
      const int r = i / m, j = i % m;
      float acc = 0.0f;
      for (int k = 0; k < d; ++k) acc = fmaf(Ks[r * d + k], W1[k * m + j], acc);
      float g, dg;
      gelu_and_grad(acc, a.gelu_tanh, &g, &dg);
      Hk[r * m + j] = g;
      Dg[r * m + j] = dg;
    }
    __syncthreads();
    // G2 = c (Hk W2 - V), in place of V
    for (int i = tid; i < n * d; i += GS_THREADS) {
      const int r = i / d, j = i % d;
      float acc = 0.0f;
      for (int k = 0; k < m; ++k) acc = fmaf(Hk[r * m + k], W2[k * d + j], acc);
      Vs[r * d + j] = a.gscale * (acc - Vs[r * d + j]);
    }
    __syncthreads();
    // G1 = (G2 W2^T) * GELU'(A), in place of GELU'(A); S = tril(Q K^T)
    for (int i = tid; i < n * m; i += GS_THREADS) {
      const int r = i / m, j = i % m;
      float acc = 0.0f;
      for (int k = 0; k < d; ++k) acc = fmaf(Vs[r * d + k], W2[j * d + k], acc);
      Dg[r * m + j] *= acc;
    }
    for (int i = tid; i < n * n; i += GS_THREADS) {
      const int r = i / n, c = i % n;
      float acc = 0.0f;
      if (c <= r)
        for (int k = 0; k < d; ++k) acc = fmaf(Qs[r * d + k], Ks[c * d + k], acc);
      S[r * b + c] = acc;
    }
    __syncthreads();
    // Hq = GELU(Q W1 - eta tril(Q K^T) G1)
    for (int i = tid; i < n * m; i += GS_THREADS) {
      const int r = i / m, j = i % m;
      float acc = 0.0f, corr = 0.0f;
      for (int k = 0; k < d; ++k) acc = fmaf(Qs[r * d + k], W1[k * m + j], acc);
      for (int c = 0; c <= r; ++c) corr = fmaf(S[r * b + c], Dg[c * m + j], corr);
      Hq[r * m + j] = gelu_f(acc - eta * corr, a.gelu_tanh);
    }
    __syncthreads();
    // P = tril(Hq Hk^T)
    for (int i = tid; i < n * n; i += GS_THREADS) {
      const int r = i / n, c = i % n;
      float acc = 0.0f;
      if (c <= r)
        for (int k = 0; k < m; ++k) acc = fmaf(Hq[r * m + k], Hk[c * m + k], acc);
      P[r * b + c] = acc;
    }
    __syncthreads();
    // Z = Hq W2 - eta tril(Hq Hk^T) G2, then the gate
    for (int i = tid; i < n * d; i += GS_THREADS) {
      const int r = i / d, j = i % d;
      float acc = 0.0f, corr = 0.0f;
      for (int k = 0; k < m; ++k) acc = fmaf(Hq[r * m + k], W2[k * d + j], acc);
      for (int c = 0; c <= r; ++c) corr = fmaf(P[r * b + c], Vs[c * d + j], corr);
      const float z = acc - eta * corr;
      const int64_t t = a.reverse ? T - 1 - (n0 + r) : n0 + r;
      const int64_t o = ((int64_t)s * T + t) * D + (int64_t)h * d + j;
      if (a.z) a.z[o] = z;
      const float x = load_io(a.xin, o, a.bf16);
      store_io(a.y, o, x + tanhf(a.alpha[h * d + j]) * z, a.bf16);
    }
    __syncthreads();
    // W1 -= eta K^T G1 ; W2 -= eta Hk^T G2
    for (int i = tid; i < d * m; i += GS_THREADS) {
      const int k = i / m, j = i % m;
      float acc = 0.0f;
      for (int r = 0; r < n; ++r) acc = fmaf(Ks[r * d + k], Dg[r * m + j], acc);
      W1[i] -= eta * acc;
    }
    for (int i = tid; i < m * d; i += GS_THREADS) {
      const int k = i / d, j = i % d;
      float acc = 0.0f;
      for (int r = 0; r < n; ++r) acc = fmaf(Hk[r * m + k], Vs[r * d + j], acc);
      W2[i] -= eta * acc;
    }
    __syncthreads();
  }
  if (a.w1_T) {
    float* o = a.w1_T + ((int64_t)s * a.H + h) * d * m;
    for (int i = tid; i < d * m; i += GS_THREADS) o[i] = W1[i];
  }
  if (a.w2_T) {
    float* o = a.w2_T + ((int64_t)s * a.H + h) * m * d;
    for (int i = tid; i < m * d; i += GS_THREADS) o[i] = W2[i];
  }
}

// ---------------------------------------------------------------------------
// generic linear scan (inner model f(u; W) = u W, W: d x d): one workgroup per
// (sequence, head), the mini-batch dual form G = c (K W - V),
// Z = Q W - eta tril(Q K^T) G, W -= eta K^T G, with W the state the mini-batch
// starts from
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(GS_THREADS) void scan_linear_generic_kernel(ScanArgs a) {
  extern __shared__ float lds[];
  const int d = a.d, b = a.b, tid = threadIdx.x;
  const int64_t T = a.T;
  const int s = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int D = a.H * d;
  const float eta = a.eta;

  float* Ks = lds;         // [b, d]
  float* Qs = Ks + b * d;  // [b, d]
  float* Vs = Qs + b * d;  // [b, d]; becomes G
  float* S = Vs + b * d;   // [b, b] tril(Q K^T), diagonal included

  float* W = a.wstate + ((int64_t)s * a.H + h) * (int64_t)d * d;
  const float* w0 = a.w1_0 + (int64_t)h * d * d;
  for (int i = tid; i < d * d; i += GS_THREADS) W[i] = w0[i];
  __syncthreads();

  const int64_t plane = a.B * a.H * T * d;
  const float* qb = a.qkv + ((int64_t)s * a.H + h) * T * d;
  const float* kb = qb + plane;
  const float* vb = kb + plane;

  for (int64_t n0 = 0; n0 < T; n0 += b) {
    const int n = (int)((T - n0) < b ? (T - n0) : b);
    for (int i = tid; i < n * d; i += GS_THREADS) {
      const int r = i / d, j = i % d;
      const int64_t t = a.reverse ? T - 1 - (n0 + r) : n0 + r;
      Ks[r * d + j] = kb[t * d + j];
      Qs[r * d + j] = qb[t * d + j];
      Vs[r * d + j] = vb[t * d + j];
    }
    __syncthreads();
    // G = c (K W - V), in place of V; S = tril(Q K^T)
    for (int i = tid; i < n * d; i += GS_THREADS) {
      const int r = i / d, j = i % d;
      float acc = 0.0f;
      for (int k = 0; k < d; ++k) acc = fmaf(Ks[r * d + k], W[k * d + j], acc);
      Vs[r * d + j] = a.gscale * (acc - Vs[r * d + j]);
    }
    for (int i = tid; i < n * n; i += GS_THREADS) {
      const int r = i / n, c = i % n;
      float acc = 0.0f;
      if (c <= r)
        for (int k = 0; k < d; ++k) acc = fmaf(Qs[r * d + k], Ks[c * d + k], acc);
      S[r * b + c] = acc;
    }
    __syncthreads();
    // Z = Q W - eta tril(Q K^T) G, then the gate
    for (int i = tid; i < n * d; i += GS_THREADS) {
      const int r = i / d, j = i % d;
      float acc = 0.0f, corr = 0.0f;
      for (int k = 0; k < d; ++k) acc = fmaf(Qs[r * d + k], W[k * d + j], acc);
      for (int c = 0; c <= r; ++c) corr = fmaf(S[r * b + c], Vs[c * d + j], corr);
      const float z = acc - eta * corr;
      const int64_t t = a.reverse ? T - 1 - (n0 + r) : n0 + r;
      const int64_t o = ((int64_t)s * T + t) * D + (int64_t)h * d + j;
      if (a.z) a.z[o] = z;
      const float x = load_io(a.xin, o, a.bf16);
      store_io(a.y, o, x + tanhf(a.alpha[h * d + j]) * z, a.bf16);
    }
    __syncthreads();
    // W -= eta K^T G
    for (int i = tid; i < d * d; i += GS_THREADS) {
      const int k = i / d, j = i % d;
      float acc = 0.0f;
      for (int r = 0; r < n; ++r) acc = fmaf(Ks[r * d + k], Vs[r * d + j], acc);
      W[i] -= eta * acc;
    }
    __syncthreads();
  }
  if (a.w1_T) {
    float* o = a.w1_T + ((int64_t)s * a.H + h) * (int64_t)d * d;
    for (int i = tid; i < d * d; i += GS_THREADS) o[i] = W[i];
  }
}

}  // namespace

hipError_t launch_project_f32out(const ProjArgs& a, hipStream_t s) {
  const int64_t M = a.B * a.T;
  const int N = 3 * a.H * a.d;
  if (M == 0) return hipSuccess;
  dim3 grid((unsigned)((M + PT_M - 1) / PT_M), (unsigned)((N + PT_N - 1) / PT_N));
  hipLaunchKernelGGL(project_f32out_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

size_t scan_generic_lds_bytes(int d, int m, int b) {
  return sizeof(float) * ((size_t)3 * b * d + (size_t)3 * b * m + (size_t)2 * b * b);
}

hipError_t launch_scan_generic(const ScanArgs& a, hipStream_t s) {
  const size_t lds = scan_generic_lds_bytes(a.d, a.m, a.b);
  hipLaunchKernelGGL(scan_generic_kernel, dim3((unsigned)(a.B * a.H)), dim3(GS_THREADS), lds, s, a);
  return hipGetLastError();
}

size_t scan_linear_generic_lds_bytes(int d, int b) {
  return sizeof(float) * ((size_t)3 * b * d + (size_t)b * b);
}

hipError_t launch_scan_linear_generic(const ScanArgs& a, hipStream_t s) {
  const size_t lds = scan_linear_generic_lds_bytes(a.d, a.b);
  hipLaunchKernelGGL(scan_linear_generic_kernel, dim3((unsigned)(a.B * a.H)), dim3(GS_THREADS), lds, s, a);
  return hipGetLastError();
}

}  // namespace ttt
