// Backward of one direction of the TTT-MLP layer ("One-Minute Video Generation
// with Test-Time Training", paper-notes page, key designs "TTT-MLP layer" and
// "gate + bidirectional"; the training section learns theta, the initial
// state and the gate through the layer): the gradients of sum(dY * Y) with
// respect to the projections' outputs Q, K, V, the initial state and the gate,
// and the two GEMMs that carry dQ, dK, dV back to X and theta.
//
// The forward pass runs first (the generic scan) and leaves the state at the
// start of every C-th mini-batch in the workspace.  The backward scan then
// walks the segments of C mini-batches from the last to the first: it replays
// the segment's forward updates from its checkpoint, keeping the state each
// mini-batch starts from, and walks the segment's mini-batches backwards,
// carrying the adjoint of the state (dW1, dW2).
//
// One mini-batch of n tokens from state (W1, W2) computes (dual form, tril
// keeps the diagonal, c = 2/d or 2):
//   A = K W1, Hk = GELU(A), S1 = GELU'(A), G2 = c (Hk W2 - V), Gh = G2 W2^T,
//   G1 = Gh * S1, M = tril(Q K^T), Aq = Q W1 - eta M G1, Hq = GELU(Aq),
//   N = tril(Hq Hk^T), Z = Hq W2 - eta N G2,
//   W1' = W1 - eta K^T G1, W2' = W2 - eta Hk^T G2.
// Given dZ = tanh(alpha) dY and the adjoints dW1', dW2' of the state after it,
// the chain rule through these lines, in reverse order, is
//   dHq = dZ W2^T + dN Hk with dN = tril(-eta dZ G2^T);  dAq = dHq * GELU'(Aq)
//   dM = tril(-eta dAq G1^T);  dQ = dAq W1^T + dM K
//   dG1 = -eta M^T dAq - eta K dW1';   dK = dM^T Q - eta G1 dW1'^T + dA W1^T
//   dG2 = -eta N^T dZ - eta Hk dW2' + dGh W2;   dGh = dG1 * S1
//   dHk = dN^T Hq - eta G2 dW2'^T + c dG2 W2^T
//   dA = dG1 * Gh * GELU''(A) + dHk * S1;   dV = -c dG2
//   dW1 = dW1' + Q^T dAq + K^T dA
//   dW2 = dW2' + Hq^T dZ + dGh^T G2 + Hk^T (c dG2)
// and dW1, dW2 are the adjoints handed to the mini-batch before.  fp32
// throughout; one workgroup per (sequence, head), the b x d and b x b
// operands in LDS, the b x m ones in a per-workgroup workspace slice.
#include "internal.h"

namespace ttt {
namespace {

constexpr int BW = 256;  // threads of the backward scan's workgroup

__device__ inline float load_io(const void* p, int64_t i, int bf16) {
  if (bf16) return __uint_as_float((uint32_t)(((const uint16_t*)p)[i]) << 16);
  return ((const float*)p)[i];
}

// GELU and its first two derivatives.  erf form: GELU = a Phi(a),
// GELU' = Phi(a) + a phi(a), GELU'' = phi(a) (2 - a^2).
__device__ inline void gelu3(float a, int tanh_form, float* g, float* dg, float* ddg) {
  if (tanh_form) {
    const float C = 0.7978845608028654f, Kc = 0.044715f;
    const float u = C * (a + Kc * a * a * a);
    const float th = tanhf(u);
    const float du = C * (1.0f + 3.0f * Kc * a * a);
    const float sech2 = 1.0f - th * th;
    *g = 0.5f * a * (1.0f + th);
    *dg = 0.5f * (1.0f + th) + 0.5f * a * sech2 * du;
    *ddg = sech2 * (du - a * th * du * du + 3.0f * C * Kc * a * a);
    return;
  }
  const float phi = 0.3989422804014327f * expf(-0.5f * a * a);
  const float cdf = 0.5f * (1.0f + erff(a * 0.7071067811865476f));
  *g = a * cdf;
  *dg = cdf + a * phi;
  *ddg = phi * (2.0f - a * a);
}

// out[r, c] (R x C, row stride ldo) = s * sum_k A(r, k) B(k, c), added to out when acc;
// tril: entries with c > r are zero.
template <class FA, class FB>
__device__ inline void mm(float* out, int ldo, int R, int C, int K, FA A, FB B, float s, bool acc, bool tril = false) {
  for (int i = threadIdx.x; i < R * C; i += BW) {
    const int r = i / C, c = i - (i / C) * C;
    float v = 0.0f;
    if (!tril || c <= r)
      for (int k = 0; k < K; ++k) v = fmaf(A(r, k), B(k, c), v);
    out[r * ldo + c] = acc ? out[r * ldo + c] + s * v : s * v;
  }
}

// Operand panels of one mini-batch.
struct MB {
  // LDS, b x d (row stride d)
  float *K, *Q, *G2, *dZ, *dG2, *dQ, *dK, *dYh;
  // LDS, b x b (row stride b)
  float *M, *N, *dM, *dN;
  // workspace slice, b x m (row stride m)
  float *A, *Hk, *S1, *Gh, *G1, *Aq, *Hq, *dAq, *dHk, *dG1, *dGh;
};

// The forward quantities of one mini-batch that the state update needs:
// A, Hk, S1, G2 (in place of V), Gh, G1.
__device__ void forward_core(const MB& t, const float* W1, const float* W2, int n, int d, int m, float gscale,
                             int gelu_tanh) {
  // A = K W1
  mm(t.A, m, n, m, d, [&](int r, int k) { return t.K[r * d + k]; }, [&](int k, int c) { return W1[k * m + c]; },
     1.0f, false);
  __syncthreads();
  for (int i = threadIdx.x; i < n * m; i += BW) {
    float g, dg, ddg;
    gelu3(t.A[i], gelu_tanh, &g, &dg, &ddg);
    t.Hk[i] = g;
    t.S1[i] = dg;
  }
  __syncthreads();
  // G2 = c (Hk W2 - V), in place of V
  for (int i = threadIdx.x; i < n * d; i += BW) {
    const int r = i / d, c = i - (i / d) * d;
    float v = 0.0f;
    for (int k = 0; k < m; ++k) v = fmaf(t.Hk[r * m + k], W2[k * d + c], v);
    t.G2[i] = gscale * (v - t.G2[i]);
  }
  __syncthreads();
  // Gh = G2 W2^T; G1 = Gh * S1
  for (int i = threadIdx.x; i < n * m; i += BW) {
    const int r = i / m, c = i - (i / m) * m;
    float v = 0.0f;
    for (int k = 0; k < d; ++k) v = fmaf(t.G2[r * d + k], W2[c * d + k], v);
    t.Gh[i] = v;
    t.G1[i] = v * t.S1[i];
  }
  __syncthreads();
}

__global__ __launch_bounds__(BW) void scan_backward_kernel(BwdArgs a) {
  extern __shared__ float lds[];
  const int d = a.d, m = a.m, b = a.b, tid = threadIdx.x;
  const int64_t T = a.T;
  const int s = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int D = a.H * d;
  const float eta = a.eta;
  const int64_t dm = (int64_t)d * m;
  const int64_t nmb = (T + b - 1) / b;
  const int C = a.ckpt_every;
  const int64_t nseg = (nmb + C - 1) / C;
  const int64_t sh = (int64_t)s * a.H + h;

  MB t;
  t.K = lds;
  t.Q = t.K + b * d;
  t.G2 = t.Q + b * d;
  t.dZ = t.G2 + b * d;
  t.dG2 = t.dZ + b * d;
  t.dQ = t.dG2 + b * d;
  t.dK = t.dQ + b * d;
  t.dYh = t.dK + b * d;
  t.M = t.dYh + b * d;
  t.N = t.M + b * b;
  t.dM = t.N + b * b;
  t.dN = t.dM + b * b;
  float* sc = a.scratch + sh * (int64_t)kBwdScratchPanels * b * m;
  float** panels[] = {&t.A, &t.Hk, &t.S1, &t.Gh, &t.G1, &t.Aq, &t.Hq, &t.dAq, &t.dHk, &t.dG1, &t.dGh};
  for (int i = 0; i < kBwdScratchPanels; ++i) *panels[i] = sc + (int64_t)i * b * m;

  float* Wc1 = a.wcur + sh * 2 * dm;  // replayed state
  float* Wc2 = Wc1 + dm;
  float* dW1 = a.dstate + sh * 2 * dm;  // adjoint of the state after the current mini-batch
  float* dW2 = dW1 + dm;
  float* seg = a.segst + sh * (int64_t)C * 2 * dm;
  for (int64_t i = tid; i < 2 * dm; i += BW) dW1[i] = 0.0f;

  const int64_t plane = a.B * a.H * T * d;
  const float* qb = a.qkv + sh * T * d;
  const float* kb = qb + plane;
  const float* vb = kb + plane;
  auto tok = [&](int64_t pos) { return a.reverse ? T - 1 - pos : pos; };
  // K, V (and Q, dZ) rows of mini-batch j into LDS
  auto load_rows = [&](int64_t j, int n, bool all) {
    for (int i = tid; i < n * d; i += BW) {
      const int r = i / d, c = i - (i / d) * d;
      const int64_t t_ = tok(j * b + r);
      t.K[i] = kb[t_ * d + c];
      t.G2[i] = vb[t_ * d + c];
      if (all) {
        t.Q[i] = qb[t_ * d + c];
        const int ch = h * d + c;
        t.dZ[i] = tanhf(a.alpha[ch]) * a.dy[((int64_t)s * T + t_) * D + ch];
      }
    }
    __syncthreads();
  };

  for (int64_t sg = nseg - 1; sg >= 0; --sg) {
    const int64_t j0 = sg * C, j1 = min(nmb, j0 + C);
    // replay the segment's forward updates from its checkpoint
    const float* ck = a.ckpt + (sh * nseg + sg) * 2 * dm;
    for (int64_t i = tid; i < 2 * dm; i += BW) Wc1[i] = ck[i];
    __syncthreads();
    for (int64_t j = j0; j < j1; ++j) {
      float* dst = seg + (j - j0) * 2 * dm;
      for (int64_t i = tid; i < 2 * dm; i += BW) dst[i] = Wc1[i];
      if (j + 1 == j1) break;
      const int n = (int)min((int64_t)b, T - j * b);
      __syncthreads();
      load_rows(j, n, false);
      forward_core(t, Wc1, Wc2, n, d, m, a.gscale, a.gelu_tanh);
      // W1 -= eta K^T G1; W2 -= eta Hk^T G2
      mm(Wc1, m, d, m, n, [&](int r, int k) { return t.K[k * d + r]; }, [&](int k, int c) { return t.G1[k * m + c]; },
         -eta, true);
      mm(Wc2, d, m, d, n, [&](int r, int k) { return t.Hk[k * m + r]; }, [&](int k, int c) { return t.G2[k * d + c]; },
         -eta, true);
      __syncthreads();
    }
    __syncthreads();
    // the segment's mini-batches, last to first
    for (int64_t j = j1 - 1; j >= j0; --j) {
      const int n = (int)min((int64_t)b, T - j * b);
      const float* W1 = seg + (j - j0) * 2 * dm;
      const float* W2 = W1 + dm;
      load_rows(j, n, true);
      forward_core(t, W1, W2, n, d, m, a.gscale, a.gelu_tanh);
      // M = tril(Q K^T)
      mm(t.M, b, n, n, d, [&](int r, int k) { return t.Q[r * d + k]; }, [&](int k, int c) { return t.K[c * d + k]; },
         1.0f, false, true);
      __syncthreads();
      // Aq = Q W1 - eta M G1; Hq = GELU(Aq), keeping GELU'(Aq) in dAq
      for (int i = tid; i < n * m; i += BW) {
        const int r = i / m, c = i - (i / m) * m;
        float v = 0.0f, corr = 0.0f;
        for (int k = 0; k < d; ++k) v = fmaf(t.Q[r * d + k], W1[k * m + c], v);
        for (int k = 0; k <= r; ++k) corr = fmaf(t.M[r * b + k], t.G1[k * m + c], corr);
        const float aq = v - eta * corr;
        float g, dg, ddg;
        gelu3(aq, a.gelu_tanh, &g, &dg, &ddg);
        t.Aq[i] = aq;
        t.Hq[i] = g;
        t.dAq[i] = dg;
      }
      __syncthreads();
      // N = tril(Hq Hk^T); dN = tril(-eta dZ G2^T)
      mm(t.N, b, n, n, m, [&](int r, int k) { return t.Hq[r * m + k]; }, [&](int k, int c) { return t.Hk[c * m + k]; },
         1.0f, false, true);
      mm(t.dN, b, n, n, d, [&](int r, int k) { return t.dZ[r * d + k]; }, [&](int k, int c) { return t.G2[c * d + k]; },
         -eta, false, true);
      __syncthreads();
      // dAq = (dZ W2^T + dN Hk) * GELU'(Aq)
      for (int i = tid; i < n * m; i += BW) {
        const int r = i / m, c = i - (i / m) * m;
        float v = 0.0f;
        for (int k = 0; k < d; ++k) v = fmaf(t.dZ[r * d + k], W2[c * d + k], v);
        for (int k = 0; k <= r; ++k) v = fmaf(t.dN[r * b + k], t.Hk[k * m + c], v);
        t.dAq[i] *= v;
      }
      // dG2 = -eta N^T dZ
      mm(t.dG2, d, n, d, n, [&](int r, int k) { return t.N[k * b + r]; }, [&](int k, int c) { return t.dZ[k * d + c]; },
         -eta, false);
      // dHk = dN^T Hq
      mm(t.dHk, m, n, m, n, [&](int r, int k) { return t.dN[k * b + r]; }, [&](int k, int c) { return t.Hq[k * m + c]; },
         1.0f, false);
      __syncthreads();
      // dQ = dAq W1^T; dM = tril(-eta dAq G1^T)
      mm(t.dQ, d, n, d, m, [&](int r, int k) { return t.dAq[r * m + k]; }, [&](int k, int c) { return W1[c * m + k]; },
         1.0f, false);
      mm(t.dM, b, n, n, m, [&](int r, int k) { return t.dAq[r * m + k]; }, [&](int k, int c) { return t.G1[c * m + k]; },
         -eta, false, true);
      // the state-update paths, with the adjoints of the state after this mini-batch:
      // dHk += -eta G2 dW2'^T; dG2 += -eta Hk dW2'
      mm(t.dHk, m, n, m, d, [&](int r, int k) { return t.G2[r * d + k]; }, [&](int k, int c) { return dW2[c * d + k]; },
         -eta, true);
      mm(t.dG2, d, n, d, m, [&](int r, int k) { return t.Hk[r * m + k]; }, [&](int k, int c) { return dW2[k * d + c]; },
         -eta, true);
      __syncthreads();
      // dG1 = -eta M^T dAq - eta K dW1'; dQ += dM K; dK = dM^T Q - eta G1 dW1'^T
      for (int i = tid; i < n * m; i += BW) {
        const int r = i / m, c = i - (i / m) * m;
        float v = 0.0f, w = 0.0f;
        for (int k = r; k < n; ++k) v = fmaf(t.M[k * b + r], t.dAq[k * m + c], v);
        for (int k = 0; k < d; ++k) w = fmaf(t.K[r * d + k], dW1[k * m + c], w);
        t.dG1[i] = -eta * (v + w);
      }
      for (int i = tid; i < n * d; i += BW) {
        const int r = i / d, c = i - (i / d) * d;
        float q = 0.0f, k1 = 0.0f, k2 = 0.0f;
        for (int k = 0; k < n; ++k) {
          q = fmaf(t.dM[r * b + k], t.K[k * d + c], q);
          k1 = fmaf(t.dM[k * b + r], t.Q[k * d + c], k1);
        }
        for (int k = 0; k < m; ++k) k2 = fmaf(t.G1[r * m + k], dW1[c * m + k], k2);
        t.dQ[i] += q;
        t.dK[i] = k1 - eta * k2;
      }
      __syncthreads();
      // dGh = dG1 * S1; dA (in dG1) = dG1 * Gh * GELU''(A)
      for (int i = tid; i < n * m; i += BW) {
        float g, dg, ddg;
        gelu3(t.A[i], a.gelu_tanh, &g, &dg, &ddg);
        const float x = t.dG1[i];
        t.dGh[i] = x * t.S1[i];
        t.dG1[i] = x * t.Gh[i] * ddg;
      }
      __syncthreads();
      // dG2 += dGh W2; then dYh = c dG2 (the gradient of Y-hat = Hk W2)
      for (int i = tid; i < n * d; i += BW) {
        const int r = i / d, c = i - (i / d) * d;
        float v = 0.0f;
        for (int k = 0; k < m; ++k) v = fmaf(t.dGh[r * m + k], W2[k * d + c], v);
        const float g2 = t.dG2[i] + v;
        t.dG2[i] = g2;
        t.dYh[i] = a.gscale * g2;
      }
      __syncthreads();
      // dHk += dYh W2^T; dA += dHk * S1
      for (int i = tid; i < n * m; i += BW) {
        const int r = i / m, c = i - (i / m) * m;
        float v = 0.0f;
        for (int k = 0; k < d; ++k) v = fmaf(t.dYh[r * d + k], W2[c * d + k], v);
        const float dhk = t.dHk[i] + v;
        t.dHk[i] = dhk;
        t.dG1[i] += dhk * t.S1[i];
      }
      __syncthreads();
      // dK += dA W1^T; write dQ, dK, dV = -dYh to their columns of [B, T, 3D]
      for (int i = tid; i < n * d; i += BW) {
        const int r = i / d, c = i - (i / d) * d;
        float v = 0.0f;
        for (int k = 0; k < m; ++k) v = fmaf(t.dG1[r * m + k], W1[c * m + k], v);
        const int64_t t_ = tok(j * b + r);
        float* row = a.dqkv + ((int64_t)s * T + t_) * 3 * D + h * d + c;
        row[0] = t.dQ[i];
        row[D] = t.dK[i] + v;
        row[2 * D] = -t.dYh[i];
      }
      // dW1 += Q^T dAq + K^T dA; dW2 += Hq^T dZ + dGh^T G2 + Hk^T dYh
      for (int64_t i = tid; i < dm; i += BW) {
        const int r = (int)(i / m), c = (int)(i - (i / m) * m);
        float v = 0.0f;
        for (int k = 0; k < n; ++k) {
          v = fmaf(t.Q[k * d + r], t.dAq[k * m + c], v);
          v = fmaf(t.K[k * d + r], t.dG1[k * m + c], v);
        }
        dW1[i] += v;
      }
      for (int64_t i = tid; i < dm; i += BW) {
        const int r = (int)(i / d), c = (int)(i - (i / d) * d);
        float v = 0.0f;
        for (int k = 0; k < n; ++k) {
          v = fmaf(t.Hq[k * m + r], t.dZ[k * d + c], v);
          v = fmaf(t.dGh[k * m + r], t.G2[k * d + c], v);
          v = fmaf(t.Hk[k * m + r], t.dYh[k * d + c], v);
        }
        dW2[i] += v;
      }
      __syncthreads();
    }
  }
  float* o = a.dw_seq + sh * 2 * dm;
  for (int64_t i = tid; i < 2 * dm; i += BW) o[i] = dW1[i];
}

// C[M x N] = (accumulate ? C : Cadd or 0) + A B, fp32; A(r, k) = A[r lda + k], or
// A[k lda + r] when AT; B(k, c) = B[k ldb + c] in fp32 or bf16.  64 x 64 tiles,
// K-steps of 16, 4 x 4 outputs per thread.
constexpr int GM = 64, GN = 64, GK = 16;

template <bool AT, bool BBF16>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* A, int64_t lda, const void* Bm, int64_t ldb,
                                                       float* C, int64_t ldc, const float* Cadd, int64_t M,
                                                       int64_t N, int64_t K, int accumulate) {
  __shared__ float As[GK][GM + 4];
  __shared__ float Bs[GK][GN + 4];
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const int64_t m0 = (int64_t)blockIdx.x * GM, n0 = (int64_t)blockIdx.y * GN;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < K; k0 += GK) {
    for (int i = tid; i < GM * GK; i += 256) {
      int r, k;
      if (AT) {  // consecutive threads walk rows of the tile: contiguous in A
        r = i % GM;
        k = i / GM;
      } else {
        r = i / GK;
        k = i % GK;
      }
      const int64_t gr = m0 + r, gk = k0 + k;
      As[k][r] = (gr < M && gk < K) ? (AT ? A[gk * lda + gr] : A[gr * lda + gk]) : 0.0f;
    }
    for (int i = tid; i < GN * GK; i += 256) {
      const int c = i % GN, k = i / GN;
      const int64_t gc = n0 + c, gk = k0 + k;
      Bs[k][c] = (gc < N && gk < K) ? load_io(Bm, gk * ldb + gc, BBF16) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < GK; ++k) {
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
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t gr = m0 + ty * 4 + i;
    if (gr >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t gc = n0 + tx * 4 + j;
      if (gc >= N) continue;
      float* p = C + gr * ldc + gc;
      const float base = accumulate ? *p : (Cadd ? Cadd[gr * ldc + gc] : 0.0f);
      *p = base + acc[i][j];
    }
  }
}

// dalpha: partial sums of dY * Z over row ranges, then the per-channel total
// (fixed order) times tanh'(alpha) = 1 - tanh(alpha)^2.
constexpr int kDalphaSplits = 256;

__global__ __launch_bounds__(256) void dalpha_partial_kernel(const float* dy, const float* z, float* part,
                                                             int64_t rows, int D) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= D) return;
  const int64_t per = (rows + kDalphaSplits - 1) / kDalphaSplits;
  const int64_t r0 = blockIdx.y * per, r1 = min(rows, r0 + per);
  float acc = 0.0f;
  for (int64_t r = r0; r < r1; ++r) acc = fmaf(dy[r * D + c], z[r * D + c], acc);
  part[(int64_t)blockIdx.y * D + c] = acc;
}

__global__ __launch_bounds__(256) void dalpha_finish_kernel(const float* part, const float* alpha, float* dalpha,
                                                            int D) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= D) return;
  float acc = 0.0f;
  for (int i = 0; i < kDalphaSplits; ++i) acc += part[(int64_t)i * D + c];
  const float th = tanhf(alpha[c]);
  dalpha[c] = acc * (1.0f - th * th);
}

// dW1_0 [H, d, m] and dW2_0 [H, m, d] (+)= sum over sequences of the per-sequence adjoints
__global__ __launch_bounds__(256) void sum_state_kernel(const float* dw_seq, float* dW1, float* dW2, int64_t B,
                                                        int H, int64_t dm, int accumulate) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)H * 2 * dm) return;
  const int64_t h = i / (2 * dm), e = i - h * 2 * dm;
  float acc = 0.0f;
  for (int64_t s = 0; s < B; ++s) acc += dw_seq[(s * H + h) * 2 * dm + e];
  float* o = e < dm ? dW1 + h * dm + e : dW2 + h * dm + (e - dm);
  *o = accumulate ? *o + acc : acc;
}

}  // namespace

size_t scan_backward_lds_bytes(int d, int b) { return sizeof(float) * ((size_t)8 * b * d + (size_t)4 * b * b); }

hipError_t launch_scan_backward(const BwdArgs& a, hipStream_t s) {
  // T = 0 runs too: no segments, and the kernel writes the zero adjoint of the initial state
  hipLaunchKernelGGL(scan_backward_kernel, dim3((unsigned)(a.B * a.H)), dim3(BW), scan_backward_lds_bytes(a.d, a.b),
                     s, a);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(bool a_transposed, bool b_bf16, const float* A, int64_t lda, const void* Bm, int64_t ldb,
                           float* C, int64_t ldc, const float* Cadd, int64_t M, int64_t N, int64_t K, int accumulate,
                           hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  dim3 grid((unsigned)((M + GM - 1) / GM), (unsigned)((N + GN - 1) / GN));
  if (a_transposed) {
    if (b_bf16)
      hipLaunchKernelGGL((gemm_f32_kernel<true, true>), grid, dim3(256), 0, s, A, lda, Bm, ldb, C, ldc, Cadd, M, N, K,
                         accumulate);
    else
      hipLaunchKernelGGL((gemm_f32_kernel<true, false>), grid, dim3(256), 0, s, A, lda, Bm, ldb, C, ldc, Cadd, M, N,
                         K, accumulate);
  } else {
    if (b_bf16)
      hipLaunchKernelGGL((gemm_f32_kernel<false, true>), grid, dim3(256), 0, s, A, lda, Bm, ldb, C, ldc, Cadd, M, N,
                         K, accumulate);
    else
      hipLaunchKernelGGL((gemm_f32_kernel<false, false>), grid, dim3(256), 0, s, A, lda, Bm, ldb, C, ldc, Cadd, M, N,
                         K, accumulate);
  }
  return hipGetLastError();
}

size_t dalpha_partial_elems(int D) { return (size_t)kDalphaSplits * D; }

hipError_t launch_dalpha(const float* dy, const float* z, const float* alpha, float* part, float* dalpha,
                         int64_t rows, int D, hipStream_t s) {
  const unsigned cb = (unsigned)((D + 255) / 256);
  hipLaunchKernelGGL(dalpha_partial_kernel, dim3(cb, kDalphaSplits), dim3(256), 0, s, dy, z, part, rows, D);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dalpha_finish_kernel, dim3(cb), dim3(256), 0, s, part, alpha, dalpha, D);
  return hipGetLastError();
}

hipError_t launch_sum_state(const float* dw_seq, float* dW1, float* dW2, int64_t B, int H, int d, int m,
                            int accumulate, hipStream_t s) {
  const int64_t n = (int64_t)H * 2 * d * m;
  hipLaunchKernelGGL(sum_state_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dw_seq, dW1, dW2, B, H,
                     (int64_t)d * m, accumulate);
  return hipGetLastError();
}

}  // namespace ttt
