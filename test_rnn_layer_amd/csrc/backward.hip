// Backward of one direction of the TTT-MLP layer ("One-Minute Video Generation
// with Test-Time Training", paper-notes page, key designs "TTT-MLP layer" and
// "gate + bidirectional"; the training section learns theta, the initial
// state and the gate through the layer): the gradients of sum(dY * Y) with
// respect to the projections' outputs Q, K, V, the initial state and the gate,
// and the two GEMMs that carry dQ, dK, dV back to X and theta.
//
// The forward pass runs first (scan_fwd_ckpt_kernel) and leaves the state at
// the start of every C-th mini-batch in the workspace.  The backward scan then
// walks the segments of C mini-batches from the last to the first: it replays
// the segment's forward updates from its checkpoint, keeping the state each
// mini-batch starts from and the forward quantities it computed (A, Hk,
// GELU'(A), G2, Gh, G1: the backward walk reads them instead of computing them
// again, for every mini-batch but the segment's last), and walks the segment's
// mini-batches backwards, carrying the adjoint of the state (dW1, dW2).
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
// throughout; one 1024-thread workgroup per (sequence, head), the state (when
// it fits) and the b x d and b x b operands in LDS, the b x m ones in a
// per-workgroup workspace slice, the adjoint in the workspace.  The products
// run on the fp32 matrix cores where d, m and the mini-batch tile by 16, on the
// vector ALU otherwise (one output column and a few rows per thread, operands
// read 16 bytes at a time; d and m multiples of 4).
#include "internal.h"
#include "mfma_common.h"
#include "phase_marks.h"
#include "token_block.h"

TTT_MARKS_BUFFER(g_marks_scan_backward);

namespace ttt {
namespace {

constexpr int BW = 1024;  // threads of the scan kernels' workgroups (16 waves, 4 per SIMD)

__device__ inline float load_io(const void* p, int64_t i, int bf16) {
  if (bf16) return __uint_as_float((uint32_t)(((const uint16_t*)p)[i]) << 16);
  return ((const float*)p)[i];
}

__device__ inline void store_io(void* p, int64_t i, float v, int bf16) {
  if (bf16) {
    uint32_t u = __float_as_uint(v);
    uint16_t r;
    if ((u & 0x7fffffffu) > 0x7f800000u) {
      r = (uint16_t)((u >> 16) | 0x40u);  // keep NaN a NaN
    } else {
      u += 0x7fffu + ((u >> 16) & 1u);  // round to nearest, ties to even
      r = (uint16_t)(u >> 16);
    }
    ((uint16_t*)p)[i] = r;
  } else {
    ((float*)p)[i] = v;
  }
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

// out[r, c] = (acc ? out[r, c] : 0) + s sum_{k<K} X[r, k] W(k, c) for r < n, c < C, with
// W(k, c) = W[k ldw + c], or W[c ldw + k] when WT.  K, ldx and ldw are multiples of 4 and
// X, W 16-byte aligned.  A thread takes one column and RG rows; k advances by 4 (X, and
// W when WT, in 16-byte loads), in order, so every sum runs k = 0, 1, ... .
template <int RG, bool WT>
__device__ void prod_valu(float* out, int ldo, int n, int C, int K, const float* X, int ldx, const float* W, int ldw,
                     float s, bool acc) {
  const int groups = (n + RG - 1) / RG;
  for (int it = threadIdx.x; it < C * groups; it += BW) {
    const int c = it % C, r0 = (it / C) * RG;
    float a[RG];
    const float* xr[RG];
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      a[i] = 0.0f;
      xr[i] = X + (int64_t)min(r0 + i, n - 1) * ldx;
    }
    for (int k = 0; k < K; k += 4) {
      float4 w;
      if (WT) {
        w = *(const float4*)(W + (int64_t)c * ldw + k);
      } else {
        w.x = W[(int64_t)k * ldw + c];
        w.y = W[(int64_t)(k + 1) * ldw + c];
        w.z = W[(int64_t)(k + 2) * ldw + c];
        w.w = W[(int64_t)(k + 3) * ldw + c];
      }
#pragma unroll
      for (int i = 0; i < RG; ++i) {
        const float4 x = *(const float4*)(xr[i] + k);
        a[i] = fmaf(x.x, w.x, a[i]);
        a[i] = fmaf(x.y, w.y, a[i]);
        a[i] = fmaf(x.z, w.z, a[i]);
        a[i] = fmaf(x.w, w.w, a[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < RG; ++i)
      if (r0 + i < n) {
        float* o = out + (r0 + i) * ldo + c;
        *o = (acc ? *o : 0.0f) + s * a[i];
      }
  }
}

// Up to three rank-n terms of a state-shaped update: S[k, c] += s sum_p sum_{r<n} P_p[r, k] Q_p[r, c]
// for k < R, c < C.  P rows are contiguous in k (row stride a multiple of 4); KG divides R.
// A thread takes one column and KG consecutive k.
struct Terms {
  int np;
  const float* P[3];
  int ldp[3];
  const float* Q[3];
  int ldq[3];
};

template <int KG>
__device__ void rank_update(float* S, int ldS, int R, int C, int n, const Terms& tm, float s) {
  const int kg = R / KG;
  for (int it = threadIdx.x; it < C * kg; it += BW) {
    const int c = it % C, k0 = (it / C) * KG;
    float a[KG];
#pragma unroll
    for (int i = 0; i < KG; ++i) a[i] = 0.0f;
    for (int p = 0; p < tm.np; ++p)
      for (int r = 0; r < n; ++r) {
        const float q = tm.Q[p][r * tm.ldq[p] + c];
        const float* pr = tm.P[p] + r * tm.ldp[p] + k0;
#pragma unroll
        for (int i = 0; i < KG; i += 4) {
          const float4 v = *(const float4*)(pr + i);
          a[i] = fmaf(v.x, q, a[i]);
          a[i + 1] = fmaf(v.y, q, a[i + 1]);
          a[i + 2] = fmaf(v.z, q, a[i + 2]);
          a[i + 3] = fmaf(v.w, q, a[i + 3]);
        }
      }
#pragma unroll
    for (int i = 0; i < KG; ++i) S[(int64_t)(k0 + i) * ldS + c] += s * a[i];
  }
}

__device__ inline void rank_update_valu(float* S, int ldS, int R, int C, int n, const Terms& tm, float s) {
  if (R % 16 == 0)
    rank_update<16>(S, ldS, R, C, n, tm, s);
  else
    rank_update<4>(S, ldS, R, C, n, tm, s);
}

// out[r, c] (n x n, row stride ldo) = s sum_{k<K} X[r, k] Y[c, k] for c <= r, 0 above the
// diagonal.  Four lanes share an output, each summing every fourth k; lane exchanges add the
// four partial sums.
__device__ void rowdot_tril_valu(float* out, int ldo, int n, int K, const float* X, int ldx, const float* Y,
                                 int ldy, float s) {
  const int nn = n * n;
  for (int base = 0; base < 4 * nn; base += BW) {  // the same trip count in every lane
    const int it = base + (int)threadIdx.x;
    const int o = it >> 2, q = it & 3;
    int r = 0, c = 0;
    float v = 0.0f;
    if (o < nn) {
      r = o / n;
      c = o - r * n;
      if (c <= r)
        for (int k = q; k < K; k += 4) v = fmaf(X[r * ldx + k], Y[c * ldy + k], v);
    }
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    if (o < nn && q == 0) out[r * ldo + c] = s * v;
  }
}

// The same three operations on the fp32 matrix cores (v_mfma_f32_16x16x4_f32, fp32
// products and sums like the VALU forms, in another order), for the shapes they tile:
// each wave takes 16 x 16 output tiles; for lane l, i = l % 16 and q = l / 16,
//   A[i][q] (row i, contraction index q), B[q][i], D[4q .. 4q+3][i].
// In the products the lane group q takes the contraction range [q K/4, (q+1) K/4), one
// index per instruction, so an operand that is contiguous along k arrives 16 bytes at a
// time.  The first wave of a call is w0: calls in one phase start on different waves.  The
// product routines stay out of line: inlined into the scan kernels, their operand addresses
// pushed the kernels past 128 registers (the limit at 16 waves per workgroup) into spills.
constexpr int kBwdWaves = BW / 64;

__device__ __forceinline__ f32x4 mfma_f32x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int bwd_wave() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); }

// sum_k X(row, k) W(k, col) over k < K (K a multiple of 16) for this lane's row and column;
// X(r, k) = X[r ldx + k], or X[k ldx + r] when XT; W(k, c) = W[k ldw + c], or W[c ldw + k] when WT
template <bool XT, bool WT>
__device__ __forceinline__ f32x4 tile_xw(const float* X, int ldx, int row, const float* W, int ldw, int col, int K,
                                         int q) {
  const int kq = K >> 2, kb = q * kq;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 2
  for (int k = 0; k < kq; k += 4) {
    float x[4], y[4];
    if (XT) {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = X[(int64_t)(kb + k + e) * ldx + row];
    } else {
      const float4 v = *(const float4*)(X + (int64_t)row * ldx + kb + k);
      x[0] = v.x, x[1] = v.y, x[2] = v.z, x[3] = v.w;
    }
    if (WT) {
      const float4 v = *(const float4*)(W + (int64_t)col * ldw + kb + k);
      y[0] = v.x, y[1] = v.y, y[2] = v.z, y[3] = v.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = W[(int64_t)(kb + k + e) * ldw + col];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = mfma_f32x4(x[e], y[e], acc);
  }
  return acc;
}

template <bool XT, bool WT>
__device__ __attribute__((noinline)) void prod_mfma(float* out, int ldo, int n, int C, int K, const float* X, int ldx,
                                                    const float* W, int ldw, float s, bool acc, int w0) {
  const int lane = threadIdx.x & 63, i = lane & 15, q = lane >> 4;
  const int ct = C >> 4, tiles = ((n + 15) >> 4) * ct;
  for (int tile = (bwd_wave() + kBwdWaves - w0 % kBwdWaves) % kBwdWaves; tile < tiles; tile += kBwdWaves) {
    const int r0 = (tile / ct) * 16, c0 = (tile % ct) * 16;
    const f32x4 v = tile_xw<XT, WT>(X, ldx, min(r0 + i, n - 1), W, ldw, c0 + i, K, q);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = r0 + 4 * q + rr;
      if (r < n) {
        float* o = out + (int64_t)r * ldo + c0 + i;
        *o = (acc ? *o : 0.0f) + s * v[rr];
      }
    }
  }
}

// out = (acc ? out : 0) + s X W (see prod_valu): on the matrix cores when C and K are multiples of 16
template <int RG, bool WT>
__device__ inline void prod(float* out, int ldo, int n, int C, int K, const float* X, int ldx, const float* W,
                            int ldw, float s, bool acc, int w0 = 0) {
  if (C % 16 == 0 && K % 16 == 0)
    prod_mfma<false, WT>(out, ldo, n, C, K, X, ldx, W, ldw, s, acc, w0);
  else
    prod_valu<RG, WT>(out, ldo, n, C, K, X, ldx, W, ldw, s, acc);
}

// S += s sum_p P_p^T Q_p (see rank_update): tile (k0, c0) takes A[i][q] = P[r][k0 + i] and
// B[q][i] = Q[r][c0 + i] with r = r4 + q, four rows per instruction (rows past n read as 0);
// the tile of S is read before the products, so that its latency overlaps theirs.
// The up to three terms come as scalar arguments (an out-of-line call would otherwise fetch
// them from private memory at every use); a tile's operands are loaded before its products.
__device__ __attribute__((noinline)) void rank_update_mfma(float* S, int ldS, int R, int C, int n, int np,
                                                           const float* P0, int lp0, const float* Q0, int lq0,
                                                           const float* P1, int lp1, const float* Q1, int lq1,
                                                           const float* P2, int lp2, const float* Q2, int lq2,
                                                           float s, int w0) {
  const int lane = threadIdx.x & 63, i = lane & 15, q = lane >> 4;
  const int ct = C >> 4, tiles = (R >> 4) * ct;
  for (int tile = (bwd_wave() + kBwdWaves - w0 % kBwdWaves) % kBwdWaves; tile < tiles; tile += kBwdWaves) {
    const int k0 = (tile / ct) * 16, c0 = (tile % ct) * 16;
    float* srow = S + (int64_t)(k0 + 4 * q) * ldS + c0 + i;
    float old[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) old[rr] = srow[(int64_t)rr * ldS];
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int r16 = 0; r16 < n; r16 += 16) {
      float a[3][4], bq[3][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = r16 + 4 * u + q;
        const bool ok = r < n;
        a[0][u] = ok ? P0[r * lp0 + k0 + i] : 0.0f;
        bq[0][u] = ok ? Q0[r * lq0 + c0 + i] : 0.0f;
        a[1][u] = ok && np > 1 ? P1[r * lp1 + k0 + i] : 0.0f;
        bq[1][u] = ok && np > 1 ? Q1[r * lq1 + c0 + i] : 0.0f;
        a[2][u] = ok && np > 2 ? P2[r * lp2 + k0 + i] : 0.0f;
        bq[2][u] = ok && np > 2 ? Q2[r * lq2 + c0 + i] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v = mfma_f32x4(a[0][u], bq[0][u], v);
        if (np > 1) v = mfma_f32x4(a[1][u], bq[1][u], v);
        if (np > 2) v = mfma_f32x4(a[2][u], bq[2][u], v);
      }
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) srow[(int64_t)rr * ldS] = old[rr] + s * v[rr];
  }
}

// The same for n <= 16 and NP terms, software-pipelined: a wave loads its next tile's operands
// and old values while the current tile's products run, so that one tile's load latency is
// paid per call rather than per tile (NP sizes the register sets: two of 8 NP + 4 floats).
template <int NP>
__device__ __attribute__((noinline)) void rank_update_pipe(float* S, int ldS, int R, int C, int n,
                                                           const float* P0, int lp0, const float* Q0, int lq0,
                                                           const float* P1, int lp1, const float* Q1, int lq1,
                                                           const float* P2, int lp2, const float* Q2, int lq2,
                                                           float s, int w0) {
  const int lane = threadIdx.x & 63, i = lane & 15, q = lane >> 4;
  const int ct = C >> 4, tiles = (R >> 4) * ct;
  const float* P[3] = {P0, P1, P2};
  const float* Q[3] = {Q0, Q1, Q2};
  const int lp[3] = {lp0, lp1, lp2}, lq[3] = {lq0, lq1, lq2};
  float a[2][NP][4], bq[2][NP][4], old[2][4];
  auto load = [&](int tile, int set) {
    const int k0 = (tile / ct) * 16, c0 = (tile % ct) * 16;
    const float* srow = S + (int64_t)(k0 + 4 * q) * ldS + c0 + i;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) old[set][rr] = srow[(int64_t)rr * ldS];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * u + q;
        const bool ok = r < n;
        a[set][p][u] = ok ? P[p][r * lp[p] + k0 + i] : 0.0f;
        bq[set][p][u] = ok ? Q[p][r * lq[p] + c0 + i] : 0.0f;
      }
  };
  auto finish = [&](int tile, int set) {
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int p = 0; p < NP; ++p) v = mfma_f32x4(a[set][p][u], bq[set][p][u], v);
    const int k0 = (tile / ct) * 16, c0 = (tile % ct) * 16;
    float* srow = S + (int64_t)(k0 + 4 * q) * ldS + c0 + i;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) srow[(int64_t)rr * ldS] = old[set][rr] + s * v[rr];
  };
  int tile = (bwd_wave() + kBwdWaves - w0 % kBwdWaves) % kBwdWaves;
  if (tile >= tiles) return;
  load(tile, 0);
  for (;;) {  // two tiles per trip, so that the register sets keep fixed names
    int next = tile + kBwdWaves;
    if (next < tiles) load(next, 1);
    finish(tile, 0);
    if (next >= tiles) return;
    tile = next;
    next = tile + kBwdWaves;
    if (next < tiles) load(next, 0);
    finish(tile, 1);
    if (next >= tiles) return;
    tile = next;
  }
}

__device__ inline void rank_update_any(float* S, int ldS, int R, int C, int n, const Terms& tm, float s,
                                       int w0 = 0) {
  if (R % 16 != 0 || C % 16 != 0) {
    rank_update_valu(S, ldS, R, C, n, tm, s);
  } else if (n > 16) {
    rank_update_mfma(S, ldS, R, C, n, tm.np, tm.P[0], tm.ldp[0], tm.Q[0], tm.ldq[0], tm.P[1], tm.ldp[1], tm.Q[1],
                     tm.ldq[1], tm.P[2], tm.ldp[2], tm.Q[2], tm.ldq[2], s, w0);
  } else if (tm.np == 1) {
    rank_update_pipe<1>(S, ldS, R, C, n, tm.P[0], tm.ldp[0], tm.Q[0], tm.ldq[0], nullptr, 0, nullptr, 0, nullptr,
                        0, nullptr, 0, s, w0);
  } else if (tm.np == 2) {
    rank_update_pipe<2>(S, ldS, R, C, n, tm.P[0], tm.ldp[0], tm.Q[0], tm.ldq[0], tm.P[1], tm.ldp[1], tm.Q[1],
                        tm.ldq[1], nullptr, 0, nullptr, 0, s, w0);
  } else {
    rank_update_pipe<3>(S, ldS, R, C, n, tm.P[0], tm.ldp[0], tm.Q[0], tm.ldq[0], tm.P[1], tm.ldp[1], tm.Q[1],
                        tm.ldq[1], tm.P[2], tm.ldp[2], tm.Q[2], tm.ldq[2], s, w0);
  }
}

// tril(s X Y^T) (see rowdot_tril_valu): one tile on wave w0 when n <= 16 and K is a multiple of 16
__device__ inline void rowdot_tril(float* out, int ldo, int n, int K, const float* X, int ldx, const float* Y,
                                   int ldy, float s, int w0 = 0) {
  if (n > 16 || K % 16 != 0) {
    rowdot_tril_valu(out, ldo, n, K, X, ldx, Y, ldy, s);
    return;
  }
  if (bwd_wave() != w0 % kBwdWaves) return;
  const int lane = threadIdx.x & 63, i = lane & 15, q = lane >> 4;
  const int ci = min(i, n - 1);
  const f32x4 v = tile_xw<false, true>(X, ldx, ci, Y, ldy, ci, K, q);
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int r = 4 * q + rr;
    if (r < n && i < n) out[r * ldo + i] = i <= r ? s * v[rr] : 0.0f;
  }
}

// Operand panels of one mini-batch.
struct MB {
  // LDS, b x d (row stride d)
  float *K, *Q, *G2, *dZ, *dG2;
  // LDS, b x b (row stride b)
  float *M, *N, *dM, *dN;
  // workspace slice: b x m (row stride m), then dQ, dK, dYh (b x d)
  float *A, *Hk, *S1, *Gh, *G1, *Aq, *Hq, *dAq, *dHk, *dG1, *dGh, *dQ, *dK, *dYh;
};

// LDS floats of the b x d and b x b panels
__host__ __device__ constexpr int64_t panel_lds_floats(int d, int b) { return 5LL * b * d + 4LL * b * b; }
constexpr int64_t kLdsBytes = 160 * 1024;
// The state is kept in LDS when it fits beside the panels, its rows padded by 4 floats
// (W1 rows of m + 4, W2 rows of d + 4), so that a transposed read, one row per lane,
// falls on distinct banks.
__host__ __device__ constexpr int64_t state_lds_floats(int d, int m) { return 2LL * d * m + 4LL * (d + m); }
__host__ __device__ constexpr bool state_in_lds(int d, int m, int b) {
  return (state_lds_floats(d, m) + panel_lds_floats(d, b)) * 4 <= kLdsBytes;
}

// Where a (W1, W2) state lives and its row strides.
struct St {
  float* w1;
  float* w2;
  int ld1, ld2;
};

__device__ inline St state_at(float* base, bool padded, int d, int m) {
  St st;
  st.ld1 = padded ? m + 4 : m;
  st.ld2 = padded ? d + 4 : d;
  st.w1 = base;
  st.w2 = base + (int64_t)d * st.ld1;
  return st;
}

// workspace floats of one replayed mini-batch: its start state (W1, W2), then A, Hk, GELU'(A),
// Gh, G1 (b x m each), G2 (b x d), and the read-out's Aq, Hq, GELU'(Aq) (b x m each) and
// M = tril(Q K^T) (b x b).  The read-out's four are written only by the fp32 matrix-core replay
// (the generic replay leaves them to the backward scan).
__host__ __device__ constexpr int64_t segment_slot_floats(int d, int m, int b) {
  return 2LL * d * m + 8LL * b * m + (int64_t)b * d + (int64_t)b * b;
}

// workspace floats of one workgroup: the b x m panels, then dQ and dK
__host__ __device__ constexpr int64_t scratch_floats(int d, int m, int b) {
  return (int64_t)kBwdScratchPanels * b * m + 3LL * b * d;
}

__device__ void bind_panels(MB& t, float* lds, float* sc, int b, int d, int m) {
  t.K = lds;
  t.Q = t.K + b * d;
  t.G2 = t.Q + b * d;
  t.dZ = t.G2 + b * d;
  t.dG2 = t.dZ + b * d;
  t.M = t.dG2 + b * d;
  t.N = t.M + b * b;
  t.dM = t.N + b * b;
  t.dN = t.dM + b * b;
  float** panels[] = {&t.A, &t.Hk, &t.S1, &t.Gh, &t.G1, &t.Aq, &t.Hq, &t.dAq, &t.dHk, &t.dG1, &t.dGh};
  for (int i = 0; i < kBwdScratchPanels; ++i) *panels[i] = sc + (int64_t)i * b * m;
  t.dQ = sc + (int64_t)kBwdScratchPanels * b * m;
  t.dK = t.dQ + b * d;
  t.dYh = t.dK + b * d;
}

// copy rows x cols floats (cols a multiple of 4, rows 16-byte aligned) between row strides
__device__ inline void copy_rows(float* dst, int ldd, const float* src, int lds_, int rows, int cols) {
  const int q = cols / 4;
  for (int i = threadIdx.x; i < rows * q; i += BW) {
    const int r = i / q, c = 4 * (i - r * q);
    *(float4*)(dst + (int64_t)r * ldd + c) = *(const float4*)(src + (int64_t)r * lds_ + c);
  }
}

// a dense state (W1 [d, m] then W2 [m, d]) to or from a St
__device__ inline void state_in(const St& st, const float* src, int d, int m) {
  copy_rows(st.w1, st.ld1, src, m, d, m);
  copy_rows(st.w2, st.ld2, src + (int64_t)d * m, d, m, d);
}
__device__ inline void state_out(float* dst, const St& st, int d, int m) {
  copy_rows(dst, m, st.w1, st.ld1, d, m);
  copy_rows(dst + (int64_t)d * m, d, st.w2, st.ld2, m, d);
}

// The forward quantities of one mini-batch that the state update needs:
// A, Hk, S1, G2 (in place of V), Gh, G1.
__device__ void forward_core(const MB& t, const St& W, int n, int d, int m, float gscale, int gelu_tanh) {
  prod<4, false>(t.A, m, n, m, d, t.K, d, W.w1, W.ld1, 1.0f, false);  // A = K W1
  __syncthreads();
  for (int i = threadIdx.x; i < n * m; i += BW) {
    float g, dg, ddg;
    gelu3(t.A[i], gelu_tanh, &g, &dg, &ddg);
    t.Hk[i] = g;
    t.S1[i] = dg;
  }
  for (int i = threadIdx.x; i < n * d; i += BW) t.G2[i] *= -gscale;  // -c V
  __syncthreads();
  prod<1, false>(t.G2, d, n, d, m, t.Hk, m, W.w2, W.ld2, gscale, true);  // G2 = c (Hk W2 - V)
  __syncthreads();
  prod<4, true>(t.Gh, m, n, m, d, t.G2, d, W.w2, W.ld2, 1.0f, false);  // Gh = G2 W2^T
  __syncthreads();
  for (int i = threadIdx.x; i < n * m; i += BW) t.G1[i] = t.Gh[i] * t.S1[i];
  __syncthreads();
}

// W1 -= eta K^T G1; W2 -= eta Hk^T G2
__device__ void state_step(const MB& t, const St& W, int n, int d, int m, float eta) {
  Terms t1{1, {t.K}, {d}, {t.G1}, {m}};
  rank_update_any(W.w1, W.ld1, d, m, n, t1, -eta);
  Terms t2{1, {t.Hk}, {m}, {t.G2}, {d}};
  rank_update_any(W.w2, W.ld2, m, d, n, t2, -eta);
}

// Aq = Q W1 - eta tril(Q K^T) G1 and Hq = GELU(Aq) (GELU'(Aq) into dq when non-null).
__device__ void readout_hidden(const MB& t, const St& W, int n, int b, int d, int m, float eta, int gelu_tanh,
                               float* dq) {
  rowdot_tril(t.M, b, n, d, t.Q, d, t.K, d, 1.0f);  // M = tril(Q K^T)
  prod<4, false>(t.Aq, m, n, m, d, t.Q, d, W.w1, W.ld1, 1.0f, false, 1);
  __syncthreads();
  const bool tiled = n % 16 == 0 && m % 16 == 0;  // M G1 on the matrix cores (M is 0 above its diagonal)
  if (tiled) {
    prod_mfma<false, false>(t.Aq, m, n, m, n, t.M, b, t.G1, m, -eta, true, 0);
    __syncthreads();
  }
  for (int i = threadIdx.x; i < n * m; i += BW) {
    const int r = i / m, c = i - r * m;
    float corr = 0.0f;
    if (!tiled)
      for (int k = 0; k <= r; ++k) corr = fmaf(t.M[r * b + k], t.G1[k * m + c], corr);
    const float aq = t.Aq[i] - eta * corr;
    float g, dg, ddg;
    gelu3(aq, gelu_tanh, &g, &dg, &ddg);
    t.Aq[i] = aq;
    t.Hq[i] = g;
    if (dq) dq[i] = dg;
  }
  __syncthreads();
}

struct Rows {
  const float *qb, *kb, *vb;
  int64_t T;
  int reverse;
  __device__ int64_t tok(int64_t pos) const { return reverse ? T - 1 - pos : pos; }
};

// K, V (into G2, unless with_v is false), Q rows of the mini-batch starting at scan position p0
__device__ void load_qkv(const MB& t, const Rows& rw, int64_t p0, int n, int d, bool with_v = true) {
  for (int i = threadIdx.x; i < n * d; i += BW) {
    const int r = i / d, c = i - r * d;
    const int64_t tt = rw.tok(p0 + r);
    t.K[i] = rw.kb[tt * d + c];
    if (with_v) t.G2[i] = rw.vb[tt * d + c];
    t.Q[i] = rw.qb[tt * d + c];
  }
}

// ---------------------------------------------------------------------------
// Forward pass for the backward: one direction, Z and Y out, and the state at
// the start of every ckpt_every-th mini-batch (the same steps the backward
// replays, so the replayed states are these states bit for bit).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(BW) void scan_fwd_ckpt_kernel(ScanArgs a) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int d = a.d, m = a.m, b = a.b;
  const int64_t T = a.T;
  const int s = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int D = a.H * d;
  const int64_t dm = (int64_t)d * m;
  const int64_t sh = (int64_t)s * a.H + h;
  const int64_t nmb = (T + b - 1) / b;
  const int64_t nseg = (nmb + a.ckpt_every - 1) / a.ckpt_every;
  const bool wl = state_in_lds(d, m, b);
  MB t;
  bind_panels(t, lds + (wl ? state_lds_floats(d, m) : 0), a.scratch + sh * scratch_floats(d, m, b), b, d, m);
  const St W = state_at(wl ? lds : a.wstate + sh * 2 * dm, wl, d, m);
  copy_rows(W.w1, W.ld1, a.w1_0 + (int64_t)h * dm, m, d, m);
  copy_rows(W.w2, W.ld2, a.w2_0 + (int64_t)h * dm, d, m, d);
  const int64_t plane = a.B * a.H * T * d;
  Rows rw{a.qkv + sh * T * d, a.qkv + plane + sh * T * d, a.qkv + 2 * plane + sh * T * d, T, a.reverse};
  __syncthreads();
  for (int64_t j = 0; j < nmb; ++j) {
    const int n = (int)min((int64_t)b, T - j * b);
    if (j % a.ckpt_every == 0) state_out(a.ckpt + (sh * nseg + j / a.ckpt_every) * 2 * dm, W, d, m);
    load_qkv(t, rw, j * b, n, d);
    __syncthreads();
    forward_core(t, W, n, d, m, a.gscale, a.gelu_tanh);
    readout_hidden(t, W, n, b, d, m, a.eta, a.gelu_tanh, nullptr);
    rowdot_tril(t.N, b, n, m, t.Hq, m, t.Hk, m, 1.0f);  // N = tril(Hq Hk^T)
    prod<1, false>(t.dZ, d, n, d, m, t.Hq, m, W.w2, W.ld2, 1.0f, false);  // Hq W2
    __syncthreads();
    // Z = Hq W2 - eta N G2, the gate, and the state step
    for (int i = threadIdx.x; i < n * d; i += BW) {
      const int r = i / d, c = i - r * d;
      float corr = 0.0f;
      for (int k = 0; k <= r; ++k) corr = fmaf(t.N[r * b + k], t.G2[k * d + c], corr);
      const float z = t.dZ[i] - a.eta * corr;
      const int64_t o = ((int64_t)s * T + rw.tok(j * b + r)) * D + (int64_t)h * d + c;
      a.z[o] = z;
      store_io(a.y, o, load_io(a.xin, o, a.bf16) + tanhf(a.alpha[h * d + c]) * z, a.bf16);
    }
    state_step(t, W, n, d, m, a.eta);
    __syncthreads();
  }
}

// REPLAYED false: one launch walks every segment, replaying each from its checkpoint;
// true: the segments seg_hi .. seg_lo were replayed into segst beforehand.
template <bool REPLAYED>
__global__ __launch_bounds__(BW) void scan_backward_kernel(BwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
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

  const bool wl = state_in_lds(d, m, b);
  MB t;
  bind_panels(t, lds + (wl ? state_lds_floats(d, m) : 0), a.scratch + sh * scratch_floats(d, m, b), b, d, m);
  // replayed state, then (state in LDS) each mini-batch's start state
  const St Wc = state_at(wl ? lds : a.wcur + sh * 2 * dm, wl, d, m);
  float* dW1 = a.dstate + sh * 2 * dm;  // adjoint of the state after the current mini-batch
  float* dW2 = dW1 + dm;
  // one slot per mini-batch of a segment: its start state, then the forward quantities the
  // replay computed for it (A, Hk, GELU'(A), Gh, G1, each b x m, and G2, b x d)
  const int64_t bm = (int64_t)b * m, slot = segment_slot_floats(d, m, b);
  float* seg = a.segst + sh * (int64_t)C * slot;
  float* const scratch_A = t.A;  // the workgroup's own b x m panels (the unkept last mini-batch)
  (void)scratch_A;
  auto bind_fwd = [&](float* base) {
    t.A = base;
    t.Hk = base + bm;
    t.S1 = base + 2 * bm;
    t.Gh = base + 3 * bm;
    t.G1 = base + 4 * bm;
  };
  if (!REPLAYED || a.first)
    for (int64_t i = tid; i < 2 * dm; i += BW) dW1[i] = 0.0f;

  const int64_t plane = a.B * a.H * T * d;
  Rows rw{a.qkv + sh * T * d, a.qkv + plane + sh * T * d, a.qkv + 2 * plane + sh * T * d, T, a.reverse};

  const int64_t sg_hi = REPLAYED ? a.seg_hi : nseg - 1, sg_lo = REPLAYED ? a.seg_lo : 0;
  for (int64_t sg = sg_hi; sg >= sg_lo; --sg) {
    const int64_t j0 = sg * C, j1 = min(nmb, j0 + C);
    if (REPLAYED) seg = a.segst + ((sh * a.seg_count + (sg - sg_lo)) * C) * slot;
    // replay the segment's forward steps from its checkpoint, keeping each mini-batch's start state
    if (!REPLAYED) state_in(Wc, a.ckpt + (sh * nseg + sg) * 2 * dm, d, m);
    __syncthreads();
    for (int64_t j = j0; j < j1 && !REPLAYED; ++j) {
      float* sl = seg + (j - j0) * slot;
      state_out(sl, Wc, d, m);
      if (j + 1 == j1) break;
      const int n = (int)min((int64_t)b, T - j * b);
      load_qkv(t, rw, j * b, n, d);
      bind_fwd(sl + 2 * dm);
      __syncthreads();
      forward_core(t, Wc, n, d, m, a.gscale, a.gelu_tanh);
      copy_rows(sl + 2 * dm + 5 * bm, d, t.G2, d, n, d);
      state_step(t, Wc, n, d, m, eta);
      __syncthreads();
    }
    __syncthreads();
    // the segment's mini-batches, last to first
    for (int64_t j = j1 - 1; j >= j0; --j) {
      // marks (measurement build): mini-batches of this launch in walking order
      const int64_t mk = (sg_hi - sg) * C + (j1 - 1 - j);
      (void)mk;
      TTT_MARK(g_marks_scan_backward, mk, 0);
      const int n = (int)min((int64_t)b, T - j * b);
      float* sl = seg + (j - j0) * slot;
      St W = state_at(sl, false, d, m);
      if (wl) {
        state_in(Wc, W.w1, d, m);
        W = Wc;
      }
      // every mini-batch but the segment's last has its forward quantities from the replay
      // (all of them when the segments were replayed beforehand)
      const bool kept = REPLAYED || j + 1 < j1;
      load_qkv(t, rw, j * b, n, d, !kept);
      if (REPLAYED) {
        // the read-out's quantities from the slot too: Hq and GELU'(Aq) (into dAq) copied to
        // this workgroup's panels (pointing the panels at the slot instead cost 30 more spilled
        // registers), M into LDS
        bind_fwd(sl + 2 * dm);
        const float* ro = sl + 2 * dm + 5 * bm + (int64_t)b * d;
        copy_rows(t.G2, d, sl + 2 * dm + 5 * bm, d, n, d);
        copy_rows(t.Hq, m, ro + bm, m, n, m);
        copy_rows(t.dAq, m, ro + 2 * bm, m, n, m);
        for (int i = tid; i < b * b; i += BW) t.M[i] = ro[3 * bm + i];
      } else if (kept) {
        bind_fwd(sl + 2 * dm);
        copy_rows(t.G2, d, sl + 2 * dm + 5 * bm, d, n, d);
      } else {
        bind_fwd(scratch_A);
      }
      for (int i = tid; i < n * d; i += BW) {
        const int r = i / d, c = i - r * d;
        const int ch = h * d + c;
        t.dZ[i] = tanhf(a.alpha[ch]) * a.dy[((int64_t)s * T + rw.tok(j * b + r)) * D + ch];
      }
      __syncthreads();
      TTT_MARK(g_marks_scan_backward, mk, 1);
      if (!kept) forward_core(t, W, n, d, m, a.gscale, a.gelu_tanh);
      if (!REPLAYED) readout_hidden(t, W, n, b, d, m, eta, a.gelu_tanh, t.dAq);  // dAq holds GELU'(Aq) for now
      TTT_MARK(g_marks_scan_backward, mk, 2);
      // N = tril(Hq Hk^T); dN = tril(-eta dZ G2^T); dZ W2^T (into dGh for now)
      rowdot_tril(t.N, b, n, m, t.Hq, m, t.Hk, m, 1.0f);
      rowdot_tril(t.dN, b, n, d, t.dZ, d, t.G2, d, -eta, 1);
      prod<4, true>(t.dGh, m, n, m, d, t.dZ, d, W.w2, W.ld2, 1.0f, false, 2);
      __syncthreads();
      TTT_MARK(g_marks_scan_backward, mk, 3);
      // dAq = (dZ W2^T + dN Hk) * GELU'(Aq); dG2 = -eta N^T dZ; dHk = dN^T Hq
      if (n % 16 == 0 && m % 16 == 0 && d % 16 == 0) {  // on the matrix cores (N, dN are 0 above the diagonal)
        prod_mfma<false, false>(t.dGh, m, n, m, n, t.dN, b, t.Hk, m, 1.0f, true, 0);
        prod_mfma<true, false>(t.dHk, m, n, m, n, t.dN, b, t.Hq, m, 1.0f, false, 0);
        prod_mfma<true, false>(t.dG2, d, n, d, n, t.N, b, t.dZ, d, -eta, false, 0);
        __syncthreads();
        for (int i = tid; i < n * m; i += BW) t.dAq[i] *= t.dGh[i];
      } else {
        for (int i = tid; i < n * m; i += BW) {
          const int r = i / m, c = i - r * m;
          float v = t.dGh[i];
          for (int k = 0; k <= r; ++k) v = fmaf(t.dN[r * b + k], t.Hk[k * m + c], v);
          t.dAq[i] *= v;
          float w = 0.0f;
          for (int k = r; k < n; ++k) w = fmaf(t.dN[k * b + r], t.Hq[k * m + c], w);
          t.dHk[i] = w;
        }
        for (int i = tid; i < n * d; i += BW) {
          const int r = i / d, c = i - r * d;
          float v = 0.0f;
          for (int k = r; k < n; ++k) v = fmaf(t.N[k * b + r], t.dZ[k * d + c], v);
          t.dG2[i] = -eta * v;
        }
      }
      __syncthreads();
      // dQ = dAq W1^T; dM = tril(-eta dAq G1^T); with the adjoints of the state after this
      // mini-batch: dHk -= eta G2 dW2'^T, dG2 -= eta Hk dW2', dG1 = -eta K dW1', dK = -eta G1 dW1'^T
      TTT_MARK(g_marks_scan_backward, mk, 4);
      prod<1, true>(t.dQ, d, n, d, m, t.dAq, m, W.w1, W.ld1, 1.0f, false);
      rowdot_tril(t.dM, b, n, m, t.dAq, m, t.G1, m, -eta, 4);
      prod<4, true>(t.dHk, m, n, m, d, t.G2, d, dW2, d, -eta, true, 5);
      prod<1, false>(t.dG2, d, n, d, m, t.Hk, m, dW2, d, -eta, true, 5);
      prod<4, false>(t.dG1, m, n, m, d, t.K, d, dW1, m, -eta, false, 9);
      prod<1, true>(t.dK, d, n, d, m, t.G1, m, dW1, m, -eta, false, 9);
      __syncthreads();
      TTT_MARK(g_marks_scan_backward, mk, 5);
      // dG1 -= eta M^T dAq; dQ += dM K; dK += dM^T Q
      for (int i = tid; i < n * m; i += BW) {
        const int r = i / m, c = i - r * m;
        float v = 0.0f;
        for (int k = r; k < n; ++k) v = fmaf(t.M[k * b + r], t.dAq[k * m + c], v);
        t.dG1[i] -= eta * v;
      }
      for (int i = tid; i < n * d; i += BW) {
        const int r = i / d, c = i - r * d;
        float q = 0.0f, k1 = 0.0f;
        for (int k = 0; k < n; ++k) {
          q = fmaf(t.dM[r * b + k], t.K[k * d + c], q);
          k1 = fmaf(t.dM[k * b + r], t.Q[k * d + c], k1);
        }
        t.dQ[i] += q;
        t.dK[i] += k1;
      }
      __syncthreads();
      // dGh = dG1 * S1; dA (in dG1) = dG1 * Gh * GELU''(A)
      TTT_MARK(g_marks_scan_backward, mk, 6);
      for (int i = tid; i < n * m; i += BW) {
        float g, dg, ddg;
        gelu3(t.A[i], a.gelu_tanh, &g, &dg, &ddg);
        const float x = t.dG1[i];
        t.dGh[i] = x * t.S1[i];
        t.dG1[i] = x * t.Gh[i] * ddg;
      }
      __syncthreads();
      prod<1, false>(t.dG2, d, n, d, m, t.dGh, m, W.w2, W.ld2, 1.0f, true);  // dG2 += dGh W2
      __syncthreads();
      for (int i = tid; i < n * d; i += BW) t.dYh[i] = a.gscale * t.dG2[i];  // gradient of Y-hat = Hk W2
      __syncthreads();
      prod<4, true>(t.dHk, m, n, m, d, t.dYh, d, W.w2, W.ld2, 1.0f, true);  // dHk += dYh W2^T
      __syncthreads();
      for (int i = tid; i < n * m; i += BW) t.dG1[i] += t.dHk[i] * t.S1[i];  // dA += dHk * S1
      __syncthreads();
      prod<1, true>(t.dK, d, n, d, m, t.dG1, m, W.w1, W.ld1, 1.0f, true);  // dK += dA W1^T
      __syncthreads();
      TTT_MARK(g_marks_scan_backward, mk, 7);
      // dQ, dK, dV = -dYh to their columns of [B, T, 3D]; the adjoints handed back:
      // dW1 += Q^T dAq + K^T dA; dW2 += Hq^T dZ + dGh^T G2 + Hk^T dYh
      for (int i = tid; i < n * d; i += BW) {
        const int r = i / d, c = i - r * d;
        float* row = a.dqkv + ((int64_t)s * T + rw.tok(j * b + r)) * 3 * D + h * d + c;
        row[0] = t.dQ[i];
        row[D] = t.dK[i];
        row[2 * D] = -t.dYh[i];
      }
      Terms u1{2, {t.Q, t.K}, {d, d}, {t.dAq, t.dG1}, {m, m}};
      rank_update_any(dW1, m, d, m, n, u1, 1.0f);
      Terms u2{3, {t.Hq, t.dGh, t.Hk}, {m, m, m}, {t.dZ, t.G2, t.dYh}, {d, d, d}};
      rank_update_any(dW2, d, m, d, n, u2, 1.0f);
      __syncthreads();
    }
  }
  if (!REPLAYED || sg_lo == 0) {
    float* o = a.dw_seq + sh * 2 * dm;
    for (int64_t i = tid; i < 2 * dm; i += BW) o[i] = dW1[i];
  }
}

// ---------------------------------------------------------------------------
// Backward scan over replayed windows with each chain's hidden units split over
// S = 2 or 4 workgroups of one cooperative launch (the notes page's on-chip tensor
// parallel: the state sharded over CUs, an all-reduce between them).  Workgroup
// part p (0 .. S-1) of chain sh takes units [p m/S, (p+1) m/S): its part of the
// mini-batch's state (W1 columns, W2 rows) and its part of the adjoint, both in
// LDS (the adjoint goes to the workspace between launches), the b x d and b x b
// panels in LDS, its b x m/S panels in the workspace.  Every product over units
// splits into the parts' partial sums.  Those that only feed outputs (dQ, dK, and
// dM, linear in them) are added by float atomics into buffers that each take two
// addends onto zero, so that the sums do not depend on their order: parts 0 and 1
// into dQ|dK|dV, parts 2 and 3 into a second [B, T, 2D] buffer added to it after
// the walk.  The one that feeds the rest of the step, dG2 = -eta N^T dZ - eta Hk
// dW2' + dGh W2 (N too is a sum over units), is exchanged: each part publishes its
// partial as tagged 64-bit device-scope stores (the mini-batch index + 1 in the
// high word, double-buffered by its parity) and polls the others'; all add them in
// the order of the parts.
// Polls are bounded: a workgroup that waits past the spin limit raises the abort
// flag, which every poll checks, and takes NaN for the missing partial, so a lost
// peer shows as NaN gradients rather than a hang.
// ---------------------------------------------------------------------------
constexpr uint32_t kSplitSpinMax = 1u << 20;
// The split walk runs at the one shape the fp32 matrix-core forward pass and replay serve
// (d = 64, m = 256, b = 16, the erf GELU): with the sizes compile-time constants its index
// arithmetic folds.
constexpr int kSplitD = 64, kSplitM = 256, kSplitB = 16;

// floats of a split workgroup's scratch: its b x m/S panels dAq, dHk, dG1 (then dA), dGh, and
// its dQ and dK partials (b x d); in LDS with four parts, in the workspace with two
__host__ __device__ constexpr int64_t split_scratch_floats(int d, int m, int b, int S) {
  return 4LL * b * (m / S) + 2LL * b * d;
}
// floats of the seven b x m/S slot panels a four-part workgroup stages in LDS (A, Hk, GELU'(A),
// Gh, G1, Hq, GELU'(Aq); rows of m/S + 4)
__host__ __device__ constexpr int64_t split_slot_panel_floats(int m, int b, int S) {
  return 7LL * b * (m / S + 4);
}
// LDS floats of a split workgroup: its part of the state and of the adjoint (W1 columns as
// [d][m/S + 4], W2 rows as [m/S][d + 4]), the b x d and b x b panels, and with four parts its
// scratch and its slot panels
__host__ __device__ constexpr int64_t split_lds_floats(int d, int m, int b, int S) {
  return 2 * ((int64_t)d * (m / S + 4) + (int64_t)(m / S) * (d + 4)) + panel_lds_floats(d, b) +
         (S == 4 ? split_scratch_floats(d, m, b, S) + split_slot_panel_floats(m, b, S) : 0);
}

__device__ float4 g_bwd_zero_chunk;  // zero-initialised, never written: the source of padding chunks

template <int S>
__global__ __launch_bounds__(BW) void scan_backward_split_kernel(BwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  constexpr int d = kSplitD, m = kSplitM, b = kSplitB, mh = m / S;  // mh: this part's units
  const int tid = threadIdx.x;
  const int64_t BH = a.B * a.H;
  const int half = (int)(blockIdx.x / BH);             // the part
  const int64_t sh = (int64_t)blockIdx.x - half * BH;  // sequence * H + head
  const int s = (int)(sh / a.H), h = (int)(sh % a.H);
  const int u0 = half * mh;
  const int64_t T = a.T;
  const int D = a.H * d;
  const float eta = a.eta;
  const int64_t dm = (int64_t)d * m, bm = (int64_t)b * m, slot = segment_slot_floats(d, m, b);
  const int64_t nmb = (T + b - 1) / b;
  const int C = a.ckpt_every;

  St W;  // the mini-batch's state, this part
  W.ld1 = mh + 4;
  W.ld2 = d + 4;
  W.w1 = lds;
  W.w2 = W.w1 + (int64_t)d * W.ld1;
  const int la1 = mh + 4, la2 = d + 4;  // the adjoint's part, same layout
  float* dW1 = W.w2 + (int64_t)mh * W.ld2;
  float* dW2 = dW1 + (int64_t)d * la1;
  MB t;  // only the b x d and b x b panels (LDS) of MB
  t.K = dW2 + (int64_t)mh * la2;
  t.Q = t.K + b * d;
  t.G2 = t.Q + b * d;
  t.M = t.G2 + b * d;
  t.dZ = t.M + b * b;
  t.dG2 = t.dZ + b * d;  // this part's partial of dG2, then the whole dG2 times c, i.e. dYh
  t.N = t.dG2 + b * d;   // this part's part of tril(Hq Hk^T)
  t.dM = t.N + b * b;    // this part's part of dM
  t.dN = t.dM + b * b;
  float* sc = S == 4 ? t.dN + b * b  // LDS, after the panels
                     : a.scratch + sh * scratch_floats(d, m, b) + half * split_scratch_floats(d, m, b, S);
  float* dAq = sc;
  float* dHk = dAq + (int64_t)b * mh;
  float* dG1 = dHk + (int64_t)b * mh;
  float* dGh = dG1 + (int64_t)b * mh;
  float* dQp = dGh + (int64_t)b * mh;
  float* dKp = dQp + (int64_t)b * d;
  // with four parts the step's slot panels in LDS (rows of mh + 4), after the scratch
  constexpr int pld = S == 4 ? mh + 4 : m;  // their row stride (in the slot: m)
  float* const spl = dKp + (int64_t)b * d;
  uint64_t* xc = a.xchg + sh * 2 * S * (int64_t)(b * d);  // [part][parity][b d]

  // the adjoint's part: zero (the window that starts the walk) or as the previous window left it
  float* gW = a.dstate + sh * 2 * dm;
  if (a.first) {
    for (int i = tid; i < d * la1; i += BW) dW1[i] = 0.0f;
    for (int i = tid; i < mh * la2; i += BW) dW2[i] = 0.0f;
  } else {
    copy_rows(dW1, la1, gW + u0, m, d, mh);
    copy_rows(dW2, la2, gW + dm + (int64_t)u0 * d, d, mh, d);
  }

  const int64_t plane = a.B * a.H * T * d;
  Rows rw{a.qkv + sh * T * d, a.qkv + plane + sh * T * d, a.qkv + 2 * plane + sh * T * d, T, a.reverse};
  bool failed = false;  // this thread saw an abort or a time-out

  for (int64_t sg = a.seg_hi; sg >= a.seg_lo; --sg) {
    const int64_t j0 = sg * C, j1 = min(nmb, j0 + C);
    const float* seg = a.segst + ((sh * a.seg_count + (sg - a.seg_lo)) * C) * slot;
    for (int64_t j = j1 - 1; j >= j0; --j) {
      const int64_t mk = (a.seg_hi - sg) * C + (j1 - 1 - j);  // marks: mini-batches of this launch
      (void)mk;
      TTT_MARK(g_marks_scan_backward, mk, 0);
      const int n = (int)min((int64_t)b, T - j * b);
      const float* sl = seg + (j - j0) * slot;
      // the slot's panels, this part's columns (row stride m)
      const float* fq = sl + 2 * dm;
      const float* ro = fq + 5 * bm + (int64_t)b * d;  // the read-out: Aq, Hq, GELU'(Aq), M
      // the seven panels this step reads: in the slot (two parts) or staged in LDS (four)
      const float *A_, *Hk_, *S1_, *Gh_, *G1_, *Hq_, *S1q_;
      if constexpr (S == 4) {
        A_ = spl, Hk_ = spl + b * pld, S1_ = spl + 2 * b * pld, Gh_ = spl + 3 * b * pld, G1_ = spl + 4 * b * pld;
        Hq_ = spl + 5 * b * pld, S1q_ = spl + 6 * b * pld;
      } else {
        A_ = fq + u0, Hk_ = fq + bm + u0, S1_ = fq + 2 * bm + u0, Gh_ = fq + 3 * bm + u0, G1_ = fq + 4 * bm + u0;
        Hq_ = ro + bm + u0, S1q_ = ro + 2 * bm + u0;
      }
      // ---- the state part, K and Q rows, G2, M (and with four parts the seven panels), dZ = tanh(alpha) dY
      __syncthreads();  // the previous step's last reads of the LDS panels and state
      if constexpr (S == 4) {
        // direct global -> LDS loads, 16 bytes a lane, all in flight at once; each wave
        // instruction fills 64 consecutive chunks of one of three LDS regions:
        //   1: W1 columns then W2 rows of this part, 17 chunks a row (the 17th: padding)
        //   2: K and Q rows (by token; rows past n zero), G2 (rows past n zero), M
        //   3: the seven panels, 17 chunks a row (rows past n zero)
        constexpr int RC = 17, N1 = (d + mh) * RC, N2 = 3 * b * d / 4 + b * b / 4, N3 = 7 * b * RC;
        constexpr int I1 = (N1 + 63) / 64, I2 = (N2 + 63) / 64, I3 = (N3 + 63) / 64;
        const int wv = tid >> 6, ln = tid & 63;
        const void* zero = (const void*)&g_bwd_zero_chunk;
        for (int i = wv; i < I1 + I2 + I3; i += kBwdWaves) {
          const void* src = zero;
          const float* base;
          int g;
          if (i < I1) {
            base = W.w1;
            g = 64 * i + ln;
            if (g >= N1) continue;
            const int r = g / RC, c = g - r * RC;
            if (c < 16)
              src = r < d ? sl + (int64_t)r * m + u0 + 4 * c : sl + dm + (int64_t)(u0 + r - d) * d + 4 * c;
          } else if (i < I1 + I2) {
            base = t.K;
            g = 64 * (i - I1) + ln;
            if (g >= N2) continue;
            const int q = g >> 4, c = g & 15;  // q: row of K (0..b-1), Q (b..2b-1), G2 (2b..3b-1), then M
            if (q < 2 * b) {
              const int r = q < b ? q : q - b;
              if (r < n) src = (q < b ? rw.kb : rw.qb) + rw.tok(j * b + r) * d + 4 * c;
            } else if (q < 3 * b) {
              if (q - 2 * b < n) src = fq + 5 * bm + (int64_t)(q - 2 * b) * d + 4 * c;
            } else {
              src = ro + 3 * bm + 4 * (g - 3 * b * d / 4);
            }
          } else {
            base = spl;
            g = 64 * (i - I1 - I2) + ln;
            if (g >= N3) continue;
            const int p = g / (b * RC), rr = g - p * (b * RC), r = rr / RC, c = rr - r * RC;
            if (c < 16 && r < n) src = (p < 5 ? fq + p * bm : ro + (p - 4) * bm) + u0 + (int64_t)r * m + 4 * c;
          }
          tb::dma16(src, tb::lds_addr_uniform(base, 1024u * (uint32_t)(g >> 6)));
        }
      } else {
        copy_rows(W.w1, W.ld1, sl + u0, m, d, mh);
        copy_rows(W.w2, W.ld2, sl + dm + (int64_t)u0 * d, d, mh, d);
        load_qkv(t, rw, j * b, n, d, false);
        copy_rows(t.G2, d, fq + 5 * bm, d, n, d);
        for (int i = tid; i < b * b; i += BW) t.M[i] = ro[3 * bm + i];
      }
      for (int i = tid; i < n * d; i += BW) {
        const int r = i / d, c = i - r * d;
        const int ch = h * d + c;
        t.dZ[i] = tanhf(a.alpha[ch]) * a.dy[((int64_t)s * T + rw.tok(j * b + r)) * D + ch];
      }
      if constexpr (S == 4) vmem_done();  // this wave's direct loads have landed
      __syncthreads();
      TTT_MARK(g_marks_scan_backward, mk, 1);
      // ---- N (this part) = tril(Hq Hk^T); dN = tril(-eta dZ G2^T); dZ W2^T (into dGh for now)
      rowdot_tril(t.N, b, n, mh, Hq_, pld, Hk_, pld, 1.0f);
      rowdot_tril(t.dN, b, n, d, t.dZ, d, t.G2, d, -eta, 1);
      prod<4, true>(dGh, mh, n, mh, d, t.dZ, d, W.w2, W.ld2, 1.0f, false, 2);
      __syncthreads();
      TTT_MARK(g_marks_scan_backward, mk, 2);
      // ---- dAq = (dZ W2^T + dN Hk) * GELU'(Aq); dHk = dN^T Hq; dG2 (this part) = -eta N^T dZ
      if (n % 16 == 0 && mh % 16 == 0 && d % 16 == 0) {  // on the matrix cores (N, dN are 0 above the diagonal)
        prod_mfma<false, false>(dGh, mh, n, mh, n, t.dN, b, Hk_, pld, 1.0f, true, 0);
        prod_mfma<true, false>(dHk, mh, n, mh, n, t.dN, b, Hq_, pld, 1.0f, false, 0);
        prod_mfma<true, false>(t.dG2, d, n, d, n, t.N, b, t.dZ, d, -eta, false, 0);
        __syncthreads();
        for (int i = tid; i < n * mh; i += BW) {
          const int r = i / mh, c = i - r * mh;
          dAq[i] = S1q_[r * pld + c] * dGh[i];
        }
      } else {
        for (int i = tid; i < n * mh; i += BW) {
          const int r = i / mh, c = i - r * mh;
          float v = dGh[i];
          for (int k = 0; k <= r; ++k) v = fmaf(t.dN[r * b + k], Hk_[k * pld + c], v);
          dAq[i] = S1q_[r * pld + c] * v;
          float w = 0.0f;
          for (int k = r; k < n; ++k) w = fmaf(t.dN[k * b + r], Hq_[k * pld + c], w);
          dHk[i] = w;
        }
        for (int i = tid; i < n * d; i += BW) {
          const int r = i / d, c = i - r * d;
          float v = 0.0f;
          for (int k = r; k < n; ++k) v = fmaf(t.N[k * b + r], t.dZ[k * d + c], v);
          t.dG2[i] = -eta * v;
        }
      }
      __syncthreads();
      TTT_MARK(g_marks_scan_backward, mk, 3);
      // ---- dQ (this part) = dAq W1^T; dM (this part) = tril(-eta dAq G1^T); with the adjoint's part:
      //      dHk -= eta G2 dW2'^T, dG2 -= eta Hk dW2', dG1 = -eta K dW1', dK (this part) = -eta G1 dW1'^T
      prod<1, true>(dQp, d, n, d, mh, dAq, mh, W.w1, W.ld1, 1.0f, false);
      rowdot_tril(t.dM, b, n, mh, dAq, mh, G1_, pld, -eta, 4);
      prod<4, true>(dHk, mh, n, mh, d, t.G2, d, dW2, la2, -eta, true, 5);
      prod<1, false>(t.dG2, d, n, d, mh, Hk_, pld, dW2, la2, -eta, true, 5);
      prod<4, false>(dG1, mh, n, mh, d, t.K, d, dW1, la1, -eta, false, 9);
      prod<1, true>(dKp, d, n, d, mh, G1_, pld, dW1, la1, -eta, false, 9);
      __syncthreads();
      TTT_MARK(g_marks_scan_backward, mk, 4);
      // ---- dG1 -= eta M^T dAq; dQ += dM K; dK += dM^T Q (this part's dM)
      for (int i = tid; i < n * mh; i += BW) {
        const int r = i / mh, c = i - r * mh;
        float v = 0.0f;
        for (int k = r; k < n; ++k) v = fmaf(t.M[k * b + r], dAq[k * mh + c], v);
        dG1[i] -= eta * v;
      }
      for (int i = tid; i < n * d; i += BW) {
        const int r = i / d, c = i - r * d;
        float q = 0.0f, k1 = 0.0f;
        for (int k = 0; k < n; ++k) {
          q = fmaf(t.dM[r * b + k], t.K[k * d + c], q);
          k1 = fmaf(t.dM[k * b + r], t.Q[k * d + c], k1);
        }
        dQp[i] += q;
        dKp[i] += k1;
      }
      __syncthreads();
      // ---- dGh = dG1 * S1; dA (in dG1) = dG1 * Gh * GELU''(A)
      for (int i = tid; i < n * mh; i += BW) {
        const int r = i / mh, c = i - r * mh;
        float g, dg, ddg;
        gelu3(A_[r * pld + c], false, &g, &dg, &ddg);
        const float x = dG1[i];
        dGh[i] = x * S1_[r * pld + c];
        dG1[i] = x * Gh_[r * pld + c] * ddg;
      }
      __syncthreads();
      prod<1, false>(t.dG2, d, n, d, mh, dGh, mh, W.w2, W.ld2, 1.0f, true);  // dG2 (this part) += dGh W2
      __syncthreads();
      TTT_MARK(g_marks_scan_backward, mk, 5);
      // ---- dG2 = the parts' partials added in the parts' order, exchanged; dYh = c dG2 (in dG2's
      //      place)
      {
        const uint32_t tag = (uint32_t)(j + 1);
        const int par = (int)(j & 1);
        uint64_t* mine = xc + (half * 2 + par) * (int64_t)(b * d);
        for (int i = tid; i < n * d; i += BW)
          __hip_atomic_store(mine + i, ((uint64_t)tag << 32) | __float_as_uint(t.dG2[i]), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        for (int i = tid; i < n * d; i += BW) {
          float sum = 0.0f;
#pragma unroll
          for (int q = 0; q < S; ++q) {
            float v = __uint_as_float(0x7fc00000u);  // NaN unless the partial arrives
            if (q == half) {
              v = t.dG2[i];
            } else {
              const uint64_t* theirs = xc + (q * 2 + par) * (int64_t)(b * d);
              for (uint32_t spin = 0; !failed; ++spin) {
                const uint64_t e = __hip_atomic_load(theirs + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if ((uint32_t)(e >> 32) == tag) {
                  v = __uint_as_float((uint32_t)e);
                  break;
                }
                if (spin >= kSplitSpinMax) {
                  __hip_atomic_store(a.abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                  failed = true;
                } else if ((spin & 15) == 15 &&
                           __hip_atomic_load(a.abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                  failed = true;
                }
                __builtin_amdgcn_s_sleep(1);
              }
            }
            sum = q == 0 ? v : sum + v;
          }
          t.dG2[i] = a.gscale * sum;
        }
      }
      __syncthreads();
      TTT_MARK(g_marks_scan_backward, mk, 6);
      prod<4, true>(dHk, mh, n, mh, d, t.dG2, d, W.w2, W.ld2, 1.0f, true);  // dHk += dYh W2^T
      __syncthreads();
      for (int i = tid; i < n * mh; i += BW) {  // dA += dHk * S1
        const int r = i / mh, c = i - r * mh;
        dG1[i] += dHk[i] * S1_[r * pld + c];
      }
      __syncthreads();
      prod<1, true>(dKp, d, n, d, mh, dG1, mh, W.w1, W.ld1, 1.0f, true);  // dK (this part) += dA W1^T
      __syncthreads();
      TTT_MARK(g_marks_scan_backward, mk, 7);
      // ---- dQ and dK: this part's sums added into [B, T, 3D] (parts 0, 1) or the [B, T, 2D] buffer
      //      (parts 2, 3), both zeroed before the walk; dV = -dYh (part 0); the adjoint's part
      //      handed to the mini-batch before: dW1 += Q^T dAq + K^T dA; dW2 += Hq^T dZ + dGh^T G2 + Hk^T dYh
      for (int i = tid; i < n * d; i += BW) {
        const int r = i / d, c = i - r * d;
        const int64_t tr = (int64_t)s * T + rw.tok(j * b + r);
        float* row = half < 2 ? a.dqkv + tr * 3 * D + h * d + c : a.dqkv_b + tr * 2 * D + h * d + c;
        atomicAdd(row, dQp[i]);
        atomicAdd(row + D, dKp[i]);
        if (half == 0) row[2 * D] = -t.dG2[i];
      }
      Terms u1{2, {t.Q, t.K}, {d, d}, {dAq, dG1}, {mh, mh}};
      rank_update_any(dW1, la1, d, mh, n, u1, 1.0f);
      Terms u2{3, {Hq_, dGh, Hk_}, {pld, mh, pld}, {t.dZ, t.G2, t.dG2}, {d, d, d}};
      rank_update_any(dW2, la2, mh, d, n, u2, 1.0f);
    }
  }
  __syncthreads();
  // the adjoint's part to the workspace for the next window, or out when the walk reached the start
  float* o = (a.seg_lo == 0 ? a.dw_seq : a.dstate) + sh * 2 * dm;
  copy_rows(o + u0, m, dW1, la1, d, mh);
  copy_rows(o + dm + (int64_t)u0 * d, d, dW2, la2, mh, d);
}

__global__ void fill_zero_u64_kernel(uint64_t* p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
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

size_t scan_backward_lds_bytes(int d, int m, int b) {
  return sizeof(float) * (size_t)(panel_lds_floats(d, b) + (state_in_lds(d, m, b) ? state_lds_floats(d, m) : 0));
}

size_t scan_backward_scratch_elems(int d, int m, int b) { return (size_t)scratch_floats(d, m, b); }
size_t scan_backward_segment_elems(int d, int m, int b) { return (size_t)segment_slot_floats(d, m, b); }

hipError_t launch_scan_fwd_ckpt(const ScanArgs& a, hipStream_t s) {
  const size_t lds = scan_backward_lds_bytes(a.d, a.m, a.b);
  hipError_t e = hipFuncSetAttribute((const void*)scan_fwd_ckpt_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scan_fwd_ckpt_kernel, dim3((unsigned)(a.B * a.H)), dim3(BW), lds,
                     s, a);
  return hipGetLastError();
}

size_t scan_backward_split_lds_bytes(int d, int m, int b, int S) {
  return sizeof(float) * (size_t)split_lds_floats(d, m, b, S);
}

size_t scan_backward_split_xchg_elems(int64_t B, int H, int d, int b, int S) {
  return (size_t)(B * H) * 2 * S * b * d;
}

const void* split_kernel_fn(int S) {
  return S == 4 ? (const void*)scan_backward_split_kernel<4> : (const void*)scan_backward_split_kernel<2>;
}

bool scan_backward_split_fits(int64_t B, int H, int d, int m, int b, int S) {
  if ((S != 2 && S != 4) || d != kSplitD || m != kSplitM || b != kSplitB) return false;
  const size_t lds = scan_backward_split_lds_bytes(d, m, b, S);
  if (lds > 160 * 1024 || S * split_scratch_floats(d, m, b, S) > scratch_floats(d, m, b)) return false;
  int dev = 0, cus = 0, coop = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop) return false;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
  if (hipFuncSetAttribute(split_kernel_fn(S), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return false;
  const hipError_t e =
      S == 4 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, scan_backward_split_kernel<4>, BW, lds)
             : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, scan_backward_split_kernel<2>, BW, lds);
  if (e != hipSuccess) return false;
  return S * B * H <= (int64_t)cus * per_cu;
}

hipError_t launch_zero_u64(uint64_t* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_zero_u64_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_scan_backward_split(const BwdArgs& a, hipStream_t s) {
  if ((a.split != 2 && a.split != 4) || a.d != kSplitD || a.m != kSplitM || a.b != kSplitB || a.gelu_tanh)
    return hipErrorInvalidValue;
  const size_t lds = scan_backward_split_lds_bytes(a.d, a.m, a.b, a.split);
  hipError_t e = hipFuncSetAttribute(split_kernel_fn(a.split), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  BwdArgs args = a;
  void* kargs[] = {(void*)&args};
  return hipLaunchCooperativeKernel(split_kernel_fn(a.split), dim3((unsigned)(a.split * a.B * a.H)), dim3(BW), kargs,
                                    (unsigned)lds, s);
}

// dQ|dK columns of dqkv [rows, 3D] += buf [rows, 2D] (the four-part walk's second buffer)
__global__ void add_dqk_kernel(float* dqkv, const float* buf, int64_t rows, int D) {
  const int64_t n = rows * 2 * D, stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t r = i / (2 * D), c = i - r * 2 * D;
    dqkv[r * 3 * D + c] += buf[i];
  }
}

hipError_t launch_add_dqk(float* dqkv, const float* buf, int64_t rows, int D, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t n = rows * 2 * D, blocks = std::min<int64_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(add_dqk_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dqkv, buf, rows, D);
  return hipGetLastError();
}

hipError_t launch_scan_backward(const BwdArgs& a, hipStream_t s) {
  // T = 0 runs too: no segments, and the kernel writes the zero adjoint of the initial state
  const size_t lds = scan_backward_lds_bytes(a.d, a.m, a.b);
  const void* fn = a.replayed ? (const void*)scan_backward_kernel<true> : (const void*)scan_backward_kernel<false>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if (a.replayed)
    hipLaunchKernelGGL(scan_backward_kernel<true>, dim3((unsigned)(a.B * a.H)), dim3(BW), lds, s, a);
  else
    hipLaunchKernelGGL(scan_backward_kernel<false>, dim3((unsigned)(a.B * a.H)), dim3(BW), lds, s, a);
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

TTT_MARKS_EXPORT(ttt_phase_marks_scan_backward, g_marks_scan_backward);
