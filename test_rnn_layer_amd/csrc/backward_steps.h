// The backward's per-mini-batch steps (products, rank updates, operand panels,
// the forward quantities a replay recomputes), shared by the walks of
// backward.hip (one workgroup per chain) and backward_split.hip (several per
// chain).  The chain rule they implement is written out at the top of
// backward.hip.  The including file defines TTT_BWD_THREADS, the workgroup size
// all of them stride by: each translation unit gets its own copy.
#pragma once

#include "internal.h"
#include "mfma_common.h"

#ifndef TTT_BWD_THREADS
#error "define TTT_BWD_THREADS (the workgroup size) before including backward_steps.h"
#endif

namespace ttt {
namespace {

constexpr int BW = TTT_BWD_THREADS;  // threads of the including file's scan workgroups

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
// X(r, k) = X[r ldx + k], or X[k ldx + r] when XT; W(k, c) = W[k ldw + c], or W[c ldw + k] when WT.
// UNR: rounds of four k issued together (their loads before their products)
template <bool XT, bool WT, int UNR = 2>
__device__ __forceinline__ f32x4 tile_xw(const float* X, int ldx, int row, const float* W, int ldw, int col, int K,
                                         int q) {
  const int kq = K >> 2, kb = q * kq;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll UNR
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

// prod_mfma with an epilogue: each finished element v of out[r][c] is stored as epi(r, c, v),
// which may also write elements of other arrays at (r, c) (the elementwise step that follows
// the product, without a pass and a barrier of its own).  Inlined: an out-of-line call would take
// the epilogue's closure through private memory.  UNR: see tile_xw.
template <bool XT, bool WT, int UNR, class Epi>
__device__ __forceinline__ void prod_mfma_epi(float* out, int ldo, int n, int C, int K, const float* X,
                                                        int ldx, const float* W, int ldw, float s, bool acc, int w0,
                                                        Epi epi) {
  const int lane = threadIdx.x & 63, i = lane & 15, q = lane >> 4;
  const int ct = C >> 4, tiles = ((n + 15) >> 4) * ct;
  for (int tile = (bwd_wave() + kBwdWaves - w0 % kBwdWaves) % kBwdWaves; tile < tiles; tile += kBwdWaves) {
    const int r0 = (tile / ct) * 16, c0 = (tile % ct) * 16;
    const f32x4 v = tile_xw<XT, WT, UNR>(X, ldx, min(r0 + i, n - 1), W, ldw, c0 + i, K, q);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = r0 + 4 * q + rr;
      if (r < n) {
        float* o = out + (int64_t)r * ldo + c0 + i;
        *o = epi(r, c0 + i, (acc ? *o : 0.0f) + s * v[rr]);
      }
    }
  }
}

// prod_mfma inlined with all UNR rounds at once (INL), or the out-of-line call
template <bool XT, bool WT, bool INL, int UNR>
__device__ __forceinline__ void prod_sel(float* out, int ldo, int n, int C, int K, const float* X, int ldx,
                                         const float* W, int ldw, float s, bool acc, int w0) {
  if constexpr (INL)
    prod_mfma_epi<XT, WT, UNR>(out, ldo, n, C, K, X, ldx, W, ldw, s, acc, w0, [](int, int, float v) { return v; });
  else
    prod_mfma<XT, WT>(out, ldo, n, C, K, X, ldx, W, ldw, s, acc, w0);
}

// The same for out = (acc ? out : 0) + s (X1 W1 + X2 W2): two contractions (lengths K1, K2, multiples
// of 16) summed per output tile, then the epilogue
template <bool XT1, bool WT1, bool XT2, bool WT2, int UNR, class Epi>
__device__ __forceinline__ void prod_mfma2_epi(float* out, int ldo, int n, int C, int K1, const float* X1, int ldx1,
                                               const float* W1, int ldw1, int K2, const float* X2, int ldx2,
                                               const float* W2, int ldw2, float s, bool acc, int w0, Epi epi) {
  const int lane = threadIdx.x & 63, i = lane & 15, q = lane >> 4;
  const int ct = C >> 4, tiles = ((n + 15) >> 4) * ct;
  for (int tile = (bwd_wave() + kBwdWaves - w0 % kBwdWaves) % kBwdWaves; tile < tiles; tile += kBwdWaves) {
    const int r0 = (tile / ct) * 16, c0 = (tile % ct) * 16;
    const f32x4 v = tile_xw<XT1, WT1, UNR>(X1, ldx1, min(r0 + i, n - 1), W1, ldw1, c0 + i, K1, q) +
                    tile_xw<XT2, WT2, UNR>(X2, ldx2, min(r0 + i, n - 1), W2, ldw2, c0 + i, K2, q);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = r0 + 4 * q + rr;
      if (r < n) {
        float* o = out + (int64_t)r * ldo + c0 + i;
        *o = epi(r, c0 + i, (acc ? *o : 0.0f) + s * v[rr]);
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
__device__ __forceinline__ void rank_update_pipe_inl(float* S, int ldS, int R, int C, int n, const float* P0, int lp0,
                                                     const float* Q0, int lq0, const float* P1, int lp1,
                                                     const float* Q1, int lq1, const float* P2, int lp2,
                                                     const float* Q2, int lq2, float s, int w0) {
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

// the same as an out-of-line call
template <int NP>
__device__ __attribute__((noinline)) void rank_update_pipe(float* S, int ldS, int R, int C, int n,
                                                           const float* P0, int lp0, const float* Q0, int lq0,
                                                           const float* P1, int lp1, const float* Q1, int lq1,
                                                           const float* P2, int lp2, const float* Q2, int lq2,
                                                           float s, int w0) {
  rank_update_pipe_inl<NP>(S, ldS, R, C, n, P0, lp0, Q0, lq0, P1, lp1, Q1, lq1, P2, lp2, Q2, lq2, s, w0);
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
// (UNR: see tile_xw)
template <int UNR = 2>
__device__ inline void rowdot_tril(float* out, int ldo, int n, int K, const float* X, int ldx, const float* Y,
                                   int ldy, float s, int w0 = 0) {
  if (n > 16 || K % 16 != 0) {
    rowdot_tril_valu(out, ldo, n, K, X, ldx, Y, ldy, s);
    return;
  }
  if (bwd_wave() != w0 % kBwdWaves) return;
  const int lane = threadIdx.x & 63, i = lane & 15, q = lane >> 4;
  const int ci = min(i, n - 1);
  const f32x4 v = tile_xw<false, true, UNR>(X, ldx, ci, Y, ldy, ci, K, q);
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

}  // namespace
}  // namespace ttt
