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
#include "phase_marks.h"

#define TTT_BWD_THREADS 1024  // 16 waves a workgroup (4 per SIMD), 128 registers a lane
#include "backward_steps.h"

TTT_MARKS_BUFFER(g_marks_scan_backward1);

namespace ttt {
namespace {

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
      TTT_MARK(g_marks_scan_backward1, mk, 0);
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
      TTT_MARK(g_marks_scan_backward1, mk, 1);
      if (!kept) forward_core(t, W, n, d, m, a.gscale, a.gelu_tanh);
      if (!REPLAYED) readout_hidden(t, W, n, b, d, m, eta, a.gelu_tanh, t.dAq);  // dAq holds GELU'(Aq) for now
      TTT_MARK(g_marks_scan_backward1, mk, 2);
      // N = tril(Hq Hk^T); dN = tril(-eta dZ G2^T); dZ W2^T (into dGh for now)
      rowdot_tril(t.N, b, n, m, t.Hq, m, t.Hk, m, 1.0f);
      rowdot_tril(t.dN, b, n, d, t.dZ, d, t.G2, d, -eta, 1);
      prod<4, true>(t.dGh, m, n, m, d, t.dZ, d, W.w2, W.ld2, 1.0f, false, 2);
      __syncthreads();
      TTT_MARK(g_marks_scan_backward1, mk, 3);
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
      TTT_MARK(g_marks_scan_backward1, mk, 4);
      prod<1, true>(t.dQ, d, n, d, m, t.dAq, m, W.w1, W.ld1, 1.0f, false);
      rowdot_tril(t.dM, b, n, m, t.dAq, m, t.G1, m, -eta, 4);
      prod<4, true>(t.dHk, m, n, m, d, t.G2, d, dW2, d, -eta, true, 5);
      prod<1, false>(t.dG2, d, n, d, m, t.Hk, m, dW2, d, -eta, true, 5);
      prod<4, false>(t.dG1, m, n, m, d, t.K, d, dW1, m, -eta, false, 9);
      prod<1, true>(t.dK, d, n, d, m, t.G1, m, dW1, m, -eta, false, 9);
      __syncthreads();
      TTT_MARK(g_marks_scan_backward1, mk, 5);
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
      TTT_MARK(g_marks_scan_backward1, mk, 6);
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
      TTT_MARK(g_marks_scan_backward1, mk, 7);
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

TTT_MARKS_EXPORT(ttt_phase_marks_scan_backward1, g_marks_scan_backward1);
