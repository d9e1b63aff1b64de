// The backward walk over replayed windows with each chain's hidden units split
// over several workgroups of one cooperative launch (the backward of one
// direction of the TTT-MLP layer, "One-Minute Video Generation with Test-Time
// Training", paper-notes page, key designs "TTT-MLP layer"; its chain rule is
// written out at the top of backward.hip).  512-thread workgroups (8 waves, 2
// per SIMD, 256 registers a lane): with the step's operands in LDS the walk
// has little memory latency left to hide, and at 16 waves its products spilled
// registers to scratch around every call.
#include "phase_marks.h"
#include "token_block.h"

#define TTT_BWD_THREADS 512
#include "backward_steps.h"

TTT_MARKS_BUFFER(g_marks_scan_backward);

namespace ttt {
namespace {

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
  // rounds of a product tile's contraction issued at once (all four with four parts; with two, the
  // registers allow two)
  constexpr int kUnr = S == 4 ? 4 : 2;
  constexpr bool kInl = S == 4;  // the products inlined (with two parts they stay out of line)
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
  // the gate factor of this thread's channel: its elements i of the b x d panels all have the
  // column tid mod d (BW is a multiple of d)
  static_assert(BW % kSplitD == 0, "a thread's column is fixed");
  const float tg = tanhf(a.alpha[h * d + tid % d]);

  for (int64_t sg = a.seg_hi; sg >= a.seg_lo; --sg) {
    const int64_t j0 = sg * C, j1 = min(nmb, j0 + C);
    const float* seg = a.segst + ((sh * a.seg_count + (sg - a.seg_lo)) * C) * slot;
    for (int64_t j = j1 - 1; j >= j0; --j) {
      const int64_t mk = (a.seg_hi - sg) * C + (j1 - 1 - j);  // marks: mini-batches of this launch
      (void)mk;
      TTT_MARK(g_marks_scan_backward, mk, 0);
      const int n = (int)min((int64_t)b, T - j * b);
      const float* sl = seg + (j - j0) * slot;
      // this part's output row of mini-batch row r: dQ | dK | dV of [B, T, 3D] (parts 0, 1), or
      // dQ | dK of the [B, T, 2D] buffer (parts 2, 3), at this head's columns
      auto out_row = [=](int r) -> float* {
        const int64_t tr = (int64_t)s * T + rw.tok(j * b + r);
        return half < 2 ? a.dqkv + tr * 3 * D + h * d : a.dqkv_b + tr * 2 * D + h * d;
      };
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
        const int r = i / d;
        t.dZ[i] = tg * a.dy[((int64_t)s * T + rw.tok(j * b + r)) * D + h * d + (i - r * d)];
      }
      if constexpr (S == 4) vmem_done();  // this wave's direct loads have landed
      __syncthreads();
      TTT_MARK(g_marks_scan_backward, mk, 1);
      // ---- N (this part) = tril(Hq Hk^T); dN = tril(-eta dZ G2^T); dZ W2^T (into dGh for now)
      rowdot_tril<kUnr>(t.N, b, n, mh, Hq_, pld, Hk_, pld, 1.0f);
      rowdot_tril<kUnr>(t.dN, b, n, d, t.dZ, d, t.G2, d, -eta, 1);
      prod_sel<false, true, kInl, kUnr>(dGh, mh, n, mh, d, t.dZ, d, W.w2, W.ld2, 1.0f, false, 2);
      __syncthreads();
      TTT_MARK(g_marks_scan_backward, mk, 2);
      // ---- dAq = (dZ W2^T + dN Hk) * GELU'(Aq); dHk = dN^T Hq; dG2 (this part) = -eta N^T dZ
      if (n % 16 == 0 && mh % 16 == 0 && d % 16 == 0) {  // on the matrix cores (N, dN are 0 above the diagonal)
        // dHq = dGh + dN Hk, and from each finished element dAq = GELU'(Aq) * dHq
        prod_mfma_epi<false, false, kUnr>(dGh, mh, n, mh, n, t.dN, b, Hk_, pld, 1.0f, true, 0,
                                    [=](int r, int c, float v) {
                                      dAq[r * mh + c] = S1q_[r * pld + c] * v;
                                      return v;
                                    });
        prod_sel<true, false, kInl, kUnr>(dHk, mh, n, mh, n, t.dN, b, Hq_, pld, 1.0f, false, 0);
        prod_sel<true, false, kInl, kUnr>(t.dG2, d, n, d, n, t.N, b, t.dZ, d, -eta, false, 0);
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
      prod_sel<false, true, kInl, kUnr>(dQp, d, n, d, mh, dAq, mh, W.w1, W.ld1, 1.0f, false, 0);
      rowdot_tril<kUnr>(t.dM, b, n, mh, dAq, mh, G1_, pld, -eta, 4);
      prod_sel<false, true, kInl, kUnr>(dHk, mh, n, mh, d, t.G2, d, dW2, la2, -eta, true, 5);
      prod_sel<false, false, kInl, kUnr>(t.dG2, d, n, d, mh, Hk_, pld, dW2, la2, -eta, true, 5);
      const bool tiled = n % 16 == 0;  // the products below on the matrix cores
      if (tiled) {  // dG1 = -eta (K dW1' + M^T dAq) (M is 0 above its diagonal), and from each finished
                    // element dGh = dG1 * S1, dA (in dG1) = dG1 * Gh * GELU''(A)
        prod_mfma2_epi<false, false, true, false, kUnr>(dG1, mh, n, mh, d, t.K, d, dW1, la1, n, t.M, b, dAq, mh, -eta, false, 1,
                                                  [=](int r, int c, float v) {
                                                    float g, dg, ddg;
                                                    gelu3(A_[r * pld + c], false, &g, &dg, &ddg);
                                                    dGh[r * mh + c] = v * S1_[r * pld + c];
                                                    return v * Gh_[r * pld + c] * ddg;
                                                  });
      } else {
        prod_sel<false, false, kInl, kUnr>(dG1, mh, n, mh, d, t.K, d, dW1, la1, -eta, false, 9);
      }
      prod_sel<false, true, kInl, kUnr>(dKp, d, n, d, mh, G1_, pld, dW1, la1, -eta, false, 9);
      __syncthreads();
      TTT_MARK(g_marks_scan_backward, mk, 4);
      // ---- dQ += dM K; dK += dM^T Q (this part's dM); dG2 (this part) += dGh W2 (the ragged last
      //      mini-batch: first dG1 -= eta M^T dAq, dGh and dA, on the vector ALU)
      if (tiled) {
        // dQ of this part is complete: each finished element goes straight to its output
        prod_mfma_epi<false, false, kUnr>(dQp, d, n, d, n, t.dM, b, t.K, d, 1.0f, true, 4, [=](int r, int c, float v) {
          atomicAdd(out_row(r) + c, v);
          return v;
        });
        prod_sel<true, false, kInl, kUnr>(dKp, d, n, d, n, t.dM, b, t.Q, d, 1.0f, true, 0);
      } else {
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
        for (int i = tid; i < n * mh; i += BW) {
          const int r = i / mh, c = i - r * mh;
          float g, dg, ddg;
          gelu3(A_[r * pld + c], false, &g, &dg, &ddg);
          const float x = dG1[i];
          dGh[i] = x * S1_[r * pld + c];
          dG1[i] = x * Gh_[r * pld + c] * ddg;
        }
        __syncthreads();
      }
      prod_sel<false, false, kInl, kUnr>(t.dG2, d, n, d, mh, dGh, mh, W.w2, W.ld2, 1.0f, true, 0);  // dG2 (this part) += dGh W2
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
        // this thread's (up to) two elements i0 = tid, i1 = tid + BW; each round issues the loads of
        // every partial still missing before looking at any, so a round costs one trip
        static_assert(kSplitB * kSplitD <= 2 * BW, "two dG2 elements per thread");
        const int i0 = tid, i1 = tid + BW;
        const bool h0 = i0 < n * d, h1 = i1 < n * d;
        float v0[S], v1[S];
        uint32_t miss = 0;  // bit 2q: element 0 of part q missing, bit 2q + 1: element 1
#pragma unroll
        for (int q = 0; q < S; ++q) {
          v0[q] = v1[q] = __uint_as_float(0x7fc00000u);  // NaN unless the partial arrives
          if (q == half) {
            if (h0) v0[q] = t.dG2[i0];
            if (h1) v1[q] = t.dG2[i1];
          } else {
            miss |= (h0 ? 1u : 0u) << (2 * q);
            miss |= (h1 ? 1u : 0u) << (2 * q + 1);
          }
        }
        for (uint32_t spin = 0; miss && !failed; ++spin) {
          uint64_t e0[S], e1[S];
#pragma unroll
          for (int q = 0; q < S; ++q) {
            const uint64_t* theirs = xc + (q * 2 + par) * (int64_t)(b * d);
            if (miss >> (2 * q) & 1u) e0[q] = __hip_atomic_load(theirs + i0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (miss >> (2 * q + 1) & 1u)
              e1[q] = __hip_atomic_load(theirs + i1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
#pragma unroll
          for (int q = 0; q < S; ++q) {
            if ((miss >> (2 * q) & 1u) && (uint32_t)(e0[q] >> 32) == tag) {
              v0[q] = __uint_as_float((uint32_t)e0[q]);
              miss &= ~(1u << (2 * q));
            }
            if ((miss >> (2 * q + 1) & 1u) && (uint32_t)(e1[q] >> 32) == tag) {
              v1[q] = __uint_as_float((uint32_t)e1[q]);
              miss &= ~(1u << (2 * q + 1));
            }
          }
          if (!miss) break;
          if (spin >= kSplitSpinMax) {
            __hip_atomic_store(a.abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            failed = true;
          } else if ((spin & 15) == 15 && __hip_atomic_load(a.abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
            failed = true;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        float s0 = v0[0], s1 = v1[0];  // the parts' partials added in the parts' order
#pragma unroll
        for (int q = 1; q < S; ++q) {
          s0 += v0[q];
          s1 += v1[q];
        }
        if (h0) t.dG2[i0] = a.gscale * s0;
        if (h1) t.dG2[i1] = a.gscale * s1;
      }
      __syncthreads();
      TTT_MARK(g_marks_scan_backward, mk, 6);
      // dHk += dYh W2^T, and from each finished element dA += dHk * S1
      prod_mfma_epi<false, true, kUnr>(dHk, mh, n, mh, d, t.dG2, d, W.w2, W.ld2, 1.0f, true, 0, [=](int r, int c, float v) {
        dG1[r * mh + c] += v * S1_[r * pld + c];
        return v;
      });
      __syncthreads();
      if (tiled) {  // dK (this part) += dA W1^T, each finished element straight to its output
        prod_mfma_epi<false, true, kUnr>(dKp, d, n, d, mh, dG1, mh, W.w1, W.ld1, 1.0f, true, 0, [=](int r, int c, float v) {
          atomicAdd(out_row(r) + D + c, v);
          return v;
        });
      } else {
        prod_sel<false, true, kInl, kUnr>(dKp, d, n, d, mh, dG1, mh, W.w1, W.ld1, 1.0f, true, 0);
        __syncthreads();
      }
      TTT_MARK(g_marks_scan_backward, mk, 7);
      // ---- dQ and dK (the ragged last mini-batch; the others' went out above): this part's sums
      //      added into [B, T, 3D] (parts 0, 1) or the [B, T, 2D] buffer (parts 2, 3), both zeroed
      //      before the walk; dV = -dYh (part 0); the adjoint's part handed to the mini-batch
      //      before: dW1 += Q^T dAq + K^T dA; dW2 += Hq^T dZ + dGh^T G2 + Hk^T dYh
      for (int i = tid; i < n * d; i += BW) {
        const int r = i / d, c = i - r * d;
        float* row = out_row(r) + c;
        if (!tiled) {
          atomicAdd(row, dQp[i]);
          atomicAdd(row + D, dKp[i]);
        }
        if (half == 0) row[2 * D] = -t.dG2[i];
      }
      if constexpr (kInl) {  // inlined, like the products
        rank_update_pipe_inl<2>(dW1, la1, d, mh, n, t.Q, d, dAq, mh, t.K, d, dG1, mh, nullptr, 0, nullptr, 0, 1.0f, 0);
        rank_update_pipe_inl<3>(dW2, la2, mh, d, n, Hq_, pld, t.dZ, d, dGh, mh, t.G2, d, Hk_, pld, t.dG2, d, 1.0f, 0);
      } else {
        Terms u1{2, {t.Q, t.K}, {d, d}, {dAq, dG1}, {mh, mh}};
        rank_update_any(dW1, la1, d, mh, n, u1, 1.0f);
        Terms u2{3, {Hq_, dGh, Hk_}, {pld, mh, pld}, {t.dZ, t.G2, t.dG2}, {d, d, d}};
        rank_update_any(dW2, la2, mh, d, n, u2, 1.0f);
      }
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

}  // namespace

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

}  // namespace ttt

TTT_MARKS_EXPORT(ttt_phase_marks_scan_backward, g_marks_scan_backward);
