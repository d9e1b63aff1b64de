// TTT-MLP scan on the bf16 matrix cores, head width d = 64, hidden m = 256,
// mini-batch b = 16 ("One-Minute Video Generation with Test-Time Training",
// paper-notes page, key designs: "TTT-MLP layer" for the inner model, its
// loss, the per-token gradient step and the read-out with the updated state;
// "gate + bidirectional" for the gate).  It computes the mini-batch dual form
// (see generic.hip) with fp32 state and fp32 accumulation; matrix operands
// are rounded to bf16.
//
// One 256-thread workgroup per (sequence, head); wave w owns hidden units
// [64w, 64w+64): its slices of W1 (64 x 64) and W2 (64 x 64) live in
// registers in the MFMA D layout for the whole sequence, so the state never
// leaves the CU.  Activations are kept "feature-major" (tokens along the 16
// lanes of a tile):
//   A^T = W1^T K^T, Hk^T = GELU(A^T)                     (local to the wave)
//   Yhat^T = W2^T Hk^T                  partial over hidden units -> LDS reduce
//   G2 = c (Yhat - V)                   each wave finishes one 16-wide d slice
//   Gh^T = W2 G2^T, G1^T = Gh^T * GELU'(A^T)
//   Aq^T = W1^T Q^T - eta G1^T tril(Q K^T)^T, Hq^T = GELU(Aq^T)
//   Z^T  = W2^T Hq^T - eta G2^T tril(Hq Hk^T)^T        partial -> LDS reduce
//   W1 -= eta K^T G1,  W2 -= eta Hk^T G2                 (K=16 MFMAs)
// A tile in the D layout is a K=16 operand of its own transpose, so an MFMA
// against the identity turns it into the D layout of the transpose: that
// gives the W2 operand of Gh (contracted over d, not m) and the token-major
// copies of Hk and G1 that the K=16 products over tokens need.
// The Z reduction, the gate y = x + tanh(alpha) z and the stores of a
// mini-batch happen during the next mini-batch, off the recurrence's path.
// Two workgroup barriers per mini-batch.
#include "internal.h"
#include "mfma_common.h"

namespace ttt {
namespace {

constexpr int SD = 64;   // head width
constexpr int SM = 256;  // hidden width
constexpr int SB = 16;   // mini-batch
constexpr int NWAVE = 4;
// Token block layout (bf16 elements), rows padded so that the 16 rows read by
// one 16-lane group fall on distinct LDS banks:
//   Q  [16 tokens][RS]  features in the pair order
//   K  [16 tokens][RS]  features in the pair order
//   KT [64 features][TS] tokens in order
//   V  [16 tokens][RS]  features in order
constexpr int RS = SD + 8;  // 72
constexpr int TS = SB + 4;  // 20
constexpr int OFF_Q = 0, OFF_K = SB * RS, OFF_KT = 2 * SB * RS, OFF_V = 2 * SB * RS + SD * TS;
constexpr int BLK = 3 * SB * RS + SD * TS;  // 4736 elements, 9472 bytes
constexpr int BLK_CHUNKS = BLK * 2 / 16;    // 592 chunks of 16 bytes
static_assert((BLK * 2) % 16 == 0, "block must be a whole number of 16-byte chunks");

// GELU and its derivative from one exponential.  erf by Abramowitz & Stegun
// 7.1.26 (Hastings' rational approximation, |error| <= 1.5e-7):
//   erf(x) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2),  t = 1 / (1 + p x),  x >= 0.
struct Gelu {
  static __device__ __forceinline__ float phi_tail(float ax_over_sqrt2, float* e) {
    const float x = ax_over_sqrt2;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
    float p = fmaf(1.061405429f, t, -1.453152027f);
    p = fmaf(p, t, 1.421413741f);
    p = fmaf(p, t, -0.284496736f);
    p = fmaf(p, t, 0.254829592f);
    p *= t;
    *e = __builtin_amdgcn_exp2f(-1.4426950408889634f * x * x);  // exp(-x^2) = exp(-a^2/2)
    return 0.5f * p * (*e);  // 1 - Phi(|a|) = erfc(|a|/sqrt2) / 2
  }
  // GELU(a) and GELU'(a) = Phi(a) + a phi(a)
  static __device__ __forceinline__ void both(float a, float* g, float* dg) {
    float e;
    const float tail = phi_tail(fabsf(a) * 0.7071067811865476f, &e);
    const float cdf = a >= 0.0f ? 1.0f - tail : tail;
    *g = a * cdf;
    *dg = fmaf(a * 0.3989422804014327f, e, cdf);
  }
  static __device__ __forceinline__ float value(float a) {
    float e;
    const float tail = phi_tail(fabsf(a) * 0.7071067811865476f, &e);
    return a * (a >= 0.0f ? 1.0f - tail : tail);
  }
};

// tanh form: 0.5 a (1 + tanh(u)), u = sqrt(2/pi) (a + 0.044715 a^3), with
// tanh(u) = 1 - 2 / (exp(2u) + 1) (exact identity; saturates to +-1 for large |u|).
struct GeluTanh {
  static __device__ __forceinline__ float tanh_u(float u) {
    const float e = __builtin_amdgcn_exp2f(2.8853900817779268f * u);  // exp(2u)
    return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
  }
  static __device__ __forceinline__ void both(float a, float* g, float* dg) {
    const float u = 0.7978845608028654f * fmaf(0.044715f * a, a * a, a);
    const float th = tanh_u(u);
    const float du = 0.7978845608028654f * fmaf(3.0f * 0.044715f * a, a, 1.0f);
    *g = 0.5f * a * (1.0f + th);
    *dg = fmaf(0.5f * a * du, fmaf(-th, th, 1.0f), 0.5f * (1.0f + th));
  }
  static __device__ __forceinline__ float value(float a) {
    const float u = 0.7978845608028654f * fmaf(0.044715f * a, a * a, a);
    return 0.5f * a * (1.0f + tanh_u(u));
  }
};

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) { return *(const bf16x8*)p; }
__device__ __forceinline__ bf16x4 ld4(const uint16_t* p) { return *(const bf16x4*)p; }

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (__bf16)0.0f;
  return v;
}

// Readers of the staged token block (LDS), masking tokens >= n of a short block.
__device__ __forceinline__ bf16x8 rd_row8(const uint16_t* blk, int off, int n, int g, int c, int cc) {
  return c < n ? *(const bf16x8*)(blk + off + c * RS + 32 * cc + 8 * g) : zero8();
}

__device__ __forceinline__ bf16x4 rd_kt(const uint16_t* blk, int n, int g, int c, int dt) {
  bf16x4 k = *(const bf16x4*)(blk + OFF_KT + (16 * dt + c) * TS + 4 * g);
  if (n < SB) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * g + i >= n) k[i] = (__bf16)0.0f;
  }
  return k;
}

__device__ __forceinline__ bf16x4 rd_v(const uint16_t* blk, int n, int w, int g, int c) {
  bf16x4 v = *(const bf16x4*)(blk + OFF_V + c * RS + 16 * w + 4 * g);
  if (c >= n) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (__bf16)0.0f;
  }
  return v;
}

template <class G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void scan_mfma_kernel(ScanArgs a) {
  __shared__ f32x4 Ypart[NWAVE][4][64];                      // partial Yhat^T per wave, d-tile, lane
  __shared__ f32x4 Zpart[NWAVE][4][64];                      // partial Z^T
  __shared__ __attribute__((aligned(16))) uint16_t G2a[SB * RS];         // G2 [token][feature, pair order]
  __shared__ __attribute__((aligned(16))) uint16_t G2b[SD * TS];         // -eta G2 [feature][token]
  __shared__ __attribute__((aligned(16))) uint16_t Stage[2][BLK];        // token blocks j (and j+1)

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int s = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int64_t T = a.T;
  const int D = a.H * SD;
  const int m0 = 64 * w;
  const float eta = a.eta, neta = -a.eta, gs = a.gscale;

  // ---- state, D layout: W1 rows d / cols m, W2 rows m / cols d
  f32x4 W1[4][4], W2[4][4];
  {
    const float* w1 = a.w1_0 + (int64_t)h * SD * SM;
    const float* w2 = a.w2_0 + (int64_t)h * SM * SD;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          W1[i][j][r] = w1[(16 * i + 4 * g + r) * SM + m0 + 16 * j + c];
          W2[i][j][r] = w2[(m0 + 16 * i + 4 * g + r) * SD + 16 * j + c];
        }
  }
  // the 16 x 16 identity as a K=16 B operand: lane holds rows 4g..4g+3 of column c
  bf16x4 ident;
#pragma unroll
  for (int r = 0; r < 4; ++r) ident[r] = (__bf16)(4 * g + r == c ? 1.0f : 0.0f);

  // gate factors of the 4 channels this lane finishes: 16w + 4g + r
  const int ch0 = h * SD + 16 * w + 4 * g;
  float tg[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) tg[r] = GeluTanh::tanh_u(a.alpha[ch0 + r]);

  const int64_t nblk = (T + SB - 1) / SB;
  const uint16_t* blocks = (const uint16_t*)a.qkv_tiles + ((int64_t)s * a.H + h) * nblk * BLK;
  const uint16_t* xin = (const uint16_t*)a.xin;
  uint16_t* yout = (uint16_t*)a.y;

  auto tok_index = [&](int64_t pos) -> int64_t { return a.reverse ? T - 1 - pos : pos; };
  auto block_n = [&](int64_t j) -> int { return (int)((T - SB * j) < SB ? (T - SB * j) : SB); };

  // reduce the Z partials of block jz, gate and store (each wave: d-tile w)
  auto finish_z = [&](int64_t jz, bf16x4 xv) {
    f32x4 z = Zpart[0][w][lane] + Zpart[1][w][lane] + Zpart[2][w][lane] + Zpart[3][w][lane];
    const int64_t pos = SB * jz + c;
    if (pos < T) {
      const int64_t o = ((int64_t)s * T + tok_index(pos)) * D + ch0;
      bf16x4 yv;
#pragma unroll
      for (int r = 0; r < 4; ++r) yv[r] = (__bf16)fmaf(tg[r], z[r], (float)xv[r]);
      *(bf16x4*)(yout + o) = yv;
      if (a.z) *(f32x4*)(a.z + o) = z;
    }
  };
  auto load_x = [&](int64_t jx) -> bf16x4 {
    const int64_t pos = SB * jx + c;
    if (pos >= T) return bf16x4{(__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f};
    return ld4(xin + ((int64_t)s * T + tok_index(pos)) * D + ch0);
  };

  // block staging: global -> registers at the start of a mini-batch, -> LDS mid-way
  uint4 pf[3];
  auto fetch = [&](int64_t jb) {
    const uint4* src = (const uint4*)(blocks + jb * BLK);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int q = tid + 256 * i;
      if (q < BLK_CHUNKS) pf[i] = src[q];
    }
  };
  auto stage = [&](int buf) {
    uint4* dst = (uint4*)Stage[buf];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int q = tid + 256 * i;
      if (q < BLK_CHUNKS) dst[q] = pf[i];
    }
  };
  if (nblk > 0) {
    fetch(0);
    stage(0);
  }
  __syncthreads();
  bf16x4 x_prev = bf16x4{(__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f, (__bf16)0.0f};

  for (int64_t j = 0; j < nblk; ++j) {
    const int n = block_n(j);
    const uint16_t* blk = Stage[j & 1];
    // prefetch the next block and this block's gate input
    if (j + 1 < nblk) fetch(j + 1);
    const bf16x4 x_cur = load_x(j);

    // ---- 1. A^T = W1^T K^T (per hidden tile), S^T = K Q^T
    f32x4 At[4];
    f32x4 St;
    {
      const bf16x8 k0 = rd_row8(blk, OFF_K, n, g, c, 0), k1 = rd_row8(blk, OFF_K, n, g, c, 1);
      const bf16x8 q0 = rd_row8(blk, OFF_Q, n, g, c, 0), q1 = rd_row8(blk, OFF_Q, n, g, c, 1);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        At[nt] = mfma32(pack8(W1[0][nt], W1[1][nt]), k0, zero4());
        At[nt] = mfma32(pack8(W1[2][nt], W1[3][nt]), k1, At[nt]);
      }
      St = mfma32(k0, q0, zero4());
      St = mfma32(k1, q1, St);
    }

    // ---- 2. Hk^T = GELU(A^T), GELU'(A^T)
    f32x4 Hk[4], Dg[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float hv, dv;
        G::both(At[nt][r], &hv, &dv);
        Hk[nt][r] = hv;
        Dg[nt][r] = dv;
      }
    bf16x8 hkB[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) hkB[cc] = pack8(Hk[2 * cc], Hk[2 * cc + 1]);

    // ---- 3. partial Yhat^T = W2^T Hk^T over this wave's hidden units
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      f32x4 yp = mfma32(pack8(W2[0][dt], W2[1][dt]), hkB[0], zero4());
      yp = mfma32(pack8(W2[2][dt], W2[3][dt]), hkB[1], yp);
      Ypart[w][dt][lane] = yp;
    }
    __syncthreads();

    // ---- 4. finish d-tile w: G2 = c (Yhat - V); publish G2 and -eta G2
    {
      const f32x4 y = Ypart[0][w][lane] + Ypart[1][w][lane] + Ypart[2][w][lane] + Ypart[3][w][lane];
      f32x4 g2;
      const bf16x4 vv = rd_v(blk, n, w, g, c);
#pragma unroll
      for (int r = 0; r < 4; ++r) g2[r] = gs * (y[r] - (float)vv[r]);
      // G2[token c][feature 16w + 4g + r] in the pair order
      *(bf16x4*)(&G2a[c * RS + 32 * (w >> 1) + 8 * g + 4 * (w & 1)]) = pack4(g2);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const __bf16 b = (__bf16)(neta * g2[r]);
        G2b[(16 * w + 4 * g + r) * TS + c] = __builtin_bit_cast(uint16_t, b);
      }
      if (j > 0) finish_z(j - 1, x_prev);
      if (j + 1 < nblk) stage((j + 1) & 1);
    }
    __syncthreads();

    // ---- 5. Gh^T = W2 G2^T (W2 slice from the transposed copy)
    bf16x8 g2B[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) g2B[cc] = *(const bf16x8*)(&G2a[c * RS + 32 * cc + 8 * g]);
    bf16x4 g2T[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) g2T[dt] = *(const bf16x4*)(&G2b[(16 * dt + c) * TS + 4 * g]);
    f32x4 G1[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      // W2 slice rows m (tile mt), contraction over d: transposes of the W2 tiles
      f32x4 t0 = mfma16(pack4(W2[mt][0]), ident, zero4());
      f32x4 t1 = mfma16(pack4(W2[mt][1]), ident, zero4());
      f32x4 t2 = mfma16(pack4(W2[mt][2]), ident, zero4());
      f32x4 t3 = mfma16(pack4(W2[mt][3]), ident, zero4());
      f32x4 gh = mfma32(pack8(t0, t1), g2B[0], zero4());
      gh = mfma32(pack8(t2, t3), g2B[1], gh);
      // ---- 6. G1^T = Gh^T * GELU'(A^T)
      G1[mt] = gh * Dg[mt];
    }
    // token-major copies of Hk and -eta G1 (tokens 4g..4g+3 of hidden unit 16mt + c)
    bf16x4 hkT[4], g1T[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      hkT[mt] = pack4(mfma16(pack4(Hk[mt]), ident, zero4()));
      g1T[mt] = pack4(mfma16(pack4(neta * G1[mt]), ident, zero4()));
    }

    // ---- 7. Aq^T = W1^T Q^T + (-eta G1)^T tril(S)^T
    bf16x4 sT;
#pragma unroll
    for (int r = 0; r < 4; ++r) sT[r] = (__bf16)(4 * g + r <= c ? St[r] : 0.0f);
    f32x4 Hq[4];
    const bf16x8 q0 = rd_row8(blk, OFF_Q, n, g, c, 0), q1 = rd_row8(blk, OFF_Q, n, g, c, 1);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      f32x4 aq = mfma32(pack8(W1[0][nt], W1[1][nt]), q0, zero4());
      aq = mfma32(pack8(W1[2][nt], W1[3][nt]), q1, aq);
      aq = mfma16(g1T[nt], sT, aq);
      // ---- 8. Hq^T = GELU(Aq^T)
#pragma unroll
      for (int r = 0; r < 4; ++r) Hq[nt][r] = G::value(aq[r]);
    }
    bf16x8 hqB[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) hqB[cc] = pack8(Hq[2 * cc], Hq[2 * cc + 1]);

    // ---- 9. partial Z^T = W2^T Hq^T + (-eta G2)^T tril(Hq Hk^T)^T
    f32x4 Pt = mfma32(hkB[0], hqB[0], zero4());
    Pt = mfma32(hkB[1], hqB[1], Pt);
    bf16x4 pT;
#pragma unroll
    for (int r = 0; r < 4; ++r) pT[r] = (__bf16)(4 * g + r <= c ? Pt[r] : 0.0f);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      f32x4 zp = mfma32(pack8(W2[0][dt], W2[1][dt]), hqB[0], zero4());
      zp = mfma32(pack8(W2[2][dt], W2[3][dt]), hqB[1], zp);
      zp = mfma16(g2T[dt], pT, zp);
      Zpart[w][dt][lane] = zp;
    }

    // ---- 10. state update: W1 += K^T (-eta G1), W2 += Hk^T (-eta G2)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const bf16x4 kt = rd_kt(blk, n, g, c, dt);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) W1[dt][nt] = mfma16(kt, g1T[nt], W1[dt][nt]);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) W2[mt][dt] = mfma16(hkT[mt], g2T[dt], W2[mt][dt]);

    x_prev = x_cur;
  }
  if (nblk > 0) {
    __syncthreads();
    finish_z(nblk - 1, x_prev);
  }
  (void)eta;

  // ---- final state
  if (a.w1_T) {
    float* o = a.w1_T + ((int64_t)s * a.H + h) * SD * SM;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[(16 * i + 4 * g + r) * SM + m0 + 16 * jj + c] = W1[i][jj][r];
  }
  if (a.w2_T) {
    float* o = a.w2_T + ((int64_t)s * a.H + h) * SM * SD;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[(m0 + 16 * i + 4 * g + r) * SD + 16 * jj + c] = W2[i][jj][r];
  }
}

}  // namespace

bool scan_mfma_supported(int d, int m, int b) { return d == SD && m == SM && b == SB; }

int scan_mfma_block_elems() { return BLK; }

size_t scan_mfma_tile_bytes(int64_t B, int64_t T, int H) {
  const int64_t nblk = (T + SB - 1) / SB;
  return (size_t)(B * H * nblk) * BLK * sizeof(uint16_t);
}

hipError_t launch_scan_mfma(const ScanArgs& a, hipStream_t s) {
  if (a.gelu_tanh)
    hipLaunchKernelGGL(scan_mfma_kernel<GeluTanh>, dim3((unsigned)(a.B * a.H)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(scan_mfma_kernel<Gelu>, dim3((unsigned)(a.B * a.H)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ttt
