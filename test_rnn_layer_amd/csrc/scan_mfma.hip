// TTT-MLP scan on the bf16 matrix cores, head width d = 64, hidden m = 256,
// mini-batch b = 16 ("One-Minute Video Generation with Test-Time Training",
// paper-notes page, key designs: "TTT-MLP layer" for the inner model, its
// loss, the per-token gradient step and the read-out with the updated state;
// "gate + bidirectional" for the gate).  It computes the mini-batch dual form
// (see generic.hip) with fp32 state and fp32 accumulation; matrix operands
// are rounded to bf16.
//
// One 512-thread workgroup per (sequence, head); wave w owns hidden units
// [32w, 32w+32): its slices of W1 (64 x 32) and W2 (32 x 64) live in
// registers in the MFMA D layout for the whole sequence, so the state never
// leaves the CU.  Activations are kept "feature-major" (tokens along the 16
// lanes of a tile).  Step j runs block j's recurrence
//   A^T = W1^T K^T, Hk^T = GELU(A^T)                     (local to the wave)
//   Yhat^T = W2^T Hk^T                  partial over hidden units -> LDS reduce
//   G2 = c (Yhat - V)                   each thread finishes two values
//   Gh^T = W2 G2^T, G1^T = Gh^T * GELU'(A^T)
//   W1 -= eta K^T G1,  W2 -= eta Hk^T G2                 (K=16 MFMAs)
// and, after the second barrier beside the update's products, block j-1's
// read-out with the state that follows block j-1 (exact):
//   Aq^T = W1'^T Q^T + eta G1^T striu(Q K^T)^T, Hq^T = GELU(Aq^T)
//   Z^T  = W2'^T Hq^T + eta G2^T striu(Hq Hk^T)^T       partial -> LDS reduce
// with the gate y = x + tanh(alpha) z and the stores one step later.  The
// transposed operands (W2 for Gh, contracted over d; token-major G1, Hk and
// K for the updates) come from LDS transpose reads.  Two workgroup barriers
// per block.
#include "internal.h"
#include "mfma_common.h"
#include "phase_marks.h"
#include "phi_poly.h"
#include "token_block.h"

TTT_MARKS_BUFFER(g_marks_scan_mfma);

namespace ttt {
namespace {

using namespace tb;  // SD = 64 head width, SB = 16 mini-batch, the token-block layout and readers
constexpr int SM = 256;  // hidden width
constexpr int NWAVE = 8;          // wave w owns hidden units [32w, 32w + 32)
constexpr int NTHR = 64 * NWAVE;
constexpr int NSTAGE = 8;         // token-block buffers in LDS (indexed by block mod 8)
constexpr int AHEAD = 3;          // blocks j+1 .. j+3 in flight during step j
constexpr int TS = SB + 8;  // 24: rows of the [feature][token] G2 copy (48 bytes: the 8-byte reads of
                            // two lane groups fall on distinct banks)
// Hk slice rows: source lane l at row l + 8 (l / 32), so that the 32 rows a transposed
// read takes in one lane group pair map to distinct banks
constexpr int HKS_ROWS = 72;
__device__ __forceinline__ int hk_row(int l) { return l + 8 * (l >> 5); }
// issue pattern after the second barrier: the step's 43 matrix-core products there (28 of
// the update, 15 of the read-out) in MIX_GROUPS groups of MIX_PRODUCTS, each followed by
// MIX_VALU vector instructions.  Measured per bidir307k call on one box: 87.6-88.2 ms with
// 11 groups of (4, 12), against 88.8 with (4, 14), 91.5 with (4, 10), 89.0-89.8 with 22
// groups of (2, 6), 90.1 with (2, 7), 91.0 with (2, 5), 89.1 with 15 groups of (3, 9),
// 91.1 with 8 of (6, 18) and 92.1 with 6 of (8, 24); on another box 43 groups of (1, 3)
// took 90.7 ms against 93.1 with (1, 2), 92.0 with (1, 4), and 92.9 with no fixed pattern.
constexpr int MIX_GROUPS = 11, MIX_PRODUCTS = 4, MIX_VALU = 12;
constexpr int DGS = SB + 4;  // 20: rows of the fp32 [hidden][token] GELU' tiles (bank spread of the column writes)

// GELU(a) = a Phi(a) and GELU'(a) = Phi(a) + a phi(a), with Phi from the
// polynomial of phi_poly.h (|error| <= 1.8e-4, no reciprocal or exponential: the
// values are rounded to bf16 matrix operands, or multiplied into them, so this
// is about 1/11 of the operands' own rounding) and the density
// phi(a) = exp(-a^2/2) / sqrt(2 pi) = 2^(-a^2 log2(e) / 2 + log2(1 / sqrt(2 pi))),
// one exponential with the constant folded into its argument.
struct Gelu {
  static __device__ __forceinline__ float cdf(float a) {
    const float c = __builtin_amdgcn_fmed3f(a, -kPhiL, kPhiL);
    const float sq = c * c;
    float q = kPhiP[kPhiDeg];
#pragma unroll
    for (int k = kPhiDeg - 1; k >= 0; --k) q = fmaf(q, sq, kPhiP[k]);
    return fmaf(c, q, 0.5f);
  }
  // GELU'(a) from a and p = Phi(a)
  static __device__ __forceinline__ float deriv(float a, float p) {
    const float dens = __builtin_amdgcn_exp2f(fmaf(-0.7213475204444817f * a, a, -1.3257480647361593f));  // phi(a)
    return fmaf(a, dens, p);
  }
  static __device__ __forceinline__ float value(float a) { return a * cdf(a); }
};

__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(2, 2))) void scan_mfma_kernel(ScanArgs a) {
  __shared__ f32x4 Ypart[NWAVE][4][64];                            // partial Yhat^T: wave, d-tile, lane
  __shared__ f32x4 Zpart[NWAVE][4][64];                            // partial Z^T
  __shared__ __attribute__((aligned(16))) uint16_t G2a[SB * RS];    // -eta G2 [token][feature, pair order]
  __shared__ __attribute__((aligned(16))) uint16_t G2b[SD * TS];    // -eta G2 [feature][token]
  __shared__ __attribute__((aligned(16))) uint16_t Stage[NSTAGE][BLK];  // token blocks j-1 .. j+3
  // per-wave slices for the transposed reads: bf16 Hk^T (one 8-byte row per source lane
  // and hidden-unit tile, see hk_row), fp32 GELU'(A^T) as [m][t]
  __shared__ __attribute__((aligned(16))) bf16x4 HkS[NWAVE][2][HKS_ROWS];
  __shared__ __attribute__((aligned(16))) float DgS[NWAVE][2][16 * DGS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int s = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int64_t T = a.T;             // whole sequence (token indexing, block layout)
  const int64_t p0 = a.p0, Tc = a.Tc;  // this launch: scan positions p0 .. p0 + Tc - 1
  const int D = a.H * SD;
  const int m0 = 32 * w;
  const float ngs = -a.eta * a.gscale;  // -eta times the loss-gradient scale

  // ---- state, D layout: W1 rows d (4 tiles) / cols m (2 tiles), W2 rows m (2 tiles) / cols d (4 tiles),
  //      and W2 once more as its transpose W2T (rows d / cols m), the operand of the
  //      contraction over d.  Both copies take the same products in the same order at
  //      every update, so W2T stays exactly the transpose of W2.
  f32x4 W1[4][2], W2[2][4], W2T[4][2];
  {
    const float* w1 = a.w1_0 + (int64_t)s * a.w_seq_stride + (int64_t)h * SD * SM;
    const float* w2 = a.w2_0 + (int64_t)s * a.w_seq_stride + (int64_t)h * SM * SD;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          W1[dt][nt][r] = w1[(16 * dt + 4 * g + r) * SM + m0 + 16 * nt + c];
          W2[nt][dt][r] = w2[(m0 + 16 * nt + 4 * g + r) * SD + 16 * dt + c];
          W2T[dt][nt][r] = w2[(m0 + 16 * nt + c) * SD + 16 * dt + 4 * g + r];
        }
    }
  }

  // The two finished values of this lane between the barriers: d-tile rd_dt,
  // source lane rd_src (of each wave's partial tile), elements 2 rd_p, 2 rd_p + 1,
  // i.e. token rd_t, features rd_d and rd_d + 1.  A wave reads 512 consecutive
  // bytes of each partial tile (lane l: bytes 8 l .. 8 l + 7 of its half).
  const int rd_dt = w >> 1;
  const int rd_src = 32 * (w & 1) + (lane >> 1);
  const int rd_p = lane & 1;
  const int rd_t = rd_src & 15;
  const int rd_d = 16 * rd_dt + 4 * (rd_src >> 4) + 2 * rd_p;
  const int ch0 = h * SD + rd_d;
  // gate factors: loop constants used once per step, kept in this thread's LDS slot
  const float2 tg = make_float2(tanh_gate(a.alpha[ch0]), tanh_gate(a.alpha[ch0 + 1]));

  const int64_t nblk = (Tc + SB - 1) / SB;  // blocks of this launch
  const uint16_t* blocks =
      (const uint16_t*)a.qkv_tiles + (((int64_t)s * a.H + h) * ((T + SB - 1) / SB) + p0 / SB) * BLK;
  // rows of this launch and of the sequence fit 32 bits (the MFMA path is chosen for T < 2^31 only)
  const int Tc32 = (int)Tc, p032 = (int)p0, T32 = (int)T;
  auto block_n = [&](int64_t j) -> int { return min(Tc32 - SB * (int)j, SB); };

  // token blocks: direct global -> LDS loads three steps ahead of use (no
  // registers); lane i of a wave fills bytes [16 i, 16 i + 16) of the wave's 1 KB
  // slice; completion is awaited (vmem_done) before the barrier that precedes the
  // block's first use
  auto stage_async = [&](int64_t jb, int buf) {
    const uint4* src = (const uint4*)(blocks + jb * BLK) + 64 * w + lane;
    const uint32_t dst = lds_addr_uniform(Stage[buf], 1024u * (uint32_t)w);
    if (64 * w + lane < BLK_CHUNKS) dma16(src, dst);
  };
  static_assert(BLK_CHUNKS <= NTHR, "one 16-byte chunk per thread");
  // Gate inputs and outputs of block jb go through buffer descriptors that span
  // the block's valid token rows (from its lowest valid token): the hardware
  // zero-fills loads and drops stores outside them, so the last, partial block of
  // a launch needs no branch, and the per-block address arithmetic is scalar.  In
  // that span this lane's pair sits at row rd_t (forward) or nv - 1 - rd_t (reverse),
  // a negative row counting as out of range.
  constexpr int kRawBufferWord3 = 0x00020000;  // 32-bit data format, raw (untyped) access
  const uint16_t* x_seq = (const uint16_t*)a.xin + (int64_t)s * T * D;
  uint16_t* y_seq = (uint16_t*)a.y + (int64_t)s * T * D;
  float* z_seq = a.z ? a.z + (int64_t)s * T * D : a.z;
  auto io_elem0 = [&](int64_t jb, int nv) -> int64_t {  // element offset of the lowest valid row
    const int p = p032 + SB * (int)jb;
    return (int64_t)(a.reverse ? T32 - p - nv : p) * D;
  };
  auto io_voff = [&](int nv, int elem_bytes) -> int {
    return ((a.reverse ? nv - 1 - rd_t : rd_t) * D + ch0) * elem_bytes;
  };
  auto load_x = [&](int64_t jb, int nv) -> uint32_t {  // two bf16 gate inputs of this lane's values (nv = 0: none)
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc((void*)(x_seq + io_elem0(jb, nv)), 0, nv * D * 2, kRawBufferWord3);
    return __builtin_amdgcn_raw_buffer_load_b32(rx, io_voff(nv, 2), 0, 0);
  };
  // the two values of a wave-summed partial tile (Ypart or Zpart) this lane
  // finishes: all loads are issued before the sum (fixed order of the sums)
  auto reduce_part = [&](const f32x4 (&part)[NWAVE][4][64]) -> float2 {
    float2 v[NWAVE];
#pragma unroll
    for (int q = 0; q < NWAVE; ++q) v[q] = *((const float2*)&part[q][rd_dt][rd_src] + rd_p);
    float2 acc = make_float2(0.0f, 0.0f);
#pragma unroll
    for (int q = 0; q < NWAVE; ++q) {
      acc.x += v[q].x;
      acc.y += v[q].y;
    }
    return acc;
  };
  // y = x + tanh(alpha) z of block jb (bf16), and z itself when it is requested
  // (without it the z descriptor spans nothing and its store is dropped); nv = 0
  // drops both
  auto store_z = [&](int64_t jb, int nv, uint32_t xv, float2 z) {
    const int64_t e0 = io_elem0(jb, nv);
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc((void*)(y_seq + e0), 0, nv * D * 2, kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rz =
        __builtin_amdgcn_make_buffer_rsrc((void*)(z_seq ? z_seq + e0 : z_seq), 0, z_seq ? nv * D * 4 : 0, kRawBufferWord3);
    const float x0 = __uint_as_float(xv << 16), x1 = __uint_as_float(xv & 0xffff0000u);
    __builtin_amdgcn_raw_buffer_store_b32(pack2(fmaf(tg.x, z.x, x0), fmaf(tg.y, z.y, x1)), ry, io_voff(nv, 2), 0, 0);
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(z.x), __float_as_uint(z.y)}, rz, io_voff(nv, 4), 0, 0);
  };

  // carried from block j-1 to its read-out during block j
  f32x4 St_prev = zero4();
  // -eta G1 and -eta G2^T of the previous block, kept in pairs of K=16
  // operands: tile 2i in the low half, 2i+1 in the high half of g?T_prev[i]
  bf16x8 g1T_prev, g2T_prev[2];
  bf16x8 hkB_prev = zero8();
  g1T_prev = zero8();
  for (int i = 0; i < 2; ++i) g2T_prev[i] = zero8();
  uint32_t x_blk = 0u;  // gate inputs of the block whose Z is finished next

  // -striu of a b x b tile in the D layout (element r: row 4g + r, column c): the
  // entries with row > column, negated, else 0, as a bf16 operand.  The selects
  // are kept in fp32 (one conversion per pair afterwards).
  bool causal[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) causal[r] = 4 * g + r > c;
  auto causal_neg = [&](f32x4 x) -> bf16x4 {
    f32x4 v;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v[r] = causal[r] ? -x[r] : 0.0f;
      asm("" : "+v"(v[r]));
    }
    return pack4(v);
  };

  // Read-out of the block staged at blk_prev with the state whose bf16 operands
  // are w1p / w2p (the state that follows that block):
  //   Aq = Q W1' + eta striu(Q K^T) G1,  Z = GELU(Aq) W2' + eta striu(Hq Hk^T) G2
  // This wave's partial Z^T (its 32 hidden units) goes to Zpart[w].
  auto readout = [&](const uint16_t* blk_prev, const bf16x8 (&w1p)[2][2], const bf16x8 (&w2p)[4]) {
    const bf16x4 sT = causal_neg(St_prev);
    // K=16 products as K=32 ones: {x, 0} picks the low tile of a pair, {0, x} the high one
    const bf16x8 sT_lo = cat8(sT, zero4b()), sT_hi = cat8(zero4b(), sT);
    const bf16x8 q0 = rd_row8(blk_prev, OFF_Q, g, c, 0), q1 = rd_row8(blk_prev, OFF_Q, g, c, 1);
    f32x4 Hq[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x4 aq = mfma32(w1p[0][nt], q0, zero4());
      aq = mfma32(w1p[1][nt], q1, aq);
      aq = mfma32(g1T_prev, nt ? sT_hi : sT_lo, aq);
#pragma unroll
      for (int r = 0; r < 4; ++r) Hq[nt][r] = Gelu::value(aq[r]);
    }
    const bf16x8 hqB = pack8(Hq[0], Hq[1]);
    const f32x4 Pt = mfma32(hkB_prev, hqB, zero4());
    const bf16x4 pT = causal_neg(Pt);
    const bf16x8 pT_lo = cat8(pT, zero4b()), pT_hi = cat8(zero4b(), pT);
    f32x4 zp[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      zp[dt] = mfma32(w2p[dt], hqB, zero4());
      zp[dt] = mfma32(g2T_prev[dt >> 1], (dt & 1) ? pT_hi : pT_lo, zp[dt]);
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) Zpart[w][dt][lane] = zp[dt];
  };
  auto pack_state = [&](bf16x8 (&w1p)[2][2], bf16x8 (&w2p)[4]) {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) w1p[cc][nt] = pack8(W1[2 * cc][nt], W1[2 * cc + 1][nt]);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) w2p[dt] = pack8(W2[0][dt], W2[1][dt]);
  };

  for (int64_t jb = 0; jb < AHEAD && jb < nblk; ++jb) stage_async(jb, (int)jb);
  vmem_done();
  __syncthreads();

  // Step j runs block j's recurrence; after its second barrier, beside the state
  // update, block j-1's read-out, whose partial Z is summed between the next step's
  // barriers and stored after them (at j = 0 a dummy read-out on zero carried operands
  // and whatever the eighth token buffer holds, whose Z is never stored).  The last
  // block's read-out follows the loop.
  for (int64_t j = 0; j < nblk; ++j) {
    const int n = block_n(j);
    const uint16_t* blk = Stage[j & (NSTAGE - 1)];
    const uint16_t* blk_prev = Stage[(j - 1) & (NSTAGE - 1)];
    TTT_MARK(g_marks_scan_mfma, j, 0);

    // ---- bf16 operands of the state that follows block j-1
    bf16x8 w1p[2][2], w2p[4];
    pack_state(w1p, w2p);

    // ---- A^T = W1^T K^T, S^T = K Q^T (block j)
    f32x4 At[2], St;
    {
      const bf16x8 k0 = rd_row8(blk, OFF_K, g, c, 0), k1 = rd_row8(blk, OFF_K, g, c, 1);
      const bf16x8 q0 = rd_row8(blk, OFF_Q, g, c, 0), q1 = rd_row8(blk, OFF_Q, g, c, 1);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        At[nt] = mfma32(w1p[0][nt], k0, zero4());
        At[nt] = mfma32(w1p[1][nt], k1, At[nt]);
      }
      St = mfma32(k0, q0, zero4());
      St = mfma32(k1, q1, St);
    }
    // ---- Hk^T = GELU(A^T) (also to this wave's LDS slice, for the transposed
    //      read), keeping Phi(A^T) for GELU' between the barriers; partial
    //      Yhat^T = W2^T Hk^T over this wave's 32 hidden units
    bf16x8 hkB;
    f32x4 Pa[2];
    {
      f32x4 Hk[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          Pa[nt][r] = Gelu::cdf(At[nt][r]);
          Hk[nt][r] = At[nt][r] * Pa[nt][r];
        }
      const bf16x4 h0 = pack4(Hk[0]), h1 = pack4(Hk[1]);
      hkB = cat8(h0, h1);
      HkS[w][0][hk_row(lane)] = h0;
      HkS[w][1][hk_row(lane)] = h1;
      f32x4 yp[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) yp[dt] = mfma32(w2p[dt], hkB, zero4());
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) Ypart[w][dt][lane] = yp[dt];
    }

    TTT_MARK(g_marks_scan_mfma, j, 1);
    __syncthreads();
    TTT_MARK(g_marks_scan_mfma, j, 2);

    // ---- between the barriers (no vector-memory operation: the second barrier
    //      waits for the wave's outstanding ones):
    //   G2 of block j from the wave-summed Yhat, this lane's two values;
    //   Z of block j-2 summed over the waves' partials;
    //   this wave's transposed operands for the update.
    {
      const float2 y = reduce_part(Ypart);
      const uint32_t vv = *(const uint32_t*)(blk + OFF_V + rd_t * RS + rd_d);
      const bool tv = rd_t < n;
      const float g2x = tv ? ngs * (y.x - __uint_as_float(vv << 16)) : 0.0f;  // -eta G2
      const float g2y = tv ? ngs * (y.y - __uint_as_float(vv & 0xffff0000u)) : 0.0f;
      const uint32_t pk = pack2(g2x, g2y);
      *(uint32_t*)&G2a[rd_t * RS + pair_order_pos(rd_d)] = pk;
      G2b[rd_d * TS + rd_t] = (uint16_t)pk;
      G2b[(rd_d + 1) * TS + rd_t] = (uint16_t)(pk >> 16);
    }
    TTT_MARK(g_marks_scan_mfma, j, 3);
    // Z of block j-2 (its read-out ran after the previous step's second barrier)
    const float2 zfin = reduce_part(Zpart);
    TTT_MARK(g_marks_scan_mfma, j, 4);
    // GELU'(A^T) to this wave's LDS slice as [m][t], read back token-major below
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) DgS[w][nt][(4 * g + r) * DGS + c] = Gelu::deriv(At[nt][r], Pa[nt][r]);
    // W2 tile (mt, dt) transposed: row m = c, features 16 dt + 4g .. +3; Hk in token-major
    // form (tokens 4g .. 4g+3 of hidden unit m0 + 16 mt + c); GELU'(A) at the same places
    bf16x4 w2t[2][4], hkT[2];
    f32x4 DgT[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) w2t[mt][dt] = pack4(W2T[dt][mt]);
      // transpose of the D-layout tile (source lane (g', c') holds hidden units
      // 4g' .. 4g'+3 of token c'): lane 16g + c addresses the row of source lane
      // 16 (c mod 4) + 4g + c/4, so that (see ld_tr) lane (g, c) receives hidden unit
      // c at tokens 4g .. 4g+3
      hkT[mt] = ld_tr(&HkS[w][mt][hk_row(16 * (c & 3) + 4 * g + (c >> 2))]);
      DgT[mt] = *(const f32x4*)&DgS[w][mt][c * DGS + 4 * g];
    }

    // this wave's vector-memory operations of the previous step (block j+2 into LDS,
    // gate inputs of block j-1, stores) have had a whole step; the barrier then
    // publishes the next block to every wave before its first use
    vmem_done();
    TTT_MARK(g_marks_scan_mfma, j, 5);
    __syncthreads();
    TTT_MARK(g_marks_scan_mfma, j, 6);

    // ---- -eta Gh = (-eta G2) W2^T (token-major, contraction over d), -eta G1 =
    //      -eta Gh * GELU'(A): directly the K=16 operand of the W1 update
    bf16x8 g2B[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) g2B[cc] = *(const bf16x8*)(&G2a[c * RS + 32 * cc + 8 * g]);
    bf16x4 g2T[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) g2T[dt] = *(const bf16x4*)(&G2b[(16 * dt + c) * TS + 4 * g]);
    bf16x4 g1T[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4 gh = mfma32(g2B[0], cat8(w2t[mt][0], w2t[mt][1]), zero4());
      gh = mfma32(g2B[1], cat8(w2t[mt][2], w2t[mt][3]), gh);
      g1T[mt] = pack4(gh * DgT[mt]);
    }
    // ---- state update: W1 += K^T (-eta G1), W2 += Hk^T (-eta G2) (and W2T += (-eta G2)^T Hk).  K^T tile dt
    //      (row d = 16 dt + c, tokens 4g .. 4g+3): lane 16g + j reads token
    //      4g + j/4, features 16 dt + 4 (j mod 4) .. +3 of the staged block
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const bf16x4 kt = ld_tr(blk + OFF_K + (4 * g + ((lane & 15) >> 2)) * RS + 16 * dt + 4 * (lane & 3));
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) W1[dt][nt] = mfma16(kt, g1T[nt], W1[dt][nt]);
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        W2[mt][dt] = mfma16(hkT[mt], g2T[dt], W2[mt][dt]);
        W2T[dt][mt] = mfma16(g2T[dt], hkT[mt], W2T[dt][mt]);
      }

    // ---- block j-1's read-out with the state that follows it (its bf16 operands
    //      w1p, w2p) -> Zpart, summed between the next step's barriers
    readout(blk_prev, w1p, w2p);
    // ---- the vector-memory work of this step, waited for just before the next
    //      step's second barrier: Y and Z of block j-2, the gate inputs of block j-1
    //      (one register, consumed before it is reloaded: no register rotation,
    //      which would make the compiler wait at once), block j+3 into the buffer
    //      that held block j-5
    store_z(j - 2, j > 1 ? block_n(j - 2) : 0, x_blk, zfin);  // nothing to store at j < 2
    x_blk = load_x(j - 1, j > 0 ? block_n(j - 1) : 0);
    // issue order after the second barrier: every matrix-core product followed by
    // two vector-ALU instructions, so that the read-out's GELU, the gate and the
    // packing work run beside the products instead of after them
#pragma unroll
    for (int i = 0; i < MIX_GROUPS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, MIX_PRODUCTS, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, MIX_VALU, 0);
    }
    if (j + AHEAD < nblk) stage_async(j + AHEAD, (int)((j + AHEAD) & (NSTAGE - 1)));

    St_prev = St;
    g1T_prev = cat8(g1T[0], g1T[1]);
    g2T_prev[0] = cat8(g2T[0], g2T[1]);
    g2T_prev[1] = cat8(g2T[2], g2T[3]);
    hkB_prev = hkB;
    TTT_MARK(g_marks_scan_mfma, j, 7);
  }

  // ---- Z of block nblk-2, then the read-out of the last block with the final
  //      state (after every wave's reads of Zpart)
  if (nblk > 0) {
    __syncthreads();
    const float2 zl = reduce_part(Zpart);
    bf16x8 w1p[2][2], w2p[4];
    pack_state(w1p, w2p);
    __syncthreads();
    store_z(nblk - 2, nblk > 1 ? block_n(nblk - 2) : 0, x_blk, zl);
    x_blk = load_x(nblk - 1, block_n(nblk - 1));
    readout(Stage[(nblk - 1) & (NSTAGE - 1)], w1p, w2p);
    __syncthreads();
    store_z(nblk - 1, block_n(nblk - 1), x_blk, reduce_part(Zpart));
  }
  // ---- final state.  The lane indices are derived afresh from an opaque copy of
  // the thread index, so that no address term is kept live across the loop.
  {
    int t2 = tid;
    asm volatile("" : "+v"(t2));
    const int l2 = t2 & 63, g2 = l2 >> 4, c2 = l2 & 15, n0 = 32 * (t2 >> 6);
    if (a.w1_T) {
      float* o = a.w1_T + ((int64_t)s * a.H + h) * SD * SM;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[(16 * dt + 4 * g2 + r) * SM + n0 + 16 * nt + c2] = W1[dt][nt][r];
    }
    if (a.w2_T) {
      float* o = a.w2_T + ((int64_t)s * a.H + h) * SM * SD;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[(n0 + 16 * mt + 4 * g2 + r) * SD + 16 * dt + c2] = W2[mt][dt][r];
    }
  }
}

}  // namespace

bool scan_mfma_supported(int d, int m, int b) { return d == SD && m == SM && b == SB; }

int scan_mfma_block_elems() { return BLK; }

size_t scan_mfma_tile_bytes(int64_t B, int64_t T, int H) {
  const int64_t nblk = (T + SB - 1) / SB;
  return (size_t)(B * H * nblk) * BLK * sizeof(uint16_t);
}

// Only the exact (erf) GELU is instantiated: the tanh form runs on the generic scan.
hipError_t launch_scan_mfma(const ScanArgs& a, hipStream_t s) {
  if (a.gelu_tanh) return hipErrorInvalidValue;
  hipLaunchKernelGGL(scan_mfma_kernel, dim3((unsigned)(a.B * a.H)), dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

}  // namespace ttt

TTT_MARKS_EXPORT(ttt_phase_marks_scan_mfma, g_marks_scan_mfma);
