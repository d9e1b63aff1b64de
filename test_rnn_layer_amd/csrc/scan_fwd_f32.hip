// Forward pass of one direction for the backward, on the fp32 matrix cores:
// head width d = 64, hidden m = 256, mini-batch b = 16, erf GELU ("One-Minute
// Video Generation with Test-Time Training", paper-notes page, key designs
// "TTT-MLP layer" and "gate + bidirectional"; the training section learns the
// outer parameters through the layer, so the backward needs this pass's Z, Y
// and the state every C mini-batches).  The same outputs as the generic
// forward with checkpoints (backward.hip), fp32 throughout: fp32 operands,
// products and sums (v_mfma_f32_16x16x4_f32), in another order.
//
// The same steps also replay checkpoint segments for the backward scan: one
// workgroup per (sequence, head, segment) of a window of segments starts from the
// segment's checkpoint and writes, for each of its mini-batches, the state it
// starts from, the forward quantities A, Hk, GELU'(A), Gh, G1 and G2, and its
// read-out's Aq, Hq, GELU'(Aq) and tril(Q K^T) into the backward scan's slot for it
// (backward.hip); no Z or Y.  The replayed states are the checkpointed trajectory
// bit for bit.
//
// One 512-thread workgroup per (sequence, head); wave w owns hidden units
// [32w, 32w + 32): its slices of W1 (64 x 32), W2 (32 x 64) and W2 once more as
// its transpose W2T (the operand of the contraction over d) stay in registers
// in the matrix-core D layout for the whole sequence.  A D-layout tile X
// (lane (g, c) = (lane / 16, lane % 16) holds X[4g + r][c] in register r) is
// directly the operand of four K=4 products over its row index: register r
// covers rows {r, 4 + r, 8 + r, 12 + r}, lane group g row 4g + r, and the other
// operand lists the contraction index in the same order.  Step j (the
// mini-batch dual form of generic.hip, c = 2/d or 2, N* = -eta *):
//   A^T = W1^T K^T, Hk^T = GELU(A^T), S1^T = GELU'(A^T)        (local)
//   Yhat^T = W2^T Hk^T         partial over the wave's units -> LDS, summed
//   G2 = c (Yhat - V)          each thread two values -> LDS
//   Gh = G2 W2^T, G1 = Gh * S1 (token-major: S1 and Hk transposed in LDS)
//   W1 += K^T NG1, W2 += Hk^T NG2, W2T += NG2^T Hk
// and, with the state that follows block j-1 (which holds the updates of all its
// tokens), block j-1's read-out, taking back the updates of the tokens after each
// one (striu keeps the entries [t][t'] with t' > t):
//   Aq^T = W1^T Q^T - NG1^T striu(Q K^T)^T, Hq^T = GELU(Aq^T)
//   Z^T  = W2^T Hq^T + eta G2^T striu(Hq Hk^T)^T            partial -> LDS, summed
// with y = x + tanh(alpha) z.  A last, short block is padded with zero tokens,
// which add exact zeros to every sum.  Two workgroup barriers per step.
//
// Two parts per chain (the forward pass only): the notes page's on-chip tensor
// parallel with the chain's hidden units split over two workgroups of one
// cooperative launch, part p taking units [128 p, 128 p + 128), 16 a wave, so
// that each CU does half the matrix-core work of a step.  The one contraction
// over units the recurrence needs, Yhat, is exchanged: each part publishes its
// sum over its units as tagged 64-bit device-scope stores (mini-batch index + 1
// in the high word, double-buffered by its parity), polls the other part's and
// adds the two (a sum of two terms does not depend on their order).  Polls are
// bounded: past the spin limit a workgroup raises the abort flag and takes NaN.
// Z, which only feeds the outputs, leaves each part as its partial in a buffer
// of its own; a small kernel adds the two and applies the gate.
#include "internal.h"
#include "mfma_common.h"
#include "token_block.h"

namespace ttt {
namespace {

constexpr int FD = 64;           // head width
constexpr int FM = 256;          // hidden width
constexpr int FB = 16;           // mini-batch
constexpr int FW = 8;            // waves; wave w owns hidden units [32 w, 32 w + 32)
constexpr int FT = 64 * FW;      // threads
constexpr int NSTG = 3;          // staged token blocks: j-1 (read-out), j, j+1 in flight
constexpr int RW = FD + 4;       // 68: row stride of the staged panels and of the NG2 panel
constexpr int GS = RW;
constexpr int PAN = FB * RW;     // floats of one staged 16 x 64 panel (Q, K or V), rows padded
constexpr int BLKF = 3 * PAN;    // floats of a staged block: Q, then K, then V
constexpr int BLK_CH = BLKF / 4; // 816 chunks of 16 bytes, 17 per row (the last one padding)
constexpr int TT = FB + 4;       // 20: row stride of the per-wave transposed tiles
constexpr int OQ = 0, OK = PAN, OV = 2 * PAN;
// a replayed mini-batch's slot: W1 [d][m], W2 [m][d], then A, Hk, GELU'(A), Gh, G1
// ([b][m] each), G2 ([b][d]), Aq, Hq, GELU'(Aq) ([b][m] each) and M = tril(Q K^T)
// ([b][b]), as the backward scan reads it
constexpr int64_t SL_W2 = (int64_t)FD * FM, SL_A = 2 * SL_W2, SL_HK = SL_A + FB * FM, SL_S1 = SL_HK + FB * FM,
                  SL_GH = SL_S1 + FB * FM, SL_G1 = SL_GH + FB * FM, SL_G2 = SL_G1 + FB * FM,
                  SL_AQ = SL_G2 + FB * FD, SL_HQ = SL_AQ + FB * FM, SL_SQ = SL_HQ + FB * FM,
                  SL_M = SL_SQ + FB * FM, SLOT = SL_M + FB * FB;

// Staged panels have rows of 68 floats (17 chunks of 16 bytes): the 16-byte reads of
// one chunk column over rows 0..7 and the 4-byte reads of 16 columns of rows 4g + r
// (g = 0, 1) fall on distinct banks, and every offset is affine in the row and column.
__device__ __forceinline__ int sw(int r, int col) { return r * RW + col; }

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// GELU and GELU' (erf form) as the generic steps compute them.
__device__ __forceinline__ void gelu2(float a, float* g, float* dg) {
  const float cdf = 0.5f * (1.0f + erff(a * 0.7071067811865476f));
  *g = a * cdf;
  *dg = cdf + a * (0.3989422804014327f * expf(-0.5f * a * a));
}
__device__ __forceinline__ float gelu1(float a) { return a * (0.5f * (1.0f + erff(a * 0.7071067811865476f))); }

__device__ float4 g_zero_chunk;  // zero-initialised, never written: the source of padding rows

// REPLAY false: the forward pass of a whole direction (grid: sequences x heads);
// REPLAY true: segments seg_lo .. seg_lo + seg_count - 1 of every (sequence, head)
// (grid: sequences x heads x seg_count)
constexpr uint32_t kFwdSpinMax = 1u << 20;

// UT: hidden-unit tiles of 16 per wave, 2 (one workgroup per chain) or 1 (two parts per chain)
template <bool REPLAY, int UT>
__global__ __launch_bounds__(FT) __attribute__((amdgpu_waves_per_eu(2, 2))) void scan_fwd_f32_kernel(ScanArgs a) {
  constexpr int PARTS = 2 / UT;
  static_assert(UT == 2 || (UT == 1 && !REPLAY), "the replay runs one workgroup per chain");
  __shared__ __attribute__((aligned(16))) float Stage[NSTG][BLKF];  // token blocks j-1 .. j+1
  __shared__ f32x4 Ypart[FW][4][64];                              // partial Yhat^T: wave, d-tile, lane
  __shared__ f32x4 Zpart[FW][4][64];                              // partial Z^T
  __shared__ __attribute__((aligned(16))) float G2s[2][FB * GS];   // G2 [token][feature], by block parity
  // per-wave transposes: Hk^T and S1^T tiles as [unit][token], read back token-major
  __shared__ __attribute__((aligned(16))) float HkS[FW][2][16 * TT];
  __shared__ __attribute__((aligned(16))) float DgS[FW][2][16 * TT];
  __shared__ float2 Tg[FT];  // this thread's two gate factors tanh(alpha), read once per step

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int part = PARTS == 1 ? 0 : (int)(blockIdx.x / (a.B * a.H));  // the chain's part (two parts)
  const int64_t chain = REPLAY ? blockIdx.x / a.seg_count : blockIdx.x - part * (a.B * a.H);  // sequence * H + head
  const int s = (int)(chain / a.H), h = (int)(chain % a.H);
  const int64_t T = a.T;
  const int D = a.H * FD;
  const int u0 = (FM / PARTS) * part + 16 * UT * w;  // this wave's first hidden unit
  const int64_t sh = (int64_t)s * a.H + h;
  const int64_t dm = (int64_t)FD * FM;
  const float neta = -a.eta, gs = a.gscale;
  const int64_t nblk_all = (T + FB - 1) / FB;
  const int C = a.ckpt_every;
  const int64_t nseg = (nblk_all + C - 1) / C;
  // mini-batches j0 .. j1 - 1: the whole sequence, or one replayed segment
  const int64_t seg = REPLAY ? a.seg_lo + blockIdx.x % a.seg_count : 0;
  const int64_t j0 = REPLAY ? seg * C : 0;
  const int64_t j1 = REPLAY ? min(nblk_all, j0 + C) : nblk_all;
  const int64_t seg_stride = a.seg_stride > 0 ? a.seg_stride : a.seg_count;
  float* const slots = REPLAY ? a.seg_slots + (chain * seg_stride + blockIdx.x % a.seg_count) * C * SLOT : nullptr;

  f32x4 W1[4][UT], W2[UT][4], W2T[4][UT];
  {
    const float* w1 = REPLAY ? a.ckpt + (chain * nseg + seg) * 2 * dm
                             : a.w1_0 + (int64_t)s * a.w_seq_stride + (int64_t)h * dm;
    const float* w2 = REPLAY ? w1 + dm : a.w2_0 + (int64_t)s * a.w_seq_stride + (int64_t)h * dm;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int ut = 0; ut < UT; ++ut) {
          W1[dt][ut][r] = w1[(16 * dt + 4 * g + r) * FM + u0 + 16 * ut + c];
          W2[ut][dt][r] = w2[(u0 + 16 * ut + 4 * g + r) * FD + 16 * dt + c];
          W2T[dt][ut][r] = w2[(u0 + 16 * ut + c) * FD + 16 * dt + 4 * g + r];
        }
  }

  // the two values this thread finishes between the barriers (Yhat, then Z of the
  // block before): d-tile rd_dt, source lane rd_src of each wave's partial tile,
  // registers 2 rd_p and 2 rd_p + 1, i.e. token row rd_t, features rd_d, rd_d + 1
  const int rd_dt = w >> 1;
  const int rd_src = 32 * (w & 1) + (lane >> 1);
  const int rd_p = lane & 1;
  const int rd_t = rd_src & 15;
  const int rd_d = 16 * rd_dt + 4 * (rd_src >> 4) + 2 * rd_p;
  const int ch0 = h * FD + rd_d;
  if (!REPLAY) Tg[tid] = make_float2(tanhf(a.alpha[ch0]), tanhf(a.alpha[ch0 + 1]));
  auto reduce_part = [&](const f32x4 (&part)[FW][4][64]) -> float2 {
    float2 v[FW];
#pragma unroll
    for (int q = 0; q < FW; ++q) v[q] = *((const float2*)&part[q][rd_dt][rd_src] + rd_p);
    float2 acc = make_float2(0.0f, 0.0f);
#pragma unroll
    for (int q = 0; q < FW; ++q) {
      acc.x += v[q].x;
      acc.y += v[q].y;
    }
    return acc;
  };
  auto tok = [&](int64_t p) -> int64_t { return a.reverse ? T - 1 - p : p; };
  // two parts: this part's sum over its units of this thread's two Yhat values of block jb,
  // published, and the other part's added (NaN for it after an abort or a time-out)
  bool failed = false;
  auto exchange = [&](float2 y, int64_t jb) -> float2 {
    const uint32_t tag = (uint32_t)(jb + 1);
    const int par = (int)(jb & 1);
    uint64_t* mine = a.xchg + ((chain * 2 + part) * 2 + par) * (2 * FT) + 2 * tid;
    const uint64_t* theirs = a.xchg + ((chain * 2 + (part ^ 1)) * 2 + par) * (2 * FT) + 2 * tid;
    __hip_atomic_store(mine, ((uint64_t)tag << 32) | __float_as_uint(y.x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(mine + 1, ((uint64_t)tag << 32) | __float_as_uint(y.y), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    float2 o = make_float2(__uint_as_float(0x7fc00000u), __uint_as_float(0x7fc00000u));
    for (uint32_t spin = 0; !failed; ++spin) {
      const uint64_t e0 = __hip_atomic_load(theirs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t e1 = __hip_atomic_load(theirs + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((uint32_t)(e0 >> 32) == tag && (uint32_t)(e1 >> 32) == tag) {
        o = make_float2(__uint_as_float((uint32_t)e0), __uint_as_float((uint32_t)e1));
        break;
      }
      if (spin >= kFwdSpinMax) {
        __hip_atomic_store(a.abort_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        failed = true;
      } else if ((spin & 15) == 15 && __hip_atomic_load(a.abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
        failed = true;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    return make_float2(y.x + o.x, y.y + o.y);
  };

  // token block jb into stage buf: chunk i (thread i, and i + 512 for the first 304
  // threads) is chunk q of row r of panel i / 272 (a wave fills 1 KB of consecutive
  // LDS); the padding chunk of each row and rows past the sequence come from the
  // zero chunk
  const int64_t plane = a.B * a.H * T * FD;
  const float* qkv_h = a.qkv + sh * T * FD;
  auto stage_async = [&](int64_t jb, int buf) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = tid + FT * k;
      if (k == 1 && 64 * w >= BLK_CH - FT) break;  // whole waves past the block
      const int pnl = i / (FB * 17), pc = i - pnl * (FB * 17), r = pc / 17, q = pc - 17 * r;
      const int64_t p = jb * FB + r;
      const bool real = i < BLK_CH && q < 16 && p < T;
      const void* src = real ? (const void*)(qkv_h + pnl * plane + tok(p) * FD + 4 * q) : (const void*)&g_zero_chunk;
      if (i < BLK_CH) tb::dma16(src, tb::lds_addr_uniform(Stage[buf], 16u * (uint32_t)(FT * k + 64 * w)));
    }
  };

  // carried from block j-1 to its read-out during step j
  f32x4 St_prev = zero4();                 // S^T = K Q^T of block j-1: [t'][t]
  f32x4 g1_prev[UT], hkT_prev[UT];  // NG1 = -eta G1 of block j-1, token-major [t][u]; Hk^T of block j-1: [u][t]
#pragma unroll
  for (int ut = 0; ut < UT; ++ut) g1_prev[ut] = hkT_prev[ut] = zero4();

  // -striu of a D-layout [t'][t] tile: the entries with t' = 4g + r > t = c, negated
  bool later[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) later[r] = 4 * g + r > c;

  // Read-out of the block staged at `prev` with the current state (the one that
  // follows that block); this wave's partial Z^T goes to Zpart[w].  Replaying, the
  // block's Aq, Hq, GELU'(Aq) and M go to its slot rs instead (no Z).
  auto readout = [&](const float* prev, const float* g2prev, float* rs) {
    f32x4 aq[UT];
#pragma unroll
    for (int ut = 0; ut < UT; ++ut) aq[ut] = zero4();
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const f32x4 qf = *(const f32x4*)&prev[OQ + sw(c, 16 * dt + 4 * g)];
#pragma unroll
      for (int ut = 0; ut < UT; ++ut)
#pragma unroll
        for (int r = 0; r < 4; ++r) aq[ut] = mfma4(W1[dt][ut][r], qf[r], aq[ut]);
    }
    f32x4 hqT[UT];
#pragma unroll
    for (int ut = 0; ut < UT; ++ut) {
#pragma unroll
      for (int r = 0; r < 4; ++r) aq[ut] = mfma4(g1_prev[ut][r], later[r] ? -St_prev[r] : 0.0f, aq[ut]);
      if (REPLAY) {  // [t][m]: lane (g, c) holds token c, units u0 + 16 ut + 4g .. +3
        f32x4 sq;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float hv, dv;
          gelu2(aq[ut][r], &hv, &dv);
          hqT[ut][r] = hv;
          sq[r] = dv;
        }
        *(f32x4*)&rs[SL_AQ + c * FM + u0 + 16 * ut + 4 * g] = aq[ut];
        *(f32x4*)&rs[SL_HQ + c * FM + u0 + 16 * ut + 4 * g] = hqT[ut];
        *(f32x4*)&rs[SL_SQ + c * FM + u0 + 16 * ut + 4 * g] = sq;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) hqT[ut][r] = gelu1(aq[ut][r]);
      }
    }
    if (REPLAY) {
      if (w == 0) {  // M[t][t'] = Q[t] . K[t'] for t' <= t: lane (g, c) holds t = c, t' = 4g .. 4g+3
        f32x4 mv;
#pragma unroll
        for (int r = 0; r < 4; ++r) mv[r] = later[r] ? 0.0f : St_prev[r];
        *(f32x4*)&rs[SL_M + c * FB + 4 * g] = mv;
      }
      return;
    }
    f32x4 pt = zero4();  // this wave's part of (Hq Hk^T)^T: [t'][t]
#pragma unroll
    for (int ut = 0; ut < UT; ++ut)
#pragma unroll
      for (int r = 0; r < 4; ++r) pt = mfma4(hkT_prev[ut][r], hqT[ut][r], pt);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      f32x4 zp = zero4();
#pragma unroll
      for (int ut = 0; ut < UT; ++ut)
#pragma unroll
        for (int r = 0; r < 4; ++r) zp = mfma4(W2[ut][dt][r], hqT[ut][r], zp);
#pragma unroll
      for (int r = 0; r < 4; ++r) zp = mfma4(g2prev[(4 * g + r) * GS + 16 * dt + c], later[r] ? a.eta * pt[r] : 0.0f, zp);
      Zpart[w][dt][lane] = zp;
    }
  };
  // z and y = x + tanh(alpha) z of this thread's two values of block jb
  auto store_z = [&](int64_t jb, float2 z) {
    const int64_t p = jb * FB + rd_t;
    if (jb < 0 || p >= T) return;
    const int64_t o = ((int64_t)s * T + tok(p)) * D + ch0;
    if (PARTS == 2) {  // this part's partial; the gate follows once both are in
      *(float2*)(a.zpart + part * (a.B * T * D) + o) = z;
      return;
    }
    *(float2*)(a.z + o) = z;
    const float2 tg = Tg[tid];
    float x0, x1;
    if (a.bf16) {
      const uint32_t xv = *(const uint32_t*)((const uint16_t*)a.xin + o);
      x0 = __uint_as_float(xv << 16);
      x1 = __uint_as_float(xv & 0xffff0000u);
      *(uint32_t*)((uint16_t*)a.y + o) = pack2(fmaf(tg.x, z.x, x0), fmaf(tg.y, z.y, x1));
    } else {
      const float2 xv = *(const float2*)((const float*)a.xin + o);
      *(float2*)((float*)a.y + o) = make_float2(fmaf(tg.x, z.x, xv.x), fmaf(tg.y, z.y, xv.y));
    }
  };

  for (int64_t jb = j0; jb < j0 + NSTG - 1 && jb < j1; ++jb) stage_async(jb, (int)(jb - j0));
  // G2s of the block before block 0 is read by the read-out at j = 0 (whose result is
  // never stored): keep it finite
  for (int i = tid; i < FB * GS; i += FT) G2s[1][i] = 0.0f;
  int sj = 0;  // stage of block j; block j-1 sits in stage (sj + 2) mod 3
  vmem_done();
  __syncthreads();

  for (int64_t j = j0; j < j1; ++j) {
    const int sp = sj == 0 ? NSTG - 1 : sj - 1;
    float* const sl = REPLAY ? slots + (j - j0) * SLOT : nullptr;
    const float* blk = Stage[sj];
    const float* blk_prev = Stage[sp];
    float* g2cur = G2s[j & 1];
    const float* g2prev = G2s[(j & 1) ^ 1];

    // ---- checkpoint (every C-th block), or the replayed block's slot: the state at the
    //      start of block j, W1 [d][m] then W2 [m][d]
    if (REPLAY || j % C == 0) {
      float* o = REPLAY ? sl : a.ckpt + (sh * nseg + j / C) * 2 * dm;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int ut = 0; ut < UT; ++ut)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            o[(16 * dt + 4 * g + r) * FM + u0 + 16 * ut + c] = W1[dt][ut][r];
            o[dm + (u0 + 16 * ut + 4 * g + r) * FD + 16 * dt + c] = W2[ut][dt][r];
          }
    }

    // ---- A^T = W1^T K^T (this wave's units), S^T = K Q^T
    f32x4 At[UT], St = zero4();
#pragma unroll
    for (int ut = 0; ut < UT; ++ut) At[ut] = zero4();
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const f32x4 kf = *(const f32x4*)&blk[OK + sw(c, 16 * dt + 4 * g)];
      const f32x4 qf = *(const f32x4*)&blk[OQ + sw(c, 16 * dt + 4 * g)];
#pragma unroll
      for (int ut = 0; ut < UT; ++ut)
#pragma unroll
        for (int r = 0; r < 4; ++r) At[ut] = mfma4(W1[dt][ut][r], kf[r], At[ut]);
#pragma unroll
      for (int r = 0; r < 4; ++r) St = mfma4(kf[r], qf[r], St);
    }
    // ---- Hk^T = GELU(A^T), S1^T = GELU'(A^T) (both also to this wave's LDS slices
    //      for the token-major reads); partial Yhat^T over this wave's units
    f32x4 hkT[UT];
#pragma unroll
    for (int ut = 0; ut < UT; ++ut)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float hv, dv;
        gelu2(At[ut][r], &hv, &dv);
        hkT[ut][r] = hv;
        HkS[w][ut][(4 * g + r) * TT + c] = hv;
        DgS[w][ut][(4 * g + r) * TT + c] = dv;
        if (REPLAY) sl[SL_S1 + c * FM + u0 + 16 * ut + 4 * g + r] = dv;
      }
    if (REPLAY)  // A and Hk [t][m]: lane (g, c) holds token c, units u0 + 16 ut + 4g .. +3
#pragma unroll
      for (int ut = 0; ut < UT; ++ut) {
        *(f32x4*)&sl[SL_A + c * FM + u0 + 16 * ut + 4 * g] = At[ut];
        *(f32x4*)&sl[SL_HK + c * FM + u0 + 16 * ut + 4 * g] = hkT[ut];
      }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      f32x4 yp = zero4();
#pragma unroll
      for (int ut = 0; ut < UT; ++ut)
#pragma unroll
        for (int r = 0; r < 4; ++r) yp = mfma4(W2[ut][dt][r], hkT[ut][r], yp);
      Ypart[w][dt][lane] = yp;
    }

    __syncthreads();

    // ---- G2 = c (Yhat - V): this thread's two values
    {
      float2 y = reduce_part(Ypart);
      if (PARTS == 2) y = exchange(y, j);
      const float2 v = *(const float2*)&blk[OV + sw(rd_t, rd_d)];
      const float2 g2 = make_float2(gs * (y.x - v.x), gs * (y.y - v.y));
      *(float2*)&g2cur[rd_t * GS + rd_d] = g2;
      if (REPLAY) *(float2*)&sl[SL_G2 + rd_t * FD + rd_d] = g2;
    }
    // ---- read-out of block j-1 (at j = 0 on zero operands, never stored; replaying, into
    //      block j-1's slot, from the segment's second block on)
    if (!REPLAY) readout(blk_prev, g2prev, nullptr);
    else if (j > j0) readout(blk_prev, g2prev, sl - SLOT);
    // ---- this wave's token-major Hk and S1: [t = 4g + r][u = c]
    f32x4 hkF[UT], s1F[UT];
#pragma unroll
    for (int ut = 0; ut < UT; ++ut) {
      hkF[ut] = *(const f32x4*)&HkS[w][ut][c * TT + 4 * g];
      s1F[ut] = *(const f32x4*)&DgS[w][ut][c * TT + 4 * g];
    }
    // block j+1's loads (issued in the previous step) are complete before the barrier
    // that publishes them
    vmem_done();
    __syncthreads();

    // ---- Gh = G2 W2^T (token-major), G1 = Gh * S1, NG1 = -eta G1
    f32x4 g1[UT];
#pragma unroll
    for (int ut = 0; ut < UT; ++ut) g1[ut] = zero4();
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const f32x4 gA = *(const f32x4*)&g2cur[c * GS + 16 * dt + 4 * g];
#pragma unroll
      for (int ut = 0; ut < UT; ++ut)
#pragma unroll
        for (int r = 0; r < 4; ++r) g1[ut] = mfma4(gA[r], W2T[dt][ut][r], g1[ut]);
    }
    if (REPLAY)  // Gh, then G1 [t][m]: lane (g, c) holds tokens 4g .. 4g+3 of unit u0 + 16 ut + c
#pragma unroll
      for (int ut = 0; ut < UT; ++ut)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sl[SL_GH + (4 * g + r) * FM + u0 + 16 * ut + c] = g1[ut][r];
          sl[SL_G1 + (4 * g + r) * FM + u0 + 16 * ut + c] = g1[ut][r] * s1F[ut][r];
        }
#pragma unroll
    for (int ut = 0; ut < UT; ++ut) g1[ut] = neta * (g1[ut] * s1F[ut]);
    // ---- state update: W1 += K^T NG1, W2 += Hk^T NG2, W2T += NG2^T Hk (contraction over
    //      the 16 tokens: register r of a token-major tile is tokens 4g + r)
    f32x4 g2c[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      f32x4 kc;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        kc[r] = blk[OK + sw(4 * g + r, 16 * dt + c)];
        g2c[dt][r] = neta * g2cur[(4 * g + r) * GS + 16 * dt + c];
      }
#pragma unroll
      for (int ut = 0; ut < UT; ++ut)
#pragma unroll
        for (int r = 0; r < 4; ++r) W1[dt][ut] = mfma4(kc[r], g1[ut][r], W1[dt][ut]);
    }
#pragma unroll
    for (int ut = 0; ut < UT; ++ut)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          W2[ut][dt] = mfma4(hkF[ut][r], g2c[dt][r], W2[ut][dt]);
          W2T[dt][ut] = mfma4(g2c[dt][r], hkF[ut][r], W2T[dt][ut]);
        }

    // ---- Z of block j-1 and its gate; block j+2 into the stage that held block j-1
    if (!REPLAY) store_z(j - 1, reduce_part(Zpart));
    if (j + NSTG - 1 < j1) stage_async(j + NSTG - 1, sp);

    St_prev = St;
#pragma unroll
    for (int ut = 0; ut < UT; ++ut) {
      g1_prev[ut] = g1[ut];
      hkT_prev[ut] = hkT[ut];
    }
    sj = sj == NSTG - 1 ? 0 : sj + 1;
  }

  // ---- read-out of the last block with the final state (after every wave's last
  //      reads of Zpart)
  if (!REPLAY && j1 > 0) {
    __syncthreads();
    readout(Stage[sj == 0 ? NSTG - 1 : sj - 1], G2s[(j1 - 1) & 1], nullptr);
    __syncthreads();
    store_z(j1 - 1, reduce_part(Zpart));
  }
  // ---- replaying: the read-out of the segment's last block (registers and its staged
  //      block only, which nothing overwrites any more)
  if (REPLAY && j1 > j0) readout(Stage[sj == 0 ? NSTG - 1 : sj - 1], nullptr, slots + (j1 - 1 - j0) * SLOT);
}

}  // namespace

bool scan_fwd_f32_supported(int d, int m, int b) { return d == FD && m == FM && b == FB; }

size_t scan_replay_f32_slot_elems() { return (size_t)SLOT; }

bool scan_fwd_f32_split_fits(int64_t B, int H) {
  int dev = 0, cus = 0, coop = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop) return false;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, scan_fwd_f32_kernel<false, 1>, FT, 0) != hipSuccess)
    return false;
  return 2 * B * H <= (int64_t)cus * per_cu;
}

size_t scan_fwd_f32_split_xchg_elems(int64_t B, int H) { return (size_t)(B * H) * 2 * 2 * 2 * FT; }

namespace {
// z = the two parts' partials added; y = x + tanh(alpha) z (io dtype); rows x D elements
__global__ void fwd_f32_gate_kernel(const float* zpart, int64_t n, int D, const float* alpha, const void* xin,
                                    void* y, float* z, int bf16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float zv = zpart[i] + zpart[n + i];
    if (z) z[i] = zv;
    if (y) {
      const float tg = tanhf(alpha[i % D]);
      if (bf16) {
        const float x = __uint_as_float((uint32_t)((const uint16_t*)xin)[i] << 16);
        ((__bf16*)y)[i] = (__bf16)fmaf(tg, zv, x);
      } else {
        ((float*)y)[i] = fmaf(tg, zv, ((const float*)xin)[i]);
      }
    }
  }
}
}  // namespace

hipError_t launch_fwd_f32_gate(const ScanArgs& a, hipStream_t s) {
  const int64_t n = a.B * a.T * a.H * FD;
  if (n == 0 || (!a.z && !a.y)) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 16384);
  hipLaunchKernelGGL(fwd_f32_gate_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a.zpart, n, (int)(a.H * FD), a.alpha,
                     a.xin, a.y, a.z, a.bf16);
  return hipGetLastError();
}

hipError_t launch_scan_fwd_f32(const ScanArgs& a, hipStream_t s) {
  if (a.gelu_tanh || !scan_fwd_f32_supported(a.d, a.m, a.b) || a.ckpt_every <= 0) return hipErrorInvalidValue;
  if (a.zpart) {  // two parts per chain, one cooperative launch
    ScanArgs args = a;
    void* kargs[] = {(void*)&args};
    return hipLaunchCooperativeKernel((const void*)scan_fwd_f32_kernel<false, 1>, dim3((unsigned)(2 * a.B * a.H)),
                                      dim3(FT), kargs, 0, s);
  }
  hipLaunchKernelGGL((scan_fwd_f32_kernel<false, 2>), dim3((unsigned)(a.B * a.H)), dim3(FT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scan_replay_f32(const ScanArgs& a, hipStream_t s) {
  if (a.gelu_tanh || !scan_fwd_f32_supported(a.d, a.m, a.b) || a.ckpt_every <= 0 || a.seg_count <= 0 ||
      !a.seg_slots || (a.seg_stride > 0 && a.seg_stride < a.seg_count))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((scan_fwd_f32_kernel<true, 2>), dim3((unsigned)(a.B * a.H * a.seg_count)), dim3(FT), 0, s, a);
  return hipGetLastError();
}

}  // namespace ttt
