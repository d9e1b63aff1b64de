// TTT-Linear scan on the bf16 matrix cores, head width d = 64, mini-batch b = 16.
// The layer is the TTT-MLP layer of "One-Minute Video Generation with
// Test-Time Training" (paper-notes page, key designs: "TTT-MLP layer",
// "gate + bidirectional") with the linear inner model f(u; W) = u W, W: d x d,
// that the page's ablation table calls TTT-Linear.  Per 16-token block, with W
// the state the block starts from (the mini-batch dual form of the per-token
// rule, gradients taken at the block's start):
//   G = c (K W - V),  Z = Q W - eta tril(Q K^T) G  (diagonal included),
//   W <- W - eta K^T G,  y = x + tanh(alpha) z.
// fp32 state and accumulation, bf16 matrix operands.
//
// One 256-thread workgroup per (sequence, head); wave w owns the output columns
// [16w, 16w+16) of W, G and Z, so W[:, cols] (64 x 16) lives in registers as
// four 16x16 accumulator tiles.  Every product above is separable by output
// column, so the waves never exchange values: they only share the staged
// blocks, and one barrier per block publishes the next one.
//
// Z is computed transposed (rows: columns of the head, columns: tokens), so that
// a lane holds 4 consecutive channels of one token and moves x, y and z with one
// access each.  A step is short (11 matrix-core products per wave), so token
// blocks and gate inputs are loaded kDist blocks ahead, by direct loads to LDS
// whose count per step is the same in every wave; a step waits only for the
// loads of the block after it (s_waitcnt vmcnt with the count of the loads and
// stores issued since), never for the most recent ones.
#include "internal.h"
#include "mfma_common.h"
#include "token_block.h"

namespace ttt {
namespace {

using namespace tb;
constexpr int LW = 4;                  // waves; wave w owns columns [16w, 16w + 16)
constexpr int LTHR = 64 * LW;
constexpr int kDist = 7;               // blocks loaded ahead of use
constexpr int NBUF = kDist + 1;        // LDS stages
constexpr int QKV_BYTES = 8192;        // a staged block (6,912 bytes) padded to two 4 KB rounds of loads
constexpr int X_BYTES = SB * SD * 2;   // gate inputs of a block: [16 tokens][64 channels] bf16
// vector-memory instructions per wave and step: block (2 rounds) + gate inputs, then y and z stores
constexpr int kLoadsPerStep = 3, kStoresPerStep = 2;
constexpr int kVmPerStep = kLoadsPerStep + kStoresPerStep;
// after the loads of block j+1 (issued at the start of step j+1-kDist): that step's stores and
// every instruction of the kDist-1 steps since
constexpr int kVmAfterNext = kStoresPerStep + kVmPerStep * (kDist - 1);
static_assert(kVmAfterNext <= 63, "vmcnt counts to 63");
constexpr int kRawBufferWord3 = 0x00020000;  // 32-bit data format, raw (untyped) access

typedef int i32x4 __attribute__((ext_vector_type(4)));

// A raw buffer descriptor over [base, base + bytes): loads outside it return
// zero, stores outside it are dropped.  base and bytes must be wave-uniform.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(p >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = kRawBufferWord3;
  return r;
}

// Direct load of 16 bytes per lane from a buffer (byte offset voff, zero outside
// the descriptor's range) into LDS bytes [lds_base + 16 lane, + 16).  A statement
// of its own for the reason given at tb::dma16; awaited by the explicit vmcnt wait.
__device__ __forceinline__ void dma16_buffer(i32x4 rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               : : "s"(lds_base), "v"(voff), "s"(rsrc) : "memory", "m0");
}

// Wait until at most kVmAfterNext vector-memory instructions of this wave are in
// flight: the loads of the block after the current one have landed.
__device__ __forceinline__ void wait_next_block() {
  __builtin_amdgcn_sched_barrier(0);
  // s_waitcnt encoding: vmcnt low bits [3:0], high bits [15:14]; expcnt [6:4] and
  // lgkmcnt [11:8] left at their maxima (no constraint)
  constexpr int v = kVmAfterNext;
  __builtin_amdgcn_s_waitcnt((v & 15) | ((v >> 4) << 14) | (7 << 4) | (15 << 8));
  __builtin_amdgcn_sched_barrier(0);
}

__global__ __launch_bounds__(LTHR) void scan_linear_mfma_kernel(ScanArgs a) {
  __shared__ __attribute__((aligned(16))) char StageQKV[NBUF][QKV_BYTES];
  __shared__ __attribute__((aligned(16))) char StageX[NBUF][X_BYTES];
  __shared__ __attribute__((aligned(16))) char Spill[2][1024];  // target of the gate-input loads of waves 2, 3

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int s = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int64_t T = a.T;
  const int Tc = (int)a.Tc, p0 = (int)a.p0, T32 = (int)T;  // rows fit 32 bits (T < 2^31 on this path)
  const int D = a.H * SD;
  const float ngs = -a.eta * a.gscale;  // -eta c

  // ---- state W[:, 16w .. 16w+15], D layout: tile dt holds rows 16 dt + 4g + r, column 16w + c
  f32x4 W[4];
  {
    const float* w0 = a.w1_0 + (int64_t)s * a.w_seq_stride + (int64_t)h * SD * SD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) W[dt][r] = w0[(16 * dt + 4 * g + r) * SD + 16 * w + c];
  }
  // this lane's outputs: token c of the block, channels h*64 + 16w + 4g .. +3
  const int col0 = 16 * w + 4 * g;
  float tg[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) tg[r] = tanh_gate(a.alpha[h * SD + col0 + r]);
  // causal mask of Z's b x b term: key tau = 4g + r at or before query t = c
  bool causal[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) causal[r] = 4 * g + r <= c;

  const int nblk = (Tc + SB - 1) / SB;
  auto block_n = [&](int jb) -> int { return min(Tc - SB * jb, SB); };
  // token blocks of this launch; loads past the last one return zeros
  const uint16_t* blocks =
      (const uint16_t*)a.qkv_tiles + (((int64_t)s * a.H + h) * ((T + SB - 1) / SB) + p0 / SB) * BLK;
  const i32x4 rsrc_blk = buffer_rsrc(blocks, (uint32_t)nblk * BLK * 2);

  // Gate inputs and outputs of block jb: descriptors spanning the block's valid
  // token rows, from its lowest valid token (scan row r sits at row r forward,
  // nv - 1 - r reversed; a negative row is out of range).
  const uint16_t* x_seq = (const uint16_t*)a.xin + (int64_t)s * T * D + h * SD;
  uint16_t* y_seq = (uint16_t*)a.y + (int64_t)s * T * D + h * SD;
  float* z_seq = a.z ? a.z + (int64_t)s * T * D + h * SD : a.z;
  auto io_elem0 = [&](int jb, int nv) -> int64_t {
    const int p = p0 + SB * jb;
    return (int64_t)(a.reverse ? T32 - p - nv : p) * D;
  };
  auto io_row = [&](int r, int nv) -> int { return a.reverse ? nv - 1 - r : r; };

  // loads of block jb into stage jb mod NBUF: two 4 KB rounds of the token block,
  // then 1 KB of gate inputs per wave (waves 0, 1: rows 8w .. 8w+7; waves 2, 3: out of
  // range, into Spill); the same three instructions in every wave and step
  auto stage = [&](int jb) {
    const int buf = jb % NBUF;
#pragma unroll
    for (int round = 0; round < 2; ++round) {
      const uint32_t chunk = 256u * round + 64u * w + lane;
      dma16_buffer(rsrc_blk, (uint32_t)jb * (BLK * 2) + 16u * chunk,
                   lds_addr_uniform(StageQKV[buf], 4096u * round + 1024u * w));
    }
    const int nv = jb < nblk ? block_n(jb) : 0;
    const i32x4 rx = buffer_rsrc(x_seq + io_elem0(jb, nv), (uint32_t)nv * D * 2);
    const int row = 8 * w + (lane >> 3), part = lane & 7;  // 8 chunks of 16 bytes per row
    const uint32_t voff = w < 2 ? (uint32_t)(io_row(row, nv) * D * 2 + 16 * part) : 0xfffffff0u;
    dma16_buffer(rx, voff, lds_addr_uniform(w < 2 ? StageX[buf] + 1024 * w : Spill[w & 1], 0u));
  };

  for (int jb = 0; jb < kDist; ++jb) stage(jb);
  vmem_done();
  __syncthreads();

  for (int j = 0; j < nblk; ++j) {
    stage(j + kDist);  // into the stage of block j-1, last read before the previous barrier
    const uint16_t* blk = (const uint16_t*)StageQKV[j % NBUF];
    const uint16_t* xs = (const uint16_t*)StageX[j % NBUF];

    // ---- bf16 operands of W: K=32 B operands over the input features, pair order
    const bf16x8 wp0 = pack8(W[0], W[1]), wp1 = pack8(W[2], W[3]);
    const bf16x8 k0 = rd_row8(blk, OFF_K, g, c, 0), k1 = rd_row8(blk, OFF_K, g, c, 1);
    const bf16x8 q0 = rd_row8(blk, OFF_Q, g, c, 0), q1 = rd_row8(blk, OFF_Q, g, c, 1);
    // A = K W (rows: tokens 4g + r, column 16w + c); S^T = K Q^T (rows: keys, columns: queries)
    f32x4 A = mfma32(k0, wp0, zero4());
    A = mfma32(k1, wp1, A);
    f32x4 St = mfma32(k0, q0, zero4());
    St = mfma32(k1, q1, St);
    // V at the same places as A: lane 16g + i addresses row 4g + i/4, columns 16w + 4 (i mod 4) ..
    const bf16x4 vv = ld_tr(blk + OFF_V + (4 * g + (c >> 2)) * RS + 16 * w + 4 * (c & 3));
    // -eta G = -eta c (A - V); rows past a short block's end are zero on both sides
    f32x4 ng;
#pragma unroll
    for (int r = 0; r < 4; ++r) ng[r] = ngs * (A[r] - (float)vv[r]);
    const bf16x4 ngb = pack4(ng);
    bf16x4 sT;
#pragma unroll
    for (int r = 0; r < 4; ++r) sT[r] = (__bf16)(causal[r] ? St[r] : 0.0f);
    // Z^T = W^T Q^T + (-eta G)^T tril(Q K^T)^T (rows: columns 16w + 4g + r, column: token c);
    // the K=16 term as a K=32 product with zero upper halves (one instruction per chain)
    f32x4 Zt = mfma32(wp0, q0, zero4());
    Zt = mfma32(wp1, q1, Zt);
    Zt = mfma32(cat8(ngb, zero4b()), cat8(sT, zero4b()), Zt);
    // ---- W += K^T (-eta G); K^T tile dt (row d = 16 dt + c, tokens 4g .. 4g+3) by transposed reads
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const bf16x4 kt = ld_tr(blk + OFF_K + (4 * g + (c >> 2)) * RS + 16 * dt + 4 * (c & 3));
      W[dt] = mfma16(kt, ngb, W[dt]);
    }
    // ---- gate: token c, channels col0 .. col0+3
    const int nv = block_n(j);
    const int64_t e0 = io_elem0(j, nv);
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc((void*)(y_seq + e0), 0, nv * D * 2, kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rz =
        __builtin_amdgcn_make_buffer_rsrc((void*)(z_seq ? z_seq + e0 : z_seq), 0, z_seq ? nv * D * 4 : 0, kRawBufferWord3);
    const bf16x4 xv = *(const bf16x4*)(xs + c * SD + col0);
    f32x4 y;
#pragma unroll
    for (int r = 0; r < 4; ++r) y[r] = fmaf(tg[r], Zt[r], (float)xv[r]);
    const int off = io_row(c, nv) * D + col0;  // elements from the descriptor's base
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, pack4(y)), ry, off * 2, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, Zt), rz, off * 4, 0, 0);
    // block j+1 has landed (this wave's part); the barrier publishes it and frees stage j
    wait_next_block();
    __syncthreads();
  }
  vmem_done();  // loads past the end, into stages no one reads, are drained before the exit

  if (a.w1_T) {
    float* o = a.w1_T + ((int64_t)s * a.H + h) * SD * SD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[(16 * dt + 4 * g + r) * SD + 16 * w + c] = W[dt][r];
  }
}

}  // namespace

bool scan_linear_mfma_supported(int d, int m, int b) { return d == SD && m == SD && b == SB; }

hipError_t launch_scan_linear_mfma(const ScanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(scan_linear_mfma_kernel, dim3((unsigned)(a.B * a.H)), dim3(LTHR), 0, s, a);
  return hipGetLastError();
}

}  // namespace ttt
