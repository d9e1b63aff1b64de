// The token-block layout shared by the projection GEMM's epilogue and the MFMA
// scans (head width 64, blocks of 16 scan positions), and its LDS readers.
//
// A block holds Q, K and V of 16 consecutive scan positions of one (sequence,
// head), each [16 tokens][RS] bf16 with the 64 features in order and rows
// padded to RS = 72 elements (144 bytes), so that the 16 rows read by one
// 16-lane group fall on distinct LDS banks.  Blocks of a (sequence, head) are
// contiguous, in scan order.  Rows past the end of a short last block are
// zero (the projection side clears them), so readers need no mask.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mfma_common.h"

namespace ttt {
namespace tb {

constexpr int SD = 64;      // head width
constexpr int SB = 16;      // scan positions per block (the mini-batch)
constexpr int RS = SD + 8;  // 72: padded row
constexpr int OFF_Q = 0, OFF_K = SB * RS, OFF_V = 2 * SB * RS;
constexpr int BLK = 3 * SB * RS;          // 3456 elements, 6912 bytes
constexpr int BLK_CHUNKS = BLK * 2 / 16;  // 432 chunks of 16 bytes
static_assert((BLK * 2) % 16 == 0, "block must be a whole number of 16-byte chunks");

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (__bf16)0.0f;
  return v;
}

// A K=32 matrix-core operand row of the staged block in the pair order: row c of
// panel `off`, features 32cc + 4g .. +3 and 32cc + 16 + 4g .. +3.
__device__ __forceinline__ bf16x8 rd_row8(const uint16_t* blk, int off, int g, int c, int cc) {
  const uint16_t* row = blk + off + c * RS + 32 * cc + 4 * g;
  const bf16x4 lo = *(const bf16x4*)row, hi = *(const bf16x4*)(row + 16);
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = lo[i];
    v[4 + i] = hi[i];
  }
  return v;
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element i mod 4 of the 8 bytes addressed by lanes
// i/4 + 4e (e = 0..3) of its group, as its element e.
__device__ __forceinline__ bf16x4 ld_tr(const void* lds_addr) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)lds_addr);
  return __builtin_bit_cast(bf16x4, v);
}

// Direct global -> LDS load of 16 bytes per lane: lane l writes LDS bytes
// [lds_base + 16 l, + 16) (lds_base wave-uniform).  Written as a statement of
// its own rather than through the compiler's builtin: the compiler makes every
// later LDS read of the destination array wait for all such loads in flight (it
// cannot tell the stages apart), which would expose their whole latency at the
// next read.  The statement has no output registers; callers wait for it
// explicitly (vmem_done) before the barrier that publishes the data.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(lds_base), "v"(src) : "memory", "m0");
}

// LDS byte address of a shared-memory pointer plus an offset, made wave-uniform
// (the offset must be the same in every lane of the wave).
__device__ __forceinline__ uint32_t lds_addr_uniform(const void* p, uint32_t off) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p) + off);
}

// tanh(u) = 1 - 2 / (exp(2u) + 1) (exact identity; saturates to +-1 for large |u|),
// used for the gate factors tanh(alpha).
__device__ __forceinline__ float tanh_gate(float u) {
  const float e = __builtin_amdgcn_exp2f(2.8853900817779268f * u);  // exp(2u)
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
}

}  // namespace tb
}  // namespace ttt
