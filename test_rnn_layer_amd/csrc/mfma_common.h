// Helpers shared by the MFMA kernels (gfx950).
//
// Lane layouts of the two bf16 matrix instructions used, for lane l of a
// 64-wide wavefront with g = l / 16 and c = l % 16:
//   v_mfma_f32_16x16x32_bf16:  A[c][8g .. 8g+7],  B[8g .. 8g+7][c],  D[4g .. 4g+3][c]
//   v_mfma_f32_16x16x16_bf16:  A[c][4g .. 4g+3],  B[4g .. 4g+3][c],  D[4g .. 4g+3][c]
// A 16x16 fp32 tile held in the D layout ("CL": lane holds rows 4g..4g+3 of
// column c) therefore feeds a K=16 operand directly when its rows are the
// contraction index, and two such tiles (rows 0-15 and 16-31 of a 32-deep
// slice) feed a K=32 operand if the other operand lists its contraction
// index in the same order: position 8g+i of a 32-slice holds index 4g+i for
// i < 4 and 16+4g+(i-4) for i >= 4 ("the pair order").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b), c,
                                                   0, 0, 0);
}

// Chains of dependent matrix-core products stay on one instruction: a 16x16x32
// result read as the accumulator of a 16x16x16 product a few instructions
// later, with no other matrix-core instruction between, gave wrong values in
// the first two result registers on gfx950, and the compiler inserts no wait for
// that case.  A K=16 product that accumulates onto a K=32 one is therefore done
// with the K=32 instruction: with A = {a0, a1} (two K=16 operands side by side)
// and B = {b, 0} the product is a0 b, with B = {0, b} it is a1 b.
__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = lo[i];
    v[4 + i] = hi[i];
  }
  return v;
}

__device__ __forceinline__ bf16x4 zero4b() {
  bf16x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (__bf16)0.0f;
  return v;
}

// Two floats as bf16 (round to nearest even), x in the low half: one conversion.
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  bf16x2 v;
  v[0] = (__bf16)x;
  v[1] = (__bf16)y;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x4 pack4(f32x4 x) {
  bf16x4 v;
  v[0] = (__bf16)x[0];
  v[1] = (__bf16)x[1];
  v[2] = (__bf16)x[2];
  v[3] = (__bf16)x[3];
  return v;
}

// Two D-layout tiles (rows 0-15 and 16-31 of a 32-deep slice) as one K=32 operand.
__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
  bf16x8 v;
  v[0] = (__bf16)lo[0];
  v[1] = (__bf16)lo[1];
  v[2] = (__bf16)lo[2];
  v[3] = (__bf16)lo[3];
  v[4] = (__bf16)hi[0];
  v[5] = (__bf16)hi[1];
  v[6] = (__bf16)hi[2];
  v[7] = (__bf16)hi[3];
  return v;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.0f, 0.0f, 0.0f, 0.0f}; }

// Wait until this wave's LDS stores have completed (lgkmcnt = 0) and keep the
// scheduler from moving anything across.  Used after storing matrix-core
// results to LDS: the store reads its data registers asynchronously, and a
// following MFMA that reuses those registers as its destination must not
// overwrite them first.
__device__ __forceinline__ void lds_stores_done() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt and expcnt unconstrained, lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
}

// Wait until this wave's vector-memory operations (including direct-to-LDS
// loads) have completed.
__device__ __forceinline__ void vmem_done() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt unconstrained
  __builtin_amdgcn_sched_barrier(0);
}

// Position of feature j inside a row stored in the pair order (32-slices).
__host__ __device__ __forceinline__ int pair_order_pos(int j) {
  const int jc = j & ~31, jl = j & 31;
  return jc + (jl < 16 ? 8 * (jl >> 2) + (jl & 3) : 8 * ((jl - 16) >> 2) + 4 + (jl & 3));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

}  // namespace ttt
