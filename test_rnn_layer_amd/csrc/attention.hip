// Segment-local attention on the bf16 matrix cores: the hybrid block's step
// before the TTT layer ("One-Minute Video Generation with Test-Time Training",
// paper-notes page, framework section: self-attention stays within each
// 3-second segment, the TTT layer runs over the whole sequence).  For every
// segment [s L, (s+1) L) of every sequence and every head h (channels
// [64 h, 64 h + 64)):  O = softmax(Q K^T / sqrt(64)) V over the segment's keys,
// no causal mask.  bf16 Q, K, V and O, fp32 scores, softmax and accumulation.
//
// One 512-thread workgroup (8 waves) takes 128 queries of one segment and
// head; each wave owns 16 queries.  Keys arrive in blocks of 64 (K and V
// staged through two LDS buffers, the next block's rows held in registers
// while this block computes).  A wave computes the transposed scores
// S^T = K Q^T (keys x its 16 queries), so that each lane holds scores of one
// query: the online softmax (running maximum and sum) is lane-local up to a
// reduction over the four lanes that share the query, and the products
// O^T += V^T P^T take the lane's own probabilities as their operand (the key
// index in "pair order", see mfma_common.h; V is staged transposed to match).
#include <algorithm>

#include "internal.h"
#include "mfma_common.h"

namespace ttt {
namespace {

constexpr int AD = 64;           // head width
constexpr int AQ = 128;          // queries per workgroup (8 waves x 16)
constexpr int AKB = 64;          // keys per block
constexpr int ARS = 72;          // LDS row stride (bf16): 144-byte rows, conflict-free fragment reads
constexpr int A_THREADS = 512;
constexpr int A_STAGE = 2 * AKB * ARS;  // bf16 elements of one stage: K rows, then V^T rows

__global__ __launch_bounds__(A_THREADS) void segment_attention_kernel(const uint16_t* __restrict__ qkv,
                                                                     uint16_t* __restrict__ out, int64_t T, int H,
                                                                     int64_t L, int64_t nseg, int nq, int64_t units) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * A_STAGE];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  // workgroup -> (unit = sequence, segment, head; query tile): the query tiles of one
  // unit go to one XCD (blockIdx mod 8), where they share the unit's K and V in L2
  const int64_t slot = blockIdx.x / 8, xcd = blockIdx.x % 8;
  const int64_t unit = (slot / nq) * 8 + xcd;
  const int qt = (int)(slot % nq);
  if (unit >= units) return;
  const int h = (int)(unit % H);
  const int64_t seg = (unit / H) % nseg, b = unit / ((int64_t)H * nseg);
  const int64_t s0 = seg * L, s1 = std::min(T, s0 + L), n = s1 - s0;
  const int64_t q0 = (int64_t)qt * AQ;
  if (q0 >= n) return;
  const int64_t D = (int64_t)H * AD, row = 3 * D;
  const uint16_t* base = qkv + (b * T + s0) * row + (int64_t)h * AD;  // Q of the segment's token 0, head h

  // this wave's 16 queries as the B operand (Q rows, 8 consecutive features per lane)
  const int64_t myq = q0 + w * 16 + c;
  const uint16_t* qrow = base + std::min(myq, n - 1) * row;
  const bf16x8 qf0 = *(const bf16x8*)(qrow + 8 * g);
  const bf16x8 qf1 = *(const bf16x8*)(qrow + 32 + 8 * g);

  // staging: thread t moves one 16-byte chunk of K and one of V per block
  const int sj = tid >> 3, sc = (tid & 7) * 8;  // key row 0..63 of the block, feature chunk
  uint4 kreg, vreg;
  auto fetch = [&](int64_t kb) {
    const int64_t key = std::min(kb * AKB + sj, n - 1);  // keys past the end load the last key (masked)
    const uint16_t* kr = base + key * row + D + sc;
    kreg = *(const uint4*)kr;
    vreg = *(const uint4*)(kr + D);
  };
  auto stage = [&](int buf) {
    uint16_t* ks = smem + buf * A_STAGE;
    uint16_t* vt = ks + AKB * ARS;
    *(uint4*)(ks + sj * ARS + sc) = kreg;
    const uint16_t* v = (const uint16_t*)&vreg;
#pragma unroll
    for (int i = 0; i < 8; ++i) vt[(sc + i) * ARS + sj] = v[i];  // V^T: feature rows, key columns
  };

  const float qk_scale = 0.125f * 1.4426950408889634f;  // 1/sqrt(64) and log2(e): p = exp2(s c - m)
  float mrun = -INFINITY, lrun = 0.0f;
  f32x4 o[4] = {zero4(), zero4(), zero4(), zero4()};  // O^T: feature tile dt, rows 4g..4g+3, query c
  const int64_t nkb = (n + AKB - 1) / AKB;
  fetch(0);
  stage(0);
  __syncthreads();
  for (int64_t kb = 0; kb < nkb; ++kb) {
    const int buf = (int)(kb & 1);
    if (kb + 1 < nkb) fetch(kb + 1);
    const uint16_t* ks = smem + buf * A_STAGE;
    const uint16_t* vt = ks + AKB * ARS;
    // S^T tiles: keys 16 t + 4g + r, query c
    f32x4 s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint16_t* kr = ks + (t * 16 + c) * ARS;
      s[t] = mfma32(*(const bf16x8*)(kr + 8 * g), qf0, zero4());
      s[t] = mfma32(*(const bf16x8*)(kr + 32 + 8 * g), qf1, s[t]);
    }
    // mask keys past the segment's end, then the block's maximum for this query
    const int64_t kvalid = n - kb * AKB;
    float bm = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (t * 16 + 4 * g + r >= kvalid) s[t][r] = -INFINITY;
        bm = fmaxf(bm, s[t][r]);
      }
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float mnew = fmaxf(mrun, bm * qk_scale);
    const float alpha = exp2f(mrun - mnew);  // 0 on the first block (mrun = -inf)
    mrun = mnew;
    float ps = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2f(fmaf(s[t][r], qk_scale, -mnew));
        s[t][r] = p;
        ps += p;
      }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    lrun = lrun * alpha + ps;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    // O^T += V^T P^T, keys of the K=32 chunk in pair order: tiles 2k (4g..4g+3) and 2k+1
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const bf16x8 pb = pack8(s[2 * k2], s[2 * k2 + 1]);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const uint16_t* vr = vt + (dt * 16 + c) * ARS + 32 * k2 + 4 * g;
        const bf16x4 lo = *(const bf16x4*)vr;
        const bf16x4 hi = *(const bf16x4*)(vr + 16);
        o[dt] = mfma32(cat8(lo, hi), pb, o[dt]);
      }
    }
    if (kb + 1 < nkb) stage(buf ^ 1);
    __syncthreads();
  }
  // O[query c][feature 16 dt + 4g + r] = O^T / l
  if (myq < n) {
    const float inv = 1.0f / lrun;
    uint16_t* orow = out + (b * T + s0 + myq) * D + (int64_t)h * AD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      uint2 v;
      v.x = pack2(o[dt][0] * inv, o[dt][1] * inv);
      v.y = pack2(o[dt][2] * inv, o[dt][3] * inv);
      *(uint2*)(orow + dt * 16 + 4 * g) = v;
    }
  }
}

}  // namespace

bool segment_attention_supported(int d) { return d == AD; }

hipError_t launch_segment_attention(const uint16_t* qkv, uint16_t* out, int64_t B, int64_t T, int H, int64_t L,
                                    hipStream_t s) {
  if (B == 0 || T == 0) return hipSuccess;
  const int64_t nseg = (T + L - 1) / L;
  const int nq = (int)((std::min(L, T) + AQ - 1) / AQ);
  const int64_t units = B * nseg * H;
  const int64_t grid = (units + 7) / 8 * 8 * nq;
  hipLaunchKernelGGL(segment_attention_kernel, dim3((unsigned)grid), dim3(A_THREADS), 0, s, qkv, out, T, H, L, nseg,
                     nq, units);
  return hipGetLastError();
}

}  // namespace ttt
