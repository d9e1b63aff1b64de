// Segment-local attention on the bf16 matrix cores: the hybrid block's step
// before the TTT layer ("One-Minute Video Generation with Test-Time Training",
// paper-notes page, framework section: self-attention stays within each
// 3-second segment, the TTT layer runs over the whole sequence).  For every
// segment [s L, (s+1) L) of every sequence and every head h (channels
// [64 h, 64 h + 64)):  O = softmax(Q K^T / sqrt(64)) V over the segment's keys,
// no causal mask.  bf16 Q, K, V and O, fp32 scores, softmax and accumulation.
//
// One 512-thread workgroup (8 waves) takes 128 QT queries of one segment and
// head; each wave owns QT tiles of 16 queries, which share every K and V
// fragment it reads from LDS.  Keys arrive in blocks of 128 (K and V
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
constexpr int QT = 2;            // 16-query tiles per wave: they share every K and V fragment read
constexpr int NW = 8;            // waves per workgroup
constexpr int AQ = NW * 16 * QT; // queries per workgroup
constexpr int AKB = 128;         // keys per block
constexpr int NT = AKB / 16;     // 16-key tiles per block
constexpr int ARS = 72;          // LDS row stride of K (bf16): 144-byte rows, conflict-free fragment reads
constexpr int VRS = AKB + 4;     // LDS row stride of V^T: 8 feature rows apart fall 16 banks apart
constexpr int A_THREADS = 64 * NW;
constexpr int SROWS = A_THREADS / 8;  // key rows staged per pass (8 threads per 128-byte row)
constexpr int A_STAGE = AKB * ARS + AD * VRS;  // bf16 elements of one stage: K rows, then V^T rows
constexpr int SCH = AKB / SROWS;  // 16-byte chunks of K (and of V) each thread stages per block
static_assert(SCH == 2, "V^T staging pairs two adjacent keys per thread");

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

  // this wave's queries (QT tiles of 16) as B operands (Q rows, 8 consecutive features per lane)
  int64_t myq[QT];
  bf16x8 qf0[QT], qf1[QT];
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    myq[u] = q0 + (w * QT + u) * 16 + c;
    const uint16_t* qrow = base + std::min(myq[u], n - 1) * row;
    qf0[u] = *(const bf16x8*)(qrow + 8 * g);
    qf1[u] = *(const bf16x8*)(qrow + 32 + 8 * g);
  }

  // staging: thread t moves SCH 16-byte chunks of K and of V per block, of the adjacent key rows
  // SCH sj + i, so that V^T takes their features two keys to a 32-bit LDS write
  const int sj = tid >> 3, sc = (tid & 7) * 8;  // key-row group of the block, feature chunk
  uint4 kreg[SCH], vreg[SCH];
  auto fetch = [&](int64_t kb) {
#pragma unroll
    for (int i = 0; i < SCH; ++i) {
      const int64_t key = std::min(kb * AKB + SCH * sj + i, n - 1);  // keys past the end load the last key
      const uint16_t* kr = base + key * row + D + sc;
      kreg[i] = *(const uint4*)kr;
      vreg[i] = *(const uint4*)(kr + D);
    }
  };
  auto stage = [&](int buf) {
    uint16_t* ks = smem + buf * A_STAGE;
    uint16_t* vt = ks + AKB * ARS;
#pragma unroll
    for (int i = 0; i < SCH; ++i) *(uint4*)(ks + (SCH * sj + i) * ARS + sc) = kreg[i];
    // V^T: feature rows, key columns; keys 2 sj and 2 sj + 1 of feature sc + e in one word
    const uint32_t* v0 = (const uint32_t*)&vreg[0];
    const uint32_t* v1 = (const uint32_t*)&vreg[1];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const uint32_t a = v0[e / 2], b = v1[e / 2];  // features sc + e (low half) and sc + e + 1
      *(uint32_t*)(vt + (sc + e) * VRS + SCH * sj) = (a & 0xffffu) | (b << 16);
      *(uint32_t*)(vt + (sc + e + 1) * VRS + SCH * sj) = (a >> 16) | (b & 0xffff0000u);
    }
  };

  const float qk_scale = 0.125f * 1.4426950408889634f;  // 1/sqrt(64) and log2(e): p = exp2(s c - m)
  float mrun[QT], lrun[QT];
  f32x4 o[QT][4];  // O^T: query tile u, feature tile dt, rows 4g..4g+3, query c
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    mrun[u] = -INFINITY;
    lrun[u] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[u][dt] = zero4();
  }
  const int64_t nkb = (n + AKB - 1) / AKB;
  fetch(0);
  stage(0);
  __syncthreads();
  for (int64_t kb = 0; kb < nkb; ++kb) {
    const int buf = (int)(kb & 1);
    if (kb + 1 < nkb) fetch(kb + 1);
    const uint16_t* ks = smem + buf * A_STAGE;
    const uint16_t* vt = ks + AKB * ARS;
    // S^T tiles: keys 16 t + 4g + r, query c of tile u
    f32x4 sc_[QT][NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint16_t* kr = ks + (t * 16 + c) * ARS;
      const bf16x8 k0 = *(const bf16x8*)(kr + 8 * g), k1 = *(const bf16x8*)(kr + 32 + 8 * g);
#pragma unroll
      for (int u = 0; u < QT; ++u) {
        sc_[u][t] = mfma32(k0, qf0[u], zero4());
        sc_[u][t] = mfma32(k1, qf1[u], sc_[u][t]);
      }
    }
    const int64_t kvalid = n - kb * AKB;
    if (kvalid < AKB) {  // the segment's last, short block: mask keys past its end
#pragma unroll
      for (int u = 0; u < QT; ++u)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (t * 16 + 4 * g + r >= kvalid) sc_[u][t][r] = -INFINITY;
    }
    bf16x8 pb[QT][NT / 2];
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      f32x4* s = sc_[u];
      // the block's maximum for this query
      float bm = -INFINITY;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) bm = fmaxf(bm, s[t][r]);
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      const float mnew = fmaxf(mrun[u], bm * qk_scale);
      // exponents are <= 0: the hardware exp2 (results below 2^-126 flush to 0, harmlessly)
      const float alpha = __builtin_amdgcn_exp2f(mrun[u] - mnew);  // 0 on the first block (mrun = -inf)
      mrun[u] = mnew;
      float ps = 0.0f;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[t][r], qk_scale, -mnew));
          s[t][r] = p;
          ps += p;
        }
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      lrun[u] = lrun[u] * alpha + ps;
      if (__any(alpha != 1.0f)) {  // once the maxima settle, most blocks leave them unchanged
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[u][dt] *= alpha;
      }
      // keys of a K=32 chunk in pair order: tiles 2k (4g..4g+3) and 2k+1
#pragma unroll
      for (int k2 = 0; k2 < NT / 2; ++k2) pb[u][k2] = pack8(s[2 * k2], s[2 * k2 + 1]);
    }
    // O^T += V^T P^T
#pragma unroll
    for (int k2 = 0; k2 < NT / 2; ++k2)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const uint16_t* vr = vt + (dt * 16 + c) * VRS + 32 * k2 + 4 * g;
        const bf16x8 v8 = cat8(*(const bf16x4*)vr, *(const bf16x4*)(vr + 16));
#pragma unroll
        for (int u = 0; u < QT; ++u) o[u][dt] = mfma32(v8, pb[u][k2], o[u][dt]);
      }
    if (kb + 1 < nkb) stage(buf ^ 1);
    __syncthreads();
  }
  // O[query c][feature 16 dt + 4g + r] = O^T / l
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    if (myq[u] >= n) continue;
    const float inv = 1.0f / lrun[u];
    uint16_t* orow = out + (b * T + s0 + myq[u]) * D + (int64_t)h * AD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      uint2 v;
      v.x = pack2(o[u][dt][0] * inv, o[u][dt][1] * inv);
      v.y = pack2(o[u][dt][2] * inv, o[u][dt][3] * inv);
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
