// Projection GEMM on the bf16 matrix cores: Q|K|V = X [theta_Q; theta_K; theta_V]^T
// ("One-Minute Video Generation with Test-Time Training", paper-notes page,
// key designs, "TTT-MLP layer": theta_K, theta_V, theta_Q are learned like
// attention's K, V, Q).  X is [B*T, D] and theta [3D, D], both with the
// contraction index contiguous, so both operands are loaded the same way.
//
// Tiling: 128 x 128 output tile per 256-thread workgroup (2 x 2 waves of
// 64 x 64), K-steps of 64 staged through double-buffered LDS (rows padded to
// 144 bytes: the 16 rows read by one 16-lane group land on distinct banks),
// fp32 accumulation in v_mfma_f32_16x16x32_bf16.
//
// Three epilogues: fp32 [3, B, H, T, d] (inspection / generic scan), the
// bf16 token-block layout the MFMA scan reads (see scan_mfma.hip), and plain
// row-major bf16 [B*T, N] with an optional bf16 residual of the same shape
// added in fp32 (the hybrid block's attention projections; N = n_out).
#include <algorithm>
#include <cmath>

#include "internal.h"
#include "mfma_common.h"

namespace ttt {
namespace {

constexpr int BM = 128, BN = 128, BK = 64, LDK = BK + 8;

__device__ __forceinline__ uint16_t to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

template <int MODE>
__global__ __launch_bounds__(256) void proj_mfma_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDK];
  const int d = a.d;
  const int D = a.H * d;
  const int64_t M = a.B * a.T;
  const int N = a.n_out > 0 ? a.n_out : 3 * D;
  const int K = D;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.x * BM;
  const int n0 = blockIdx.y * BN;
  const uint16_t* X = (const uint16_t*)a.X;
  const uint16_t* Th = (const uint16_t*)a.theta;

  uint4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i, row = q >> 3, kc = (q & 7) * 8;
      const int64_t gr = m0 + row;
      const int gn = n0 + row;
      const bool kin = k0 + kc < K;
      ra[i] = (gr < M && kin) ? *(const uint4*)(X + gr * K + k0 + kc) : uint4{0, 0, 0, 0};
      rb[i] = (gn < N && kin) ? *(const uint4*)(Th + (int64_t)gn * K + k0 + kc) : uint4{0, 0, 0, 0};
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i, row = q >> 3, kc = (q & 7) * 8;
      *(uint4*)(&As[buf][row * LDK + kc]) = ra[i];
      *(uint4*)(&Bs[buf][row * LDK + kc]) = rb[i];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero4();

  gload(0);
  sstore(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < K; k0 += BK) {
    const bool more = k0 + BK < K;
    if (more) gload(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        af[t] = *(const bf16x8*)(&As[buf][(wm * 64 + t * 16 + c) * LDK + kk + 8 * g]);
        bfr[t] = *(const bf16x8*)(&Bs[buf][(wn * 64 + t * 16 + c) * LDK + kk + 8 * g]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    if (more) sstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // epilogue: lane holds rows m0 + wm*64 + i*16 + 4g + r, column n0 + wn*64 + j*16 + c
  const int64_t nblk = (a.T + 15) / 16;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = n0 + wn * 64 + j * 16 + c;
    if (col >= N) continue;
    if (MODE == 2) {
      uint16_t* out = (uint16_t*)a.out;
      const uint16_t* res = (const uint16_t*)a.resid;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t row = m0 + wm * 64 + i * 16 + 4 * g + r;
          if (row >= M) continue;
          float v = acc[i][j][r];
          if (res) v += bf16_to_f32(res[row * N + col]);
          out[row * N + col] = to_bf16_bits(v);
        }
      continue;
    }
    const int p = col / D, rem = col - p * D, h = rem / d, jj = rem - h * d;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wm * 64 + i * 16 + 4 * g + r;
        if (row >= M) continue;
        const int64_t s = row / a.T, t = row - s * a.T;
        const float v = acc[i][j][r];
        if (MODE == 0) {
          float* out = (float*)a.out;
          out[((((int64_t)p * a.B + s) * a.H + h) * a.T + t) * d + jj] = v;
        } else {
          uint16_t* out = (uint16_t*)a.out;
          const int64_t pos = a.reverse ? a.T - 1 - t : t;
          const int64_t jb = pos >> 4;
          const int tl = (int)(pos & 15);
          // token block of the MFMA scan (d = 64): Q, K, V rows of 72
          uint16_t* blk = out + (((int64_t)s * a.H + h) * nblk + jb) * (int64_t)a.blk_elems;
          blk[(p * 16 + tl) * 72 + jj] = to_bf16_bits(v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Token-block projection for the MFMA scan: 256 x 256 output tiles per
// 512-thread workgroup (2 x 4 waves of 128 x 64), K-steps of 64 staged by
// direct global -> LDS loads into two buffers (the next step loads while this
// one computes).  Each step reads both 32-deep halves of its operands from LDS
// up front, the second half's reads spread over the first half's products, so
// the matrix cores do not wait on LDS inside a step.  LDS rows are 128 bytes
// with the 16-byte chunks XOR-swizzled by (row / 2) mod 8, so the 16 rows one
// 16-lane group reads hit 16 distinct bank groups.  Tiles are grouped group_m (M) x
// all (N) and handed out per XCD so the workgroups resident on one XCD share A
// and theta slices in its L2; a workgroup takes the tiles of its XCD's range
// in turn.  Rows past the end of X load its last row (never stored), so every
// step issues the same loads.  The epilogue stages each wave's 128 x 64 bf16
// sub-tile through LDS and writes whole 128-byte token rows of the scan's
// token blocks, or (row-major mode) 128-byte row pieces of [B*T, N] with the
// residual added; in the fp32 mode (mode 0, [3, B, H, T, d] with d a multiple
// of 64) each lane stores its accumulators directly, 64-byte row pieces.
// ---------------------------------------------------------------------------
constexpr int T_BM = 256, T_BN = 256, T_BK = 64, T_THREADS = 512;
constexpr int T_STAGE = (T_BM + T_BN) * T_BK;  // bf16 elements per stage (64 KB)
constexpr int TOK_RS = 72;                     // row stride of a token block (bf16)

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

__global__ __launch_bounds__(T_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void proj_tiles_kernel(
    ProjArgs a, int mtiles, int ntiles, int group_m, int mode) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T_STAGE];
  const int d = a.d;
  const int D = a.H * d;
  const int64_t Tw = a.tt1 - a.tt0;  // tokens [tt0, tt1) of every sequence: GEMM row r is token
  const int64_t M = a.B * Tw;        // tt0 + r mod Tw of sequence r / Tw
  const int N = a.n_out > 0 ? a.n_out : 3 * D;
  const int K = D;
  const int tid = threadIdx.x, lane_ = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 2, wn = w & 3;

  // tiles: XCD-contiguous ranges (workgroup b runs on XCD b mod 8), grouped group_m
  // m-tiles at a time; the workgroups of an XCD take its range in turn
  const int total = mtiles * ntiles;
  const int per_xcd = (total + 7) / 8;
  const int slots = (int)(gridDim.x / 8);
  for (int ti = (int)(blockIdx.x / 8); ti < per_xcd; ti += slots) {
    const int t = (int)(blockIdx.x % 8) * per_xcd + ti;
    if (t >= total) break;
    // lane-derived addresses are recomputed per tile: hoisted out of the tile
    // loop they would stay live across it and spill
    int lane = lane_, g = lane_ >> 4, c = lane_ & 15;
    asm volatile("" : "+v"(lane), "+v"(g), "+v"(c));
    const int group = t / (group_m * ntiles);
    const int first_m = group * group_m;
    const int gm = min(mtiles - first_m, group_m);
    const int rem = t - group * group_m * ntiles;
    const int mt = first_m + rem % gm;
    const int nt = rem / gm;
    const int64_t m0 = (int64_t)mt * T_BM;
    const int n0 = nt * T_BN;
    const uint16_t* X = (const uint16_t*)a.X;
    const uint16_t* Th = (const uint16_t*)a.theta;

    // direct loads of one K-step: per matrix 256 rows x 8 chunks; instruction i of
    // wave w fills LDS rows 8 (8 i + w) .. +8, lane -> row + lane / 8, chunk lane % 8
    int64_t xrow[4];  // X row of this lane's A rows (rows past the end load the last row, never stored)
  #pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t ga = min(m0 + 8 * (8 * i + w) + (lane >> 3), M - 1);
      xrow[i] = (ga / Tw) * a.T + a.tt0 + ga % Tw;
    }
    auto issue = [&](int k0, int buf) {
      uint16_t* base = smem + buf * T_STAGE;
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 8 * (8 * i + w) + (lane >> 3);
        const int gch = swz(row, lane & 7);
        uint16_t* ldsA = base + (8 * (8 * i + w)) * T_BK;
        uint16_t* ldsB = base + T_BM * T_BK + (8 * (8 * i + w)) * T_BK;
        const int gb = min(n0 + row, N - 1);
        __builtin_amdgcn_global_load_lds((const void*)(X + xrow[i] * K + k0 + 8 * gch),
                                         (__attribute__((address_space(3))) void*)ldsA, 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(Th + (int64_t)gb * K + k0 + 8 * gch),
                                           (__attribute__((address_space(3))) void*)ldsB, 16, 0, 0);
      }
    };

    f32x4 acc[8][4];
  #pragma unroll
    for (int i = 0; i < 8; ++i)
  #pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = zero4();

    const int nk = K / T_BK;
    issue(0, 0);
    for (int ks = 0; ks < nk; ++ks) {
      vmem_done();  // this wave's loads of step ks have landed
      __syncthreads();  // ... everyone's, and everyone is done with step ks - 1
      if (ks + 1 < nk) issue((ks + 1) * T_BK, (ks + 1) & 1);
      const uint16_t* As = smem + (ks & 1) * T_STAGE;
      const uint16_t* Bs = As + T_BM * T_BK;
      bf16x8 af[2][8], bfr[2][4];
  #pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
  #pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = wm * 128 + i * 16 + c;
          af[kk][i] = *(const bf16x8*)(As + row * T_BK + 8 * swz(row, 4 * kk + g));
        }
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = wn * 64 + j * 16 + c;
          bfr[kk][j] = *(const bf16x8*)(Bs + row * T_BK + 8 * swz(row, 4 * kk + g));
        }
      }
  #pragma unroll
      for (int kk = 0; kk < 2; ++kk)
  #pragma unroll
        for (int i = 0; i < 8; ++i)
  #pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[kk][i], bfr[kk][j], acc[i][j]);
      // the first half's operands, then the second half's reads spread over the first half's products
      __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
  #pragma unroll
      for (int q = 0; q < 12; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 40, 0);
    }

    // ---- epilogue, fp32 mode: the 64 columns of this wave are features jj0 .. jj0 + 63
    //      of one head and one of Q, K, V
    __syncthreads();
    if (mode == 0) {
      const int col0 = n0 + wn * 64;
      if (col0 < N) {
        const int p = col0 / D, hh = (col0 - p * D) / d, jj0 = (col0 - p * D) - hh * d;
        float* out = (float*)a.out;
  #pragma unroll
        for (int i = 0; i < 8; ++i)
  #pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t grow = m0 + wm * 128 + i * 16 + 4 * g + r;
            if (grow >= M) continue;
            const int64_t sq = grow / Tw, tt = a.tt0 + (grow - sq * Tw);
            float* o = out + ((((int64_t)p * a.B + sq) * a.H + hh) * a.T + tt) * d + jj0 + c;
  #pragma unroll
            for (int j = 0; j < 4; ++j) o[16 * j] = acc[i][j][r];
          }
      }
      continue;  // the stages were last read before the barrier above
    }
    // ---- epilogue: this wave's 128 x 64 sub-tile as bf16 rows in LDS, then 16-byte stores
    uint16_t* ctile = smem + w * (128 * 64);
  #pragma unroll
    for (int i = 0; i < 8; ++i)
  #pragma unroll
      for (int j = 0; j < 4; ++j)
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = i * 16 + 4 * g + r, col = j * 16 + c;
          ctile[row * 64 + 8 * swz(row, col >> 3) + (col & 7)] = __builtin_bit_cast(uint16_t, (__bf16)acc[i][j][r]);
        }
    lds_stores_done();
    __builtin_amdgcn_wave_barrier();
    const int col0 = n0 + wn * 64;
    if (a.n_out > 0) {
      // row-major bf16 [M, N], plus the residual
      uint16_t* out = (uint16_t*)a.out;
      const uint16_t* res = (const uint16_t*)a.resid;
  #pragma unroll 4
      for (int it = 0; it < 16; ++it) {
        const int q = it * 64 + lane;
        const int row = q >> 3, ch = q & 7;
        const int64_t grow = m0 + wm * 128 + row;
        if (grow >= M || col0 + 8 * ch >= N) continue;
        uint4 v = *(const uint4*)(ctile + row * 64 + 8 * swz(row, ch));
        if (res) {
          const uint4 rv = *(const uint4*)(res + grow * N + col0 + 8 * ch);
          const uint16_t* a16 = (const uint16_t*)&v;
          const uint16_t* r16 = (const uint16_t*)&rv;
          uint16_t o16[8];
  #pragma unroll
          for (int e = 0; e < 8; ++e) o16[e] = to_bf16_bits(bf16_to_f32(a16[e]) + bf16_to_f32(r16[e]));
          v = *(const uint4*)o16;
        }
        *(uint4*)(out + grow * N + col0 + 8 * ch) = v;
      }
    } else if (col0 < N) {
      const int p = col0 / D, h = (col0 - p * D) / d;
      const int64_t nblk = (a.T + 15) / 16;
      uint16_t* out = (uint16_t*)a.out;
  #pragma unroll 4
      for (int it = 0; it < 16; ++it) {
        const int q = it * 64 + lane;
        const int row = q >> 3, ch = q & 7;
        const int64_t grow = m0 + wm * 128 + row;
        if (grow >= M) continue;
        const uint4 v = *(const uint4*)(ctile + row * 64 + 8 * swz(row, ch));
        const int64_t s = grow / Tw, tt = a.tt0 + (grow - s * Tw);
        const int64_t pos = a.reverse ? a.T - 1 - tt : tt;
        uint16_t* blk = out + (((int64_t)s * a.H + h) * nblk + (pos >> 4)) * (int64_t)a.blk_elems;
        *(uint4*)(blk + (p * 16 + (int)(pos & 15)) * TOK_RS + 8 * ch) = v;
      }
    }
    __syncthreads();  // every wave has read its sub-tile before the next tile's loads reuse the stages
  }
}

// Rows of the last token block past the end of the sequence (T mod 16 of
// them valid): zero in all three panels, so that the scan reads them
// unmasked.  One workgroup per (sequence, head).
__global__ void zero_block_padding_kernel(uint16_t* out, int64_t T, int H, int blk_elems) {
  const int n = (int)(T & 15);
  const int64_t nblk = (T + 15) / 16;
  uint16_t* blk = out + ((int64_t)blockIdx.x * nblk + nblk - 1) * blk_elems;
  const int rows = 16 - n;  // per panel
  for (int i = threadIdx.x; i < 3 * rows * TOK_RS; i += blockDim.x) {
    const int p = i / (rows * TOK_RS), r = n + (i / TOK_RS) % rows, col = i % TOK_RS;
    blk[(p * 16 + r) * TOK_RS + col] = 0;
  }
}

}  // namespace

hipError_t launch_zero_block_padding(const ProjArgs& a, hipStream_t s) {
  if (a.T % 16 == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_block_padding_kernel, dim3((unsigned)(a.B * a.H)), dim3(256), 0, s, (uint16_t*)a.out, a.T,
                     a.H, a.blk_elems);
  return hipGetLastError();
}

bool project_mfma_supported(const ProjArgs& a) { return a.bf16 && (a.H * a.d) % 8 == 0; }

hipError_t launch_project_mfma(const ProjArgs& a, int mode, hipStream_t s) {
  const int N = 3 * a.H * a.d;
  // fp32 output (mode 0, d a multiple of 64), token blocks (mode 1, d = 64) and row-major output
  // (mode 2, N a multiple of 8) on the 256 x 256 tiles
  if (((mode == 0 && a.n_out <= 0 && a.d % 64 == 0) || (mode == 1 && a.n_out <= 0 && a.d == 64) ||
       (mode == 2 && a.n_out % 8 == 0)) &&
      (a.H * a.d) % T_BK == 0) {
    const int64_t M = a.B * (a.tt1 - a.tt0);
    if (M == 0) return hipSuccess;
    const int Nt = mode == 2 ? a.n_out : N;
    const int mtiles = (int)((M + T_BM - 1) / T_BM), ntiles = (Nt + T_BN - 1) / T_BN;
    const int total = mtiles * ntiles;
    int grid = (total + 7) / 8 * 8;
    if (a.max_wg > 0) grid = std::min(grid, std::max(8, a.max_wg / 8 * 8));
    // the tiles an XCD runs at once (one workgroup per CU, 32 CUs per XCD) span
    // group_m m-tiles x (that many / group_m) n-tiles: about square, so they
    // share the fewest A and theta slices in the XCD's L2
    const int resident = std::min(grid / 8, 32);
    const int group_m = std::max(1, std::min(8, (int)std::lround(std::sqrt((double)resident))));
    hipLaunchKernelGGL(proj_tiles_kernel, dim3((unsigned)grid), dim3(T_THREADS), 0, s, a, mtiles, ntiles, group_m,
                       mode);
    return hipGetLastError();
  }
  if (a.tt0 != 0 || a.tt1 != a.T) return hipErrorInvalidValue;  // the other kernels cover whole sequences
  const int64_t M = a.B * a.T;
  if (M == 0) return hipSuccess;
  const int Nk = a.n_out > 0 ? a.n_out : N;
  dim3 grid((unsigned)((M + BM - 1) / BM), (unsigned)((Nk + BN - 1) / BN));
  if (mode == 0)
    hipLaunchKernelGGL(proj_mfma_kernel<0>, grid, dim3(256), 0, s, a);
  else if (mode == 1)
    hipLaunchKernelGGL(proj_mfma_kernel<1>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(proj_mfma_kernel<2>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ttt
