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
// Two epilogues: fp32 [3, B, H, T, d] (inspection / generic scan) and the
// bf16 token-block layout the MFMA scan reads (see scan_mfma.hip).
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
  const int N = 3 * D;
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

}  // namespace

bool project_mfma_supported(const ProjArgs& a) { return a.bf16 && (a.H * a.d) % 8 == 0; }

hipError_t launch_project_mfma(const ProjArgs& a, int mode, hipStream_t s) {
  const int64_t M = a.B * a.T;
  const int N = 3 * a.H * a.d;
  if (M == 0) return hipSuccess;
  dim3 grid((unsigned)((M + BM - 1) / BM), (unsigned)((N + BN - 1) / BN));
  if (mode == 0)
    hipLaunchKernelGGL(proj_mfma_kernel<0>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(proj_mfma_kernel<1>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ttt
