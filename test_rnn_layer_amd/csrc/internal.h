// Internal interfaces between the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

// Projection: QKV = X theta^T for theta_Q, theta_K, theta_V.
struct ProjArgs {
  const void* X;      // [B, T, D] io dtype
  const void* theta;  // [3, D, D] io dtype, [out, in]
  void* out;          // layout depends on the kernel
  int64_t B, T;
  int32_t H, d;
  int32_t bf16;       // 1: X and theta are bf16, 0: fp32
  int32_t reverse;    // token-block layout only: blocks follow the reversed sequence
  int32_t blk_elems;  // token-block layout only: bf16 elements per 16-token block
  int64_t tt0, tt1;   // token-block GEMM only: tokens [tt0, tt1) of every sequence (others: 0, T)
  int32_t max_wg;     // token-block GEMM only: at most this many workgroups, each taking several
                      // tiles in turn (0: one workgroup per tile)
  int32_t n_out;      // row-major mode only: output columns N (theta is [N, D]); 0 elsewhere (N = 3 D)
  const void* resid;  // row-major mode only: bf16 [B*T, N] added to the product, or null
};

// fp32 output, [3, B, H, T, d] (VALU kernel, any dtype and shape).
hipError_t launch_project_f32out(const ProjArgs& a, hipStream_t s);

// bf16 MFMA GEMM; mode 0: fp32 [3, B, H, T, d]; mode 1: the MFMA scan's token blocks;
// mode 2: bf16 row-major [B*T, n_out] (+ resid).
bool project_mfma_supported(const ProjArgs& a);
hipError_t launch_project_mfma(const ProjArgs& a, int mode, hipStream_t s);
// Zeroes the rows past the end of each sequence's last token block (mode 1 layout).
hipError_t launch_zero_block_padding(const ProjArgs& a, hipStream_t s);

// One direction of the scan.
struct ScanArgs {
  const float* qkv;      // generic path: fp32 [3, B, H, T, d]
  const void* qkv_tiles; // MFMA path: bf16 tiled layout (see scan_mfma)
  const void* xin;       // [B, T, D] io dtype: gate input
  void* y;               // [B, T, D] io dtype: gated output (may equal xin)
  float* z;              // [B, T, D] fp32 or null
  const float* alpha;    // [D]
  const float* w1_0;     // [H, d, m], or per sequence (see w_seq_stride)
  const float* w2_0;     // [H, m, d], or per sequence
  int64_t w_seq_stride;  // elements between sequences' initial states (0: shared by all)
  float* wstate;         // workspace, [B, H, d*m + m*d] fp32 (generic path)
  uint64_t* xchg;        // cooperative path: exchange slots (see scan_coop)
  uint32_t* abort_flag;  // cooperative path: raised by a workgroup that timed out
  int32_t clear_abort;   // cooperative path: 1 clears abort_flag before the launch (the first
                         // launch of a call), 0 keeps it (a bidirectional call's reversed pass)
  float* w1_T;           // [B, H, d, m] or null
  float* w2_T;           // [B, H, m, d] or null
  int64_t B, T;
  int64_t p0, Tc;        // this launch covers scan positions [p0, p0 + Tc) (MFMA scan; others: 0, T)
  int32_t H, d, m, b;
  float eta;
  float gscale;          // 2/d (mean) or 2 (sum)
  int32_t gelu_tanh;     // 0: erf form, 1: tanh form
  int32_t reverse;
  int32_t bf16;          // io dtype of xin / y
  int32_t linear;        // 1: linear inner model f(u; W) = u W (W = w1, d x d; w2 unused)
  float* ckpt;           // forward pass for the backward only: the state (W1 then W2) at the
  int32_t ckpt_every;    // start of every ckpt_every-th mini-batch, [B, H, nseg, 2 d m],
  float* scratch;        // and its operand panels, scan_backward_scratch_elems per (sequence, head)
  float* seg_slots;      // segment replay only: [B, H, seg_stride, ckpt_every, slot] (see backward.hip)
  int64_t seg_lo;        // segment replay only: segments seg_lo .. seg_lo + seg_count - 1
  int32_t seg_count;
  int32_t seg_stride;    // segment replay only: slots of a chain in seg_slots (0: seg_count)
  // the forward pass on two parts per chain (its exchange entries, scan_fwd_f32_split_xchg_elems,
  // and abort flag in xchg and abort_flag): the parts' Z partials [2, B, T, D] (fp32)
  float* zpart;
};

// LDS bytes the generic scan needs for (d, m, b).
size_t scan_generic_lds_bytes(int d, int m, int b);
hipError_t launch_scan_generic(const ScanArgs& a, hipStream_t s);

// MFMA scan (d = 64, m = 256, b = 16, bf16 io).
bool scan_mfma_supported(int d, int m, int b);
size_t scan_mfma_tile_bytes(int64_t B, int64_t T, int H);
int scan_mfma_block_elems();
hipError_t launch_scan_mfma(const ScanArgs& a, hipStream_t s);

// Linear inner model.  MFMA scan: d = m = 64, b = 16, bf16 io (token blocks as for
// the MFMA scan); generic scan: any supported shape and dtype (fp32 Q/K/V).
bool scan_linear_mfma_supported(int d, int m, int b);
hipError_t launch_scan_linear_mfma(const ScanArgs& a, hipStream_t s);
size_t scan_linear_generic_lds_bytes(int d, int b);
hipError_t launch_scan_linear_generic(const ScanArgs& a, hipStream_t s);

// Cooperative per-token scan (d = 128, m = 512, b = 1): each head's state is
// split over 8 co-resident workgroups that exchange partial sums every token.
bool scan_coop_supported(int d, int m, int b, int64_t T);
bool scan_coop_fits(int64_t B, int H);  // co-residency on the current device
size_t scan_coop_xchg_bytes(int64_t B, int H);  // exchange slots
hipError_t launch_scan_coop(const ScanArgs& a, hipStream_t s);

// Backward of one direction of the MLP layer (generic, fp32): the backward scan
// (one workgroup per (sequence, head)) walks segments of ckpt_every
// mini-batches from the last, replaying each from its checkpoint.
constexpr int kBwdScratchPanels = 11;  // b x m fp32 panels per workgroup (plus dQ, dK)
struct BwdArgs {
  const float* qkv;    // [3, B, H, T, d] fp32: the direction's projections of its input
  const float* dy;     // [B, T, D] fp32: gradient of the direction's output Y
  const float* alpha;  // [D] the direction's gate
  const float* ckpt;   // [B, H, nseg, 2 d m]: written by the generic scan
  float* segst;        // [B, H, ckpt_every, segment elems] workspace: one segment's start states and
                       // forward quantities
  float* wcur;         // [B, H, 2 d m] workspace: replayed state
  float* dstate;       // [B, H, 2 d m] workspace: adjoint of the state
  float* scratch;      // workspace, scan_backward_scratch_elems per (sequence, head)
  float* dqkv;         // [B, T, 3 D] out: dQ | dK | dV per token
  float* dw_seq;       // [B, H, 2 d m] out: adjoint of the initial state, per sequence
  int64_t B, T;
  int32_t H, d, m, b, ckpt_every;
  float eta, gscale;
  int32_t gelu_tanh, reverse;
  // 1: the segments were replayed beforehand (launch_scan_replay_f32): this launch walks
  // segments seg_hi down to seg_lo from segst laid out [B, H, seg_count, ckpt_every, slot],
  // clearing the adjoint first when `first` is set and writing dw_seq when seg_lo is 0;
  // 0: one launch walks every segment, replaying each itself (segst: one segment per chain)
  int32_t replayed, first, seg_count;
  int64_t seg_lo, seg_hi;
  // the split backward scan only: exchange entries (scan_backward_split_xchg_elems, zero before a
  // direction's walk) and the abort flag; dqkv must be zero before the walk (dQ and dK are added)
  uint64_t* xchg;
  uint32_t* abort_flag;
  int32_t split;   // workgroups per chain: 2 or 4
  float* dqkv_b;   // four parts: [B, T, 2D], zero before the walk, added to dqkv's dQ|dK after it
                   // (by the bf16 split of the gradient GEMMs, else by launch_add_dqk)
};
// LDS bytes of the backward's scan kernels (the forward pass below too): the b x d and
// b x b panels, and the state when it fits beside them (at most 160 KB); workspace
// floats per workgroup (the b x m panels, dQ, dK)
size_t scan_backward_lds_bytes(int d, int m, int b);
size_t scan_backward_scratch_elems(int d, int m, int b);
// workspace floats per (sequence, head) and replayed mini-batch: the start state, then the
// forward quantities the replay keeps for the backward walk
size_t scan_backward_segment_elems(int d, int m, int b);
// The forward pass of one direction with the backward's own steps, writing Z, Y and
// the checkpoints (ScanArgs: qkv, xin, y, z, alpha, w1_0, w2_0, wstate, ckpt, scratch).
hipError_t launch_scan_fwd_ckpt(const ScanArgs& a, hipStream_t s);
// The same forward pass on the fp32 matrix cores with the state in registers (d = 64, m = 256,
// b = 16, erf GELU; ScanArgs: qkv, xin, y, z, alpha, w1_0, w2_0, ckpt, ckpt_every).
bool scan_fwd_f32_supported(int d, int m, int b);
hipError_t launch_scan_fwd_f32(const ScanArgs& a, hipStream_t s);
// The same steps replaying segments seg_lo .. seg_lo + seg_count - 1 of every (sequence, head)
// from their checkpoints (ScanArgs: qkv, ckpt, ckpt_every, seg_slots, seg_lo, seg_count): each
// mini-batch's slot gets its start state and forward quantities (scan_replay_f32_slot_elems
// floats, the layout scan_backward_segment_elems describes).
size_t scan_replay_f32_slot_elems();
// The forward pass split over two workgroups per chain (launch_scan_fwd_f32 with ScanArgs zpart set:
// one cooperative launch; xchg and abort_flag point at scan_fwd_f32_split_xchg_elems entries and a
// flag, zeroed before the launch), where 2 B H of them fit co-resident; launch_fwd_f32_gate then
// adds the parts' Z and writes Z and Y.
bool scan_fwd_f32_split_fits(int64_t B, int H);
size_t scan_fwd_f32_split_xchg_elems(int64_t B, int H);
hipError_t launch_fwd_f32_gate(const ScanArgs& a, hipStream_t s);
hipError_t launch_scan_replay_f32(const ScanArgs& a, hipStream_t s);
hipError_t launch_scan_backward(const BwdArgs& a, hipStream_t s);
// The replayed windows' walk with each chain's hidden units split over S co-resident workgroups
// (S = 4 or 2; one cooperative launch of S B H workgroups; the state and adjoint parts in LDS).
bool scan_backward_split_fits(int64_t B, int H, int d, int m, int b, int S);
size_t scan_backward_split_xchg_elems(int64_t B, int H, int d, int b, int S);
hipError_t launch_scan_backward_split(const BwdArgs& a, hipStream_t s);
hipError_t launch_add_dqk(float* dqkv, const float* buf, int64_t rows, int D, hipStream_t s);
hipError_t launch_zero_u64(uint64_t* p, int64_t n, hipStream_t s);
// C = (accumulate ? C : Cadd or 0) + A B, fp32 (A [M, K] row-major, or [K, M] when
// a_transposed; B [K, N] row-major, fp32 or bf16)
hipError_t launch_gemm_f32(bool a_transposed, bool b_bf16, const float* A, int64_t lda, const void* Bm, int64_t ldb,
                           float* C, int64_t ldc, const float* Cadd, int64_t M, int64_t N, int64_t K, int accumulate,
                           hipStream_t s);
// The same two gradient GEMMs on rocBLAS (grad_gemm.hip): dX [BT, D] = dY + dQKV [BT, 3D] theta
// [3D, D], and dtheta [3D, D] (+)= dQKV^T X [BT, D], all fp32 row-major.  slot 0: the caller's
// stream, 1: the side stream; ws: a workspace slice of grad_gemm_workspace_bytes() for that slot.
// Return NULL or rocBLAS's description of its error.
size_t grad_gemm_workspace_bytes();
const char* grad_gemm_dx(int slot, const float* dqkv, const float* theta32, const float* dy, float* dx, int64_t BT,
                         int64_t D, void* ws, size_t ws_bytes, hipStream_t s);
const char* grad_gemm_dtheta(int slot, const float* dqkv, const float* x32, float* dtheta, int64_t BT, int64_t D,
                             int accumulate, void* ws, size_t ws_bytes, hipStream_t s);
// With bf16 X and theta: S [BT, 9D] = the exact bf16 split [h | m | l] of dQKV [BT, 3D]
// (split_bf16x3; cols % 4 == 0; in2, if not null, [rows, cols2] is added to the first cols2
// columns of in before the split, cols2 % 4 == 0), theta3 [9D, D] = theta stacked three times
// (stack3_u16), and the same two GEMMs on the bf16 matrix cores with fp32 accumulation.
hipError_t split_bf16x3(const float* in, const float* in2, int64_t cols2, uint16_t* out, int64_t rows, int64_t cols,
                        hipStream_t s);
hipError_t stack3_u16(const uint16_t* in, uint16_t* out, int64_t n, hipStream_t s);
const char* grad_gemm_dx_split(int slot, const uint16_t* sp, const uint16_t* theta3, const float* dy, float* dx,
                               int64_t BT, int64_t D, void* ws, size_t ws_bytes, hipStream_t s);
// (p3: [9D, D] fp32 scratch for the three parts' products)
const char* grad_gemm_dtheta_split(int slot, const uint16_t* sp, const uint16_t* x16, float* dtheta, float* p3,
                                   int64_t BT, int64_t D, int accumulate, void* ws, size_t ws_bytes, hipStream_t s);
// dalpha[c] = (1 - tanh(alpha[c])^2) sum_r dy[r, c] z[r, c]; part: dalpha_partial_elems(D) floats
size_t dalpha_partial_elems(int D);
hipError_t launch_dalpha(const float* dy, const float* z, const float* alpha, float* part, float* dalpha,
                         int64_t rows, int D, hipStream_t s);
// dW1 [H, d, m], dW2 [H, m, d] (+)= sum over sequences of dw_seq [B, H, 2 d m]
hipError_t launch_sum_state(const float* dw_seq, float* dW1, float* dW2, int64_t B, int H, int d, int m,
                            int accumulate, hipStream_t s);

// Segment-local attention (head width 64, bf16): qkv [B, T, 3 D] (Q | K | V, head h at
// columns 64 h of each), out [B, T, D]; segments of L tokens (the last one shorter).
bool segment_attention_supported(int d);
hipError_t launch_segment_attention(const uint16_t* qkv, uint16_t* out, int64_t B, int64_t T, int H, int64_t L,
                                    hipStream_t s);

}  // namespace ttt
