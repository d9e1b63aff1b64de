// Shader-clock marks at the phase boundaries of a scan's steps, for measuring
// where a step's time goes.  Only the measurement build defines TTT_PHASE_MARKS
// (python -m test_rnn_layer_amd.build --phase-marks, which writes
// libttt_mlp_marks.so); in the library itself every mark compiles to nothing.
//
// With marks, lane 0 of wave 0 of workgroup 0 stores the 64-bit shader clock
// (s_memtime) when it passes mark p of step j, for kMarkSteps steps from step
// kMarkFirst of every launch (a later launch overwrites an earlier one's marks).
// The store waits for the clock read; that wait is what the marks cost.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {
constexpr int kMarkFirst = 32;    // skip the first steps of a launch (staging fills)
constexpr int kMarkSteps = 256;   // steps recorded per launch
constexpr int kMarkPhases = 8;    // marks per step
}  // namespace ttt

#ifdef TTT_PHASE_MARKS
#define TTT_MARKS_BUFFER(name) __device__ uint64_t name[ttt::kMarkSteps * ttt::kMarkPhases]
#define TTT_MARK(buf, step, phase)                                                                    \
  do {                                                                                                \
    const int64_t mk_j_ = (int64_t)(step) - ttt::kMarkFirst;                                          \
    if (blockIdx.x == 0 && threadIdx.x == 0 && mk_j_ >= 0 && mk_j_ < ttt::kMarkSteps)                 \
      buf[mk_j_ * ttt::kMarkPhases + (phase)] = __builtin_amdgcn_s_memtime();                          \
  } while (0)
// Host side: copies a kernel's marks ([kMarkSteps][kMarkPhases] clock values) out of
// its device buffer after the launches have finished.
#define TTT_MARKS_EXPORT(fn, buf)                                                                      \
  extern "C" int32_t fn(uint64_t* out, int64_t n) {                                                   \
    if (!out || n < (int64_t)ttt::kMarkSteps * ttt::kMarkPhases) return -1;                           \
    return hipMemcpyFromSymbol(out, HIP_SYMBOL(buf), sizeof(uint64_t) * ttt::kMarkSteps * ttt::kMarkPhases, 0, \
                               hipMemcpyDeviceToHost) == hipSuccess ? 0 : -4;                         \
  }
#else
#define TTT_MARKS_BUFFER(name) static_assert(true, "")
#define TTT_MARK(buf, step, phase) \
  do {                             \
  } while (0)
#define TTT_MARKS_EXPORT(fn, buf) static_assert(true, "")
#endif
