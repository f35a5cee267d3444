// Timeline hooks of the measurement build (built with -DFH_TRACE by
// `python -m two_stage_retrieval_amd.build --trace` into
// libflashhead_trace.so; empty in the library itself).
//
// The hooks store timestamps into a device array of the translation unit
// that includes this header; flashhead_trace_read (fh_stage1.hip) copies the
// single-launch decode's array to the host.  Cross-workgroup events use the
// constant-rate device clock (s_memrealtime, the wall-clock rate the device
// reports); the selection's phases, which run on one compute unit, also get
// shader-clock cycles (s_memtime).
//   FH_TRACE_BLOCK(ev)   thread 0 of the workgroup: block event ev
//   FH_TRACE_WAVE(ev)    lane 0 of each wave: wave event ev
//   FH_TRACE_SEL(i)      thread 0: selection phase i
//   FH_TRACE_COUNT(i, n) thread 0: counter i = n
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fh {

constexpr int kTraceBlockEvents = 8;
constexpr int kTraceMaxBlocks = 512;
constexpr int kTraceWaveEvents = 4;
constexpr int kTraceMaxWaves = kTraceMaxBlocks * 16;
constexpr int kTraceSelPhases = 16;
constexpr int kTraceCounters = 16;
constexpr int64_t kTraceWaveOff = (int64_t)kTraceBlockEvents * kTraceMaxBlocks;
constexpr int64_t kTraceSelOff = kTraceWaveOff + (int64_t)kTraceWaveEvents * kTraceMaxWaves;
constexpr int64_t kTraceCountOff = kTraceSelOff + 2 * kTraceSelPhases;
constexpr int64_t kTraceWords = kTraceCountOff + kTraceCounters;

}  // namespace fh

#ifdef FH_TRACE
namespace fh {
static __device__ uint64_t fh_trace_buf[kTraceWords];
}
#define FH_TRACE_BLOCK(ev)                                                              \
  do {                                                                                  \
    if (threadIdx.x == 0 && blockIdx.x < ::fh::kTraceMaxBlocks)                         \
      ::fh::fh_trace_buf[(ev) * ::fh::kTraceMaxBlocks + blockIdx.x] =                   \
          __builtin_amdgcn_s_memrealtime();                                             \
  } while (0)
#define FH_TRACE_WAVE(ev)                                                               \
  do {                                                                                  \
    const uint32_t w_ = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);            \
    if ((threadIdx.x & 63) == 0 && w_ < (uint32_t)::fh::kTraceMaxWaves)                 \
      ::fh::fh_trace_buf[::fh::kTraceWaveOff + (ev) * ::fh::kTraceMaxWaves + w_] =      \
          __builtin_amdgcn_s_memrealtime();                                             \
  } while (0)
#define FH_TRACE_SEL(i)                                                                 \
  do {                                                                                  \
    if (threadIdx.x == 0) {                                                             \
      ::fh::fh_trace_buf[::fh::kTraceSelOff + 2 * (i)] = __builtin_amdgcn_s_memtime();  \
      ::fh::fh_trace_buf[::fh::kTraceSelOff + 2 * (i) + 1] =                            \
          __builtin_amdgcn_s_memrealtime();                                             \
    }                                                                                   \
  } while (0)
#define FH_TRACE_COUNT(i, n)                                                            \
  do {                                                                                  \
    if (threadIdx.x == 0) ::fh::fh_trace_buf[::fh::kTraceCountOff + (i)] = (uint64_t)(n); \
  } while (0)
#else
#define FH_TRACE_BLOCK(ev) \
  do {                     \
  } while (0)
#define FH_TRACE_WAVE(ev) \
  do {                    \
  } while (0)
#define FH_TRACE_SEL(i) \
  do {                  \
  } while (0)
#define FH_TRACE_COUNT(i, n) \
  do {                       \
  } while (0)
#endif
