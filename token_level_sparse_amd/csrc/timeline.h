// Per-wave timeline of the kernels, for measurement builds only.
//
// Built with -DTS_TIMELINE (libtokenselect_timeline.so beside the library), every
// instrumented kernel records, for each of its waves, the wall clock
// (s_memrealtime, 100 MHz) at entry and at exit, up to six marks taken at phase
// boundaries, its workgroup and its XCD, into a device buffer of its source file
// that ts_timeline_read_<file> copies out. TS_TIMELINE_MARK first waits for the
// wave's outstanding memory operations, so it records when the phase's data had
// arrived; TS_TIMELINE_MARK_HERE records when the wave gets there. Without TS_TIMELINE every macro below expands to nothing and the
// kernels are those of the library.
#pragma once

#ifdef TS_TIMELINE

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ts {

constexpr int kTimelineKernels = 10;      // kernel ids 0..9 per source file
constexpr int kTimelineWaves = 16384;     // waves recorded per kernel (later waves are dropped)
constexpr int kTimelineWords = 10;        // u64 per wave record

// Kernel ids.
enum TimelineKernel {
  kTlScore = 0, kTlStats = 1, kTlVote = 2, kTlRefine1 = 3, kTlRefine2 = 4, kTlWrite = 6,
  kTlChunkAttn = 7, kTlAttn = 8, kTlCombine = 9
};

// One wave's record: [0] entry, [1] exit, [2..7] marks (0 if not taken), [8] marks
// taken | XCD << 8 | workgroup << 16, [9] 1 (a record is present). Lane 0 stores each
// time as it is taken, so the scope holds only the record's address and the mark count.
struct TimelineScope {
  unsigned long long* rec;     // wave-uniform; null past kTimelineWaves
  int n;
  __device__ explicit TimelineScope(unsigned long long* buf, int kid) : n(0) {
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
    rec = (w < kTimelineWaves) ? buf + ((int64_t)kid * kTimelineWaves + w) * kTimelineWords : nullptr;
    if (rec && (threadIdx.x & 63) == 0) rec[0] = t0;
  }
  // Marks are stored in program order, at most six. mark() first waits for the
  // wave's outstanding memory operations; mark_here() records when the wave reaches
  // the point (for points whose data the control flow already waited for).
  __device__ void mark_here() {
    const unsigned long long t = __builtin_amdgcn_s_memrealtime();
    if (rec && n < 6 && (threadIdx.x & 63) == 0) rec[2 + n] = t;
    ++n;
  }
  __device__ void mark() {
    __builtin_amdgcn_s_waitcnt(0);
    mark_here();
  }
  __device__ ~TimelineScope() {
    __builtin_amdgcn_s_waitcnt(0);
    const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
    if (rec && (threadIdx.x & 63) == 0) {
      unsigned xcc;
      asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
      rec[1] = t1;
      rec[8] = (unsigned long long)(n < 6 ? n : 6) | ((unsigned long long)(xcc & 0xf) << 8) |
               ((unsigned long long)blockIdx.x << 16);
      rec[9] = 1;
    }
  }
};

}  // namespace ts

// The buffer of one source file and its host readers (extern "C": copy the whole
// buffer of kTimelineKernels x kTimelineWaves x kTimelineWords u64 out, or clear it).
#define TS_TIMELINE_DEFINE(NAME)                                                                        \
  namespace ts {                                                                                        \
  __device__ unsigned long long g_timeline_##NAME[kTimelineKernels * kTimelineWaves * kTimelineWords]; \
  }                                                                                                     \
  extern "C" int ts_timeline_read_##NAME(void* dst) {                                                   \
    return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(ts::g_timeline_##NAME), sizeof(ts::g_timeline_##NAME), 0, \
                                    hipMemcpyDeviceToHost);                                             \
  }                                                                                                     \
  extern "C" int ts_timeline_clear_##NAME() {                                                           \
    void* p = nullptr;                                                                                  \
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(ts::g_timeline_##NAME));                    \
    if (e != hipSuccess) return (int)e;                                                                 \
    return (int)hipMemset(p, 0, sizeof(ts::g_timeline_##NAME));                                         \
  }
#define TS_TIMELINE_SCOPE(NAME, KID) ts::TimelineScope ts_timeline_(ts::g_timeline_##NAME, (KID))
#define TS_TIMELINE_MARK() ts_timeline_.mark()
#define TS_TIMELINE_MARK_HERE() ts_timeline_.mark_here()
// a device function that marks takes the kernel's scope as a trailing parameter
#define TS_TIMELINE_PARAM , ts::TimelineScope& ts_timeline_
#define TS_TIMELINE_ARG , ts_timeline_

#else

#define TS_TIMELINE_DEFINE(NAME)
#define TS_TIMELINE_SCOPE(NAME, KID)
#define TS_TIMELINE_MARK()
#define TS_TIMELINE_MARK_HERE()
#define TS_TIMELINE_PARAM
#define TS_TIMELINE_ARG

#endif
