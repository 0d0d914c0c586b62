// Per-workgroup timeline of the decode kernels, compiled in only when OSCAR_TIMELINE is defined
// (the diagnostic library liboscar_timeline.so; the product library has no stamps).
//
// Thread 0 of a workgroup writes the constant-rate real-time counter (s_memrealtime, 100 MHz) at
// fixed points of its run into a device table, one row per workgroup; the host copies the table
// out with oscar_timeline_read. Split kernel columns: 0 entry, 1 work plan known, 2 step and
// window segments done, 3 query operands ready, 4 page loop done (wavefront 0), 5 exit,
// 6 segments (bit 0 step, 1 window, 2 INT2, 3 INT4) | history pages of the unit << 8,
// 7 XCC_ID << 32 | HW_ID, 8 every wavefront past its page loop (last history segment), 9 step
// segment loads done, 10 step rotation done, 11 step codes stored, 12 workgroup merge: own state
// in LDS, 13 past its barrier, 14 partial stored. History units of the interleaved one-request
// launch reuse 9 (first page loads issued), 10 (first page pair done), 11 (query products formed)
// and 15 (past the query prologue's first barrier). Merge kernel rows follow the split rows:
// 0 entry, 1 slots folded, 3 groups combined, 5 exit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oscar {

constexpr int kTimelineSplitRows = 16384;
constexpr int kTimelineMergeRows = 2048;
constexpr int kTimelineCols = 16;

#ifdef OSCAR_TIMELINE
extern __device__ uint64_t g_timeline[kTimelineSplitRows + kTimelineMergeRows][kTimelineCols];

__device__ __forceinline__ void timeline_put(int row, int col, uint64_t v) {
  if (threadIdx.x == 0 && row < kTimelineSplitRows + kTimelineMergeRows) g_timeline[row][col] = v;
}
__device__ __forceinline__ uint64_t timeline_now() { return __builtin_amdgcn_s_memrealtime(); }
__device__ __forceinline__ uint64_t timeline_placement() {
  // hardware registers HW_ID (id 4) and XCC_ID (id 20), whole 32-bit fields
  const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);
  const uint32_t xcc = __builtin_amdgcn_s_getreg((31 << 11) | 20);
  return ((uint64_t)xcc << 32) | hw;
}
#define OSCAR_TL_SPLIT(col) ::oscar::timeline_put((int)blockIdx.x, (col), ::oscar::timeline_now())
#define OSCAR_TL_SPLIT_VALUE(col, v) ::oscar::timeline_put((int)blockIdx.x, (col), (uint64_t)(v))
#define OSCAR_TL_MERGE(col) \
  ::oscar::timeline_put(::oscar::kTimelineSplitRows + (int)blockIdx.x, (col), ::oscar::timeline_now())
#else
#define OSCAR_TL_SPLIT(col) ((void)0)
#define OSCAR_TL_SPLIT_VALUE(col, v) ((void)0)
#define OSCAR_TL_MERGE(col) ((void)0)
#endif

}  // namespace oscar
