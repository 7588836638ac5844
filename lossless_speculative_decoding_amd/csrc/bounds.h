// Address-range checking of every launch and copy (a debug mode of the library).
//
// Mode VC_DEBUG_CHECK: before a kernel launch or a copy, the launcher states every byte range
// the kernel or copy can touch (derived from its arguments and the kernel's own loop bounds);
// each range must lie inside one buffer the caller registered (vc_debug_register), else the
// call fails with VC_ERR_ARG and a message naming the kernel, the operand and the range, and
// nothing is launched.  Mode VC_DEBUG_DRY: the same checks, after which no HIP call is made at
// all (no launch, copy, event, synchronisation or allocation on a device; host "pinned"
// allocations become ordinary lazily-mapped memory and are counted), so a whole workload's
// sequence of calls can be replayed on a machine without a GPU, with host memory standing in
// for device memory.
#pragma once
#include <initializer_list>

#include "common.h"

namespace vc {

int dbg_mode();
inline bool dbg_on() { return dbg_mode() != VC_DEBUG_OFF; }
inline bool dbg_dry() { return dbg_mode() == VC_DEBUG_DRY; }

struct DbgRange {
  const char* what;
  const void* p;
  int64_t bytes;  // <= 0: nothing touched
};

// Every range inside a registered buffer; counts one launch.
vc_status dbg_check(const char* kernel, std::initializer_list<DbgRange> ranges);
vc_status dbg_check_one(const char* kernel, const DbgRange& r);
// The block of `rows` rows of `width` bytes at pitch `pitch` starting at p.
inline DbgRange dbg_2d(const char* what, const void* p, int64_t pitch, int64_t width, int64_t rows) {
  return DbgRange{what, p, rows > 0 && width > 0 ? (rows - 1) * pitch + width : 0};
}
// Counts a check failure caused elsewhere (a launch-shape contract) with its message.
vc_status dbg_fail(const char* fmt, ...);
// Host allocations standing in for device or pinned memory in dry mode (registered).
void* dbg_alloc(size_t bytes, bool pinned);
void dbg_free(void* p, bool pinned);
void dbg_register(const void* p, size_t bytes);
void dbg_forget(const void* p);

}  // namespace vc

// In a launcher: check the ranges (when checking is on) and, in dry mode, return before the launch.
#define VC_DBG_LAUNCH(kernel, ...)                                          \
  do {                                                                       \
    if (::vc::dbg_on()) {                                                    \
      if (vc_status dst_ = ::vc::dbg_check(kernel, {__VA_ARGS__})) return dst_; \
      if (::vc::dbg_dry()) return VC_OK;                                     \
    }                                                                        \
  } while (0)
