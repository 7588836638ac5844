// Registry of caller buffers and the range checks of the debug mode (bounds.h).
#include <cstdarg>
#include <cstdlib>
#include <iterator>
#include <map>
#include <mutex>

#include "bounds.h"

namespace vc {

namespace {
std::mutex g_mu;
int g_mode = VC_DEBUG_OFF;
std::map<uintptr_t, size_t> g_reg;  // base -> bytes
vc_debug_stats g_stats{};
}  // namespace

int dbg_mode() { return g_mode; }

void dbg_register(const void* p, size_t bytes) {
  if (!p || !bytes) return;
  // Live allocations never overlap, so any registered range this one overlaps belongs to freed
  // memory the allocator has handed out again: it is dropped, and this registration wins.
  const uintptr_t a = uintptr_t(p), b = a + bytes;
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_reg.upper_bound(a);
  if (it != g_reg.begin()) {
    auto prev = std::prev(it);
    if (prev->first + prev->second > a) it = prev;
  }
  while (it != g_reg.end() && it->first < b) it = g_reg.erase(it);
  g_reg[a] = bytes;
}

void dbg_forget(const void* p) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_reg.erase(uintptr_t(p));
}

vc_status dbg_fail(const char* fmt, ...) {
  char buf[768];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_stats.violations++;
  }
  set_error("bounds check: %s", buf);
  return VC_ERR_ARG;
}

vc_status dbg_check_one(const char* kernel, const DbgRange& r) {
  if (r.bytes <= 0) return VC_OK;
  const uintptr_t a = uintptr_t(r.p), b = a + uintptr_t(r.bytes);
  uintptr_t base = 0;
  size_t size = 0;
  bool ok = false;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_stats.ranges++;
    auto it = g_reg.upper_bound(a);
    if (it != g_reg.begin()) {
      --it;
      base = it->first;
      size = it->second;
      ok = b <= base + size;
    }
  }
  if (ok) return VC_OK;
  return dbg_fail("%s: %s [0x%llx, +%lld) lies outside every registered buffer (nearest below: [0x%llx, +%zu))",
                  kernel, r.what, (unsigned long long)a, (long long)r.bytes, (unsigned long long)base, size);
}

vc_status dbg_check(const char* kernel, std::initializer_list<DbgRange> ranges) {
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_stats.launches++;
  }
  for (const DbgRange& r : ranges)
    if (vc_status st = dbg_check_one(kernel, r)) return st;
  return VC_OK;
}

void* dbg_alloc(size_t bytes, bool pinned) {
  void* p = std::malloc(bytes ? bytes : 1);  // large blocks are mapped lazily: nothing is touched
  if (!p) return nullptr;
  dbg_register(p, bytes);
  if (pinned) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_stats.pinned_bytes += double(bytes);
    if (g_stats.pinned_bytes > g_stats.pinned_peak) g_stats.pinned_peak = g_stats.pinned_bytes;
  }
  return p;
}

void dbg_free(void* p, bool pinned) {
  if (!p) return;
  size_t bytes = 0;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_reg.find(uintptr_t(p));
    if (it != g_reg.end()) {
      bytes = it->second;
      g_reg.erase(it);
    }
    if (pinned) g_stats.pinned_bytes -= double(bytes);
  }
  std::free(p);
}

}  // namespace vc

using namespace vc;

extern "C" {

vc_status vc_debug_mode(int32_t mode) {
  VC_REQUIRE(mode == VC_DEBUG_OFF || mode == VC_DEBUG_CHECK || mode == VC_DEBUG_DRY, VC_ERR_ARG,
             "vc_debug_mode: bad mode %d", mode);
  std::lock_guard<std::mutex> lk(g_mu);
  g_mode = mode;
  return VC_OK;
}

vc_status vc_debug_register(const void* p, size_t bytes) {
  VC_REQUIRE(p != nullptr, VC_ERR_ARG, "vc_debug_register: null pointer");
  dbg_register(p, bytes);
  return VC_OK;
}

vc_status vc_debug_forget(const void* p) {
  dbg_forget(p);
  return VC_OK;
}

vc_status vc_debug_stats_read(vc_debug_stats* out, int32_t reset) {
  VC_REQUIRE(out != nullptr, VC_ERR_ARG, "vc_debug_stats_read: null output");
  std::lock_guard<std::mutex> lk(g_mu);
  *out = g_stats;
  if (reset) {
    const double pinned = g_stats.pinned_bytes;
    g_stats = vc_debug_stats{};
    g_stats.pinned_bytes = g_stats.pinned_peak = pinned;
  }
  return VC_OK;
}

}  // extern "C"
