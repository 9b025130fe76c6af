// Optional per-kernel timing with HIP events (see msda_profile_start in msda.h).
#include "msda_bench.h"
#include "msda_launch.h"

#include <cstring>
#include <string>
#include <vector>

namespace msda {
namespace {

struct Record {
  const char *name;
  hipEvent_t begin, end;
};

struct Session {
  bool on = false;
  int capacity = 0;
  int dropped = 0;
  std::vector<Record> records;
  std::vector<hipEvent_t> pool;  // events kept for reuse across sessions
  size_t next = 0;               // next free pool entry in this session
  bool failed = false;
  hipEvent_t pending = nullptr;  // begin event of the launch being enqueued
  std::string only;              // record only kernels of this name ("" = all)
};

thread_local Session g_session;

hipEvent_t take_event(Session &s) {
  if (s.next == s.pool.size()) {
    hipEvent_t e = nullptr;
    // timing-only events: no system-scope fence, so recording one does not
    // write back and invalidate the caches in the middle of the measured work
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
      s.failed = true;
      return nullptr;
    }
    s.pool.push_back(e);
  }
  return s.pool[s.next++];
}

}  // namespace

static bool selected(const Session &s, const char *name) {
  return s.only.empty() || std::strcmp(s.only.c_str(), name) == 0;
}

void prof_begin(hipStream_t stream, const char *name) {
  Session &s = g_session;
  s.pending = nullptr;
  if (!s.on || !selected(s, name) || (int)s.records.size() >= s.capacity) return;
  hipEvent_t e = take_event(s);
  if (e && hipEventRecord(e, stream) == hipSuccess) s.pending = e;
  else s.failed = true;
}

void prof_end(hipStream_t stream, const char *name) {
  Session &s = g_session;
  if (!s.on || !selected(s, name)) return;
  if (!s.pending) {
    ++s.dropped;
    return;
  }
  hipEvent_t e = take_event(s);
  if (e && hipEventRecord(e, stream) == hipSuccess) s.records.push_back({name, s.pending, e});
  else s.failed = true;
  s.pending = nullptr;
}

}  // namespace msda

extern "C" {

msda_status msda_profile_start(int capacity) {
  msda::Session &s = msda::g_session;
  if (capacity < 0) return MSDA_ERR_INVALID_DIMS;
  s.on = true;
  s.capacity = capacity;
  s.dropped = 0;
  s.records.clear();
  s.records.reserve(capacity);
  s.next = 0;
  s.failed = false;
  s.pending = nullptr;
  return MSDA_OK;
}

void msda_profile_select(const char *name) { msda::g_session.only = name ? name : ""; }

int msda_profile_stop(msda_kernel_time *out, int max) {
  msda::Session &s = msda::g_session;
  s.on = false;
  if (s.failed) return -1;
  if (!s.records.empty() && hipEventSynchronize(s.records.back().end) != hipSuccess) return -1;
  int n = 0;
  for (const auto &r : s.records) {
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.begin, r.end) != hipSuccess) return -1;
    if (out && n < max) out[n] = msda_kernel_time{r.name, ms};
    ++n;
  }
  s.records.clear();
  s.next = 0;
  return n + s.dropped;
}

}  // extern "C"
