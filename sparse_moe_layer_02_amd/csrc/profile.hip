// Opt-in per-kernel timing with HIP events (a diagnostic, off by default).
// While enabled, every kernel the library enqueues -- or only the kernels
// named by moe_profile_select -- is bracketed by two events recorded on the
// same stream; the summary waits for them and reports, per kernel name, the
// number of launches and the summed elapsed time.  Each bracketed launch
// costs a few microseconds of stream time, so a timed loop should select
// only the kernels it needs.  When disabled the cost is one relaxed atomic
// load per launch.
#include <atomic>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "moe_internal.h"

namespace moe {
namespace {

struct Rec {
  const char* name;
  hipEvent_t a, b;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_recs;            // this profiling session
std::vector<hipEvent_t> g_pool;     // events kept for reuse across sessions
std::vector<std::string> g_sel;     // kernels to time; empty: every kernel

bool selected_locked(const char* name) {
  if (g_sel.empty()) return true;
  for (const auto& s : g_sel)
    if (s == name) return true;
  return false;
}

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void recycle_locked() {
  for (auto& r : g_recs) {
    if (r.a) g_pool.push_back(r.a);
    if (r.b) g_pool.push_back(r.b);
  }
  g_recs.clear();
}

}  // namespace

int prof_begin(const char* name, hipStream_t s) {
  if (!g_on.load(std::memory_order_relaxed)) return -1;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!selected_locked(name)) return -1;
  Rec r{name, take_event(), take_event()};
  if (!r.a || !r.b || hipEventRecord(r.a, s) != hipSuccess) {
    if (r.a) g_pool.push_back(r.a);
    if (r.b) g_pool.push_back(r.b);
    return -1;
  }
  g_recs.push_back(r);
  return (int)g_recs.size() - 1;
}

void prof_end(int token, hipStream_t s) {
  if (token < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  // a failed record leaves the end event unrecorded: the summary then
  // reports the failure instead of a time
  if (token < (int)g_recs.size()) (void)hipEventRecord(g_recs[token].b, s);
}

}  // namespace moe

extern "C" {

/* Turn per-kernel event timing on (1) or off (0).  Turning it on discards the
 * previous session's records.  Returns the previous state. */
int moe_profile_enable(int on) {
  using namespace moe;
  std::lock_guard<std::mutex> lk(g_mu);
  const bool was = g_on.load();
  if (on) recycle_locked();
  g_on.store(on != 0);
  return was ? 1 : 0;
}

/* Time only the kernels named in `names`, a comma-separated list (e.g.
 * "ffn_gateup_bf16,ffn_down_bf16"); NULL or "" times every kernel.  Applies
 * from the next launch.  Returns the number of names selected. */
int moe_profile_select(const char* names) {
  using namespace moe;
  std::lock_guard<std::mutex> lk(g_mu);
  g_sel.clear();
  if (names) {
    std::string cur;
    for (const char* p = names;; ++p) {
      if (*p == ',' || *p == 0) {
        if (!cur.empty()) g_sel.push_back(cur);
        cur.clear();
        if (*p == 0) break;
      } else if (*p != ' ') {
        cur += *p;
      }
    }
  }
  return (int)g_sel.size();
}

/* Waits for the recorded events and writes one line per kernel name,
 * "name launches total_ms\n", into buf (truncated to len, NUL-terminated).
 * Returns the length of the full text, or -1 if an event failed. */
int moe_profile_summary(char* buf, size_t len) {
  using namespace moe;
  std::lock_guard<std::mutex> lk(g_mu);
  std::map<std::string, std::pair<int, double>> agg;
  std::vector<std::string> order;
  for (auto& r : g_recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return -1;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return -1;
    auto it = agg.find(r.name);
    if (it == agg.end()) {
      order.push_back(r.name);
      agg[r.name] = {1, (double)ms};
    } else {
      it->second.first += 1;
      it->second.second += ms;
    }
  }
  std::string text;
  char line[256];
  for (auto& n : order) {
    snprintf(line, sizeof line, "%s %d %.6f\n", n.c_str(), agg[n].first, agg[n].second);
    text += line;
  }
  if (buf && len) {
    size_t n = text.size() < len - 1 ? text.size() : len - 1;
    memcpy(buf, text.data(), n);
    buf[n] = 0;
  }
  return (int)text.size();
}

}  // extern "C"
