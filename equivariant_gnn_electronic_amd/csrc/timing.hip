// Event pool behind egnn_timing_* (see egnn.h, "Kernel timing").
#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "timing.h"

namespace egnn {
namespace {

constexpr int kPool = 16384;

struct Rec {
  int begin, end;
  std::string name;
  double flops, bytes;
};

struct Totals {
  int64_t launches = 0;
  double ms = 0, flops = 0, bytes = 0;
};

struct State {
  std::mutex mu;
  std::atomic<bool> on{false};
  std::vector<hipEvent_t> ev;
  int next = 0;
  std::vector<Rec> pending;
  std::map<std::string, Totals> totals;
  int64_t dropped = 0;
};

State &st() {
  static State s;
  return s;
}

}  // namespace

bool timing_on() { return st().on.load(std::memory_order_relaxed); }

void timing_begin(hipStream_t s, int *slot) {
  State &S = st();
  std::lock_guard<std::mutex> lock(S.mu);
  if (S.next + 2 > static_cast<int>(S.ev.size())) {
    ++S.dropped;
    *slot = -1;
    return;
  }
  *slot = S.next;
  S.next += 2;
  (void)hipEventRecord(S.ev[*slot], s);
}

void timing_end(hipStream_t s, int slot, const char *name, double flops, double bytes) {
  State &S = st();
  std::lock_guard<std::mutex> lock(S.mu);
  (void)hipEventRecord(S.ev[slot + 1], s);
  S.pending.push_back({slot, slot + 1, name, flops, bytes});
}

}  // namespace egnn

using namespace egnn;

extern "C" egnn_status egnn_timing_enable(int on) {
  clear_error();
  State &S = st();
  std::lock_guard<std::mutex> lock(S.mu);
  if (on && S.ev.empty()) {
    S.ev.resize(kPool);
    for (auto &e : S.ev) EGNN_TRY_HIP(hipEventCreate(&e));
  }
  S.on.store(on != 0);
  return EGNN_OK;
}

extern "C" int egnn_timing_collect(egnn_timing_entry *out, int max_entries, int64_t *dropped) {
  State &S = st();
  std::lock_guard<std::mutex> lock(S.mu);
  for (const Rec &r : S.pending) {
    (void)hipEventSynchronize(S.ev[r.end]);
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, S.ev[r.begin], S.ev[r.end]) != hipSuccess) continue;
    Totals &t = S.totals[r.name];
    t.launches += 1;
    t.ms += ms;
    t.flops += r.flops;
    t.bytes += r.bytes;
  }
  S.pending.clear();
  S.next = 0;
  int n = 0;
  for (const auto &kv : S.totals) {
    if (n >= max_entries || !out) break;
    std::memset(&out[n], 0, sizeof(out[n]));
    std::strncpy(out[n].name, kv.first.c_str(), sizeof(out[n].name) - 1);
    out[n].launches = kv.second.launches;
    out[n].total_ms = kv.second.ms;
    out[n].flops = kv.second.flops;
    out[n].bytes = kv.second.bytes;
    ++n;
  }
  if (dropped) *dropped = S.dropped;
  return n;
}

extern "C" void egnn_timing_reset(void) {
  State &S = st();
  std::lock_guard<std::mutex> lock(S.mu);
  S.totals.clear();
  S.dropped = 0;
}
