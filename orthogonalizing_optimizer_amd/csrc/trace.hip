// Kernel timing trace for benchmarks.  While enabled, each kernel the
// library launches is timed by HIP events on the caller's stream and its
// algorithmic work (flops or bytes the method needs, on unpadded sizes) is
// recorded, so a benchmark can time every kernel of the step live.  Within
// one library call the kernels run back to back on the call's stream, so a
// kernel's start event is the previous kernel's end event: one event record
// per kernel instead of two (each record costs a few microseconds of GPU
// time between kernels).
#include <mutex>
#include <vector>

#include "../../include/dion3.h"
#include "dion3_internal.h"

namespace dion3 {
namespace {

struct TraceRec {
  const char* name;
  double flops, bytes;
  hipEvent_t e0, e1;
  int from;   // the record whose end event is this one's start, or -1: e0
  bool ok;    // the start and end events were recorded
};

std::mutex g_mu;
std::vector<TraceRec> g_recs;
int g_count = 0;
bool g_on = false;
// the open chain: its stream, and the record whose end event was the last
// thing enqueued on it (-1: none)
bool g_chain_on = false;
hipStream_t g_chain = nullptr;
int g_last = -1;

}  // namespace

TraceScope::TraceScope(const char* name, double flops, double bytes, hipStream_t s)
    : slot(-1), stream(s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on || g_count >= (int)g_recs.size()) return;
  slot = g_count++;
  TraceRec& r = g_recs[slot];
  r.name = name;
  r.flops = flops;
  r.bytes = bytes;
  if (g_chain_on && s == g_chain && g_last >= 0) {
    r.from = g_last;
    r.ok = true;
  } else {
    r.from = -1;
    r.ok = hipEventRecord(r.e0, s) == hipSuccess;
  }
  g_last = -1;   // until this launch's end event is recorded
}

TraceScope::~TraceScope() {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  TraceRec& r = g_recs[slot];
  if (r.ok) r.ok = hipEventRecord(r.e1, stream) == hipSuccess;
  if (r.ok && g_chain_on && stream == g_chain) g_last = slot;
}

TraceChain::TraceChain(hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_chain_on = g_on;
  g_chain = s;
  g_last = -1;
}

TraceChain::~TraceChain() {
  std::lock_guard<std::mutex> lk(g_mu);
  g_chain_on = false;
  g_last = -1;
}

void trace_break() {
  std::lock_guard<std::mutex> lk(g_mu);
  g_last = -1;
}

}  // namespace dion3

using namespace dion3;

extern "C" {

dion3_status dion3_trace_enable(int32_t capacity) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (TraceRec& r : g_recs) {   // nothing to do about a failed destroy
    (void)hipEventDestroy(r.e0);
    (void)hipEventDestroy(r.e1);
  }
  g_recs.clear();
  g_count = 0;
  g_on = false;
  g_chain_on = false;
  g_last = -1;
  if (capacity <= 0) return DION3_OK;
  if (capacity > (1 << 20)) return DION3_ERR_ARG;
  g_recs.resize(capacity);
  for (int i = 0; i < capacity; ++i) {
    TraceRec& r = g_recs[i];
    if (hipEventCreate(&r.e0) != hipSuccess) {
      g_recs.resize(i);
      return DION3_ERR_HIP;
    }
    if (hipEventCreate(&r.e1) != hipSuccess) {
      (void)hipEventDestroy(r.e0);   // this slot's first event; nothing to do if it fails
      g_recs.resize(i);
      return DION3_ERR_HIP;
    }
  }
  g_on = true;
  return DION3_OK;
}

int32_t dion3_trace_count(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  return g_count;
}

void dion3_trace_reset(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_count = 0;
  g_last = -1;
}

dion3_status dion3_trace_record(int32_t i, const char** name, double* ms, double* flops,
                                double* bytes) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (i < 0 || i >= g_count || !name || !ms || !flops || !bytes) return DION3_ERR_ARG;
  TraceRec& r = g_recs[i];
  if (!r.ok || (r.from >= 0 && !g_recs[r.from].ok) || hipEventSynchronize(r.e1) != hipSuccess)
    return DION3_ERR_HIP;
  float t = 0.0f;
  if (hipEventElapsedTime(&t, r.from >= 0 ? g_recs[r.from].e1 : r.e0, r.e1) != hipSuccess)
    return DION3_ERR_HIP;
  *name = r.name;
  *ms = t;
  *flops = r.flops;
  *bytes = r.bytes;
  return DION3_OK;
}

}  // extern "C"
