// Optional timing of every launch (dit_profile_begin / dit_profile_end):
// when on, each launch is bracketed by a pair of HIP events on its stream.
#pragma once

#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

namespace dit {
namespace prof {

struct Record {
  int kind;
  double flops, bytes;
  hipEvent_t start, stop;
};
struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<Record> recs;
  std::vector<hipEvent_t> pool;
};
Profiler& state();  // the process-wide profiler (abi.cpp)

inline hipEvent_t event(Profiler& p) {
  if (!p.pool.empty()) {
    hipEvent_t e = p.pool.back();
    p.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` (returning hipError_t); when profiling, brackets it with events.
template <class F>
hipError_t timed(int kind, double flops, double bytes, hipStream_t st, F&& launch) {
  Profiler& p = state();
  if (!p.on) return launch();
  std::lock_guard<std::mutex> lock(p.mu);
  Record r{kind, flops, bytes, event(p), event(p)};
  if (!r.start || !r.stop) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(r.start, st);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(r.stop, st);
  if (e != hipSuccess) return e;
  p.recs.push_back(r);
  return hipSuccess;
}

}  // namespace prof
}  // namespace dit
