// Test shim: exposes the library's host CPU branch and worker pool (csrc/cpu_ffn.cpp)
// through a C interface so the CPU suite can exercise them without a GPU.
#include <atomic>
#include <vector>

#include "../../routed_expert_ffn_02_amd/csrc/internal.hpp"

using namespace rmoe;

extern "C" int shim_cpu_ffn(int wfmt, int H, int I, int T, int k, long long rec_bytes, const float* x, const float* w,
                            const int* slot_idx, const void* const* recs, int ncpu, float* h, float* y, int threads) {
  CpuPool pool(threads);
  CpuFfnJob job;
  job.wfmt = wfmt;
  job.H = H;
  job.I = I;
  job.T = T;
  job.k = k;
  job.rec_bytes = rec_bytes;
  job.x = x;
  job.w = w;
  job.slot_idx = slot_idx;
  for (int c = 0; c < ncpu; ++c) job.rec.push_back(static_cast<const uint8_t*>(recs[c]));
  job.h = h;
  job.y = y;
  cpu_ffn(pool, job);
  return 0;
}

// Many generations of varying size: returns the number of tasks run with an index
// outside their generation, or run a number of times other than once.
extern "C" long long shim_pool_stress(int threads, int iters) {
  CpuPool pool(threads);
  long long bad = 0;
  for (int it = 0; it < iters; ++it) {
    const int n = 1 + (it * 7919) % 9;
    std::vector<std::atomic<int>> hits(n);
    for (auto& v : hits) v = 0;
    std::atomic<long long> out_of_range{0};
    pool.run(n, [&](int i) {
      if (i < 0 || i >= n) out_of_range++;
      else hits[i]++;
    });
    bad += out_of_range.load();
    for (int i = 0; i < n; ++i) bad += (hits[i].load() != 1);
  }
  return bad;
}

// Create / run / destroy cycles, including pools destroyed before their threads start.
extern "C" int shim_pool_lifecycle(int threads, int reps) {
  for (int rep = 0; rep < reps; ++rep) {
    CpuPool* p = new CpuPool(threads);
    for (int r = 0; r < rep % 4; ++r) {
      std::atomic<int> c{0};
      p->run(1 + r, [&](int) { c++; });
    }
    delete p;
  }
  return 0;
}
