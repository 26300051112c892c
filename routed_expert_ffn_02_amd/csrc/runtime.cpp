// Host runtime and C ABI of the routed-MoE library.
//
// Owns the residency tables, work lists, pinned staging, the copy stream and the
// CPU worker pool; sequences the per-layer hot path:
//   decode   route -> lookup (one device kernel) -> [read the step's fill / CPU
//            lists from host-mapped staging] -> CPU branch started first ->
//            fills on the copy stream -> GEMV phases on the compute stream ->
//            exact merge y = y_GPU + y_CPU
//            (FreeToken summary, "측정된 대역폭이 분할을 결정합니다");
//   prefill  two full-layer buffers from the shared slot pool; the copy stream
//            loads layer l+2 into the buffer layer l frees while later layers
//            compute (FreeToken summary, "전층 이중 버퍼링");
//   resize   rebuild the cache for a new slot budget at a safe point without
//            touching the host pool (FreeToken summary, "탄력적 메모리 관리").
#include <hip/hip_runtime.h>
#include <immintrin.h>
#include <sched.h>

#include <algorithm>
#include <chrono>
#include <cstdlib>
#include <cstring>
#include <numeric>
#include <string>
#include <vector>

#include "internal.hpp"

using namespace rmoe;

namespace {

moe_status fail(moe_ctx* c, moe_status st, const std::string& msg) {
  if (c) c->err = msg;
  return st;
}

#define HIPCHK(expr)                                                                           \
  do {                                                                                         \
    hipError_t e_ = (expr);                                                                    \
    if (e_ != hipSuccess) return fail(ctx, MOE_EHIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

#define CHECK_ARG(cond, msg) \
  do {                       \
    if (!(cond)) return fail(ctx, MOE_EINVAL, msg); \
  } while (0)

// Entries of both GEMMs' tile tables for up to Pmax prefill pairs (sets ctx->tiles1_max).
int64_t prefill_tables_max(moe_ctx* ctx, int64_t Pmax) {
  const moe_config& c = ctx->cfg;
  const int bm = prefill_bm();
  const int max_tiles_m = (int)((Pmax + bm - 1) / bm + std::min<int64_t>(c.n_experts, Pmax));
  ctx->tiles1_max = prefill_tile_slots(max_tiles_m, c.inter / 128);
  return ctx->tiles1_max + prefill_tile_slots(max_tiles_m, c.hidden / 256);
}

int64_t record_bytes(const moe_config& c) {
  const int64_t n = (int64_t)c.hidden * c.inter;
  switch (c.wfmt) {
    case MOE_WFMT_F32: return 3 * n * 4;
    case MOE_WFMT_BF16: return 3 * n * 2;
    case MOE_WFMT_FP4: return 3 * (n / 2) + 3 * (n / 32) * 2;
    case MOE_WFMT_MXFP4: return 3 * (n / 2) + 3 * (n / 32);
  }
  return -1;
}

int64_t weight_row_bytes(const moe_config& c, int cols) {
  switch (c.wfmt) {
    case MOE_WFMT_F32: return (int64_t)cols * 4;
    case MOE_WFMT_BF16: return (int64_t)cols * 2;
    case MOE_WFMT_MXFP4: return (int64_t)cols / 2 + (int64_t)cols / 32;
    default: return (int64_t)cols / 2 + (int64_t)cols / 32 * 2;
  }
}

int act_bytes(const moe_config& c) { return c.afmt == MOE_AFMT_BF16 ? 2 : 4; }

template <typename T>
hipError_t dev_alloc(T** p, size_t n) {
  return hipMalloc(reinterpret_cast<void**>(p), std::max<size_t>(n, 1) * sizeof(T));
}

const uint8_t* pool_record(const moe_ctx* c, int64_t key) {
  const int64_t b = (c->pool_records > 0) ? key % c->pool_records : key;
  return c->pool + b * c->S;
}

// Enqueue copies of keys [k0, k0+n) into consecutive arena slots starting at dst_slot,
// merging runs that are contiguous in the pool.
hipError_t copy_keys(moe_ctx* c, int64_t k0, int64_t n, int64_t dst_slot, hipStream_t s) {
  int64_t i = 0;
  while (i < n) {
    const uint8_t* src = pool_record(c, k0 + i);
    int64_t run = 1;
    while (i + run < n && pool_record(c, k0 + i + run) == src + run * c->S) ++run;
    hipError_t e = hipMemcpyAsync(c->arena + (dst_slot + i) * c->S, src, run * c->S, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return e;
    c->stats.fill_bytes += run * c->S;
    i += run;
  }
  return hipSuccess;
}

hipEvent_t take_event(moe_ctx* c) {
  if (!c->event_pool.empty()) {
    hipEvent_t e = c->event_pool.back();
    c->event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

enum TimedKind { TK_P1 = 0, TK_P2 = 1, TK_G1 = 2, TK_G2 = 3, TK_COPY = 4, TK_FILL = 5 };
constexpr size_t kStepLogMax = size_t(1) << 20;

// Work enqueued while `s` is being captured into a graph runs later, at each replay:
// nothing may be read on the host then, and per-launch profiling is skipped.
bool capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &st) == hipSuccess && st == hipStreamCaptureStatusActive;
}

// Events for one timed launch (none unless MOE_FLAG_PROFILE).  Kernels receive them
// through hipExtLaunchKernelGGL, so the interval is the kernel's own execution; copies
// are bracketed by records on their stream.
struct TimedScope {
  moe_ctx* c;
  hipStream_t s;
  int kind;
  bool record;
  int64_t rec;  // TK_FILL: the step-log record the interval belongs to
  Timing tm;
  TimedScope(moe_ctx* c_, hipStream_t s_, int kind_, bool record_around = false, int64_t rec_ = -1)
      : c(c_), s(s_), kind(kind_), record(record_around), rec(rec_) {
    if (kind >= 0 && (c->cfg.flags & MOE_FLAG_PROFILE) && !capturing(s)) {
      tm.start = take_event(c);
      tm.stop = take_event(c);
      if (record && tm.start) hipEventRecord(tm.start, s);
    }
  }
  ~TimedScope() {
    if (tm.start && tm.stop) {
      if (record) hipEventRecord(tm.stop, s);
      c->pending_timed.push_back({tm.start, tm.stop, kind, rec});
    }
  }
};

void drain_timed(moe_ctx* c) {
  for (auto& t : c->pending_timed) {
    float ms = 0.f;
    if (hipEventSynchronize(t.b) == hipSuccess && hipEventElapsedTime(&ms, t.a, t.b) == hipSuccess) {
      switch (t.kind) {
        case TK_P1: c->stats.phase1_ms += ms; break;
        case TK_P2: c->stats.phase2_ms += ms; break;
        case TK_G1: c->stats.gemm1_ms += ms; break;
        case TK_G2: c->stats.gemm2_ms += ms; break;
        case TK_COPY: c->stats.copy_ms += ms; break;
        case TK_FILL:
          if (t.rec >= 0 && t.rec < (int64_t)c->step_log.size() && c->step_log[t.rec].fills > 0)
            c->step_log[t.rec].fill_ms += ms;
          break;
      }
    }
    c->event_pool.push_back(t.a);
    c->event_pool.push_back(t.b);
  }
  c->pending_timed.clear();
}

// The CPU branch's pool.  By default it leaves two of the process's CPUs free: one for the
// application thread, which keeps a core busy while it waits on the stream as a replayed
// step's branch runs on the library's branch thread, and one for the runtime's own threads.
// Measured on a 16-CPU process replaying DSV4-shaped hybrid steps: with 16 pool threads
// the branch took 4x as long as eagerly (it ends with its slowest task, and a worker
// sharing a core stalls it), with 15 1.7x, with 14 the same as eagerly.
rmoe::CpuPool& cpu_pool(moe_ctx* c) {
  if (!c->cpu) {
    int n = c->cfg.cpu_threads;
    if (n <= 0) {
      cpu_set_t set;
      CPU_ZERO(&set);
      const int cpus = (sched_getaffinity(0, sizeof(set), &set) == 0) ? CPU_COUNT(&set) : 1;
      n = std::max(1, cpus - 2);
    }
    c->cpu = new rmoe::CpuPool(n);
  }
  return *c->cpu;
}

void fill_lookup_args(moe_ctx* c, LookupArgs& a, int layer, const int32_t* idx, int T, int mode) {
  std::memset(&a, 0, sizeof(a));
  a.topk_idx = idx;
  a.T = T;
  a.k = c->cfg.top_k;
  a.E = c->cfg.n_experts;
  a.layer = layer;
  a.mode = mode;
  a.n_slots = c->n_slots;
  a.bw_pcie = c->cfg.bw_pcie;
  a.bw_host = c->cfg.bw_host;
  a.ctrl = c->ctrl;
  a.mode_from_ctrl = 0;
  a.slot_of = c->slot_of;
  a.key_of = c->key_of;
  a.stamp = c->stamp;
  a.reserved = c->reserved;
  a.counter = c->counter;
  a.u_key = c->u_key;
  a.u_kind = c->u_kind;
  a.u_slot = c->u_slot;
  a.u_evict = c->u_evict;
  a.fill_key = c->fill_key;
  a.fill_slot = c->fill_slot;
  a.cpu_key = c->cpu_key;
  a.grp_slot = c->grp_slot;
  a.grp_pair0 = c->grp_pair0;
  a.pair_grp = c->pair_grp;
  a.cnt = c->cnt;
}

int lookup_mode_of(int mode) {
  switch (mode) {
    case MOE_MODE_FUSED: return LK_FUSED;
    case MOE_MODE_OFFLOAD: return LK_OFFLOAD;
    case MOE_MODE_CPU: return LK_CPU;
    default: return LK_HYBRID;
  }
}

// The device control block from the host state, once all work on the device has finished
// (kernels read it when they run, so it changes only between steps).
moe_status write_ctrl(moe_ctx* ctx) {
  DevCtrl h{};
  h.arena = ctx->arena;
  h.n_slots = ctx->n_slots;
  h.lk_mode = lookup_mode_of(ctx->cfg.mode);
  h.bw_pcie = ctx->cfg.bw_pcie;
  h.bw_host = ctx->cfg.bw_host;
  h.cpu_wait_ticks = (uint64_t)(ctx->cpu_wait_ms * (double)ctx->wall_khz);
  HIPCHK(hipDeviceSynchronize());
  HIPCHK(hipMemcpy(ctx->ctrl, &h, sizeof h, hipMemcpyHostToDevice));
  return MOE_OK;
}

// Copy the step's counts and work lists (one contiguous block) to pinned host memory,
// with the CPU branch's inputs when `inputs` is set, and wait: the one device -> host
// decision point of a cached step.
// The step block (and, with inputs, x, gates and slot ids for the CPU branch) copied to
// pinned staging behind the lookup on stream s; read_step_finish waits for the copies.
moe_status read_step_issue(moe_ctx* ctx, hipStream_t s, bool inputs, const void* x, const float* w,
                           const int32_t* slot_idx, int T) {
  const int E = ctx->cfg.n_experts;
  HIPCHK(hipMemcpyAsync(ctx->step_host, ctx->step_dev, (size_t)(C_COUNT + 5 * E) * sizeof(int32_t),
                        hipMemcpyDeviceToHost, s));
  if (inputs) {
    const int P = T * ctx->cfg.top_k;
    HIPCHK(hipEventSynchronize(ctx->ev_ycpu));  // the previous H2D from the host staging has finished
    HIPCHK(hipMemcpyAsync(ctx->h_x, x, (size_t)T * ctx->cfg.hidden * act_bytes(ctx->cfg), hipMemcpyDeviceToHost, s));
    HIPCHK(hipMemcpyAsync(ctx->h_w, w, (size_t)P * sizeof(float), hipMemcpyDeviceToHost, s));
    HIPCHK(hipMemcpyAsync(ctx->h_slot_idx, slot_idx, (size_t)P * sizeof(int32_t), hipMemcpyDeviceToHost, s));
  }
  HIPCHK(hipEventRecord(ctx->ev_sync, s));
  return MOE_OK;
}

moe_status read_step_finish(moe_ctx* ctx) {
  HIPCHK(hipEventSynchronize(ctx->ev_sync));
  if (ctx->h_cnt[C_ERR]) return fail(ctx, MOE_EINVAL, "expert id out of range in topk_idx");
  ctx->stats.lookups += 1;
  ctx->stats.hits += ctx->h_cnt[C_HIT];
  ctx->stats.fills += ctx->h_cnt[C_FILL];
  ctx->stats.cpu_experts += ctx->h_cnt[C_CPU];
  ctx->stats.evictions += ctx->h_cnt[C_EVICT];
  return MOE_OK;
}

moe_status read_step(moe_ctx* ctx, hipStream_t s, bool inputs, const void* x, const float* w, const int32_t* slot_idx,
                     int T) {
  moe_status st = read_step_issue(ctx, s, inputs, x, w, slot_idx, T);
  return st != MOE_OK ? st : read_step_finish(ctx);
}

// Fills of the current step: pinned pool -> victim slots on the copy stream; the
// compute stream waits for them.  The compute stream is idle up to the lookup here
// (read_step synchronised it), so no kernel still reads a victim slot.
moe_status issue_fills(moe_ctx* ctx, hipStream_t s, int64_t log_rec = -1) {
  const int nf = ctx->h_cnt[C_FILL];
  if (nf <= 0) return MOE_OK;
  if (!ctx->pool_pinned) return fail(ctx, MOE_ENOPIN, "fills need a page-locked host pool");
  TimedScope ts(ctx, ctx->copy_stream, TK_COPY, true);
  TimedScope tl(ctx, ctx->copy_stream, log_rec >= 0 ? TK_FILL : -1, true, log_rec);
  for (int i = 0; i < nf; ++i) {
    const int key = ctx->h_fill_key[i], slot = ctx->h_fill_slot[i];
    HIPCHK(hipMemcpyAsync(ctx->arena + (int64_t)slot * ctx->S, pool_record(ctx, key), ctx->S, hipMemcpyHostToDevice,
                          ctx->copy_stream));
    ctx->stats.fill_bytes += ctx->S;
  }
  HIPCHK(hipEventRecord(ctx->ev_fill, ctx->copy_stream));
  HIPCHK(hipStreamWaitEvent(s, ctx->ev_fill, 0));
  return MOE_OK;
}

// CPU branch over the step's CPU list.  x, w and slot ids are already in pinned
// staging (read_step with inputs); the GPU work of the step is enqueued before this
// runs, so both branches proceed together.  Ends with the H2D copy of the partial sum.
moe_status run_cpu_branch(moe_ctx* ctx, int T, hipStream_t s, float** y_cpu_dev_out) {
  *y_cpu_dev_out = nullptr;
  const int ncpu = ctx->h_cnt[C_CPU];
  if (ncpu <= 0) return MOE_OK;
  const int H = ctx->cfg.hidden;
  if (ctx->cfg.afmt == MOE_AFMT_BF16) {
    const uint16_t* xb = static_cast<const uint16_t*>(ctx->h_x);
    for (int64_t i = 0; i < (int64_t)T * H; ++i) {
      uint32_t u = (uint32_t)xb[i] << 16;
      std::memcpy(&ctx->h_xf[i], &u, 4);
    }
  } else {
    std::memcpy(ctx->h_xf, ctx->h_x, (size_t)T * H * sizeof(float));
  }
  CpuFfnJob job;
  job.wfmt = ctx->cfg.wfmt;
  job.H = H;
  job.I = ctx->cfg.inter;
  job.T = T;
  job.k = ctx->cfg.top_k;
  job.rec_bytes = ctx->S;
  job.x = ctx->h_xf;
  job.w = ctx->h_w;
  job.slot_idx = ctx->h_slot_idx;
  for (int c = 0; c < ncpu; ++c) job.rec.push_back(pool_record(ctx, ctx->h_cpu_key[c]));
  job.h = ctx->h_hbuf;
  job.y = ctx->h_y;
  std::memset(ctx->h_y, 0, (size_t)T * H * sizeof(float));
  const auto t0 = std::chrono::steady_clock::now();
  cpu_ffn(cpu_pool(ctx), job);
  ctx->stats.cpu_ms += std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
  HIPCHK(hipMemcpyAsync(ctx->y_cpu_dev, ctx->h_y, (size_t)T * H * sizeof(float), hipMemcpyHostToDevice, s));
  HIPCHK(hipEventRecord(ctx->ev_ycpu, s));
  *y_cpu_dev_out = ctx->y_cpu_dev;
  return MOE_OK;
}

// The CPU branch of a captured step, run by the branch worker once the step block and the
// inputs are in the pinned staging: it reads the CPU list there and leaves the partial sum
// (zeros without CPU work) in h_y, which the device reads through its mapping.  It calls
// no HIP API.
void cpu_branch_staged(moe_ctx* ctx) {
  const int T = ctx->h_cnt[C_T], H = ctx->cfg.hidden;
  std::memset(ctx->h_y, 0, (size_t)T * H * sizeof(float));
  const int ncpu = ctx->h_cnt[C_ERR] ? 0 : ctx->h_cnt[C_CPU];
  if (ncpu <= 0) return;
  if (ctx->cfg.afmt == MOE_AFMT_BF16) {
    const uint16_t* xb = static_cast<const uint16_t*>(ctx->h_x);
    for (int64_t i = 0; i < (int64_t)T * H; ++i) {
      uint32_t u = (uint32_t)xb[i] << 16;
      std::memcpy(&ctx->h_xf[i], &u, 4);
    }
  } else {
    std::memcpy(ctx->h_xf, ctx->h_x, (size_t)T * H * sizeof(float));
  }
  CpuFfnJob job;
  job.wfmt = ctx->cfg.wfmt;
  job.H = H;
  job.I = ctx->cfg.inter;
  job.T = T;
  job.k = ctx->cfg.top_k;
  job.rec_bytes = ctx->S;
  job.x = ctx->h_xf;
  job.w = ctx->h_w;
  job.slot_idx = ctx->h_slot_idx;
  for (int c = 0; c < ncpu; ++c) job.rec.push_back(pool_record(ctx, ctx->h_cpu_key[c]));
  job.h = ctx->h_hbuf;
  job.y = ctx->h_y;
  const auto t0 = std::chrono::steady_clock::now();
  cpu_ffn(cpu_pool(ctx), job);
  ctx->stats.cpu_ms += std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
}

// The branch worker of captured steps: it waits for the device to publish a new sequence
// number in the pinned go word, runs that step's CPU branch from the staging, and answers
// with the same number in the done word, which the step's wait kernel polls.  It spins
// while steps keep coming (the branch then starts within a microsecond of the signal) and
// sleeps in short naps after 2 ms without one.  Numbers only grow; a number the device
// publishes while the previous branch still runs is taken next (the device waits for each
// branch before it stages the next step, so a step is never overwritten while it is read).
void branch_worker(moe_ctx* ctx) {
  uint32_t* go = ctx->sig_host + kSigGo;
  uint32_t* done = ctx->sig_host + kSigDone;
  // failure tests only: a delay before each answer, so that a short wait bound expires
  const char* env = std::getenv("RMOE_CPU_BRANCH_DELAY_US");
  const long delay_us = env ? std::max(0L, std::atol(env)) : 0L;
  uint32_t last = __atomic_load_n(done, __ATOMIC_ACQUIRE);
  auto idle = std::chrono::steady_clock::now();
  while (!ctx->branch_stop.load(std::memory_order_acquire)) {
    const uint32_t g = __atomic_load_n(go, __ATOMIC_ACQUIRE);
    if (g != last) {
      if (delay_us) std::this_thread::sleep_for(std::chrono::microseconds(delay_us));
      cpu_branch_staged(ctx);
      __atomic_store_n(done, g, __ATOMIC_RELEASE);
      last = g;
      idle = std::chrono::steady_clock::now();
      continue;
    }
    if (std::chrono::steady_clock::now() - idle < std::chrono::milliseconds(2)) _mm_pause();
    else std::this_thread::sleep_for(std::chrono::microseconds(50));
  }
}

// The step block and the CPU branch's inputs written into the pinned staging by one
// launch on s (through the staging's device mapping), in place of four copies.
StageArgs stage_args(moe_ctx* ctx, const void* x, const float* w, const int32_t* slot_idx, int T) {
  StageArgs sa;
  sa.step = ctx->step_dev;
  sa.step_h = ctx->step_host_dev;
  sa.n_step = C_COUNT + 5 * ctx->cfg.n_experts;
  sa.x = static_cast<const uint32_t*>(x);
  sa.x_h = static_cast<uint32_t*>(ctx->h_x_dev);
  sa.n_x = (int)((int64_t)T * ctx->cfg.hidden * act_bytes(ctx->cfg) / 4);
  sa.w = w;
  sa.w_h = ctx->h_w_dev;
  sa.slot = slot_idx;
  sa.slot_h = ctx->h_slot_idx_dev;
  sa.P = T * ctx->cfg.top_k;
  return sa;
}

void stage_step(moe_ctx* ctx, const void* x, const float* w, const int32_t* slot_idx, int T, hipStream_t s) {
  launch_stage_step(stage_args(ctx, x, w, slot_idx, T), s);
}

// The CPU branch of a captured step, first half (right after the lookup on s): the step
// block and inputs to the pinned staging and the signal to the branch worker, which starts
// with the first such step.  The GPU work enqueued next runs while the CPU computes;
// join_cpu_branch then makes s wait for the partial sum.
moe_status enqueue_cpu_branch(moe_ctx* ctx, const void* x, const float* w, const int32_t* slot_idx, int T,
                              hipStream_t s) {
  if (!ctx->step_host_dev || !ctx->sig_dev || !ctx->h_y_dev)
    return fail(ctx, MOE_ENOTSUP, "a captured step with a CPU branch needs device-mapped pinned staging");
  if (!ctx->branch_thread.joinable()) ctx->branch_thread = std::thread(branch_worker, ctx);
  StageArgs sa = stage_args(ctx, x, w, slot_idx, T);
  sa.cnt = ctx->cnt;
  sa.seq = ctx->seq_dev;
  sa.go_h = ctx->sig_dev + kSigGo;
  launch_stage_signal(sa, s);
  return MOE_OK;
}

// Second half, before the combine: the bounded wait for the worker's answer and the copy of
// the partial sum to y_cpu_dev.
void join_cpu_branch(moe_ctx* ctx, int T, hipStream_t s) {
  CpuWaitArgs w;
  w.cnt = ctx->cnt;
  w.seq = ctx->seq_dev;
  w.done_h = ctx->sig_dev + kSigDone;
  w.y_h = reinterpret_cast<uint32_t*>(ctx->h_y_dev);
  w.y = ctx->y_cpu_dev;
  w.n = T * ctx->cfg.hidden;
  w.ctrl = ctx->ctrl;
  w.dstats = ctx->dstats;
  launch_cpu_wait(w, s);
}

// A step may send experts to the CPU: CPU and HYBRID modes, or too few slots.
bool may_use_cpu(const moe_ctx* c, int P) {
  return c->cfg.mode == MOE_MODE_CPU || c->cfg.mode == MOE_MODE_HYBRID || c->n_slots < 2 * P;
}

bool valid_mode(int m) { return m >= MOE_MODE_FUSED && m <= MOE_MODE_HYBRID; }

}  // namespace

// ============================================================================
extern "C" {

MOE_API int64_t moe_record_bytes(const moe_config* cfg) {
  if (!cfg || cfg->hidden <= 0 || cfg->inter <= 0) return -1;
  return record_bytes(*cfg);
}

MOE_API int32_t qstar_split(int32_t m, uint64_t bw_pcie, uint64_t bw_host, int32_t mode, int32_t evictable) {
  if (m < 0 || evictable < 0 || !valid_mode(mode)) return -1;
  if (mode == MOE_MODE_FUSED || mode == MOE_MODE_CPU) return 0;
  const int32_t cap = std::min(m, evictable);
  if (mode == MOE_MODE_OFFLOAD) return cap;
  if (m == 0 || evictable == 0) return 0;
  if (bw_host <= bw_pcie) return cap;
  // round-half-up of m * B_P / B_H in exact integer arithmetic
  const unsigned __int128 num = (unsigned __int128)2 * (unsigned __int128)m * bw_pcie + bw_host;
  const unsigned __int128 q = num / ((unsigned __int128)2 * bw_host);
  const int64_t qi = std::max<int64_t>(1, (int64_t)std::min<unsigned __int128>(q, (unsigned __int128)INT32_MAX));
  return (int32_t)std::min<int64_t>(cap, qi);
}

MOE_API const char* moe_last_error(const moe_ctx* ctx) { return ctx ? ctx->err.c_str() : "null context"; }

MOE_API moe_status moe_create(const moe_config* cfg, moe_ctx** out) {
  moe_ctx* ctx = nullptr;
  if (!cfg || !out) return MOE_EINVAL;
  *out = nullptr;
  const moe_config& c = *cfg;
  if (c.n_layers < 1 || c.n_experts < 1 || c.n_experts > kMaxExperts || c.top_k < 1 || c.top_k > c.n_experts ||
      c.hidden < 64 || c.hidden % 64 || c.inter < 64 || c.inter % 64 || c.max_tokens < 1 ||
      (int64_t)c.n_layers * c.n_experts > (1 << 24) || c.wfmt < MOE_WFMT_F32 || c.wfmt > MOE_WFMT_MXFP4 ||
      c.afmt < MOE_AFMT_F32 || c.afmt > MOE_AFMT_BF16 || !valid_mode(c.mode) ||
      (int64_t)c.max_tokens * c.top_k > (1 << 22))
    return MOE_EINVAL;
  // MXFP4 runs the LDS-staged prefill GEMMs only: 256-k chunks, 32-bit byte offsets
  if ((c.flags & MOE_FLAG_MX_PREFILL) && c.wfmt != MOE_WFMT_MXFP4) return MOE_ENOTSUP;
  if (c.wfmt == MOE_WFMT_MXFP4 &&
      (c.hidden % 256 || c.inter % 256 || (int64_t)c.max_tokens * c.hidden >= (1ll << 31) ||
       (int64_t)c.max_tokens * c.top_k * c.inter >= (1ll << 31) || record_bytes(c) >= (1ll << 32)))
    return MOE_ENOTSUP;
  ctx = new moe_ctx();
  ctx->cfg = c;
  ctx->S = record_bytes(c);
  ctx->stats = moe_stats{};
  HIPCHK(hipGetDevice(&ctx->device));
  const int L = c.n_layers, E = c.n_experts, H = c.hidden, I = c.inter, k = c.top_k;
  const int64_t Pmax = (int64_t)c.max_tokens * k;
  const int64_t Pdec = (int64_t)std::min(c.max_tokens, kDecodeMaxTok) * k;
  auto cleanup_fail = [&](moe_status st) {
    moe_destroy(ctx);
    return st;
  };
  if (dev_alloc(&ctx->slot_of, (size_t)L * E) || dev_alloc(&ctx->key_of, kMaxCachedSlots) ||
      dev_alloc(&ctx->stamp, kMaxCachedSlots) || dev_alloc(&ctx->reserved, kMaxCachedSlots) ||
      dev_alloc(&ctx->counter, 1) || dev_alloc(&ctx->step_dev, C_COUNT + 5 * E) ||
      dev_alloc(&ctx->u_slot, E) || dev_alloc(&ctx->u_evict, E) ||
      dev_alloc(&ctx->grp_slot, std::max<int64_t>(E, Pmax)) || dev_alloc(&ctx->grp_pair0, std::max<int64_t>(E, Pmax)) ||
      dev_alloc(&ctx->slot_scratch, Pmax) ||
      dev_alloc(&ctx->pair_grp, Pmax) ||
      dev_alloc(&ctx->logits, (size_t)c.max_tokens * E) || dev_alloc(&ctx->h, (size_t)Pdec * I) || dev_alloc(&ctx->h16, (size_t)Pdec * I) ||
      dev_alloc(&ctx->dpair, (size_t)Pdec * H) ||
      dev_alloc(&ctx->y_cpu_dev, (size_t)c.max_tokens * H) || dev_alloc(&ctx->perm, Pmax) ||
      dev_alloc(&ctx->inv, Pmax) || dev_alloc(&ctx->offsets, std::max<int64_t>(E, Pmax) + 1) ||
      dev_alloc(&ctx->tile_base, std::max<int64_t>(E, Pmax) + 1) ||
      dev_alloc(&ctx->tiles, prefill_tables_max(ctx, Pmax)) ||
      dev_alloc(&ctx->hist, (size_t)((Pmax + 255) / 256) * kMaxExperts) || dev_alloc(&ctx->cand, E) ||
      dev_alloc(reinterpret_cast<uint8_t**>(&ctx->act), (size_t)Pmax * I * 4) ||
      dev_alloc(&ctx->ypair, (size_t)Pmax * H) || dev_alloc(&ctx->flags, std::max<int64_t>((int64_t)L * E, kMaxCachedSlots)) ||
      dev_alloc(&ctx->dstats, D_COUNT) || dev_alloc(&ctx->ctrl, 1) || dev_alloc(&ctx->seq_dev, 1))
    return cleanup_fail(MOE_ENOMEM);
  if (prefill_needs_act_operands(c.wfmt, c.afmt) &&
      dev_alloc(reinterpret_cast<uint8_t**>(&ctx->xo), (size_t)c.max_tokens * H * 2))
    return cleanup_fail(MOE_ENOMEM);
  ctx->cnt = ctx->step_dev;
  ctx->fill_key = ctx->cnt + C_COUNT;
  ctx->fill_slot = ctx->fill_key + E;
  ctx->cpu_key = ctx->fill_slot + E;
  ctx->u_key = ctx->cpu_key + E;
  ctx->u_kind = ctx->u_key + E;
  if (hipMemset(ctx->slot_of, 0xff, (size_t)L * E * 4) || hipMemset(ctx->key_of, 0xff, kMaxCachedSlots * 4) ||
      hipMemset(ctx->stamp, 0, kMaxCachedSlots * 8) || hipMemset(ctx->reserved, 0, kMaxCachedSlots) ||
      hipMemset(ctx->counter, 0, 8) || hipMemset(ctx->dstats, 0, D_COUNT * 8) || hipMemset(ctx->seq_dev, 0, 4) ||
      hipMemset(ctx->step_dev, 0, (C_COUNT + 5 * E) * 4))
    return cleanup_fail(MOE_EHIP);
  // pinned host staging
  if (hipHostMalloc(reinterpret_cast<void**>(&ctx->step_host), (C_COUNT + 5 * E) * 4, 0) ||
      hipHostMalloc(reinterpret_cast<void**>(&ctx->h_slot_idx), Pmax * 4, 0) ||
      hipHostMalloc(reinterpret_cast<void**>(&ctx->h_w), Pmax * 4, 0) ||
      hipHostMalloc(&ctx->h_x, (size_t)c.max_tokens * H * 4, 0) ||
      hipHostMalloc(reinterpret_cast<void**>(&ctx->h_xf), (size_t)c.max_tokens * H * 4, 0) ||
      hipHostMalloc(reinterpret_cast<void**>(&ctx->h_y), (size_t)c.max_tokens * H * 4, 0) ||
      hipHostMalloc(reinterpret_cast<void**>(&ctx->h_hbuf), (size_t)Pmax * I * 4, 0) ||
      hipHostMalloc(reinterpret_cast<void**>(&ctx->sig_host), 256, 0))
    return cleanup_fail(MOE_ENOMEM);
  std::memset(ctx->sig_host, 0, 256);
  {  // device addresses of the staging the step-staging kernel writes (optional)
    void *a = nullptr, *b = nullptr, *c2 = nullptr, *d = nullptr;
    if (hipHostGetDevicePointer(&a, ctx->step_host, 0) == hipSuccess &&
        hipHostGetDevicePointer(&b, ctx->h_x, 0) == hipSuccess && hipHostGetDevicePointer(&c2, ctx->h_w, 0) == hipSuccess &&
        hipHostGetDevicePointer(&d, ctx->h_slot_idx, 0) == hipSuccess) {
      ctx->step_host_dev = static_cast<int32_t*>(a);
      ctx->h_x_dev = b;
      ctx->h_w_dev = static_cast<float*>(c2);
      ctx->h_slot_idx_dev = static_cast<int32_t*>(d);
    }
    void *g = nullptr, *yh = nullptr;
    if (hipHostGetDevicePointer(&g, ctx->sig_host, 0) == hipSuccess &&
        hipHostGetDevicePointer(&yh, ctx->h_y, 0) == hipSuccess) {
      ctx->sig_dev = static_cast<uint32_t*>(g);
      ctx->h_y_dev = static_cast<float*>(yh);
    }
    (void)hipGetLastError();
  }
  {
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, ctx->device) != hipSuccess || khz <= 0)
      khz = 100000;  // 100 MHz, the rate of the device's constant wall clock
    ctx->wall_khz = khz;
  }
  ctx->h_cnt = ctx->step_host;
  ctx->h_fill_key = ctx->h_cnt + C_COUNT;
  ctx->h_fill_slot = ctx->h_fill_key + E;
  ctx->h_cpu_key = ctx->h_fill_slot + E;
  ctx->h_u_key = ctx->h_cpu_key + E;
  ctx->h_u_kind = ctx->h_u_key + E;
  std::memset(ctx->h_cnt, 0, C_COUNT * 4);
  if (hipStreamCreateWithFlags(&ctx->copy_stream, hipStreamNonBlocking) ||
      hipEventCreateWithFlags(&ctx->ev_sync, hipEventDisableTiming) ||
      hipEventCreateWithFlags(&ctx->ev_fill, hipEventDisableTiming) ||
      hipEventCreateWithFlags(&ctx->ev_ycpu, hipEventDisableTiming) ||
      hipEventCreateWithFlags(&ctx->ev_layer_copied[0], hipEventDisableTiming) ||
      hipEventCreateWithFlags(&ctx->ev_layer_copied[1], hipEventDisableTiming) ||
      hipEventCreateWithFlags(&ctx->ev_layer_done[0], hipEventDisableTiming) ||
      hipEventCreateWithFlags(&ctx->ev_layer_done[1], hipEventDisableTiming))
    return cleanup_fail(MOE_EHIP);
  if (write_ctrl(ctx) != MOE_OK) return cleanup_fail(MOE_EHIP);
  *out = ctx;
  return MOE_OK;
}

MOE_API moe_status moe_destroy(moe_ctx* ctx) {
  if (!ctx) return MOE_EINVAL;
  if (ctx->copy_stream) hipStreamSynchronize(ctx->copy_stream);
  hipDeviceSynchronize();  // a captured step's wait for its branch ends first (bounded)
  if (ctx->branch_thread.joinable()) {
    ctx->branch_stop.store(true, std::memory_order_release);
    ctx->branch_thread.join();
  }
  delete ctx->cpu;
  ctx->cpu = nullptr;
  for (auto& t : ctx->pending_timed) {
    hipEventDestroy(t.a);
    hipEventDestroy(t.b);
  }
  for (auto e : ctx->event_pool) hipEventDestroy(e);
  void* dev[] = {ctx->slot_of, ctx->key_of, ctx->stamp, ctx->reserved, ctx->counter, ctx->step_dev,
                 ctx->u_slot, ctx->u_evict, ctx->grp_slot, ctx->grp_pair0, ctx->slot_scratch, ctx->pair_grp, ctx->logits, ctx->h, ctx->h16, ctx->dpair, ctx->y_cpu_dev,
                 ctx->perm, ctx->inv, ctx->offsets, ctx->tile_base, ctx->tiles, ctx->hist, ctx->cand, ctx->act, ctx->ypair,
                 ctx->flags, ctx->xo, ctx->dstats, ctx->ctrl, ctx->seq_dev};
  for (void* p : dev)
    if (p) hipFree(p);
  void* host[] = {ctx->step_host, ctx->h_slot_idx, ctx->h_w, ctx->h_x, ctx->h_xf, ctx->h_y, ctx->h_hbuf, ctx->sig_host};
  for (void* p : host)
    if (p) hipHostFree(p);
  if (ctx->pool_owned && ctx->pool) hipHostFree(ctx->pool);
  hipEvent_t evs[] = {ctx->ev_sync, ctx->ev_fill, ctx->ev_ycpu, ctx->ev_layer_copied[0],
                      ctx->ev_layer_copied[1],
                      ctx->ev_layer_done[0], ctx->ev_layer_done[1]};
  for (auto e : evs)
    if (e) hipEventDestroy(e);
  if (ctx->copy_stream) hipStreamDestroy(ctx->copy_stream);
  delete ctx;
  return MOE_OK;
}

MOE_API moe_status moe_pool_alloc(moe_ctx* ctx, int64_t n_records, void** host_pool) {
  if (!ctx || !host_pool) return MOE_EINVAL;
  const int64_t nkeys = (int64_t)ctx->cfg.n_layers * ctx->cfg.n_experts;
  CHECK_ARG(n_records >= 1 && n_records <= nkeys, "n_records must be in [1, L*E]");
  CHECK_ARG(!ctx->pool, "a pool is already set");
  void* p = nullptr;
  HIPCHK(hipHostMalloc(&p, (size_t)n_records * ctx->S, 0));
  void* pd = nullptr;
  if (hipHostGetDevicePointer(&pd, p, 0) != hipSuccess) {
    hipHostFree(p);
    return fail(ctx, MOE_EHIP, "page-locked pool without a device mapping");
  }
  ctx->pool_dev = static_cast<const uint8_t*>(pd);
  ctx->pool = static_cast<uint8_t*>(p);
  ctx->pool_records = n_records;
  ctx->pool_owned = true;
  ctx->pool_pinned = true;
  *host_pool = p;
  return MOE_OK;
}

MOE_API moe_status moe_pool_register(moe_ctx* ctx, void* host_pool, int64_t n_records, int32_t pinned) {
  if (!ctx) return MOE_EINVAL;
  const int64_t nkeys = (int64_t)ctx->cfg.n_layers * ctx->cfg.n_experts;
  CHECK_ARG(host_pool && n_records >= 1 && n_records <= nkeys, "bad pool");
  CHECK_ARG(!ctx->pool, "a pool is already set");
  ctx->pool = static_cast<uint8_t*>(host_pool);
  ctx->pool_records = n_records;
  ctx->pool_owned = false;
  ctx->pool_pinned = pinned != 0;
  if (!ctx->pool_pinned && ctx->cfg.mode != MOE_MODE_CPU)
    return fail(ctx, MOE_ENOPIN, "pageable pool: only MOE_MODE_CPU can run (every expert on the host)");
  if (ctx->pool_pinned) {  // a device mapping enables device fills; without one they are refused
    void* pd = nullptr;
    if (hipHostGetDevicePointer(&pd, host_pool, 0) == hipSuccess) ctx->pool_dev = static_cast<const uint8_t*>(pd);
    else (void)hipGetLastError();
  }
  return MOE_OK;
}

MOE_API moe_status moe_bind(moe_ctx* ctx, const float* router_w, void* arena, size_t arena_bytes, int32_t n_slots) {
  if (!ctx) return MOE_EINVAL;
  CHECK_ARG(router_w, "router weights required");
  CHECK_ARG(!ctx->in_prefill, "bind inside prefill");
  const int64_t nkeys = (int64_t)ctx->cfg.n_layers * ctx->cfg.n_experts;
  if (ctx->cfg.mode == MOE_MODE_FUSED) {
    CHECK_ARG(n_slots >= nkeys, "FUSED mode needs n_slots >= L*E");
  } else {
    CHECK_ARG(n_slots >= 0 && n_slots <= kMaxCachedSlots, "n_slots must be in [0, 4096]");
  }
  CHECK_ARG(n_slots == 0 || (arena && arena_bytes >= (size_t)n_slots * ctx->S), "arena too small");
  HIPCHK(hipDeviceSynchronize());
  HIPCHK(hipMemset(ctx->slot_of, 0xff, (size_t)nkeys * 4));
  HIPCHK(hipMemset(ctx->key_of, 0xff, kMaxCachedSlots * 4));
  HIPCHK(hipMemset(ctx->stamp, 0, kMaxCachedSlots * 8));
  HIPCHK(hipMemset(ctx->reserved, 0, kMaxCachedSlots));
  HIPCHK(hipMemset(ctx->counter, 0, 8));
  HIPCHK(hipDeviceSynchronize());
  ctx->router_w = router_w;
  ctx->arena = static_cast<uint8_t*>(arena);
  ctx->arena_bytes = arena_bytes;
  ctx->n_slots = n_slots;
  ctx->bound = true;
  ctx->last_lookup_layer = -1;
  return write_ctrl(ctx);
}

MOE_API moe_status moe_fused_load(moe_ctx* ctx, moe_stream_t stream) {
  if (!ctx) return MOE_EINVAL;
  CHECK_ARG(ctx->bound && ctx->pool, "bind and pool first");
  CHECK_ARG(ctx->cfg.mode == MOE_MODE_FUSED, "FUSED mode only");
  const int64_t nkeys = (int64_t)ctx->cfg.n_layers * ctx->cfg.n_experts;
  HIPCHK(copy_keys(ctx, 0, nkeys, 0, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

MOE_API moe_status moe_set_bandwidths(moe_ctx* ctx, uint64_t bw_pcie, uint64_t bw_host) {
  if (!ctx) return MOE_EINVAL;
  CHECK_ARG(bw_pcie > 0 && bw_host > 0 && bw_pcie < (1ull << 53) && bw_host < (1ull << 53), "bandwidths out of range");
  ctx->cfg.bw_pcie = bw_pcie;
  ctx->cfg.bw_host = bw_host;
  return write_ctrl(ctx);
}

MOE_API moe_status moe_set_mode(moe_ctx* ctx, int32_t mode) {
  if (!ctx) return MOE_EINVAL;
  CHECK_ARG(valid_mode(mode), "bad mode");
  CHECK_ARG((mode == MOE_MODE_FUSED) == (ctx->cfg.mode == MOE_MODE_FUSED), "FUSED <-> cached needs a new context");
  CHECK_ARG(ctx->pool_pinned || mode == MOE_MODE_CPU, "pageable pool: only MOE_MODE_CPU");
  ctx->cfg.mode = mode;
  return write_ctrl(ctx);
}

MOE_API moe_status moe_set_cpu_wait(moe_ctx* ctx, double timeout_ms) {
  if (!ctx) return MOE_EINVAL;
  CHECK_ARG(timeout_ms > 0.0 && timeout_ms <= 60000.0, "timeout_ms must be in (0, 60000]");
  ctx->cpu_wait_ms = timeout_ms;
  return write_ctrl(ctx);
}

MOE_API moe_status moe_route(moe_ctx* ctx, int32_t layer, const void* x, int32_t T, const float* logit_bias,
                             float* logits_out, int32_t* topk_idx, float* topk_w, moe_stream_t stream) {
  if (!ctx) return MOE_EINVAL;
  CHECK_ARG(ctx->router_w, "bind router weights first");
  CHECK_ARG(layer >= 0 && layer < ctx->cfg.n_layers, "layer out of range");
  CHECK_ARG(T >= 1 && T <= ctx->cfg.max_tokens, "T out of range");
  CHECK_ARG(x && topk_idx && topk_w, "null pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int E = ctx->cfg.n_experts, H = ctx->cfg.hidden;
  float* z = logits_out ? logits_out : ctx->logits;
  launch_route_logits(x, ctx->cfg.afmt, ctx->router_w + (int64_t)layer * E * H, logit_bias, z, T, E, H, s);
  launch_topk(z, T, E, ctx->cfg.top_k, ctx->cfg.renorm, topk_idx, topk_w, s);
  HIPCHK(hipGetLastError());
  return MOE_OK;
}

MOE_API moe_status moe_topk(moe_ctx* ctx, const float* logits, int32_t T, int32_t* topk_idx, float* topk_w,
                            moe_stream_t stream) {
  if (!ctx) return MOE_EINVAL;
  CHECK_ARG(T >= 1 && logits && topk_idx && topk_w, "bad arguments");
  launch_topk(logits, T, ctx->cfg.n_experts, ctx->cfg.top_k, ctx->cfg.renorm, topk_idx, topk_w,
              static_cast<hipStream_t>(stream));
  HIPCHK(hipGetLastError());
  return MOE_OK;
}

MOE_API moe_status expert_cache_lookup(moe_ctx* ctx, int32_t layer, const int32_t* topk_idx, int32_t T,
                                       int32_t* slot_idx, moe_trace_rec* trace, int32_t* counts, moe_stream_t stream) {
  if (!ctx) return MOE_EINVAL;
  CHECK_ARG(ctx->bound, "bind first");
  CHECK_ARG(!ctx->in_prefill, "decode lookup inside prefill");
  CHECK_ARG(layer >= 0 && layer < ctx->cfg.n_layers, "layer out of range");
  CHECK_ARG(T >= 1 && T <= ctx->cfg.max_tokens, "T out of range");
  CHECK_ARG(topk_idx && slot_idx, "null pointer");
  LookupArgs a;
  fill_lookup_args(ctx, a, layer, topk_idx, T, lookup_mode_of(ctx->cfg.mode));
  a.mode_from_ctrl = 1;
  a.slot_idx = slot_idx;
  a.trace = trace;
  a.counts_out = counts;
  launch_lookup(a, static_cast<hipStream_t>(stream));
  HIPCHK(hipGetLastError());
  ctx->last_lookup_layer = layer;
  ctx->last_lookup_T = T;
  return MOE_OK;
}

MOE_API moe_status moe_route_lookup(moe_ctx* ctx, int32_t layer, const void* x, int32_t T, const float* logit_bias,
                                    float* logits_out, int32_t* topk_idx, float* topk_w, int32_t* slot_idx,
                                    moe_trace_rec* trace, int32_t* counts, moe_stream_t stream) {
  if (!ctx) return MOE_EINVAL;
  CHECK_ARG(ctx->bound && ctx->router_w, "bind first");
  CHECK_ARG(!ctx->in_prefill, "decode lookup inside prefill");
  CHECK_ARG(layer >= 0 && layer < ctx->cfg.n_layers, "layer out of range");
  CHECK_ARG(T >= 1 && T <= ctx->cfg.max_tokens, "T out of range");
  CHECK_ARG(x && topk_idx && topk_w && slot_idx, "null pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int E = ctx->cfg.n_experts, H = ctx->cfg.hidden, k = ctx->cfg.top_k;
  float* z = logits_out ? logits_out : ctx->logits;
  launch_route_logits(x, ctx->cfg.afmt, ctx->router_w + (int64_t)layer * E * H, logit_bias, z, T, E, H, s);
  LookupArgs a;
  fill_lookup_args(ctx, a, layer, topk_idx, T, lookup_mode_of(ctx->cfg.mode));
  a.mode_from_ctrl = 1;
  if (T * k <= kSmallLookupPairs && T <= kLookupThreads / 64) {
    // the lookup kernel takes the top k from the logits itself: one launch fewer
    a.topk_idx = nullptr;
    a.logits = z;
    a.topk_out = topk_idx;
    a.topk_w = topk_w;
    a.renorm = ctx->cfg.renorm;
  } else {
    launch_topk(z, T, E, k, ctx->cfg.renorm, topk_idx, topk_w, s);
  }
  a.slot_idx = slot_idx;
  a.trace = trace;
  a.counts_out = counts;
  launch_lookup(a, s);
  HIPCHK(hipGetLastError());
  ctx->last_lookup_layer = layer;
  ctx->last_lookup_T = T;
  return MOE_OK;
}

MOE_API moe_status moe_decode_layer(moe_ctx* ctx, int32_t layer, const void* x, int32_t T, const float* logit_bias,
                                    int32_t* topk_idx, float* topk_w, int32_t* slot_idx, float* y, moe_stream_t stream) {
  if (!ctx) return MOE_EINVAL;
  CHECK_ARG(ctx->bound && ctx->router_w, "bind first");
  CHECK_ARG(!ctx->in_prefill, "decode inside prefill");
  CHECK_ARG(layer >= 0 && layer < ctx->cfg.n_layers, "layer out of range");
  CHECK_ARG(x && topk_idx && topk_w && slot_idx && y, "null pointer");
  CHECK_ARG(T >= 1 && T <= kDecodeMaxTok && T <= ctx->cfg.max_tokens && (int64_t)T * ctx->cfg.hidden <= kDecodeMaxTH,
            "decode needs T <= 8, T <= max_tokens and T*H <= 16384");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int k = ctx->cfg.top_k, E = ctx->cfg.n_experts, H = ctx->cfg.hidden, I = ctx->cfg.inter;
  if (ctx->cfg.mode == MOE_MODE_FUSED && T == 1 && decode_phase1_routed_ok(ctx->cfg.wfmt, ctx->cfg.afmt, H, k)) {
    // all resident, one token: the lookup is the identity, so phase 1 routes itself and
    // the step takes four launches: router GEMV, phase 1, phase 2, combine
    DecodeArgs d{};
    d.x = x;
    d.w = topk_w;
    d.ctrl = ctx->ctrl;
    d.rec_bytes = ctx->S;
    d.T = 1;
    d.k = k;
    d.H = H;
    d.I = I;
    d.grp_slot = ctx->grp_slot;
    d.grp_pair0 = ctx->grp_pair0;
    d.pair_grp = ctx->pair_grp;
    d.cnt = ctx->cnt;
    d.slot_idx = slot_idx;
    d.h = ctx->h;
    d.h16 = ctx->h16;
    d.d = ctx->dpair;
    d.y = y;
    d.logits = ctx->logits;
    d.E = E;
    d.renorm = ctx->cfg.renorm;
    d.layer = layer;
    d.topk_out = topk_idx;
    d.topk_w_out = topk_w;
    d.slot_out = slot_idx;
    d.grp_slot_out = ctx->grp_slot;
    d.grp_pair0_out = ctx->grp_pair0;
    d.pair_grp_out = ctx->pair_grp;
    d.cnt_out = ctx->cnt;
    launch_route_logits(x, ctx->cfg.afmt, ctx->router_w + (int64_t)layer * E * H, logit_bias, ctx->logits, 1, E, H, s);
    bool routed;
    {
      TimedScope t1(ctx, s, TK_P1);
      routed = launch_decode_phase1_routed(ctx->cfg.wfmt, ctx->cfg.afmt, d, s, t1.tm);
    }
    if (routed) {
      {
        TimedScope t2(ctx, s, TK_P2);
        if (!launch_decode_phase2_combine(ctx->cfg.wfmt, d, s, t2.tm)) {
          launch_decode_phase2(ctx->cfg.wfmt, d, k, s, t2.tm);
          launch_decode_combine(d, nullptr, s);
        }
      }
      HIPCHK(hipGetLastError());
      if ((ctx->cfg.flags & MOE_FLAG_PROFILE) && !capturing(s)) {
        const int64_t wrow_h = weight_row_bytes(ctx->cfg, H), wrow_i = weight_row_bytes(ctx->cfg, I);
        ctx->stats.phase1_launches += 1;
        ctx->stats.phase2_launches += 1;
        // h out as fp32 and bf16 (6 bytes a value); phase 2 reads one of them
        const uint64_t h_in = decode_phase2_reads_h16(ctx->cfg.wfmt, I, 1, k) ? 2 : 4;
        ctx->stats.phase1_bytes += (uint64_t)k * 2 * I * wrow_h + (uint64_t)H * act_bytes(ctx->cfg) + (uint64_t)k * I * 6;
        ctx->stats.phase2_bytes += (uint64_t)k * H * wrow_i + (uint64_t)k * I * h_in + (uint64_t)H * 4;
      }
      ctx->stats.lookups += 1;
      ctx->stats.hits += k;
      ctx->stats.decode_calls += 1;
      ctx->last_lookup_layer = -1;
      return MOE_OK;
    }
  }
  moe_status st = moe_route_lookup(ctx, layer, x, T, logit_bias, nullptr, topk_idx, topk_w, slot_idx, nullptr, nullptr,
                                   stream);
  if (st != MOE_OK) return st;
  return moe_ffn_decode(ctx, layer, x, T, topk_idx, topk_w, slot_idx, y, stream);
}

MOE_API moe_status moe_ffn_decode(moe_ctx* ctx, int32_t layer, const void* x, int32_t T, const int32_t* topk_idx,
                                  const float* topk_w, const int32_t* slot_idx, float* y, moe_stream_t stream) {
  if (!ctx) return MOE_EINVAL;
  CHECK_ARG(x && topk_idx && topk_w && slot_idx && y, "null pointer");
  CHECK_ARG(T >= 1 && T <= kDecodeMaxTok && (int64_t)T * ctx->cfg.hidden <= kDecodeMaxTH,
            "decode needs T <= 8 and T*H <= 16384 (use moe_ffn_prefill)");
  if (ctx->last_lookup_layer != layer || ctx->last_lookup_T != T)
    return fail(ctx, MOE_ESTATE, "moe_ffn_decode must follow expert_cache_lookup of the same layer and T");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int k = ctx->cfg.top_k, E = ctx->cfg.n_experts, H = ctx->cfg.hidden, I = ctx->cfg.inter;
  const int P = T * k;
  const bool fused = ctx->cfg.mode == MOE_MODE_FUSED;
  const bool captured = capturing(s);
  const bool profile = (ctx->cfg.flags & MOE_FLAG_PROFILE) != 0 && !captured;
  float* y_cpu = nullptr;
  const bool inputs = !fused && may_use_cpu(ctx, P);
  // device fills: no host read of the step (its counts and profiled bytes stay on the
  // device).  A step that may send work to the CPU hands it to the branch thread while the
  // stream is being captured (signal and bounded wait on the device, no host node).
  // Eagerly the calling thread reads the step and runs the branch itself; the fill kernel,
  // queued behind the step's copies to the host, moves the records meanwhile, so no host
  // round trip precedes the fills.
  const bool devfill_flag = (ctx->cfg.flags & MOE_FLAG_DEVICE_FILLS) && !fused;
  const bool async_cpu = devfill_flag && inputs && captured;
  const bool devfill = devfill_flag && (!inputs || captured);
  const bool devfill_host = devfill_flag && inputs && !captured && ctx->pool_dev;
  if (devfill && !ctx->pool_dev) return fail(ctx, MOE_ENOPIN, "device fills need a mapped page-locked pool");
  // a profiled step whose lists the host reads is logged with its split and branch times
  int64_t log_rec = -1;
  if (profile && !fused && !devfill && ctx->step_log.size() < kStepLogMax) {
    ctx->step_log.push_back(moe_step_rec{layer, 0, 0, 0, 0.0, 0.0});
    log_rec = (int64_t)ctx->step_log.size() - 1;
  }
  const double cpu_ms0 = ctx->stats.cpu_ms;
  if (captured && !fused && !devfill)
    return fail(ctx, MOE_ESTATE, "a captured decode step reads nothing on the host: use FUSED mode or a cached "
                                 "mode with MOE_FLAG_DEVICE_FILLS");
  if (devfill_host && ctx->step_host_dev) {
    // one staging launch writes the step block and the CPU branch's inputs straight into
    // the pinned staging, and the fill kernel follows it at once
    HIPCHK(hipEventSynchronize(ctx->ev_ycpu));  // the previous partial sum has left h_y's staging
    stage_step(ctx, x, topk_w, slot_idx, T, s);
    HIPCHK(hipEventRecord(ctx->ev_sync, s));
  } else if (devfill_host) {
    moe_status st = read_step_issue(ctx, s, true, x, topk_w, slot_idx, T);
    if (st != MOE_OK) return st;
  } else if ((!fused && !devfill) || (fused && profile)) {
    moe_status st = read_step(ctx, s, inputs, x, topk_w, slot_idx, T);
    if (st != MOE_OK) return st;
  }
  bool has_cpu = !fused && !devfill && !devfill_host && ctx->h_cnt[C_CPU] > 0;
  if (has_cpu && !inputs) {  // unexpected CPU work (e.g. every slot protected): fetch its inputs
    moe_status st = read_step(ctx, s, true, x, topk_w, slot_idx, T);
    if (st != MOE_OK) return st;
  }
  DecodeArgs d{};
  d.x = x;
  d.w = topk_w;
  d.ctrl = ctx->ctrl;
  d.rec_bytes = ctx->S;
  d.T = T;
  d.k = k;
  d.H = H;
  d.I = I;
  d.grp_slot = ctx->grp_slot;
  d.grp_pair0 = ctx->grp_pair0;
  d.pair_grp = ctx->pair_grp;
  d.cnt = ctx->cnt;
  d.slot_idx = slot_idx;
  d.h = ctx->h;
  d.h16 = ctx->h16;
  d.d = ctx->dpair;
  d.y = y;
  const int max_groups = std::min(P, E);
  if (async_cpu) {
    moe_status st = enqueue_cpu_branch(ctx, x, topk_w, slot_idx, T, s);
    if (st != MOE_OK) return st;
    y_cpu = ctx->y_cpu_dev;
  }
  if (devfill || devfill_host) {
    FillArgs f;
    f.cnt = ctx->cnt;
    f.fill_key = ctx->fill_key;
    f.fill_slot = ctx->fill_slot;
    f.pool = ctx->pool_dev;
    f.pool_records = ctx->pool_records;
    f.ctrl = ctx->ctrl;
    f.no_cpu_branch = devfill && !async_cpu;
    f.rec_bytes = ctx->S;
    f.dstats = devfill ? ctx->dstats : nullptr;  // a step the host reads is counted there
    const int64_t wrow_h = weight_row_bytes(ctx->cfg, H), wrow_i = weight_row_bytes(ctx->cfg, I);
    const bool dprof = profile && devfill;
    f.p1_grp = dprof ? (uint64_t)2 * I * wrow_h : 0;
    f.p1_fixed = dprof ? (uint64_t)T * H * act_bytes(ctx->cfg) : 0;
    f.p2_grp = dprof ? (uint64_t)H * wrow_i : 0;
    f.p2_fixed = dprof ? (uint64_t)T * H * 4 : 0;
    f.p1_pair = dprof ? (uint64_t)I * 6 : 0;  // h out, fp32 and bf16
    f.p2_pair = dprof ? (uint64_t)I * (decode_phase2_reads_h16(ctx->cfg.wfmt, I, T, k) ? 2 : 4) : 0;
    TimedScope tf(ctx, s, log_rec >= 0 ? TK_FILL : -1, false, log_rec);
    launch_fill_pull(f, max_groups, s, tf.tm);
  } else if (!fused) {
    moe_status st = issue_fills(ctx, s, log_rec);
    if (st != MOE_OK) return st;
  }
  {
    TimedScope t1(ctx, s, TK_P1);
    launch_decode_phase1(ctx->cfg.wfmt, ctx->cfg.afmt, d, max_groups, s, t1.tm);
  }
  // one token with no CPU branch possible: phase 2 and the combine in one launch
  const bool p2c = T == 1 && !inputs && !has_cpu && !async_cpu;
  bool combined = false;
  {
    TimedScope t2(ctx, s, TK_P2);
    if (p2c) combined = launch_decode_phase2_combine(ctx->cfg.wfmt, d, s, t2.tm);
    if (!combined) launch_decode_phase2(ctx->cfg.wfmt, d, max_groups, s, t2.tm);
  }
  if (devfill_host) {  // the GPU path (fills included) is enqueued: read the step now
    moe_status st = read_step_finish(ctx);
    if (st != MOE_OK) return st;
    has_cpu = ctx->h_cnt[C_CPU] > 0;
    if (ctx->h_cnt[C_FILL] > 0) ctx->stats.fill_bytes += (uint64_t)ctx->h_cnt[C_FILL] * ctx->S;
  }
  if (has_cpu) {
    // the GPU path is enqueued; the CPU branch runs now, concurrently, then merges exactly
    moe_status st = run_cpu_branch(ctx, T, s, &y_cpu);
    if (st != MOE_OK) return st;
  }
  if (async_cpu) join_cpu_branch(ctx, T, s);
  if (!combined) launch_decode_combine(d, y_cpu, s);
  if (log_rec >= 0) {
    moe_step_rec& r = ctx->step_log[log_rec];
    r.fills = ctx->h_cnt[C_FILL];
    r.cpu = ctx->h_cnt[C_CPU];
    r.misses = r.fills + r.cpu;
    r.cpu_ms = ctx->stats.cpu_ms - cpu_ms0;
  }
  HIPCHK(hipGetLastError());
  if (profile && devfill) {  // bytes are added on the device
    ctx->stats.phase1_launches += 1;
    ctx->stats.phase2_launches += 1;
  } else if (profile) {
    const int ngrp = ctx->h_cnt[C_NGRP];
    const int64_t wrow_h = weight_row_bytes(ctx->cfg, H), wrow_i = weight_row_bytes(ctx->cfg, I);
    ctx->stats.phase1_launches += 1;
    ctx->stats.phase2_launches += 1;
    // algorithmic bytes: the GPU experts' gate+up rows, x once, h out (fp32 and bf16) / down
    // rows, h in (the copy phase 2 reads), y out
    const uint64_t npair = (uint64_t)ctx->h_cnt[C_NPAIR_GPU];
    const uint64_t h_in = decode_phase2_reads_h16(ctx->cfg.wfmt, I, T, k) ? 2 : 4;
    ctx->stats.phase1_bytes += (uint64_t)ngrp * 2 * I * wrow_h + (uint64_t)T * H * act_bytes(ctx->cfg) + npair * I * 6;
    ctx->stats.phase2_bytes += (uint64_t)ngrp * H * wrow_i + npair * I * h_in + (uint64_t)T * H * 4;
  }
  ctx->stats.decode_calls += 1;
  ctx->last_lookup_layer = -1;
  return MOE_OK;
}

// ---------------------------------------------------------------- prefill
namespace {

moe_status prefill_gpu_part(moe_ctx* ctx, const void* x, int T, const float* w, float* y, const int32_t* pair_gpu,
                            const float* y_cpu, bool do_combine, hipStream_t s) {
  const int k = ctx->cfg.top_k, E = ctx->cfg.n_experts, H = ctx->cfg.hidden, I = ctx->cfg.inter;
  const int P = T * k;
  const int bm = prefill_bm();
  launch_permute(ctx->pair_grp, ctx->cnt, P, E, ctx->hist, ctx->perm, ctx->inv, ctx->offsets, ctx->tile_base, bm, s);
  PrefillArgs a;
  a.x = x;
  a.xa = x;
  a.xs = nullptr;
  a.acts = nullptr;
  // MX prefill: activations as MXFP8 codes (xo) with their scales after them
  const bool mx = (ctx->cfg.flags & MOE_FLAG_MX_PREFILL) != 0;
  if (mx) {
    uint8_t* codes = reinterpret_cast<uint8_t*>(ctx->xo);
    launch_mx_quant(ctx->cfg.afmt, x, codes, codes + (int64_t)T * H, (int64_t)T * H, s);
    a.xa = codes;
    a.xs = codes + (int64_t)T * H;
  } else if (prefill_needs_act_operands(ctx->cfg.wfmt, ctx->cfg.afmt)) {
    launch_act_operands(ctx->cfg.wfmt, ctx->cfg.afmt, x, ctx->xo, (int64_t)T * H, s);
    a.xa = ctx->xo;
  }
  a.w = w;
  a.arena = ctx->arena;
  a.rec_bytes = ctx->S;
  a.T = T;
  a.k = k;
  a.H = H;
  a.I = I;
  a.E = E;
  a.grp_slot = ctx->grp_slot;
  a.perm = ctx->perm;
  a.inv = ctx->inv;
  a.offsets = ctx->offsets;
  a.tile_base = ctx->tile_base;
  a.cnt = ctx->cnt;
  const int max_tiles_m = (P + bm - 1) / bm + std::min(E, P);
  a.tiles1 = ctx->tiles;
  a.tiles2 = ctx->tiles + ctx->tiles1_max;
  if (ctx->cfg.wfmt != MOE_WFMT_F32) launch_tile_tables(a, ctx->cfg.wfmt, mx, max_tiles_m, s);
  a.act = ctx->act;
  if (mx) a.acts = reinterpret_cast<uint8_t*>(ctx->act) + (int64_t)P * I;
  a.ypair = ctx->ypair;
  a.y = y;
  a.y_cpu = y_cpu;
  a.pair_gpu = pair_gpu;
  {
    TimedScope t(ctx, s, TK_G1);
    if (mx) launch_prefill_gemm1_mx(a, max_tiles_m, s, t.tm);
    else launch_prefill_gemm1(ctx->cfg.wfmt, ctx->cfg.afmt, a, max_tiles_m, s, t.tm);
  }
  {
    TimedScope t(ctx, s, TK_G2);
    if (mx) launch_prefill_gemm2_mx(a, max_tiles_m, s, t.tm);
    else launch_prefill_gemm2(ctx->cfg.wfmt, a, max_tiles_m, s, t.tm);
  }
  if (ctx->cfg.flags & MOE_FLAG_PROFILE) {
    ctx->stats.gemm1_launches += 1;
    ctx->stats.gemm2_launches += 1;
  }
  if (do_combine) launch_prefill_combine(a, s);
  HIPCHK(hipGetLastError());
  return MOE_OK;
}

// Write the caller's trace (device) from host records.
moe_status put_trace(moe_ctx* ctx, moe_trace_rec* trace, const std::vector<moe_trace_rec>& recs, hipStream_t s) {
  if (!trace || recs.empty()) return MOE_OK;
  HIPCHK(hipMemcpyAsync(trace, recs.data(), recs.size() * sizeof(moe_trace_rec), hipMemcpyHostToDevice, s));
  HIPCHK(hipStreamSynchronize(s));
  return MOE_OK;
}

moe_status put_counts(moe_ctx* ctx, int32_t* counts, const int32_t v[4], hipStream_t s) {
  if (!counts) return MOE_OK;
  HIPCHK(hipMemcpyAsync(counts, v, 4 * sizeof(int32_t), hipMemcpyHostToDevice, s));
  HIPCHK(hipStreamSynchronize(s));
  return MOE_OK;
}

}  // namespace

MOE_API moe_status moe_prefill_begin(moe_ctx* ctx, moe_stream_t stream) {
  if (!ctx) return MOE_EINVAL;
  CHECK_ARG(ctx->bound, "bind first");
  if (ctx->in_prefill) return fail(ctx, MOE_ESTATE, "prefill already begun");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int E = ctx->cfg.n_experts, L = ctx->cfg.n_layers;
  ctx->in_prefill = true;
  ctx->prefill_buffers = false;
  ctx->buffer_layer[0] = ctx->buffer_layer[1] = -1;
  ctx->next_prefill_layer = 0;
  const int mode = ctx->cfg.mode;
  if ((mode == MOE_MODE_OFFLOAD || mode == MOE_MODE_HYBRID) && ctx->n_slots >= 2 * E) {
    if (!ctx->pool_pinned) return fail(ctx, MOE_ENOPIN, "prefill buffers need a page-locked pool");
    HIPCHK(hipStreamSynchronize(s));
    launch_evict_range(ctx->slot_of, ctx->key_of, ctx->stamp, ctx->reserved, 0, 2 * E, 1, s);
    HIPCHK(hipGetLastError());
    HIPCHK(hipStreamSynchronize(s));
    ctx->prefill_buffers = true;
    for (int l = 0; l < std::min(2, L); ++l) {
      TimedScope ts(ctx, ctx->copy_stream, TK_COPY, true);
      HIPCHK(copy_keys(ctx, (int64_t)l * E, E, (int64_t)(l % 2) * E, ctx->copy_stream));
      HIPCHK(hipEventRecord(ctx->ev_layer_copied[l % 2], ctx->copy_stream));
      ctx->stats.copy_bytes += (uint64_t)E * ctx->S;
    }
  }
  return MOE_OK;
}

MOE_API moe_status moe_ffn_prefill(moe_ctx* ctx, int32_t layer, const void* x, int32_t T, const int32_t* topk_idx,
                                   const float* topk_w, float* y, moe_trace_rec* trace, int32_t* counts,
                                   moe_stream_t stream) {
  if (!ctx) return MOE_EINVAL;
  if (!ctx->in_prefill) return fail(ctx, MOE_ESTATE, "moe_prefill_begin first");
  CHECK_ARG(layer >= 0 && layer < ctx->cfg.n_layers, "layer out of range");
  CHECK_ARG(T >= 1 && T <= ctx->cfg.max_tokens, "T out of range");
  CHECK_ARG(x && topk_idx && topk_w && y, "null pointer");
  if (ctx->cfg.wfmt != MOE_WFMT_F32 && (ctx->cfg.hidden % 256 || ctx->cfg.inter % 128))
    return fail(ctx, MOE_ENOTSUP, "MFMA prefill needs hidden % 256 == 0 and inter % 128 == 0");
  // the bf16 GEMMs (LDS-staged) hold byte offsets of activations and records in 32 bits
  if (ctx->cfg.wfmt == MOE_WFMT_BF16 &&
      ((int64_t)T * ctx->cfg.hidden >= (1ll << 31) || (int64_t)T * ctx->cfg.top_k * ctx->cfg.inter >= (1ll << 31) ||
       ctx->S >= (1ll << 32)))
    return fail(ctx, MOE_ENOTSUP, "bf16 prefill needs T * hidden and T * top_k * inter below 2^31, records below 4 GiB");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int k = ctx->cfg.top_k, E = ctx->cfg.n_experts, L = ctx->cfg.n_layers, P = T * k;
  const int mode = ctx->cfg.mode;
  ctx->stats.prefill_calls += 1;
  if (ctx->cfg.flags & MOE_FLAG_PROFILE) ctx->stats.gemm_flops += 2.0 * P * 3.0 * ctx->cfg.hidden * ctx->cfg.inter;

  if (ctx->prefill_buffers) {
    if (layer != ctx->next_prefill_layer)
      return fail(ctx, MOE_ESTATE, "buffered prefill runs layers 0..L-1 in ascending order");
    const int b = layer % 2;
    HIPCHK(hipStreamWaitEvent(s, ctx->ev_layer_copied[b], 0));
    LookupArgs a;
    fill_lookup_args(ctx, a, layer, topk_idx, T, LK_BUFFER);
    a.buffer_base = b * E;
    a.slot_idx = ctx->slot_scratch;
    a.trace = trace;
    a.counts_out = counts;
    launch_lookup(a, s);
    moe_status st = prefill_gpu_part(ctx, x, T, topk_w, y, nullptr, nullptr, true, s);
    if (st != MOE_OK) return st;
    HIPCHK(hipEventRecord(ctx->ev_layer_done[b], s));
    ctx->buffer_layer[b] = layer;
    if (layer + 2 < L) {
      HIPCHK(hipStreamWaitEvent(ctx->copy_stream, ctx->ev_layer_done[b], 0));
      TimedScope ts(ctx, ctx->copy_stream, TK_COPY, true);
      HIPCHK(copy_keys(ctx, (int64_t)(layer + 2) * E, E, (int64_t)b * E, ctx->copy_stream));
      HIPCHK(hipEventRecord(ctx->ev_layer_copied[b], ctx->copy_stream));
      ctx->stats.copy_bytes += (uint64_t)E * ctx->S;
    }
    ctx->next_prefill_layer = layer + 1;
    return MOE_OK;
  }

  if (mode == MOE_MODE_FUSED || mode == MOE_MODE_CPU) {
    LookupArgs a;
    fill_lookup_args(ctx, a, layer, topk_idx, T, lookup_mode_of(mode));
    a.slot_idx = ctx->slot_scratch;
    a.trace = trace;
    a.counts_out = counts;
    launch_lookup(a, s);
    HIPCHK(hipGetLastError());
    float* y_cpu = nullptr;
    if (mode == MOE_MODE_CPU) {
      moe_status st = read_step(ctx, s, true, x, topk_w, ctx->slot_scratch, T);
      if (st != MOE_OK) return st;
      // GPU part for the hits first, then the CPU branch; the combine adds both
      st = prefill_gpu_part(ctx, x, T, topk_w, y, ctx->pair_grp, nullptr, false, s);
      if (st != MOE_OK) return st;
      st = run_cpu_branch(ctx, T, s, &y_cpu);
      if (st != MOE_OK) return st;
      PrefillArgs c{};
      c.w = topk_w;
      c.T = T;
      c.k = k;
      c.H = ctx->cfg.hidden;
      c.ypair = ctx->ypair;
      c.y = y;
      c.y_cpu = y_cpu;
      c.pair_gpu = ctx->pair_grp;
      launch_prefill_combine(c, s);
      HIPCHK(hipGetLastError());
      return MOE_OK;
    }
    return prefill_gpu_part(ctx, x, T, topk_w, y, ctx->pair_grp, y_cpu, true, s);
  }

  // On-demand prefill: offload lookups in rounds; a round's leftover misses wait for the next.
  if (ctx->n_slots == 0) return fail(ctx, MOE_ENOTSUP, "on-demand prefill needs at least one slot");
  if (!ctx->pool_pinned) return fail(ctx, MOE_ENOPIN, "fills need a page-locked host pool");
  std::vector<moe_trace_rec> final_recs;
  std::vector<int> pending;
  int32_t tot[4] = {0, 0, 0, 0};
  bool first = true;
  int guard = 0;
  while (first || !pending.empty()) {
    if (++guard > 4 * E + 4) return fail(ctx, MOE_ESTATE, "on-demand prefill did not converge");
    LookupArgs a;
    fill_lookup_args(ctx, a, layer, topk_idx, T, LK_OFFLOAD);
    a.slot_idx = ctx->slot_scratch;
    if (!first) {
      HIPCHK(hipMemcpyAsync(ctx->cand, pending.data(), pending.size() * 4, hipMemcpyHostToDevice, s));
      a.cand = ctx->cand;
      a.n_cand = (int)pending.size();
    }
    launch_lookup(a, s);
    HIPCHK(hipGetLastError());
    moe_status st = read_step(ctx, s, false, nullptr, nullptr, nullptr, T);
    if (st != MOE_OK) return st;
    const int nU = ctx->h_cnt[C_NU];
    std::vector<int32_t> u_slot(nU), u_evict(nU);
    HIPCHK(hipMemcpy(u_slot.data(), ctx->u_slot, nU * 4, hipMemcpyDeviceToHost));
    HIPCHK(hipMemcpy(u_evict.data(), ctx->u_evict, nU * 4, hipMemcpyDeviceToHost));
    pending.clear();
    for (int u = 0; u < nU; ++u) {
      const int kind = ctx->h_u_kind[u];
      if (kind == MOE_KIND_CPU) {
        pending.push_back(ctx->h_u_key[u]);
      } else {
        final_recs.push_back(moe_trace_rec{ctx->h_u_key[u], kind, u_slot[u], u_evict[u]});
      }
    }
    tot[0] += ctx->h_cnt[C_HIT];
    tot[1] += ctx->h_cnt[C_FILL];
    tot[3] += ctx->h_cnt[C_EVICT];
    st = issue_fills(ctx, s);
    if (st != MOE_OK) return st;
    st = prefill_gpu_part(ctx, x, T, topk_w, y, nullptr, nullptr, false, s);
    if (st != MOE_OK) return st;
    if (!pending.empty()) HIPCHK(hipStreamSynchronize(s));  // the next round may evict this round's slots
    first = false;
  }
  // records in U order of the first appearance over (token, rank) pairs
  {
    std::vector<int32_t> idx((size_t)P);
    HIPCHK(hipMemcpy(idx.data(), topk_idx, (size_t)P * 4, hipMemcpyDeviceToHost));
    std::vector<int> order;
    std::vector<char> seen(E, 0);
    for (int p = 0; p < P; ++p)
      if (idx[p] >= 0 && idx[p] < E && !seen[idx[p]]) {
        seen[idx[p]] = 1;
        order.push_back(layer * E + idx[p]);
      }
    std::vector<moe_trace_rec> sorted;
    for (int key : order)
      for (auto& r : final_recs)
        if (r.key == key) {
          sorted.push_back(r);
          break;
        }
    moe_status st = put_trace(ctx, trace, sorted, s);
    if (st != MOE_OK) return st;
  }
  moe_status st = put_counts(ctx, counts, tot, s);
  if (st != MOE_OK) return st;
  PrefillArgs a{};
  a.w = topk_w;
  a.T = T;
  a.k = k;
  a.H = ctx->cfg.hidden;
  a.ypair = ctx->ypair;
  a.y = y;
  launch_prefill_combine(a, s);
  HIPCHK(hipGetLastError());
  return MOE_OK;
}

MOE_API moe_status moe_prefill_end(moe_ctx* ctx, moe_stream_t stream) {
  if (!ctx) return MOE_EINVAL;
  if (!ctx->in_prefill) return fail(ctx, MOE_ESTATE, "no prefill in progress");
  hipStream_t s = static_cast<hipStream_t>(stream);
  HIPCHK(hipStreamSynchronize(ctx->copy_stream));
  HIPCHK(hipStreamSynchronize(s));
  const int E = ctx->cfg.n_experts;
  if (ctx->prefill_buffers) {
    std::vector<std::pair<int, int>> held;
    for (int b = 0; b < 2; ++b)
      if (ctx->buffer_layer[b] >= 0) held.push_back({ctx->buffer_layer[b], b});
    std::sort(held.begin(), held.end());
    for (auto& hb : held)
      launch_admit_buffer(ctx->slot_of, ctx->key_of, ctx->stamp, ctx->counter, hb.first, E, hb.second * E, s);
    launch_evict_range(ctx->slot_of, ctx->key_of, ctx->stamp, ctx->reserved, 0, 2 * E, 0, s);
    HIPCHK(hipGetLastError());
    HIPCHK(hipStreamSynchronize(s));
  }
  ctx->in_prefill = false;
  ctx->prefill_buffers = false;
  ctx->buffer_layer[0] = ctx->buffer_layer[1] = -1;
  ctx->last_lookup_layer = -1;
  return MOE_OK;
}

MOE_API moe_status moe_permute(moe_ctx* ctx, const int32_t* slot_idx, int32_t T, int32_t* perm, int32_t* offsets,
                               int32_t* group_slot, int32_t* n_groups, moe_stream_t stream) {
  if (!ctx) return MOE_EINVAL;
  CHECK_ARG(T >= 1 && T <= ctx->cfg.max_tokens, "T out of range");
  CHECK_ARG(slot_idx && perm && offsets && group_slot && n_groups, "null pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int P = T * ctx->cfg.top_k;
  const int nrange = (int)std::max<int64_t>((int64_t)ctx->cfg.n_layers * ctx->cfg.n_experts, kMaxCachedSlots);
  // groups are indexed by distinct slot; up to min(P, 1024) of them
  const int gmax = std::min(P, kMaxExperts);
  launch_groups_from_slots(slot_idx, P, ctx->pair_grp, group_slot, ctx->cnt, ctx->flags, nrange, gmax, nullptr, s);
  HIPCHK(hipMemcpyAsync(ctx->h_cnt, ctx->cnt, C_COUNT * 4, hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  if (ctx->h_cnt[C_ERR] == 1) return fail(ctx, MOE_EINVAL, "slot id out of range");
  if (ctx->h_cnt[C_ERR] == 2) return fail(ctx, MOE_ENOTSUP, "more than 1024 distinct slots");
  launch_permute(ctx->pair_grp, ctx->cnt, P, gmax, ctx->hist, perm, ctx->inv, offsets, ctx->tile_base, prefill_bm(), s);
  HIPCHK(hipMemcpyAsync(n_groups, ctx->cnt + C_NGRP, 4, hipMemcpyDeviceToDevice, s));
  HIPCHK(hipGetLastError());
  return MOE_OK;
}

MOE_API moe_status expert_cache_resize(moe_ctx* ctx, int32_t new_n_slots, void* new_arena, size_t new_arena_bytes,
                                       moe_stream_t stream) {
  if (!ctx) return MOE_EINVAL;
  if (ctx->in_prefill) return fail(ctx, MOE_ESTATE, "resize inside prefill");
  if (ctx->cfg.mode == MOE_MODE_FUSED) return fail(ctx, MOE_ENOTSUP, "FUSED mode has no cache to resize");
  CHECK_ARG(ctx->bound, "bind first");
  CHECK_ARG(new_n_slots >= 0 && new_n_slots <= kMaxCachedSlots, "n_slots must be in [0, 4096]");
  uint8_t* dst = new_arena ? static_cast<uint8_t*>(new_arena) : ctx->arena;
  const size_t dst_bytes = new_arena ? new_arena_bytes : ctx->arena_bytes;
  CHECK_ARG(new_n_slots == 0 || (dst && dst_bytes >= (size_t)new_n_slots * ctx->S), "arena too small");
  hipStream_t s = static_cast<hipStream_t>(stream);
  HIPCHK(hipStreamSynchronize(s));
  HIPCHK(hipStreamSynchronize(ctx->copy_stream));
  const int N = ctx->n_slots;
  const int64_t nkeys = (int64_t)ctx->cfg.n_layers * ctx->cfg.n_experts;
  std::vector<int32_t> key_of(std::max(N, 1));
  std::vector<uint64_t> stamp(std::max(N, 1));
  if (N > 0) {
    HIPCHK(hipMemcpy(key_of.data(), ctx->key_of, N * 4, hipMemcpyDeviceToHost));
    HIPCHK(hipMemcpy(stamp.data(), ctx->stamp, N * 8, hipMemcpyDeviceToHost));
  }
  std::vector<int> occupied;
  for (int sl = 0; sl < N; ++sl)
    if (key_of[sl] >= 0) occupied.push_back(sl);
  std::vector<std::pair<int, int>> moves;  // (old slot, new slot)
  if (new_n_slots < N) {
    std::vector<int> by_recency = occupied;
    std::sort(by_recency.begin(), by_recency.end(), [&](int a, int b) {
      return stamp[a] != stamp[b] ? stamp[a] > stamp[b] : a < b;
    });
    if ((int)by_recency.size() > new_n_slots) by_recency.resize(new_n_slots);
    std::sort(by_recency.begin(), by_recency.end());
    for (int i = 0; i < (int)by_recency.size(); ++i) moves.push_back({by_recency[i], i});
  } else {
    for (int sl : occupied) moves.push_back({sl, sl});
  }
  // move records: ascending old slots; a destination never precedes a source still unread
  for (auto& mv : moves) {
    if (mv.first == mv.second && dst == ctx->arena) continue;
    HIPCHK(hipMemcpyAsync(dst + (int64_t)mv.second * ctx->S, ctx->arena + (int64_t)mv.first * ctx->S, ctx->S,
                          hipMemcpyDeviceToDevice, s));
  }
  std::vector<int32_t> new_key(std::max(new_n_slots, 1), -1), slot_of(nkeys, -1);
  std::vector<uint64_t> new_stamp(std::max(new_n_slots, 1), 0);
  for (auto& mv : moves) {
    new_key[mv.second] = key_of[mv.first];
    new_stamp[mv.second] = stamp[mv.first];
    slot_of[key_of[mv.first]] = mv.second;
  }
  HIPCHK(hipMemcpyAsync(ctx->slot_of, slot_of.data(), nkeys * 4, hipMemcpyHostToDevice, s));
  HIPCHK(hipMemsetAsync(ctx->key_of, 0xff, kMaxCachedSlots * 4, s));
  HIPCHK(hipMemsetAsync(ctx->stamp, 0, kMaxCachedSlots * 8, s));
  HIPCHK(hipMemsetAsync(ctx->reserved, 0, kMaxCachedSlots, s));
  if (new_n_slots > 0) {
    HIPCHK(hipMemcpyAsync(ctx->key_of, new_key.data(), new_n_slots * 4, hipMemcpyHostToDevice, s));
    HIPCHK(hipMemcpyAsync(ctx->stamp, new_stamp.data(), new_n_slots * 8, hipMemcpyHostToDevice, s));
  }
  HIPCHK(hipStreamSynchronize(s));
  ctx->arena = dst;
  ctx->arena_bytes = dst_bytes;
  ctx->n_slots = new_n_slots;
  ctx->last_lookup_layer = -1;
  return write_ctrl(ctx);
}

MOE_API moe_status moe_bench_bw(moe_ctx* ctx, uint64_t* bw_pcie, uint64_t* bw_host) {
  if (!ctx) return MOE_EINVAL;
  CHECK_ARG(ctx->pool && bw_pcie && bw_host, "pool and outputs required");
  const int64_t S = ctx->S;
  const int nrec = (int)std::min<int64_t>(ctx->pool_records, 32);
  // B_P: pinned pool -> device, whole records
  uint8_t* scratch = nullptr;
  HIPCHK(hipMalloc(&scratch, (size_t)S * 2));
  hipEvent_t e0, e1;
  HIPCHK(hipEventCreate(&e0));
  HIPCHK(hipEventCreate(&e1));
  double best_p = 0.0;
  if (ctx->pool_pinned) {
    for (int rep = 0; rep < 3; ++rep) {
      HIPCHK(hipEventRecord(e0, ctx->copy_stream));
      for (int i = 0; i < 4 * nrec; ++i)
        HIPCHK(hipMemcpyAsync(scratch + (i & 1) * S, ctx->pool + (int64_t)(i % nrec) * S, S, hipMemcpyHostToDevice,
                              ctx->copy_stream));
      HIPCHK(hipEventRecord(e1, ctx->copy_stream));
      HIPCHK(hipEventSynchronize(e1));
      float ms = 0.f;
      HIPCHK(hipEventElapsedTime(&ms, e0, e1));
      if (rep > 0) best_p = std::max(best_p, (double)S * 4 * nrec / (ms * 1e-3));
    }
  }
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  hipFree(scratch);
  // B_H: the CPU branch at batch 1 over distinct records
  const int H = ctx->cfg.hidden, I = ctx->cfg.inter, k = ctx->cfg.top_k;
  const int ncpu = std::min(nrec, k);
  std::vector<float> x(H, 0.01f), w(k, 1.0f / k), y(H), h((size_t)k * I);
  std::vector<int32_t> sidx(k);
  for (int j = 0; j < k; ++j) sidx[j] = (j < ncpu) ? -1 - j : 0;
  double best_h = 0.0;
  for (int rep = 0; rep < 4; ++rep) {
    CpuFfnJob job;
    job.wfmt = ctx->cfg.wfmt;
    job.H = H;
    job.I = I;
    job.T = 1;
    job.k = k;
    job.rec_bytes = S;
    job.x = x.data();
    job.w = w.data();
    job.slot_idx = sidx.data();
    for (int c = 0; c < ncpu; ++c) job.rec.push_back(ctx->pool + (int64_t)((rep * ncpu + c) % nrec) * S);
    job.h = h.data();
    job.y = y.data();
    const auto t0 = std::chrono::steady_clock::now();
    cpu_ffn(cpu_pool(ctx), job);
    const double sec = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    if (rep > 0) best_h = std::max(best_h, (double)S * ncpu / sec);
  }
  *bw_pcie = (uint64_t)best_p;
  *bw_host = (uint64_t)best_h;
  return MOE_OK;
}

MOE_API moe_status moe_bench_hbm(const void* buf, size_t buf_bytes, size_t read_bytes, int32_t reps,
                                 double* seconds_out, moe_stream_t stream) {
  if (!buf || !seconds_out || reps < 1 || read_bytes < 16 || read_bytes > buf_bytes) return MOE_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Timing tm;
  if (hipEventCreate(&tm.start) != hipSuccess) return MOE_EHIP;
  if (hipEventCreate(&tm.stop) != hipSuccess) {
    hipEventDestroy(tm.start);
    return MOE_EHIP;
  }
  moe_status st = MOE_OK;
  const size_t span = buf_bytes - read_bytes + 1;
  for (int r = 0; r < reps && st == MOE_OK; ++r) {
    const size_t off = (size_t)(((unsigned __int128)r * read_bytes) % span) & ~(size_t)255;
    launch_read_probe(static_cast<const uint8_t*>(buf) + off, (int64_t)read_bytes, s, tm);
    float ms = 0.f;
    if (hipGetLastError() != hipSuccess || hipEventSynchronize(tm.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, tm.start, tm.stop) != hipSuccess)
      st = MOE_EHIP;
    seconds_out[r] = ms * 1e-3;
  }
  hipEventDestroy(tm.start);
  hipEventDestroy(tm.stop);
  return st;
}

MOE_API moe_status moe_cache_snapshot(moe_ctx* ctx, int32_t* slot_of, int32_t* key_of, uint64_t* stamp,
                                      uint64_t* counter, int32_t* n_slots) {
  if (!ctx) return MOE_EINVAL;
  HIPCHK(hipDeviceSynchronize());
  const int64_t nkeys = (int64_t)ctx->cfg.n_layers * ctx->cfg.n_experts;
  const int N = ctx->n_slots;
  const int Ncap = std::min(N, kMaxCachedSlots);
  if (slot_of) HIPCHK(hipMemcpy(slot_of, ctx->slot_of, nkeys * 4, hipMemcpyDeviceToHost));
  if (key_of && Ncap > 0) HIPCHK(hipMemcpy(key_of, ctx->key_of, Ncap * 4, hipMemcpyDeviceToHost));
  if (stamp && Ncap > 0) HIPCHK(hipMemcpy(stamp, ctx->stamp, Ncap * 8, hipMemcpyDeviceToHost));
  if (counter) HIPCHK(hipMemcpy(counter, ctx->counter, 8, hipMemcpyDeviceToHost));
  if (n_slots) *n_slots = N;
  return MOE_OK;
}

MOE_API moe_status moe_sync(moe_ctx* ctx, moe_stream_t stream) {
  if (!ctx) return MOE_EINVAL;
  HIPCHK(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
  uint64_t err = 0, nocpu = 0, waits = 0;
  HIPCHK(hipMemcpy(&err, ctx->dstats + D_ERR, 8, hipMemcpyDeviceToHost));
  HIPCHK(hipMemcpy(&nocpu, ctx->dstats + D_NOCPU, 8, hipMemcpyDeviceToHost));
  HIPCHK(hipMemcpy(&waits, ctx->dstats + D_CPUWAIT, 8, hipMemcpyDeviceToHost));
  const uint64_t zero = 0;
  if (err) {
    HIPCHK(hipMemcpy(ctx->dstats + D_ERR, &zero, 8, hipMemcpyHostToDevice));
    return fail(ctx, MOE_EINVAL, "expert id out of range in topk_idx (device-fill step)");
  }
  if (nocpu) {
    HIPCHK(hipMemcpy(ctx->dstats + D_NOCPU, &zero, 8, hipMemcpyHostToDevice));
    return fail(ctx, MOE_ESTATE, "a step without a CPU branch had experts sent to the CPU (a graph captured "
                                 "before a shrink or a mode change: capture it again)");
  }
  if (waits) {
    HIPCHK(hipMemcpy(ctx->dstats + D_CPUWAIT, &zero, 8, hipMemcpyHostToDevice));
    return fail(ctx, MOE_ETIMEDOUT, "a captured step's wait for its CPU branch expired (its CPU experts are "
                                    "missing from y)");
  }
  return MOE_OK;
}

MOE_API moe_status moe_get_stats(moe_ctx* ctx, moe_stats* out) {
  if (!ctx || !out) return MOE_EINVAL;
  drain_timed(ctx);
  *out = ctx->stats;
  // counts of device-fill steps live on the device
  HIPCHK(hipDeviceSynchronize());
  uint64_t d[D_COUNT];
  HIPCHK(hipMemcpy(d, ctx->dstats, sizeof d, hipMemcpyDeviceToHost));
  out->lookups += d[D_LOOKUP];
  out->hits += d[D_HIT];
  out->fills += d[D_FILL];
  out->cpu_experts += d[D_CPU];
  out->evictions += d[D_EVICT];
  out->fill_bytes += d[D_FILL] * (uint64_t)ctx->S;
  out->phase1_bytes += d[D_P1_BYTES];
  out->phase2_bytes += d[D_P2_BYTES];
  return MOE_OK;
}

MOE_API moe_status moe_step_log(moe_ctx* ctx, moe_step_rec* out, int32_t capacity, int32_t* n_out) {
  if (!ctx) return MOE_EINVAL;
  CHECK_ARG(n_out && capacity >= 0 && (out || capacity == 0), "bad arguments");
  HIPCHK(hipDeviceSynchronize());
  drain_timed(ctx);
  const int32_t n = (int32_t)std::min<size_t>((size_t)capacity, ctx->step_log.size());
  if (n > 0) std::memcpy(out, ctx->step_log.data(), (size_t)n * sizeof(moe_step_rec));
  ctx->step_log.clear();
  *n_out = n;
  return MOE_OK;
}

MOE_API moe_status moe_reset_stats(moe_ctx* ctx) {
  if (!ctx) return MOE_EINVAL;
  drain_timed(ctx);
  ctx->stats = moe_stats{};
  ctx->step_log.clear();
  HIPCHK(hipDeviceSynchronize());
  uint64_t d[D_COUNT];
  HIPCHK(hipMemcpy(d, ctx->dstats, sizeof d, hipMemcpyDeviceToHost));
  const uint64_t err = d[D_ERR], nocpu = d[D_NOCPU];  // pending errors stay pending for moe_sync
  for (auto& v : d) v = 0;
  d[D_ERR] = err;
  d[D_NOCPU] = nocpu;
  HIPCHK(hipMemcpy(ctx->dstats, d, sizeof d, hipMemcpyHostToDevice));
  return MOE_OK;
}

}  // extern "C"
