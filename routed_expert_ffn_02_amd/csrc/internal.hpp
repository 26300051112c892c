// Internal declarations of the routed-MoE library: context state, kernel
// launchers and device helpers.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <condition_variable>
#include <cstdint>
#include <functional>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/routed_moe.h"

namespace rmoe {

// ---------------------------------------------------------------- limits
constexpr int kMaxExperts = 1024;       // E (lookup kernel keeps per-expert tables in LDS)
constexpr int kMaxCachedSlots = 4096;   // slots of a cached (non-FUSED) context
constexpr int kLookupThreads = 1024;
constexpr int kSlotsPerThread = kMaxCachedSlots / kLookupThreads;
constexpr int kDecodeMaxTH = 16384;     // decode: T * H fp32 activations staged in 64 KiB of LDS
constexpr int kDecodeMaxTok = 8;        // decode: tokens routed to one expert within a call
constexpr int kSmallLookupPairs = 64;   // lookup steps of at most this many pairs take the one-wavefront path

// lookup counters (device int32 array)
enum {
  C_NU = 0, C_HIT = 1, C_FILL = 2, C_CPU = 3, C_EVICT = 4, C_NGRP = 5, C_M = 6, C_EV = 7,
  C_NPAIR_GPU = 8, C_ERR = 9, C_T = 10, C_COUNT = 16
};

// device-side step statistics of device-fill steps (uint64 array)
// D_NOCPU: steps whose lookup sent experts to the CPU although the step, as enqueued or
// captured, had no CPU branch (a graph replayed after a shrink or a mode change)
// D_CPUWAIT: captured steps whose bounded wait for the CPU branch's partial sum expired
enum { D_LOOKUP = 0, D_HIT = 1, D_FILL = 2, D_CPU = 3, D_EVICT = 4, D_ERR = 5, D_P1_BYTES = 6, D_P2_BYTES = 7,
       D_NOCPU = 8, D_CPUWAIT = 9, D_COUNT = 10 };

// Cache parameters the kernels read on the device when they run, not from their launch
// arguments, so a step captured into a graph and replayed sees the current values after
// expert_cache_resize, moe_set_mode and moe_set_bandwidths.
constexpr int kSigGo = 0, kSigDone = 32;  // words, 128 bytes apart

struct DevCtrl {
  uint8_t* arena;      // the bound slot arena
  int32_t n_slots;
  int32_t lk_mode;     // LookupMode of decode lookups (the context's backend mode)
  uint64_t bw_pcie, bw_host;
  uint64_t cpu_wait_ticks;  // bound of a captured step's wait for its CPU branch (wall-clock ticks)
};

enum LookupMode { LK_FUSED = 0, LK_OFFLOAD = 1, LK_CPU = 2, LK_HYBRID = 3, LK_BUFFER = 4 };

struct LookupArgs {
  const int32_t* topk_idx;   // [T,k] experts (or nullptr when cand is used or logits is set)
  const float* logits;       // [T,E]: the kernel takes the top k itself (decode-sized steps), or nullptr
  int32_t* topk_out;         // [T,k] experts and
  float* topk_w;             // [T,k] gates written with the top k (logits set)
  int32_t renorm;
  const int32_t* cand;       // candidate key list (on-demand prefill rounds) or nullptr
  int32_t n_cand;
  int32_t T, k, E, layer;
  int32_t mode;              // LookupMode
  int32_t n_slots;
  // decode lookups: n_slots, mode and bandwidths are read from the control block when the
  // kernel runs (prefill lookups: n_slots only, the mode as given)
  const DevCtrl* ctrl;
  int32_t mode_from_ctrl;
  int32_t buffer_base;       // LK_BUFFER: slot of expert 0 of this layer
  uint64_t bw_pcie, bw_host;
  // cache tables
  int32_t* slot_of;          // [L*E]
  int32_t* key_of;           // [cap]
  uint64_t* stamp;           // [cap]
  const uint8_t* reserved;   // [cap]
  uint64_t* counter;         // [1]
  // outputs
  int32_t* slot_idx;         // [T,k]
  moe_trace_rec* trace;      // [<=E] or nullptr (caller's)
  int32_t* counts_out;       // [4] or nullptr (caller's)
  int32_t* u_key; int32_t* u_kind; int32_t* u_slot; int32_t* u_evict;  // [E]
  int32_t* fill_key; int32_t* fill_slot; int32_t* cpu_key;              // [E]
  int32_t* grp_slot;         // [E]
  int32_t* grp_pair0;        // [E] first pair of each group (-1 in candidate mode)
  int32_t* pair_grp;         // [T*k]
  int32_t* cnt;              // [C_COUNT]
};

struct DecodeArgs {
  const void* x;             // [T,H] afmt
  const float* w;            // [T,k]
  const DevCtrl* ctrl;       // the arena base is read from here when the kernel runs
  int64_t rec_bytes;
  int32_t T, k, H, I;
  const int32_t* grp_slot;   // [G]
  const int32_t* grp_pair0;  // [G] first pair routed to group g (the only one when T == 1)
  const int32_t* pair_grp;   // [T*k]
  const int32_t* cnt;        // device counters (C_NGRP)
  const int32_t* slot_idx;   // [T,k] slot of each pair (or a CPU flag), as the lookup wrote it
  float* h;                  // [T*k, I] scratch
  uint16_t* h16;             // [T*k, I] the same values rounded to bf16
  float* d;                  // [T*k, H] scratch (per-pair expert outputs)
  float* y;                  // [T,H]
  // all-resident batch-1 steps routed inside phase 1 (logits != nullptr): every workgroup
  // takes the top k itself; group g is rank g, its slot layer * E + expert
  const float* logits;       // [E]
  int32_t E, renorm, layer;
  int32_t* topk_out;         // [k] written by workgroup (0, 0), with
  float* topk_w_out;         // [k] the gates,
  int32_t* slot_out;         // [k] the slot ids (or nullptr),
  int32_t* grp_slot_out;     // [k] and the group tables phase 2 and the combine read
  int32_t* grp_pair0_out;    // [k]
  int32_t* pair_grp_out;     // [k]
  int32_t* cnt_out;          // C_NGRP, C_NPAIR_GPU, C_ERR, C_T
};

struct FillArgs {
  const int32_t* cnt;        // [C_COUNT]: C_FILL, C_ERR (and the step counts for dstats)
  const int32_t* fill_key;   // [E]
  const int32_t* fill_slot;  // [E]
  const uint8_t* pool;       // device address of the page-locked host pool
  int64_t pool_records;      // the pool holds records key % pool_records
  const DevCtrl* ctrl;       // the arena base is read from here when the kernel runs
  int32_t no_cpu_branch;     // the step has no CPU branch: CPU work from the lookup is an error
  int64_t rec_bytes;
  uint64_t* dstats;          // [D_COUNT] accumulated step counts, or nullptr
  // algorithmic bytes of the step's GEMV phases (zero unless profiling):
  // phase 1 = groups * p1_grp + p1_fixed + gpu pairs * p1_pair, phase 2 likewise
  uint64_t p1_grp, p1_fixed, p2_grp, p2_fixed, p1_pair, p2_pair;
};

struct PrefillArgs {
  const void* x;             // [T,H] afmt
  const void* xa;            // [T,H] 16-bit MFMA operands (x itself, or its converted copy);
                             // MX prefill: E4M3 codes
  const uint8_t* xs;         // MX prefill: E8M0 scales of xa [T, H/32]
  const float* w;            // [T,k]
  const uint8_t* arena;
  int64_t rec_bytes;
  int32_t T, k, H, I, E;
  const int32_t* grp_slot;   // [G]
  const int32_t* perm;       // [P] sorted position -> pair
  const int32_t* inv;        // [P] pair -> sorted position or -1
  const int32_t* offsets;    // [G+1]
  const int32_t* tile_base;  // [G+1] cumulative m-tiles
  const int4* tiles1;        // GEMM1's tile per workgroup (group, first row, rows, column tile); rows 0: none
  const int4* tiles2;        // GEMM2's
  const int32_t* cnt;        // C_NGRP, C_NPAIR_GPU
  void* act;                 // [P, I] bf16/f16 (sorted order); MX prefill: E4M3 codes
  uint8_t* acts;             // MX prefill: E8M0 scales of act [P, I/32]
  float* ypair;              // [P, H] fp32 (sorted order)
  float* y;                  // [T, H]
  const float* y_cpu;        // [T, H] or nullptr
  const int32_t* pair_gpu;   // [T*k]: >= 0 for pairs evaluated on the GPU; nullptr = every pair
};

// ---------------------------------------------------------------- launchers
void launch_route_logits(const void* x, int afmt, const float* wr, const float* bias, float* logits, int T, int E,
                         int H, hipStream_t s);
void launch_topk(const float* logits, int T, int E, int k, int renorm, int32_t* idx, float* w, hipStream_t s);
void launch_lookup(const LookupArgs& a, hipStream_t s);
void launch_evict_range(int32_t* slot_of, int32_t* key_of, uint64_t* stamp, uint8_t* reserved, int lo, int hi,
                        uint8_t reserve_value, hipStream_t s);
void launch_admit_buffer(int32_t* slot_of, int32_t* key_of, uint64_t* stamp, uint64_t* counter, int layer, int E,
                         int base, hipStream_t s);
// Launchers of timed kernels take optional start / stop events that the dispatch
// itself timestamps (hipExtLaunchKernelGGL): the elapsed time is the kernel's own.
struct Timing {
  hipEvent_t start = nullptr, stop = nullptr;
};
void launch_decode_phase1(int wfmt, int afmt, const DecodeArgs& a, int max_groups, hipStream_t s, Timing tm = {});
void launch_decode_phase2(int wfmt, const DecodeArgs& a, int max_groups, hipStream_t s, Timing tm = {});
bool decode_phase1_routed_ok(int wfmt, int afmt, int H, int k);
bool decode_phase2_reads_h16(int wfmt, int I, int T, int k);
bool launch_decode_phase2_combine(int wfmt, const DecodeArgs& a, hipStream_t s, Timing tm = {});
bool launch_decode_phase1_routed(int wfmt, int afmt, const DecodeArgs& a, hipStream_t s, Timing tm = {});
int decode_phase2_rowblocks(int H);
void launch_decode_combine(const DecodeArgs& a, const float* y_cpu, hipStream_t s);
int fill_blocks_per_record(int64_t rec_bytes);
// One launch writing the step block and the CPU branch's inputs into pinned host staging
// through its device mapping (system-scope stores), in place of four device-to-host copies.
struct StageArgs {
  const int32_t* step;  // [n_step] device step block
  int32_t* step_h;      // its pinned mirror (device address)
  int n_step;
  const uint32_t* x;    // [n_x] activations as 32-bit words
  uint32_t* x_h;
  int n_x;
  const float* w;       // [P] gates
  float* w_h;
  const int32_t* slot;  // [P] slot ids
  int32_t* slot_h;
  int P;
  // signalling variant only: the step's counts (nothing is staged without CPU work), the
  // device sequence number of signalled steps, and the pinned go word (device address)
  const int32_t* cnt = nullptr;
  uint32_t* seq = nullptr;
  uint32_t* go_h = nullptr;
};
void launch_stage_step(const StageArgs& a, hipStream_t s);
// The staging of a captured step with CPU work followed by its signal to the library's
// CPU-branch worker (sequence number to the go word); a step without CPU work stages nothing.
void launch_stage_signal(const StageArgs& a, hipStream_t s);
// The captured step's join with its CPU branch: waits (bounded by ctrl->cpu_wait_ticks) for
// the worker to publish the step's sequence number in the pinned done word, then copies the
// partial sum from pinned memory to y; zeros y when the step has no CPU work or the wait
// expires (counted in dstats[D_CPUWAIT]).
struct CpuWaitArgs {
  const int32_t* cnt;
  const uint32_t* seq;
  uint32_t* done_h;   // pinned done word (device address)
  uint32_t* y_h;      // [n] the partial sum in pinned memory (device address), fp32 bits
  float* y;           // [n] device copy read by the combine
  int n;
  const DevCtrl* ctrl;
  uint64_t* dstats;
};
void launch_cpu_wait(const CpuWaitArgs& a, hipStream_t s);
void launch_fill_pull(const FillArgs& a, int max_fills, hipStream_t s, Timing tm = {});
void launch_read_probe(const void* p, int64_t bytes, hipStream_t s, Timing tm);
void launch_permute(const int32_t* pair_grp, const int32_t* cnt, int P, int G_max, int32_t* hist, int32_t* perm,
                    int32_t* inv, int32_t* offsets, int32_t* tile_base, int bm, hipStream_t s);
void launch_groups_from_slots(const int32_t* slot_idx, int P, int32_t* pair_grp, int32_t* grp_slot, int32_t* cnt,
                              int32_t* scratch_flags, int n_slot_range, int gmax, int32_t* n_groups_out,
                              hipStream_t s);
int prefill_bm();
// Workgroups (table entries) of a GEMM launch over at most max_tiles_m row tiles of nt
// column tiles each.
int prefill_tile_slots(int max_tiles_m, int nt);
struct PrefillArgs;
// Both GEMMs' tile tables (a.tiles1, a.tiles2) from the permutation's counts.
void launch_tile_tables(const PrefillArgs& a, int wfmt, bool mx, int max_tiles_m, hipStream_t s);
bool prefill_needs_act_operands(int wfmt, int afmt);
void launch_act_operands(int wfmt, int afmt, const void* x, void* xo, int64_t n, hipStream_t s);
void launch_prefill_gemm1(int wfmt, int afmt, const PrefillArgs& a, int max_tiles_m, hipStream_t s, Timing tm = {});
void launch_prefill_gemm2(int wfmt, const PrefillArgs& a, int max_tiles_m, hipStream_t s, Timing tm = {});
// MX prefill of MXFP4 experts: activations to MXFP8 (codes [T,H], scales [T,H/32]) and the
// scaled-MFMA GEMMs (a.xa / a.xs in, a.act / a.acts between them)
void launch_mx_quant(int afmt, const void* x, uint8_t* codes, uint8_t* scales, int64_t n, hipStream_t s);
void launch_prefill_gemm1_mx(const PrefillArgs& a, int max_tiles_m, hipStream_t s, Timing tm = {});
void launch_prefill_gemm2_mx(const PrefillArgs& a, int max_tiles_m, hipStream_t s, Timing tm = {});
void launch_prefill_combine(const PrefillArgs& a, hipStream_t s);

// ---------------------------------------------------------------- CPU branch
struct CpuPool {
  explicit CpuPool(int threads);
  ~CpuPool();
  // Run fn(i) for i in [0, n) on the pool (caller participates); returns when all are done.
  void run(int n, const std::function<void(int)>& fn);
  int size() const { return nthreads_; }

 private:
  void worker(int id);
  int nthreads_;
  std::vector<std::thread> threads_;
  std::mutex mu_;
  std::condition_variable cv_;
  std::atomic<uint64_t> gen_{0};    // bumped once per run(): wakes the workers
  // One word per generation: (generation << 44) | (task count << 22) | next task index.
  // A claim succeeds only while next < count of the word it read, so a worker that is
  // late for one generation can never claim a task index that generation does not have.
  std::atomic<uint64_t> claim_{0};
  std::atomic<int> done_{0};
  std::atomic<const std::function<void(int)>*> fn_{nullptr};
  std::atomic<bool> stop_{false};
};

struct CpuFfnJob {
  int wfmt;
  int H, I, T, k;
  int64_t rec_bytes;
  const float* x;                   // [T,H] fp32 (host)
  const float* w;                   // [T,k] gates (host)
  const int32_t* slot_idx;          // [T,k] (host): CPU pairs are < 0
  std::vector<const uint8_t*> rec;  // record address of CPU list entry c
  float* h;                         // [T*k, I] scratch (host)
  float* y;                         // [T,H] out (host), CPU partial sum
};
void cpu_ffn(CpuPool& pool, const CpuFfnJob& job);

}  // namespace rmoe

// ---------------------------------------------------------------- context
struct moe_ctx {
  moe_config cfg{};
  int device = 0;
  int64_t S = 0;                 // record bytes
  std::string err;

  // host pool
  uint8_t* pool = nullptr;
  const uint8_t* pool_dev = nullptr;  // its device mapping (page-locked pools), for device fills
  int64_t pool_records = 0;
  bool pool_owned = false, pool_pinned = false;

  // bound device memory
  const float* router_w = nullptr;
  uint8_t* arena = nullptr;
  size_t arena_bytes = 0;
  int32_t n_slots = 0;
  bool bound = false;

  // residency tables (device)
  int32_t* slot_of = nullptr;    // [L*E]
  int32_t* key_of = nullptr;     // [kMaxCachedSlots]
  uint64_t* stamp = nullptr;     // [kMaxCachedSlots]
  uint8_t* reserved = nullptr;   // [kMaxCachedSlots]
  uint64_t* counter = nullptr;   // [1]

  // per-step work lists (device).  cnt, fill_key, fill_slot, cpu_key, u_key and u_kind
  // are consecutive pieces of one block (step_dev) so the host reads them with one copy.
  int32_t* step_dev = nullptr;   // [C_COUNT + 5E]
  int32_t *cnt = nullptr, *fill_key = nullptr, *fill_slot = nullptr, *cpu_key = nullptr;
  int32_t *u_key = nullptr, *u_kind = nullptr;
  int32_t *u_slot = nullptr, *u_evict = nullptr, *grp_slot = nullptr, *grp_pair0 = nullptr;
  int32_t* pair_grp = nullptr;   // [Pmax]
  int32_t* slot_scratch = nullptr;  // [Pmax] slot ids of steps whose caller passes none

  // scratch (device)
  float* logits = nullptr;       // [max_tokens*E]
  float* h = nullptr;            // [decode pairs * I]
  uint16_t* h16 = nullptr;       // [decode pairs * I] h rounded to bf16
  float* dpair = nullptr;        // [decode pairs * H]
  float* y_cpu_dev = nullptr;    // [max_tokens*H]
  // prefill scratch (device, sized for max_tokens)
  int32_t *perm = nullptr, *inv = nullptr, *offsets = nullptr, *tile_base = nullptr, *hist = nullptr;
  int4* tiles = nullptr;         // the GEMMs' tile tables (GEMM1's, then GEMM2's)
  int64_t tiles1_max = 0;        // entries reserved for GEMM1's
  int32_t* cand = nullptr;       // [E]
  void* act = nullptr;
  void* xo = nullptr;        // [max_tokens, H] 16-bit MFMA operands of the prefill activations
  float* ypair = nullptr;
  int32_t* flags = nullptr;
  uint64_t* dstats = nullptr;    // [D_COUNT] counts of device-fill steps
  rmoe::DevCtrl* ctrl = nullptr; // device control block (arena, n_slots, mode, bandwidths)

  // pinned host staging; h_cnt .. h_u_kind mirror step_dev
  int32_t* step_host = nullptr;
  int32_t* h_cnt = nullptr;      // [C_COUNT]
  int32_t* h_fill_key = nullptr;
  int32_t* h_fill_slot = nullptr;
  int32_t* h_cpu_key = nullptr;
  int32_t* h_u_key = nullptr;
  int32_t* h_u_kind = nullptr;
  int32_t* h_slot_idx = nullptr; // [Pmax]
  float* h_w = nullptr;          // [Pmax]
  void* h_x = nullptr;           // [max_tokens*H] in afmt
  float* h_xf = nullptr;         // [max_tokens*H] fp32
  float* h_y = nullptr;          // [max_tokens*H] fp32 (pinned, CPU partial)
  float* h_hbuf = nullptr;       // [Pmax*I] fp32 (CPU intermediate)
  // device addresses of step_host, h_x, h_w, h_slot_idx (nullptr: no mapping, copies instead)
  int32_t* step_host_dev = nullptr;
  void* h_x_dev = nullptr;
  float* h_w_dev = nullptr;
  int32_t* h_slot_idx_dev = nullptr;

  // captured steps with CPU work: a library thread runs the branch when the device publishes
  // a step's sequence number in the pinned go word, and answers in the done word
  uint32_t* sig_host = nullptr;   // pinned: go word at [kSigGo], done word at [kSigDone]
  uint32_t* sig_dev = nullptr;    // its device mapping
  float* h_y_dev = nullptr;       // device mapping of h_y
  uint32_t* seq_dev = nullptr;    // [1] sequence number of the last signalled step (device)
  int64_t wall_khz = 0;           // device wall-clock rate
  double cpu_wait_ms = 5000.0;    // bound of the device's wait for the branch
  std::thread branch_thread;
  std::atomic<bool> branch_stop{false};

  hipStream_t copy_stream = nullptr;
  hipEvent_t ev_sync = nullptr, ev_fill = nullptr, ev_ycpu = nullptr;
  hipEvent_t ev_layer_copied[2] = {nullptr, nullptr};
  hipEvent_t ev_layer_done[2] = {nullptr, nullptr};

  // state machine
  int last_lookup_layer = -1;
  int last_lookup_T = 0;
  bool in_prefill = false;
  bool prefill_buffers = false;
  int buffer_layer[2] = {-1, -1};
  int next_prefill_layer = 0;

  // stats and profiling
  moe_stats stats{};
  std::vector<moe_step_rec> step_log;   // profiled steps read on the host (moe_step_log)
  struct Timed { hipEvent_t a, b; int kind; int64_t rec; };
  std::vector<Timed> pending_timed;
  std::vector<hipEvent_t> event_pool;

  rmoe::CpuPool* cpu = nullptr;
};
