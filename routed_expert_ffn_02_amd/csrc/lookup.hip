// Device-side control of the bounded expert cache shared by all MoE layers.
//
// One workgroup per layer step (FreeToken summary, "CUDA Graph와 공존하는 LRU
// 캐시"; FreeToken reading notes, 05 Implementation): dedupe the routed experts,
// classify them against the residency table, derive the fill count q from the
// integer bandwidths, find the q least recently used evictable slots in a single
// selection pass, admit the fills, refresh recency, and rewrite logical ids to
// slot ids or CPU flags.  Every decision is integer arithmetic and every
// ordering is total, so the trace is deterministic.
//
// Ordering rules (fixed here where the pages leave them open):
//  - U: distinct keys in first-appearance order over (token, rank) pairs;
//  - F: the first q misses of U; the other misses form the CPU list C;
//  - victims: smallest (stamp, slot) among unreserved slots holding no hit of
//    this step (empty slots carry stamp 0);
//  - recency: after admission each key of U in H or F takes the next value of
//    one global counter, in U order.
#include <climits>

#include "common.hpp"

namespace rmoe {

constexpr int kWaves = kLookupThreads / 64;

__device__ uint64_t block_min_u64(uint64_t v, uint64_t* s_red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint64_t o = __shfl_xor(v, off);
    v = (o < v) ? o : v;
  }
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  uint64_t r = s_red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = (s_red[i] < r) ? s_red[i] : r;
  __syncthreads();
  return r;
}

__device__ int block_sum(int v, int* s_tmp) {
  int total;
  block_excl_scan(v, s_tmp, &total);
  return total;
}

// Minimum of an unsigned value over the 64 lanes, by DPP row moves (all ones is the
// identity); every lane receives it.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  auto step = [](uint32_t x, uint32_t y) { return y < x ? y : x; };
  const int id = -1;
  v = step(v, (uint32_t)dpp_move_i<0xB1, 0xf>((int)v, id));
  v = step(v, (uint32_t)dpp_move_i<0x4E, 0xf>((int)v, id));
  v = step(v, (uint32_t)dpp_move_i<0x141, 0xf>((int)v, id));
  v = step(v, (uint32_t)dpp_move_i<0x140, 0xf>((int)v, id));
  v = step(v, (uint32_t)dpp_move_i<0x142, 0xa>((int)v, id));
  v = step(v, (uint32_t)dpp_move_i<0x143, 0xc>((int)v, id));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// 64-bit minimum as two 32-bit ones: the high words, then the low words of the lanes
// holding the smallest high word (no LDS round trips).
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
  const uint32_t hi = wave_min_u32((uint32_t)(v >> 32));
  const uint32_t lo = wave_min_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0xffffffffu);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ int lanes_below(uint64_t mask, int lane) {  // set bits of mask below lane
  return __popcll(mask & ((1ull << lane) - 1ull));
}

constexpr int kSmallP = kSmallLookupPairs;  // pairs a step may have for the one-wavefront path

// Decode-sized steps (T*k <= 64, routed ids given): wavefront 0 holds one (token,
// rank) pair per lane and does every per-key step (dedupe, classify, miss ranks,
// admission, stamps, groups, outputs) with ballots and lane reads; the whole block
// joins only for the per-slot scan (evictable count and each wavefront's smallest
// (stamp, slot) candidates).  Three block barriers in all; the decisions and their
// order are those of the general path below.
__device__ __forceinline__ void lookup_small(const LookupArgs& a, int* s_slotrow, int* s_keyof, unsigned char* s_prot,
                             uint64_t (*s_cand)[kSmallP], int* s_evc, int* s_ufirst, int* s_sc, int* s_tk) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, P = a.T * a.k;
  const int kbase = a.layer * E;
  const bool cached = (a.mode == LK_OFFLOAD || a.mode == LK_CPU || a.mode == LK_HYBRID);

  // ---- 0. every piece of state requested at once (as in the general path)
  int slotrow_r = -1;
  uint64_t st_r[kSlotsPerThread];
  uint8_t rs_r[kSlotsPerThread];
  int ko_r[kSlotsPerThread];
  uint64_t c0 = 0;
  int e = -1;
  if (!a.logits && wave == 0 && lane < P) e = a.topk_idx[lane];
  if (cached) {
    if (tid < E) slotrow_r = a.slot_of[kbase + tid];
#pragma unroll
    for (int j = 0; j < kSlotsPerThread; ++j) {
      const int sl = tid + j * kLookupThreads;
      const bool in = sl < a.n_slots;
      st_r[j] = in ? a.stamp[sl] : 0;
      rs_r[j] = in ? a.reserved[sl] : 1;
      ko_r[j] = in ? a.key_of[sl] : -1;
    }
    if (wave == 0) c0 = *a.counter;
  }
  // routing fused in: wavefront t takes token t's top k from its logits while the state
  // loads above are in flight (the same selection and gates as the top-k kernel)
  if (a.logits && wave < a.T)
    topk_wave(a.logits + (size_t)wave * E, E, a.k, a.renorm, a.topk_out + wave * a.k, a.topk_w + wave * a.k,
              s_tk + wave * a.k);
  reinterpret_cast<uint32_t*>(s_prot)[tid] = 0u;  // kMaxCachedSlots bytes = one word per thread
  if (cached) {
    if (tid < E) s_slotrow[tid] = slotrow_r;
#pragma unroll
    for (int j = 0; j < kSlotsPerThread; ++j) {
      const int sl = tid + j * kLookupThreads;
      if (sl < a.n_slots) s_keyof[sl] = ko_r[j];
    }
  }
  __syncthreads();  // #1

  // ---- 1. wavefront 0: U, classification, miss ranks
  const bool valid = lane < P;
  if (a.logits && wave == 0 && valid) e = s_tk[lane];
  int nU = 0, m = 0, upos_p = 0;       // pair lanes: U position of the pair's expert
  int key = -1, slot = -1, kind = 9, p0 = 0;  // U lanes (lane < nU)
  uint64_t missmask = 0;
  if (wave == 0) {
    const bool bad = valid && (e < 0 || e >= E);
    if (__ballot(bad)) {
      if (valid) a.pair_grp[lane] = -1;  // nothing runs for this step
      if (lane == 0) {
        a.cnt[C_ERR] = 1;
        a.cnt[C_NGRP] = 0;
        a.cnt[C_T] = a.T;
        s_sc[0] = 1;
      }
    } else {
      if (lane == 0) s_sc[0] = 0;
      int first = lane;  // first pair routed to the same expert
      for (int q = 0; q < P; ++q) {
        const int eq = __builtin_amdgcn_readlane(e, q);
        if (q < first && eq == e) first = q;
      }
      const uint64_t fmask = __ballot(valid && first == lane);
      nU = __popcll(fmask);
      if (valid && first == lane) s_ufirst[lanes_below(fmask, lane)] = lane;
      upos_p = lanes_below(fmask, first);
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): s_ufirst written before it is read
      __builtin_amdgcn_wave_barrier();
      if (lane < nU) {
        p0 = s_ufirst[lane];
      }
      const int ue = __shfl(e, p0);
      if (lane < nU) {
        key = kbase + ue;
        if (a.mode == LK_FUSED) {
          slot = key;
          kind = MOE_KIND_HIT;
        } else if (a.mode == LK_BUFFER) {
          slot = a.buffer_base + ue;
          kind = MOE_KIND_BUF;
        } else {
          slot = s_slotrow[ue];
          if (slot >= 0) {
            kind = MOE_KIND_HIT;
            s_prot[slot] = 1;
          }
        }
      }
      missmask = __ballot(lane < nU && kind == 9);
      m = __popcll(missmask);
      if (lane == 0) s_sc[1] = m;
    }
  }
  __syncthreads();  // #2
  if (s_sc[0]) return;  // range error: reported above
  const int m_all = s_sc[1];

  // ---- 2. every wavefront: evictable slots and its own smallest (stamp, slot) keys
  if (cached) {
    uint64_t keys[kSlotsPerThread];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < kSlotsPerThread; ++j) {
      const int sl = tid + j * kLookupThreads;
      const bool elig = (sl < a.n_slots) && !s_prot[sl] && !rs_r[j];
      cnt += elig;
      keys[j] = elig ? ((st_r[j] << 16) | (uint64_t)sl) : ~0ull;
    }
    // a wavefront's count: lanes hold 0..4
    int wc = cnt;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) wc += __shfl_xor(wc, off);
    if (lane == 0) s_evc[wave] = wc;
    if (a.mode != LK_CPU) {
      uint64_t last = 0;
      for (int r = 0; r < m_all; ++r) {
        uint64_t best = ~0ull;
#pragma unroll
        for (int j = 0; j < kSlotsPerThread; ++j)
          if ((r == 0 || keys[j] > last) && keys[j] < best) best = keys[j];
        best = wave_min_u64(best);
        if (lane == 0) s_cand[wave][r] = best;
        last = best;
      }
    }
  }
  __syncthreads();  // #3
  if (wave != 0) return;

  // ---- 3. wavefront 0: q, victims, admission, stamps, groups, outputs
  int ev = 0, q = 0;
  if (cached) {
    int w = lane < kWaves ? s_evc[lane] : 0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) w += __shfl_xor(w, off);
    ev = w;
    if (a.mode == LK_OFFLOAD) {
      q = min(m, ev);
    } else if (a.mode == LK_HYBRID) {
      if (m == 0 || ev == 0) {
        q = 0;
      } else if (a.bw_host <= a.bw_pcie) {
        q = min(m, ev);
      } else {
        const uint64_t num = 2ull * (uint64_t)m * a.bw_pcie + a.bw_host;
        const uint64_t qq = num / (2ull * a.bw_host);
        const int qi = (int)max<uint64_t>(1ull, qq);
        q = min(min(m, ev), qi);
      }
    }
  }
  const bool miss = (missmask >> lane) & 1ull;
  const int mrank = miss ? lanes_below(missmask, lane) : -1;
  // the q smallest of the union of every wavefront's m smallest (q <= m, so it holds them)
  uint64_t victim = ~0ull;
  if (q > 0) {
    const int nc = kWaves * m;  // candidates s_cand[w][r], r < m
    uint64_t last = 0;
    for (int r = 0; r < q; ++r) {
      uint64_t best = ~0ull;
      for (int i = lane; i < nc; i += 64) {
        const uint64_t c = s_cand[i / m][i % m];
        if ((r == 0 || c > last) && c < best) best = c;
      }
      best = wave_min_u64(best);
      if (mrank == r) victim = best;
      last = best;
    }
  }
  int evicted = -1;
  if (miss) {
    if (mrank < q) {
      slot = (int)(victim & 0xffffull);
      evicted = s_keyof[slot];
      if (evicted >= 0) a.slot_of[evicted] = -1;
      a.slot_of[key] = slot;
      a.key_of[slot] = key;
      kind = MOE_KIND_FILL;
    } else {
      kind = MOE_KIND_CPU;
      slot = -1;
    }
  }
  const int n_evict = __popcll(__ballot(miss && mrank < q && evicted >= 0));
  const bool is_gpu = lane < nU && (kind == MOE_KIND_HIT || kind == MOE_KIND_FILL || kind == MOE_KIND_BUF);
  const uint64_t gmask = __ballot(is_gpu);
  const int nG = __popcll(gmask);
  if (cached && is_gpu) a.stamp[slot] = c0 + (uint64_t)lanes_below(gmask, lane) + 1ull;
  // group id: GPU entries ordered by slot
  int g = 0;
  for (int u = 0; u < nU; ++u) {
    const int su = __builtin_amdgcn_readlane(slot, u);
    if (((gmask >> u) & 1ull) && su < slot) ++g;
  }
  if (is_gpu) {
    a.grp_slot[g] = slot;
    a.grp_pair0[g] = p0;
  }
  if (lane < nU) {
    a.u_key[lane] = key;
    a.u_kind[lane] = kind;
    a.u_slot[lane] = slot;
    a.u_evict[lane] = evicted;
    if (a.trace) a.trace[lane] = moe_trace_rec{key, kind, slot, evicted};
    if (miss) {
      if (mrank < q) {
        a.fill_key[mrank] = key;
        a.fill_slot[mrank] = slot;
      } else {
        a.cpu_key[mrank - q] = key;
      }
    }
  }
  // per pair: the data of its expert's U entry
  const int pk = __shfl(kind, upos_p), ps = __shfl(slot, upos_p), pg = __shfl(g, upos_p);
  const int pr = __shfl(mrank, upos_p);
  if (valid) {
    a.slot_idx[lane] = (pk == MOE_KIND_CPU) ? -1 - (pr - q) : ps;
    a.pair_grp[lane] = (pk == MOE_KIND_CPU) ? -1 : pg;
  }
  const int gpu_pairs = __popcll(__ballot(valid && pk != MOE_KIND_CPU));
  if (lane == 0) {
    if (cached) *a.counter = c0 + (uint64_t)nG;
    a.cnt[C_NU] = nU;
    a.cnt[C_HIT] = nU - m;
    a.cnt[C_FILL] = q;
    a.cnt[C_CPU] = m - q;
    a.cnt[C_EVICT] = n_evict;
    a.cnt[C_NGRP] = nG;
    a.cnt[C_M] = m;
    a.cnt[C_EV] = ev;
    a.cnt[C_NPAIR_GPU] = gpu_pairs;
    a.cnt[C_ERR] = 0;
    a.cnt[C_T] = a.T;
    if (a.counts_out) {
      a.counts_out[MOE_CNT_HIT] = nU - m;
      a.counts_out[MOE_CNT_FILL] = q;
      a.counts_out[MOE_CNT_CPU] = m - q;
      a.counts_out[MOE_CNT_EVICT] = n_evict;
    }
  }
}

__global__ __launch_bounds__(kLookupThreads) void lookup_kernel(LookupArgs args) {
  // the cache's current size (and for decode lookups mode and bandwidths) as they are when
  // the kernel runs: a replayed graph follows resizes and mode changes made after capture
  LookupArgs a = args;
  if (args.ctrl) {
    a.n_slots = args.ctrl->n_slots;
    if (args.mode_from_ctrl) {
      a.mode = args.ctrl->lk_mode;
      a.bw_pcie = args.ctrl->bw_pcie;
      a.bw_host = args.ctrl->bw_host;
    }
  }
  __shared__ int s_first[kMaxExperts];   // first pair index of expert e, or INT_MAX
  __shared__ int s_upos[kMaxExperts];    // position of expert e in U, or -1
  __shared__ int s_ukey[kMaxExperts];
  __shared__ int s_uslot[kMaxExperts];
  __shared__ int s_ukind[kMaxExperts];   // HIT, FILL, CPU, BUF; 9 = miss (undecided)
  __shared__ int s_uevict[kMaxExperts];
  __shared__ int s_uaux[kMaxExperts];    // miss rank (misses) ; group id (GPU entries)
  __shared__ int s_miss_u[kMaxExperts];  // U position of the r-th miss
  __shared__ __attribute__((aligned(4))) unsigned char s_prot[kMaxCachedSlots];
  __shared__ uint64_t s_victim[kMaxExperts];
  __shared__ uint64_t s_red[kWaves];
  __shared__ int s_tmp[64];
  __shared__ int s_sc[8];

  __shared__ int s_slotrow[kMaxExperts];       // slot_of of this layer's keys at kernel start
  __shared__ int s_keyof[kMaxCachedSlots];     // key_of at kernel start
  __shared__ uint64_t s_c0;

  if (a.cand == nullptr && a.T * a.k <= kSmallP) {  // uniform
    __shared__ uint64_t s_cand[kWaves][kSmallP];
    __shared__ int s_evc[kWaves];
    __shared__ int s_ufirst[kSmallP];
    __shared__ int s_tk[kSmallP];
    lookup_small(a, s_slotrow, s_keyof, s_prot, s_cand, s_evc, s_ufirst, s_sc, s_tk);
    return;
  }

  const int tid = threadIdx.x;
  const int E = a.E, k = a.k, P = a.T * a.k;
  const int kbase = a.layer * E;
  const bool cached = (a.mode == LK_OFFLOAD || a.mode == LK_CPU || a.mode == LK_HYBRID);

  // Every piece of cache state this step reads is requested now, in parallel, instead of
  // one dependent round trip per stage: this layer's slot_of row, and per slot the
  // stamp, the reservation flag and the resident key (E <= kLookupThreads).
  int slotrow_r = -1;
  uint64_t st_r[kSlotsPerThread];
  uint8_t rs_r[kSlotsPerThread];
  int ko_r[kSlotsPerThread];
  uint64_t c0_r = 0;
  if (cached) {
    if (tid < E) slotrow_r = a.slot_of[kbase + tid];
#pragma unroll
    for (int j = 0; j < kSlotsPerThread; ++j) {
      const int s = tid + j * kLookupThreads;
      const bool in = s < a.n_slots;
      st_r[j] = in ? a.stamp[s] : 0;
      rs_r[j] = in ? a.reserved[s] : 1;
      ko_r[j] = in ? a.key_of[s] : -1;
    }
    if (tid == 0) c0_r = *a.counter;
  }

  // ---- 1. U in first-appearance order --------------------------------------
  for (int e = tid; e < E; e += kLookupThreads) {
    s_first[e] = INT_MAX;
    s_upos[e] = -1;
  }
  for (int s = tid; s < kMaxCachedSlots; s += kLookupThreads) s_prot[s] = 0;
  if (cached) {
    if (tid < E) s_slotrow[tid] = slotrow_r;
#pragma unroll
    for (int j = 0; j < kSlotsPerThread; ++j) {
      const int s = tid + j * kLookupThreads;
      if (s < a.n_slots) s_keyof[s] = ko_r[j];
    }
    if (tid == 0) s_c0 = c0_r;
  }
  __syncthreads();
  if (tid == 0) s_sc[0] = 0;
  __syncthreads();
  int nU;
  if (a.cand == nullptr) {
    for (int p = tid; p < P; p += kLookupThreads) {
      const int e = a.topk_idx[p];
      if (e < 0 || e >= E) s_sc[0] = 1;  // invalid expert id: reported, never used as an index
      else atomicMin(&s_first[e], p);
    }
    __syncthreads();
    if (s_sc[0]) {  // uniform: every thread read the same flag after the barrier
      for (int p = tid; p < P; p += kLookupThreads) a.pair_grp[p] = -1;  // nothing runs for this step
      if (tid == 0) {
        a.cnt[C_ERR] = 1;
        a.cnt[C_NGRP] = 0;
        a.cnt[C_T] = a.T;
      }
      return;
    }
    // each thread owns a contiguous range of pairs; count the first appearances in it
    const int cpt = (P + kLookupThreads - 1) / kLookupThreads;
    const int p0 = tid * cpt, p1 = min(P, p0 + cpt);
    int local = 0;
    for (int p = p0; p < p1; ++p) local += (s_first[a.topk_idx[p]] == p);
    int total;
    int pos = block_excl_scan(local, s_tmp, &total);
    for (int p = p0; p < p1; ++p) {
      int e = a.topk_idx[p];
      if (s_first[e] == p) {
        s_upos[e] = pos;
        s_ukey[pos] = kbase + e;
        ++pos;
      }
    }
    nU = total;
  } else {
    for (int i = tid; i < a.n_cand; i += kLookupThreads) {
      int key = a.cand[i];
      s_upos[key - kbase] = i;
      s_ukey[i] = key;
    }
    nU = a.n_cand;
  }
  __syncthreads();

  // ---- 2. classify ----------------------------------------------------------
  int is_miss = 0;
  if (tid < nU) {
    const int key = s_ukey[tid];
    int slot = -1, kind = 9;
    if (a.mode == LK_FUSED) {
      slot = key;
      kind = MOE_KIND_HIT;
    } else if (a.mode == LK_BUFFER) {
      slot = a.buffer_base + (key - kbase);
      kind = MOE_KIND_BUF;
    } else {
      slot = s_slotrow[key - kbase];
      if (slot >= 0) {
        kind = MOE_KIND_HIT;
        s_prot[slot] = 1;
      }
    }
    s_uslot[tid] = slot;
    s_ukind[tid] = kind;
    s_uevict[tid] = -1;
    is_miss = (kind == 9);
  }
  int m;
  const int miss_rank = block_excl_scan(is_miss, s_tmp, &m);
  if (is_miss) {
    s_uaux[tid] = miss_rank;
    s_miss_u[miss_rank] = tid;
  }
  __syncthreads();

  // ---- 3. evictable slots ----------------------------------------------------
  int q = 0, ev = 0;
  if (cached) {
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < kSlotsPerThread; ++j) {
      const int s = tid + j * kLookupThreads;
      cnt += (s < a.n_slots && !s_prot[s] && !rs_r[j]);
    }
    ev = block_sum(cnt, s_tmp);
    // ---- 4. q: same rule as the host qstar_split ---------------------------
    if (a.mode == LK_OFFLOAD) {
      q = min(m, ev);
    } else if (a.mode == LK_HYBRID) {
      if (m == 0 || ev == 0) {
        q = 0;
      } else if (a.bw_host <= a.bw_pcie) {
        q = min(m, ev);
      } else {
        uint64_t num = 2ull * (uint64_t)m * a.bw_pcie + a.bw_host;
        uint64_t qq = num / (2ull * a.bw_host);
        int qi = (int)max<uint64_t>(1ull, qq);
        q = min(min(m, ev), qi);
      }
    } else {
      q = 0;  // CPU mode
    }
  }

  // ---- 5. the q smallest (stamp, slot) among evictable slots: one selection pass
  if (q > 0) {
    uint64_t keys[kSlotsPerThread];
#pragma unroll
    for (int j = 0; j < kSlotsPerThread; ++j) {
      int s = tid + j * kLookupThreads;
      bool elig = (s < a.n_slots) && !s_prot[s] && !rs_r[j];
      keys[j] = elig ? ((st_r[j] << 16) | (uint64_t)s) : ~0ull;
    }
    uint64_t last = 0;
    bool first = true;
    for (int r = 0; r < q; ++r) {
      uint64_t best = ~0ull;
#pragma unroll
      for (int j = 0; j < kSlotsPerThread; ++j)
        if ((first || keys[j] > last) && keys[j] < best) best = keys[j];
      best = block_min_u64(best, s_red);
      if (tid == 0) s_victim[r] = best;
      last = best;
      first = false;
    }
  }
  __syncthreads();

  // ---- 6. admit fills -----------------------------------------------------------
  uint64_t c0 = cached ? s_c0 : 0;
  int n_evict_local = 0;
  for (int r = tid; r < m; r += kLookupThreads) {
    const int u = s_miss_u[r];
    if (r < q) {
      const int slot = (int)(s_victim[r] & 0xffffull);
      const int key = s_ukey[u];
      const int old = s_keyof[slot];
      if (old >= 0) {
        a.slot_of[old] = -1;
        ++n_evict_local;
      }
      a.slot_of[key] = slot;
      a.key_of[slot] = key;
      s_uslot[u] = slot;
      s_ukind[u] = MOE_KIND_FILL;
      s_uevict[u] = old;
    } else {
      s_ukind[u] = MOE_KIND_CPU;
      s_uslot[u] = -1;
    }
  }
  const int n_evict = block_sum(n_evict_local, s_tmp);
  __syncthreads();

  // ---- 7. recency stamps in U order; GPU groups ordered by slot -------------------
  int is_gpu = 0;
  if (tid < nU) {
    const int kd = s_ukind[tid];
    is_gpu = (kd == MOE_KIND_HIT || kd == MOE_KIND_FILL || kd == MOE_KIND_BUF);
  }
  int nG;
  const int grank = block_excl_scan(is_gpu, s_tmp, &nG);
  if (cached && is_gpu) a.stamp[s_uslot[tid]] = c0 + (uint64_t)grank + 1ull;
  if (is_gpu) {
    const int my = s_uslot[tid];
    int g = 0;
    for (int u = 0; u < nU; ++u) {
      const int kd = s_ukind[u];
      if ((kd == MOE_KIND_HIT || kd == MOE_KIND_FILL || kd == MOE_KIND_BUF) && s_uslot[u] < my) ++g;
    }
    s_uaux[tid] = g;  // group id (misses that became fills are GPU now; their miss rank is no longer needed)
    a.grp_slot[g] = my;
    a.grp_pair0[g] = (a.cand == nullptr) ? s_first[s_ukey[tid] - kbase] : -1;
  }
  __syncthreads();

  // ---- 8. outputs ----------------------------------------------------------------
  if (tid < nU) {
    const int key = s_ukey[tid], kind = s_ukind[tid], slot = s_uslot[tid], evicted = s_uevict[tid];
    a.u_key[tid] = key;
    a.u_kind[tid] = kind;
    a.u_slot[tid] = slot;
    a.u_evict[tid] = evicted;
    if (a.trace) a.trace[tid] = moe_trace_rec{key, kind, slot, evicted};
  }
  for (int r = tid; r < m; r += kLookupThreads) {
    const int u = s_miss_u[r];
    if (r < q) {
      a.fill_key[r] = s_ukey[u];
      a.fill_slot[r] = s_uslot[u];
    } else {
      a.cpu_key[r - q] = s_ukey[u];
    }
  }
  int gpu_pairs_local = 0;
  for (int p = tid; p < P; p += kLookupThreads) {
    const int e = a.topk_idx[p];
    const int u = s_upos[e];
    int sl, pg = -1;
    if (u < 0) {
      sl = INT_MIN;  // not part of this round (on-demand prefill)
    } else {
      const int kd = s_ukind[u];
      if (kd == MOE_KIND_CPU) {
        sl = -1 - (s_uaux[u] - q);  // CPU list index = miss rank - q
      } else {
        sl = s_uslot[u];
        pg = s_uaux[u];
        ++gpu_pairs_local;
      }
    }
    a.slot_idx[p] = sl;
    a.pair_grp[p] = pg;
  }
  const int gpu_pairs = block_sum(gpu_pairs_local, s_tmp);
  if (tid == 0) {
    if (cached) *a.counter = c0 + (uint64_t)nG;
    a.cnt[C_NU] = nU;
    a.cnt[C_HIT] = nU - m;
    a.cnt[C_FILL] = q;
    a.cnt[C_CPU] = m - q;
    a.cnt[C_EVICT] = n_evict;
    a.cnt[C_NGRP] = nG;
    a.cnt[C_M] = m;
    a.cnt[C_EV] = ev;
    a.cnt[C_NPAIR_GPU] = gpu_pairs;
    a.cnt[C_ERR] = 0;
    a.cnt[C_T] = a.T;
    if (a.counts_out) {
      a.counts_out[MOE_CNT_HIT] = nU - m;
      a.counts_out[MOE_CNT_FILL] = q;
      a.counts_out[MOE_CNT_CPU] = m - q;
      a.counts_out[MOE_CNT_EVICT] = n_evict;
    }
  }
}

void launch_lookup(const LookupArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(lookup_kernel, dim3(1), dim3(kLookupThreads), 0, s, a);
}

// Evict (optionally) and (un)reserve slots [lo, hi).
__global__ void evict_range_kernel(int32_t* slot_of, int32_t* key_of, uint64_t* stamp, uint8_t* reserved, int lo,
                                   int hi, uint8_t reserve_value, int do_evict) {
  int s = lo + blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= hi) return;
  if (do_evict) {
    int old = key_of[s];
    if (old >= 0) slot_of[old] = -1;
    key_of[s] = -1;
    stamp[s] = 0;
  }
  reserved[s] = reserve_value;
}

void launch_evict_range(int32_t* slot_of, int32_t* key_of, uint64_t* stamp, uint8_t* reserved, int lo, int hi,
                        uint8_t reserve_value, hipStream_t s) {
  if (hi <= lo) return;
  int do_evict = reserve_value ? 1 : 0;  // reserving evicts; releasing keeps the entries
  hipLaunchKernelGGL(evict_range_kernel, dim3((hi - lo + 255) / 256), dim3(256), 0, s, slot_of, key_of, stamp,
                     reserved, lo, hi, reserve_value, do_evict);
}

// Prefill end: admit the full layer held in a buffer, expert e at slot base + e,
// stamps in ascending expert order; an older copy of the same key elsewhere is freed.
__global__ void admit_buffer_kernel(int32_t* slot_of, int32_t* key_of, uint64_t* stamp, uint64_t* counter, int layer,
                                    int E, int base) {
  const int e = threadIdx.x;
  const uint64_t c0 = *counter;
  __syncthreads();
  if (e < E) {
    const int key = layer * E + e;
    const int old = slot_of[key];
    if (old >= 0 && (old < base || old >= base + E)) {
      key_of[old] = -1;
      stamp[old] = 0;
    }
    slot_of[key] = base + e;
    key_of[base + e] = key;
    stamp[base + e] = c0 + (uint64_t)e + 1ull;
  }
  if (e == 0) *counter = c0 + (uint64_t)E;
}

void launch_admit_buffer(int32_t* slot_of, int32_t* key_of, uint64_t* stamp, uint64_t* counter, int layer, int E,
                         int base, hipStream_t s) {
  hipLaunchKernelGGL(admit_buffer_kernel, dim3(1), dim3(kMaxExperts), 0, s, slot_of, key_of, stamp, counter, layer, E,
                     base);
}

}  // namespace rmoe
