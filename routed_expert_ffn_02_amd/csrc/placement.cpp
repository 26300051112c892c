// Placement-policy replay on the host: the decode-time miss rate of a GPU expert
// placement policy over a recorded routing trace.
//
// The FreeToken summary ("무엇이 성능을 만들었나", expert-locality paragraph) and the
// reading notes (Figure 4b) replay one routing trace against several engines' placement
// policies at equal cache capacity and compare the fraction of decode expert reads that
// miss the GPU: FreeToken's global LRU, KTransformers' placement updated at prefill
// time, and llama.cpp's routing-blind static split.  The Luce Spark post adds a set
// pinned from measured routing frequencies plus a bounded ring of spare slots evicted
// least-recently-used first.  The LRU here is the shared cache of this library in
// offload mode (the cache-control kernel's victim order, in list form).
#include <algorithm>
#include <cstdint>
#include <vector>

#include "../../include/routed_moe.h"

namespace {

// Global LRU in list form: slots ordered least to most recently used, with the never
// used (empty) slots first in slot order, which is the (stamp, slot) order the lookup
// kernel selects victims by when every access takes the next stamp.
struct ListLru {
  int32_t n;
  std::vector<int32_t> prev, next;  // n slots + sentinel n
  std::vector<int32_t> key_of;      // key in slot, -1 empty
  std::vector<int32_t> slot_of;     // slot of key, -1 absent

  ListLru(int32_t n_slots, int64_t n_keys) : n(n_slots), prev(n_slots + 1), next(n_slots + 1),
                                             key_of(n_slots, -1), slot_of(n_keys, -1) {
    // sentinel n: next[n] = least recently used, prev[n] = most recently used
    for (int32_t s = 0; s <= n; ++s) {
      next[s] = (s == n) ? (n ? 0 : n) : (s + 1);
      prev[s] = (s == 0) ? n : (s - 1);
    }
    prev[n] = n ? n - 1 : n;
  }
  void unlink(int32_t s) {
    next[prev[s]] = next[s];
    prev[next[s]] = prev[s];
  }
  void push_mru(int32_t s) {
    const int32_t last = prev[n];
    next[last] = s;
    prev[s] = last;
    next[s] = n;
    prev[n] = s;
  }
  // victims: walk from the least recent end, skipping slots that hold a hit of this step
  void victims(int32_t q, const std::vector<int32_t>& hit_step, int32_t step_id, std::vector<int32_t>& out) {
    out.clear();
    for (int32_t s = next[n]; s != n && (int32_t)out.size() < q; s = next[s])
      if (hit_step[s] != step_id) out.push_back(s);
  }
};

// One layer's ring, most recently used key first.
struct Ring {
  int32_t cap = 0;
  std::vector<int32_t> keys;
};

bool by_count_then_key(const std::vector<int64_t>& cnt, int32_t a, int32_t b) {
  return cnt[a] != cnt[b] ? cnt[a] > cnt[b] : a < b;
}

}  // namespace

extern "C" MOE_API moe_status moe_placement_replay(const moe_replay_config* cfg, const int32_t* decode, int32_t steps,
                                                   const int32_t* calib, int32_t calib_tokens, int32_t calib_k,
                                                   uint8_t* miss_out, moe_replay_result* out) {
  if (!cfg || !out || steps < 0 || (steps > 0 && !decode)) return MOE_EINVAL;
  const int32_t L = cfg->n_layers, E = cfg->n_experts, P = cfg->pairs, C = cfg->capacity, pol = cfg->policy;
  if (L < 1 || E < 1 || P < 1 || (int64_t)L * E > (1 << 26) || C < 0 || C > L * E) return MOE_EINVAL;
  if (pol < MOE_PLACE_LRU || pol > MOE_PLACE_PINNED_RING) return MOE_EINVAL;
  const int32_t R = (pol == MOE_PLACE_PINNED_RING) ? cfg->ring_per_layer : 0;
  if (R < 0 || (int64_t)L * R > C) return MOE_EINVAL;
  const bool needs_calib = pol == MOE_PLACE_PREFILL || pol == MOE_PLACE_PINNED_RING;
  if (needs_calib && (calib_tokens < 0 || calib_k < 1 || (calib_tokens > 0 && !calib))) return MOE_EINVAL;
  const int64_t n_keys = (int64_t)L * E;
  const int64_t n_reads = (int64_t)steps * L * P;
  for (int64_t i = 0; i < n_reads; ++i)
    if (decode[i] < 0 || decode[i] >= E) return MOE_EINVAL;

  // resident sets of the placement-time policies
  std::vector<uint8_t> resident(n_keys, 0);
  if (needs_calib) {
    std::vector<int64_t> cnt(n_keys, 0);
    for (int64_t t = 0; t < calib_tokens; ++t)
      for (int32_t l = 0; l < L; ++l)
        for (int32_t j = 0; j < calib_k; ++j) {
          const int32_t e = calib[(t * L + l) * calib_k + j];
          if (e < 0 || e >= E) return MOE_EINVAL;
          ++cnt[(int64_t)l * E + e];
        }
    const int64_t n_pin = (pol == MOE_PLACE_PREFILL) ? C : (int64_t)C - (int64_t)L * R;
    std::vector<int32_t> order(n_keys);
    for (int64_t i = 0; i < n_keys; ++i) order[i] = (int32_t)i;
    std::partial_sort(order.begin(), order.begin() + n_pin, order.end(),
                      [&](int32_t a, int32_t b) { return by_count_then_key(cnt, a, b); });
    for (int64_t i = 0; i < n_pin; ++i) resident[order[i]] = 1;
  } else if (pol == MOE_PLACE_STATIC) {
    const int32_t full = C / E, rest = C % E;
    for (int32_t l = L - full; l < L; ++l)
      for (int32_t e = 0; e < E; ++e) resident[(int64_t)l * E + e] = 1;
    if (rest)
      for (int32_t e = 0; e < rest; ++e) resident[(int64_t)(L - full - 1) * E + e] = 1;
  }

  ListLru lru(pol == MOE_PLACE_LRU ? C : 0, pol == MOE_PLACE_LRU ? n_keys : 0);
  std::vector<Ring> rings(pol == MOE_PLACE_PINNED_RING ? L : 0);
  for (auto& r : rings) r.cap = R;
  std::vector<int32_t> seen(n_keys, -1), hit_step(std::max(C, 1), -1);
  std::vector<uint8_t> key_miss(n_keys, 0);
  std::vector<int32_t> U, misses, vict, unp_hits;
  uint64_t n_u = 0, n_miss = 0;
  int32_t step_id = 0;
  for (int32_t s = 0; s < steps; ++s) {
    for (int32_t l = 0; l < L; ++l, ++step_id) {
      const int32_t* row = decode + ((int64_t)s * L + l) * P;
      U.clear();
      for (int32_t p = 0; p < P; ++p) {
        const int32_t key = l * E + row[p];
        if (seen[key] != step_id) {
          seen[key] = step_id;
          U.push_back(key);
        }
      }
      if (pol == MOE_PLACE_LRU) {
        misses.clear();
        int32_t n_hit = 0;
        for (int32_t u : U) {
          const int32_t sl = lru.slot_of[u];
          key_miss[u] = sl < 0;
          if (sl >= 0) {
            hit_step[sl] = step_id;
            ++n_hit;
          } else {
            misses.push_back(u);
          }
        }
        const int32_t q = std::min<int32_t>((int32_t)misses.size(), C - n_hit);
        lru.victims(q, hit_step, step_id, vict);
        for (int32_t i = 0; i < q; ++i) {
          const int32_t v = vict[i], u = misses[i];
          if (lru.key_of[v] >= 0) lru.slot_of[lru.key_of[v]] = -1;
          lru.key_of[v] = u;
          lru.slot_of[u] = v;
        }
        // every key of U now resident (hits and admitted misses) becomes the most recent, in U order
        for (int32_t u : U) {
          const int32_t sl = lru.slot_of[u];
          if (sl >= 0) {
            lru.unlink(sl);
            lru.push_mru(sl);
          }
        }
      } else if (pol == MOE_PLACE_PINNED_RING) {
        Ring& rg = rings[l];
        misses.clear();
        unp_hits.clear();
        for (int32_t u : U) {
          if (resident[u]) {
            key_miss[u] = 0;
            continue;
          }
          const bool hit = std::find(rg.keys.begin(), rg.keys.end(), u) != rg.keys.end();
          key_miss[u] = !hit;
          (hit ? unp_hits : misses).push_back(u);
        }
        const int32_t free_slots = rg.cap - (int32_t)rg.keys.size();
        vict.clear();  // evictable keys, least recent first, none a hit of this step
        for (auto it = rg.keys.rbegin(); it != rg.keys.rend(); ++it)
          if (std::find(unp_hits.begin(), unp_hits.end(), *it) == unp_hits.end()) vict.push_back(*it);
        const int32_t admit = std::min<int32_t>((int32_t)misses.size(), free_slots + (int32_t)vict.size());
        for (int32_t i = 0; i < std::max(0, admit - free_slots); ++i)
          rg.keys.erase(std::find(rg.keys.begin(), rg.keys.end(), vict[i]));
        for (int32_t u : U) {
          if (resident[u]) continue;
          const bool admitted = std::find(misses.begin(), misses.begin() + admit, u) != misses.begin() + admit;
          const bool hit = std::find(unp_hits.begin(), unp_hits.end(), u) != unp_hits.end();
          if (!admitted && !hit) continue;
          auto it = std::find(rg.keys.begin(), rg.keys.end(), u);
          if (it != rg.keys.end()) rg.keys.erase(it);
          rg.keys.insert(rg.keys.begin(), u);
        }
      } else {
        for (int32_t u : U) key_miss[u] = !resident[u];
      }
      n_u += U.size();
      for (int32_t u : U) n_miss += key_miss[u];
      if (miss_out) {
        uint8_t* m = miss_out + ((int64_t)s * L + l) * P;
        for (int32_t p = 0; p < P; ++p) m[p] = key_miss[l * E + row[p]];
      }
    }
  }
  out->keys = n_u;
  out->misses = n_miss;
  out->reads = (uint64_t)n_reads;
  return MOE_OK;
}
