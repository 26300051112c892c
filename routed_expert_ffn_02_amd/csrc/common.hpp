// Device helpers shared by the HIP kernels of the routed-MoE library (gfx950,
// wavefront 64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.hpp"

namespace rmoe {

// Launch with dispatch-timestamped events when timing is requested.
template <typename... KArgs, typename... Args>
inline void launch_timed(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t lds, hipStream_t s, Timing tm,
                         Args... args) {
  if (tm.start && tm.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, tm.start, tm.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int AFMT>
__device__ __forceinline__ float load_act(const void* x, size_t i) {
  if constexpr (AFMT == MOE_AFMT_BF16) {
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(x)[i]);
  } else {
    return reinterpret_cast<const float*>(x)[i];
  }
}

// Sum over the 64 lanes of a wavefront, returned to every lane.  Data-parallel
// primitives (DPP) move values between lanes inside the VALU: quad permutes and the
// (half-)row mirrors sum each 16-lane row, then the row broadcasts of lanes 15 and
// 31 carry the partial sums up to lane 63, which is read out as a uniform value.
// No LDS round trips, unlike lane shuffles.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<0xB1, 0xf>(v);   // quad_perm [1,0,3,2]: pairs
  v += dpp_move<0x4E, 0xf>(v);   // quad_perm [2,3,0,1]: quads
  v += dpp_move<0x141, 0xf>(v);  // row_half_mirror: 8 lanes
  v += dpp_move<0x140, 0xf>(v);  // row_mirror: 16 lanes
  v += dpp_move<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_move<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Maximum over the 64 lanes (same DPP pattern as wave_sum; lanes a row broadcast does
// not write read -inf, the identity).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_move_or(float v, float ident) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, ident), __builtin_bit_cast(int, v),
                                                               CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_max(float v) {
  const float ni = -INFINITY;
  v = fmaxf(v, dpp_move_or<0xB1, 0xf>(v, ni));
  v = fmaxf(v, dpp_move_or<0x4E, 0xf>(v, ni));
  v = fmaxf(v, dpp_move_or<0x141, 0xf>(v, ni));
  v = fmaxf(v, dpp_move_or<0x140, 0xf>(v, ni));
  v = fmaxf(v, dpp_move_or<0x142, 0xa>(v, ni));
  v = fmaxf(v, dpp_move_or<0x143, 0xc>(v, ni));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Minimum of an int over the 64 lanes (INT_MAX is the identity).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_move_i(int v, int ident) {
  return __builtin_amdgcn_update_dpp(ident, v, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ int wave_min_i32(int v) {
  const int id = 0x7fffffff;
  v = min(v, dpp_move_i<0xB1, 0xf>(v, id));
  v = min(v, dpp_move_i<0x4E, 0xf>(v, id));
  v = min(v, dpp_move_i<0x141, 0xf>(v, id));
  v = min(v, dpp_move_i<0x140, 0xf>(v, id));
  v = min(v, dpp_move_i<0x142, 0xa>(v, id));
  v = min(v, dpp_move_i<0x143, 0xc>(v, id));
  return __builtin_amdgcn_readlane(v, 63);
}

// Maximum of an int over the 64 lanes (INT_MIN is the identity).
__device__ __forceinline__ int wave_max_i32(int v) {
  const int id = (int)0x80000000;
  v = max(v, dpp_move_i<0xB1, 0xf>(v, id));
  v = max(v, dpp_move_i<0x4E, 0xf>(v, id));
  v = max(v, dpp_move_i<0x141, 0xf>(v, id));
  v = max(v, dpp_move_i<0x140, 0xf>(v, id));
  v = max(v, dpp_move_i<0x142, 0xa>(v, id));
  v = max(v, dpp_move_i<0x143, 0xc>(v, id));
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// ---------------------------------------------------------------------------
// Softmax over E logits and the top k of one token, by one wavefront.  Selection order:
// the larger logit, then the lower index (-0 and +0 compare equal).  Gates are the
// softmax values at the chosen experts, renormalised over the k when renorm is set.
// Writes idx_out[j], w_out[j] (global) and, when lds_idx is given, lds_idx[j].
constexpr int kTopkPerLane = kMaxExperts / 64;

__device__ __forceinline__ bool topk_better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Order-preserving int key of a finite logit or -inf (-0 taken as +0, so equal values
// have equal keys), and back.
__device__ __forceinline__ int topk_key(float v) {
  const int b = __float_as_int(v == 0.f ? 0.f : v);
  return b >= 0 ? b : b ^ 0x7fffffff;
}
__device__ __forceinline__ float topk_unkey(int key) { return __int_as_float(key >= 0 ? key : key ^ 0x7fffffff); }

// PL logits per lane (E <= 64 * PL).  A lane first sorts its own logits under the
// selection order (PL <= 8; an insertion network of selects), so its best is always its
// first; a round takes the wave maximum of the lanes' firsts as int keys (one DPP max
// per step), breaks a tie between lanes by the lower index, and the winning lane shifts
// its list up.  (PL = 16 keeps a scan of the lane's logits per round: its network would
// cost more than the scans.)  A chosen logit (and every slot past E) is held as
// (-inf, INT_MAX), which loses to any candidate under the order, so the rounds are
// branch-free selects.  Logits are finite (the router's inputs are).
// GATES = false: the selection alone (lds_idx only; no softmax, no global outputs), for
// readers that need only which experts were chosen.
template <int PL, bool GATES = true>
__device__ __forceinline__ void topk_wave_pl(const float* __restrict__ z, int E, int k, int renorm,
                                             int32_t* __restrict__ idx_out, float* __restrict__ w_out, int* lds_idx) {
  constexpr bool SORTED = PL <= 8;
  const int lane = threadIdx.x & 63;
  float v[PL];
  int ev[PL];  // the logit's expert, INT_MAX once chosen or past E
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int e = lane + 64 * i;
    v[i] = (e < E) ? z[e] : -INFINITY;
    ev[i] = (e < E) ? e : 0x7fffffff;
    mx = fmaxf(mx, v[i]);
  }
  float sum = 0.f;
  if constexpr (GATES) {
    mx = wave_max(mx);
#pragma unroll
    for (int i = 0; i < PL; ++i)
      if (lane + 64 * i < E) sum += __expf(v[i] - mx);
    sum = wave_sum(sum);
  }
  if constexpr (SORTED) {
#pragma unroll
    for (int i = 1; i < PL; ++i) {
#pragma unroll
      for (int j = i; j > 0; --j) {
        // entry j before entry j - 1 under the order (no short-circuit evaluation)
        const bool sw = (v[j] > v[j - 1]) | ((v[j] == v[j - 1]) & (ev[j] < ev[j - 1]));
        const float va = v[j - 1], vb = v[j];
        const int ia = ev[j - 1], ib = ev[j];
        v[j - 1] = sw ? vb : va;
        v[j] = sw ? va : vb;
        ev[j - 1] = sw ? ib : ia;
        ev[j] = sw ? ia : ib;
      }
    }
  }
  // selection rounds carry only the arg-max; lane j keeps the j-th winner (k <= 64) and
  // the gates are formed after the loop, all lanes at once
  int my_idx = 0;
  float my_v = -INFINITY;
  for (int j = 0; j < k; ++j) {
    float wv;
    int bi;
    if constexpr (SORTED) {
      const int key = topk_key(v[0]);
      const int wkey = wave_max_i32(key);
      wv = topk_unkey(wkey);
      const uint64_t holders = __ballot(key == wkey);
      if (__popcll(holders) == 1)
        bi = __builtin_amdgcn_readlane(ev[0], __ffsll((unsigned long long)holders) - 1);
      else
        bi = wave_min_i32(key == wkey ? ev[0] : 0x7fffffff);
      const bool hit = ev[0] == bi;
#pragma unroll
      for (int i = 0; i + 1 < PL; ++i) {
        v[i] = hit ? v[i + 1] : v[i];
        ev[i] = hit ? ev[i + 1] : ev[i];
      }
      v[PL - 1] = hit ? -INFINITY : v[PL - 1];
      ev[PL - 1] = hit ? 0x7fffffff : ev[PL - 1];
    } else {
      float bv = -INFINITY;
      bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const bool better = (v[i] > bv) | ((v[i] == bv) & (ev[i] < bi));
        bv = better ? v[i] : bv;
        bi = better ? ev[i] : bi;
      }
      // wave arg-max under the same order: the largest value, then the lowest index among
      // the lanes holding it (a single holder, the usual case, is read from its lane)
      wv = wave_max(bv);
      const uint64_t holders = __ballot(bv == wv);
      if (__popcll(holders) == 1)
        bi = __builtin_amdgcn_readlane(bi, __ffsll((unsigned long long)holders) - 1);
      else
        bi = wave_min_i32(bv == wv ? bi : 0x7fffffff);
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const bool hit = ev[i] == bi;
        v[i] = hit ? -INFINITY : v[i];
        ev[i] = hit ? 0x7fffffff : ev[i];
      }
    }
    if (k <= 64) {
      if (lane == j) { my_idx = bi; my_v = wv; }
    } else if (!GATES) {
      if (lane == 0) lds_idx[j] = bi;
    } else if (lane == 0) {  // more than one selection per lane: written as found
      idx_out[j] = bi;
      w_out[j] = __expf(wv - mx) / sum;
      if (lds_idx) lds_idx[j] = bi;
    }
  }
  if (!GATES) {
    if (k <= 64 && lane < k) lds_idx[lane] = my_idx;
    return;
  }
  if (k <= 64) {
    const float p = __expf(my_v - mx) / sum;
    if (lane < k) {
      idx_out[lane] = my_idx;
      w_out[lane] = p;
      if (lds_idx) lds_idx[lane] = my_idx;
    }
    if (renorm) {
      float sel_sum = 0.f;  // in rank order
      for (int j = 0; j < k; ++j) sel_sum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), j));
      if (lane < k) w_out[lane] = p / sel_sum;
    }
  } else if (renorm && lane == 0) {
    float sel_sum = 0.f;
    for (int j = 0; j < k; ++j) sel_sum += w_out[j];
    for (int j = 0; j < k; ++j) w_out[j] = w_out[j] / sel_sum;
  }
}

__device__ __forceinline__ void topk_wave(const float* __restrict__ z, int E, int k, int renorm,
                                          int32_t* __restrict__ idx_out, float* __restrict__ w_out,
                                          int* lds_idx = nullptr) {
  if (E <= 64) topk_wave_pl<1>(z, E, k, renorm, idx_out, w_out, lds_idx);
  else if (E <= 128) topk_wave_pl<2>(z, E, k, renorm, idx_out, w_out, lds_idx);
  else if (E <= 256) topk_wave_pl<4>(z, E, k, renorm, idx_out, w_out, lds_idx);
  else if (E <= 512) topk_wave_pl<8>(z, E, k, renorm, idx_out, w_out, lds_idx);
  else topk_wave_pl<kTopkPerLane>(z, E, k, renorm, idx_out, w_out, lds_idx);
}

// The selection of topk_wave into lds_idx alone (k <= 64 or not): no softmax, no gates.
__device__ __forceinline__ void topk_wave_select(const float* __restrict__ z, int E, int k, int* lds_idx) {
  if (E <= 64) topk_wave_pl<1, false>(z, E, k, 0, nullptr, nullptr, lds_idx);
  else if (E <= 128) topk_wave_pl<2, false>(z, E, k, 0, nullptr, nullptr, lds_idx);
  else if (E <= 256) topk_wave_pl<4, false>(z, E, k, 0, nullptr, nullptr, lds_idx);
  else if (E <= 512) topk_wave_pl<8, false>(z, E, k, 0, nullptr, nullptr, lds_idx);
  else topk_wave_pl<kTopkPerLane, false>(z, E, k, 0, nullptr, nullptr, lds_idx);
}

// Two e2m1 codes (byte `sel` of w, low nibble first) -> two fp32 values, exact.
template <int SEL>
__device__ __forceinline__ void fp4x2_to_f32(uint32_t w, float& a, float& b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  a = v[0];
  b = v[1];
}

// 32 e2m1 codes in 16 bytes -> 32 fp32 values (element i = nibble i, low nibble first).
__device__ __forceinline__ void fp4x32_to_f32(const uint4& q, float* v) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fp4x2_to_f32<0>(w[i], v[8 * i + 0], v[8 * i + 1]);
    fp4x2_to_f32<1>(w[i], v[8 * i + 2], v[8 * i + 3]);
    fp4x2_to_f32<2>(w[i], v[8 * i + 4], v[8 * i + 5]);
    fp4x2_to_f32<3>(w[i], v[8 * i + 6], v[8 * i + 7]);
  }
}

// Block-wide exclusive scan of one int per thread (1024 threads); returns the
// thread's exclusive prefix and writes the total to *total.
__device__ int block_excl_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_tmp[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = (lane < (kLookupThreads / 64)) ? s_tmp[lane] : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int y = __shfl_up(w, off);
      if (lane >= off) w += y;
    }
    if (lane < (kLookupThreads / 64)) s_tmp[32 + lane] = w;  // inclusive wave totals
  }
  __syncthreads();
  int base = (wave > 0) ? s_tmp[32 + wave - 1] : 0;
  *total = s_tmp[32 + (kLookupThreads / 64) - 1];
  __syncthreads();
  return base + x - v;
}

}  // namespace rmoe
