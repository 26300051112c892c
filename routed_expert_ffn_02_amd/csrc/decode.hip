// Decode expert FFN over cache slots: HBM-bound GEMVs.
//
// Small-batch expert execution is memory bound: each routed expert's weights
// are read once per step (FreeToken summary, "decode" challenge section; the
// host/GPU bandwidth comparison).  So the kernels are built around streaming
// each resident record exactly once with 16-byte lane loads:
//
//  phase 1  grid (I / 4, groups): each wavefront reads gate row i and up row i
//           of one expert and forms h = silu(W_g x) * (W_u x) for every token
//           routed to that expert; activations are staged once per block in LDS.
//  phase 2  grid (H / 16, groups): each wavefront reads 4 rows of W_down of one
//           expert and writes per-pair outputs d[pair][row]; the last block to
//           finish a row range (atomic arrival count) combines
//           y[t] = sum_j w[t,j] d[(t,j)] over the GPU pairs in rank order.
// The per-pair values never depend on which slot an expert sits in, and the
// combine order is fixed, so a fully resident cache reproduces the all-resident
// (FUSED) result bit for bit (the Luce Spark post reports the same property
// for its fused path at full residency).
//
// Weight formats: F32 and BF16 rows; FP4 = e2m1 codes (16 bytes = one 32-element
// block per lane load) with one bf16 scale per block, converted exactly by the
// gfx950 scaled-convert instruction with unit scale and scaled after the block dot.
#include "common.hpp"

namespace rmoe {

constexpr int kP1Waves = 4;          // rows (gate/up pairs) per phase-1 block
constexpr int kP2RowsPerWave = 4;
constexpr int kP2Rows = 4 * kP2RowsPerWave;  // rows per phase-2 block

int decode_phase2_rowblocks(int H) { return (H + kP2Rows - 1) / kP2Rows; }

// Pairs routed to group g: (pair index, token) lists in LDS; returns the count.
__device__ __forceinline__ int group_pairs(const DecodeArgs& a, int g, int* s_pair, int* s_n) {
  const int P = a.T * a.k;
  if (threadIdx.x == 0) *s_n = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    if (a.pair_grp[p] == g) {
      int i = atomicAdd(s_n, 1);
      if (i < kDecodeMaxTok) s_pair[i] = p;
    }
  }
  __syncthreads();
  return min(*s_n, kDecodeMaxTok);
}

// ---------------------------------------------------------------------------
// Row dot products against LDS activations.  Each lane covers elements
// [16*c/bpe, ...) of the row for c = lane, lane+64, ...
template <int WFMT>
struct RowDot;

template <>
struct RowDot<MOE_WFMT_F32> {
  static constexpr int kElems = 4;  // per 16-byte chunk
  static __device__ __forceinline__ void chunk(const uint8_t* row, int c, const float* scales_row, float* v) {
    float4 q = reinterpret_cast<const float4*>(row)[c];
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  static __device__ __forceinline__ float scale(const uint8_t*, int) { return 1.f; }
};

template <>
struct RowDot<MOE_WFMT_BF16> {
  static constexpr int kElems = 8;
  static __device__ __forceinline__ void chunk(const uint8_t* row, int c, const float*, float* v) {
    uint4 q = reinterpret_cast<const uint4*>(row)[c];
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
  }
  static __device__ __forceinline__ float scale(const uint8_t*, int) { return 1.f; }
};

template <>
struct RowDot<MOE_WFMT_FP4> {
  static constexpr int kElems = 32;
  static __device__ __forceinline__ void chunk(const uint8_t* row, int c, const float*, float* v) {
    uint4 q = reinterpret_cast<const uint4*>(row)[c];
    fp4x32_to_f32(q, v);
  }
  // scale row pointer holds bf16 scales, one per 32-element block (= one per chunk)
  static __device__ __forceinline__ float scale(const uint8_t* srow, int c) {
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(srow)[c]);
  }
};

template <int WFMT>
__device__ __forceinline__ int64_t row_bytes(int cols) {
  if constexpr (WFMT == MOE_WFMT_F32) return (int64_t)cols * 4;
  else if constexpr (WFMT == MOE_WFMT_BF16) return (int64_t)cols * 2;
  else return (int64_t)cols / 2;
}

// Bytes of one tensor of a record (gate and up are [I,H], down is [H,I]: same count).
template <int WFMT>
__device__ __forceinline__ int64_t tensor_bytes(int H, int I) {
  const int64_t n = (int64_t)H * I;
  if constexpr (WFMT == MOE_WFMT_F32) return n * 4;
  else if constexpr (WFMT == MOE_WFMT_BF16) return n * 2;
  else return n / 2;
}

// Tensor t (0 gate, 1 up, 2 down) row r of a record; FP4 scale rows follow all codes.
template <int WFMT>
__device__ __forceinline__ const uint8_t* tensor_row(const uint8_t* rec, int t, int r, int H, int I) {
  const int cols = (t < 2) ? H : I;
  return rec + (int64_t)t * tensor_bytes<WFMT>(H, I) + (int64_t)r * row_bytes<WFMT>(cols);
}

template <int WFMT>
__device__ __forceinline__ const uint8_t* scale_row(const uint8_t* rec, int t, int r, int H, int I) {
  if constexpr (WFMT != MOE_WFMT_FP4) return nullptr;
  const int64_t n = (int64_t)H * I;
  const int cols = (t < 2) ? H : I;
  return rec + 3 * (n / 2) + (int64_t)t * (n / 32) * 2 + (int64_t)r * (cols / 32) * 2;
}

// ---------------------------------------------------------------------------
template <int WFMT, int AFMT>
__global__ __launch_bounds__(256) void dec_phase1(DecodeArgs a) {
  const int g = blockIdx.y;
  if (g >= a.cnt[C_NGRP]) return;
  __shared__ int s_pair[kDecodeMaxTok];
  __shared__ int s_n;
  extern __shared__ float s_x[];  // [n][H]
  const int n = group_pairs(a, g, s_pair, &s_n);
  const int H = a.H, I = a.I;
  for (int i = threadIdx.x; i < n * H; i += blockDim.x) {
    const int t = s_pair[i / H] / a.k;
    s_x[i] = load_act<AFMT>(a.x, (size_t)t * H + (i % H));
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * kP1Waves + wave;
  if (row >= I) return;
  const uint8_t* rec = a.arena + (int64_t)a.grp_slot[g] * a.rec_bytes;
  const uint8_t* grow = tensor_row<WFMT>(rec, 0, row, H, I);
  const uint8_t* urow = tensor_row<WFMT>(rec, 1, row, H, I);
  const uint8_t* gsrow = scale_row<WFMT>(rec, 0, row, H, I);
  const uint8_t* usrow = scale_row<WFMT>(rec, 1, row, H, I);
  using RD = RowDot<WFMT>;
  constexpr int EPC = RD::kElems;
  const int chunks = H / EPC;
  float accg[kDecodeMaxTok], accu[kDecodeMaxTok];
#pragma unroll
  for (int t = 0; t < kDecodeMaxTok; ++t) { accg[t] = 0.f; accu[t] = 0.f; }
#pragma unroll 4
  for (int c = lane; c < chunks; c += 64) {
    float vg[EPC], vu[EPC];
    RD::chunk(grow, c, nullptr, vg);
    RD::chunk(urow, c, nullptr, vu);
    const float sg = RD::scale(gsrow, c), su = RD::scale(usrow, c);
#pragma unroll
    for (int t = 0; t < kDecodeMaxTok; ++t) {
      if (t < n) {
        const float* xs = &s_x[t * H + c * EPC];
        float pg = 0.f, pu = 0.f;
#pragma unroll
        for (int i = 0; i < EPC; i += 4) {
          const float4 x4 = *reinterpret_cast<const float4*>(xs + i);
          pg += vg[i] * x4.x + vg[i + 1] * x4.y + vg[i + 2] * x4.z + vg[i + 3] * x4.w;
          pu += vu[i] * x4.x + vu[i + 1] * x4.y + vu[i + 2] * x4.z + vu[i + 3] * x4.w;
        }
        accg[t] += sg * pg;
        accu[t] += su * pu;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kDecodeMaxTok; ++t) {
    if (t < n) {
      const float gs = wave_sum(accg[t]);
      const float us = wave_sum(accu[t]);
      if (lane == 0) a.h[(int64_t)s_pair[t] * I + row] = silu(gs) * us;
    }
  }
}

// ---------------------------------------------------------------------------
template <int WFMT, int MAXT>
__global__ __launch_bounds__(256) void dec_phase2(DecodeArgs a) {
  const int g = blockIdx.y;
  const int H = a.H, I = a.I;
  __shared__ int s_pair[kDecodeMaxTok];
  __shared__ int s_n;
  __shared__ int s_last;
  const int ngrp = a.cnt[C_NGRP];
  if (g < ngrp) {
    const int n = min(group_pairs(a, g, s_pair, &s_n), MAXT);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint8_t* rec = a.arena + (int64_t)a.grp_slot[g] * a.rec_bytes;
    using RD = RowDot<WFMT>;
    constexpr int EPC = RD::kElems;
    const int chunks = I / EPC;
    const int r0 = blockIdx.x * kP2Rows + wave * kP2RowsPerWave;
    float acc[kP2RowsPerWave][MAXT];
#pragma unroll
    for (int r = 0; r < kP2RowsPerWave; ++r)
#pragma unroll
      for (int t = 0; t < MAXT; ++t) acc[r][t] = 0.f;
    for (int c = lane; c < chunks; c += 64) {
      // this lane's slice of h for every token of the group
      float hv[MAXT][EPC];
#pragma unroll
      for (int t = 0; t < MAXT; ++t) {
        if (t < n) {
          const float4* hp = reinterpret_cast<const float4*>(a.h + (int64_t)s_pair[t] * I + c * EPC);
#pragma unroll
          for (int i = 0; i < EPC / 4; ++i) {
            float4 q = hp[i];
            hv[t][4 * i] = q.x; hv[t][4 * i + 1] = q.y; hv[t][4 * i + 2] = q.z; hv[t][4 * i + 3] = q.w;
          }
        }
      }
#pragma unroll
      for (int r = 0; r < kP2RowsPerWave; ++r) {
        const int row = r0 + r;
        if (row < H) {
          float v[EPC];
          RD::chunk(tensor_row<WFMT>(rec, 2, row, H, I), c, nullptr, v);
          const float sc = RD::scale(scale_row<WFMT>(rec, 2, row, H, I), c);
#pragma unroll
          for (int t = 0; t < MAXT; ++t) {
            if (t < n) {
              float p = 0.f;
#pragma unroll
              for (int i = 0; i < EPC; ++i) p += v[i] * hv[t][i];
              acc[r][t] += sc * p;
            }
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kP2RowsPerWave; ++r) {
#pragma unroll
      for (int t = 0; t < MAXT; ++t) {
        if (t < n) {
          const float s = wave_sum(acc[r][t]);
          const int row = r0 + r;
          if (lane == 0 && row < H) a.d[(int64_t)s_pair[t] * H + row] = s;
        }
      }
    }
  }
  // arrival count for this row range; the last block combines in rank order
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(&a.rowblock_done[blockIdx.x], 1);
    s_last = (prev == (int)gridDim.y - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const int P = a.T * a.k;
  for (int i = threadIdx.x; i < a.T * kP2Rows; i += blockDim.x) {
    const int t = i / kP2Rows, row = blockIdx.x * kP2Rows + (i % kP2Rows);
    if (row >= H) continue;
    float y = 0.f;
    for (int j = 0; j < a.k; ++j) {
      const int p = t * a.k + j;
      if (p < P && a.pair_grp[p] >= 0) y += a.w[p] * __builtin_nontemporal_load(&a.d[(int64_t)p * H + row]);
    }
    a.y[(int64_t)t * H + row] = y;
  }
  if (threadIdx.x == 0) a.rowblock_done[blockIdx.x] = 0;
}

void launch_decode_phase1(int wfmt, int afmt, const DecodeArgs& a, int max_groups, hipStream_t s) {
  dim3 grid((a.I + kP1Waves - 1) / kP1Waves, max_groups);
  const size_t lds = (size_t)min(a.T, kDecodeMaxTok) * a.H * sizeof(float);
#define P1(W, A) hipLaunchKernelGGL((dec_phase1<W, A>), grid, dim3(256), lds, s, a)
  if (afmt == MOE_AFMT_BF16) {
    if (wfmt == MOE_WFMT_BF16) P1(MOE_WFMT_BF16, MOE_AFMT_BF16);
    else if (wfmt == MOE_WFMT_FP4) P1(MOE_WFMT_FP4, MOE_AFMT_BF16);
    else P1(MOE_WFMT_F32, MOE_AFMT_BF16);
  } else {
    if (wfmt == MOE_WFMT_BF16) P1(MOE_WFMT_BF16, MOE_AFMT_F32);
    else if (wfmt == MOE_WFMT_FP4) P1(MOE_WFMT_FP4, MOE_AFMT_F32);
    else P1(MOE_WFMT_F32, MOE_AFMT_F32);
  }
#undef P1
}

void launch_decode_phase2(int wfmt, const DecodeArgs& a, int max_groups, hipStream_t s) {
  dim3 grid(decode_phase2_rowblocks(a.H), max_groups);
#define P2(W, M) hipLaunchKernelGGL((dec_phase2<W, M>), grid, dim3(256), 0, s, a)
  const int maxt = a.T;  // tokens routed to one expert <= T
  if (wfmt == MOE_WFMT_BF16) {
    if (maxt <= 1) P2(MOE_WFMT_BF16, 1); else if (maxt <= 4) P2(MOE_WFMT_BF16, 4); else P2(MOE_WFMT_BF16, 8);
  } else if (wfmt == MOE_WFMT_FP4) {
    if (maxt <= 1) P2(MOE_WFMT_FP4, 1); else if (maxt <= 4) P2(MOE_WFMT_FP4, 4); else P2(MOE_WFMT_FP4, 8);
  } else {
    if (maxt <= 1) P2(MOE_WFMT_F32, 1); else if (maxt <= 4) P2(MOE_WFMT_F32, 4); else P2(MOE_WFMT_F32, 8);
  }
#undef P2
}

__global__ void add_inplace_kernel(float* y, const float* src, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] += src[i];
}

void launch_add_inplace(float* y, const float* src, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  hipLaunchKernelGGL(add_inplace_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, y, src, n);
}

}  // namespace rmoe
