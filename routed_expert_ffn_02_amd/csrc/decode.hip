// Decode expert FFN over cache slots: HBM-bound GEMVs.
//
// Small-batch expert execution is memory bound: each routed expert's weights
// are read once per step (FreeToken summary, "decode" challenge section; the
// host/GPU bandwidth comparison).  So the kernels are built around streaming
// each resident record exactly once with 16-byte lane loads:
//
//  phase 1  grid (I / rows per block, groups): each wavefront reads a few gate
//           and up rows of one expert and forms h = silu(W_g x) * (W_u x) for
//           every token routed to that expert; activations are staged in LDS
//           while the weight loads are already in flight.
//  phase 2  grid (H / 32, groups): each wavefront reads 8 rows of W_down of one
//           expert and writes per-pair outputs d[pair][row].
//  combine  y[t] = sum_j w[t,j] d[(t,j)] over the GPU pairs in rank order
//           (plus the CPU branch's partial sum when there is one).
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

constexpr int kP2RowsPerWave = 8;
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

// Stage the activation rows of the group's tokens into LDS as fp32 with one
// 16-byte global load per thread per 8 (bf16) or 4 (fp32) elements.
template <int AFMT>
__device__ __forceinline__ void stage_rows(const void* x, const int* s_pair, int k, int n, int H, float* s_x) {
  constexpr int EV = (AFMT == MOE_AFMT_BF16) ? 8 : 4;
  const int per_row = H / EV;
  for (int i = threadIdx.x; i < n * per_row; i += blockDim.x) {
    const int r = i / per_row, c = i % per_row;
    const int t = s_pair[r] / k;
    const uint4 q = reinterpret_cast<const uint4*>(x)[((size_t)t * H) / EV + c];
    float* dst = s_x + r * H + c * EV;
    if constexpr (AFMT == MOE_AFMT_BF16) {
      *reinterpret_cast<float4*>(dst) = make_float4(bf16_lo(q.x), bf16_hi(q.x), bf16_lo(q.y), bf16_hi(q.y));
      *reinterpret_cast<float4*>(dst + 4) = make_float4(bf16_lo(q.z), bf16_hi(q.z), bf16_lo(q.w), bf16_hi(q.w));
    } else {
      *reinterpret_cast<float4*>(dst) = make_float4(__uint_as_float(q.x), __uint_as_float(q.y),
                                                    __uint_as_float(q.z), __uint_as_float(q.w));
    }
  }
}

// ---------------------------------------------------------------------------
// Row dot products against LDS activations.  Each lane covers elements
// [16*c/bpe, ...) of the row for c = lane, lane+64, ...
template <int WFMT>
struct RowDot;

template <>
struct RowDot<MOE_WFMT_F32> {
  static constexpr int kElems = 4;  // per 16-byte chunk
  static __device__ __forceinline__ void unpack(const uint4& q, float* v) {
    v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y); v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
  }
  static __device__ __forceinline__ void chunk(const uint8_t* row, int c, const float*, float* v) {
    unpack(reinterpret_cast<const uint4*>(row)[c], v);
  }
  static __device__ __forceinline__ float scale(const uint8_t*, int) { return 1.f; }
};

template <>
struct RowDot<MOE_WFMT_BF16> {
  static constexpr int kElems = 8;
  static __device__ __forceinline__ void unpack(const uint4& q, float* v) {
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
  }
  static __device__ __forceinline__ void chunk(const uint8_t* row, int c, const float*, float* v) {
    unpack(reinterpret_cast<const uint4*>(row)[c], v);
  }
  static __device__ __forceinline__ float scale(const uint8_t*, int) { return 1.f; }
};

template <>
struct RowDot<MOE_WFMT_FP4> {
  static constexpr int kElems = 32;
  static __device__ __forceinline__ void unpack(const uint4& q, float* v) { fp4x32_to_f32(q, v); }
  static __device__ __forceinline__ void chunk(const uint8_t* row, int c, const float*, float* v) {
    unpack(reinterpret_cast<const uint4*>(row)[c], v);
  }
  // scale row pointer holds bf16 scales, one per 32-element block (= one per chunk)
  static __device__ __forceinline__ float scale(const uint8_t* srow, int c) {
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(srow)[c]);
  }
};

// MXFP4: the same codes with one E8M0 scale byte per block, 2^(e - 127); the byte is
// the exponent field of that power of two as an fp32 (bytes 1..254).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) { return __uint_as_float(e << 23); }

template <>
struct RowDot<MOE_WFMT_MXFP4> {
  static constexpr int kElems = 32;
  static __device__ __forceinline__ void unpack(const uint4& q, float* v) { fp4x32_to_f32(q, v); }
  static __device__ __forceinline__ void chunk(const uint8_t* row, int c, const float*, float* v) {
    unpack(reinterpret_cast<const uint4*>(row)[c], v);
  }
  static __device__ __forceinline__ float scale(const uint8_t* srow, int c) { return e8m0_to_f32(srow[c]); }
};

// e2m1 code formats: bf16 block scales (FP4) or E8M0 block scales (MXFP4)
template <int WFMT>
constexpr bool kIsFp4 = (WFMT == MOE_WFMT_FP4 || WFMT == MOE_WFMT_MXFP4);

// An activated value v = h[pair, row] is stored twice: fp32 in h (the fp32 phase-2 paths)
// and rounded to bf16 (to nearest even) in h16, the operand of the bf16 phase-2 paths,
// which read half the bytes and convert nothing.
__device__ __forceinline__ void store_h(const DecodeArgs& a, int64_t i, float v) {
  a.h[i] = v;
  a.h16[i] = __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Raw block scale c of a scale row (bf16 bits or the E8M0 byte) and its value.
template <int WFMT>
__device__ __forceinline__ uint32_t scale_raw(const uint8_t* srow, int c) {
  if constexpr (WFMT == MOE_WFMT_MXFP4) return srow[c];
  else return reinterpret_cast<const uint16_t*>(srow)[c];
}
template <int WFMT>
__device__ __forceinline__ float scale_value(uint32_t raw) {
  if constexpr (WFMT == MOE_WFMT_MXFP4) return e8m0_to_f32(raw);
  else return bf16_to_f32((uint16_t)raw);
}

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
  if constexpr (!kIsFp4<WFMT>) return nullptr;
  constexpr int SB = (WFMT == MOE_WFMT_MXFP4) ? 1 : 2;  // bytes per block scale
  const int64_t n = (int64_t)H * I;
  const int cols = (t < 2) ? H : I;
  return rec + 3 * (n / 2) + (int64_t)t * (n / 32) * SB + (int64_t)r * (cols / 32) * SB;
}

// Pairs of group g, found by one wavefront with a ballot (no block barrier, so no
// fence waits on the weight loads already in flight).  P <= 64 on the fast path.
__device__ __forceinline__ uint64_t group_mask(const DecodeArgs& a, int g) {
  const int lane = threadIdx.x & 63;
  const int P = a.T * a.k;
  const bool mine = lane < P && a.pair_grp[lane] == g;
  return __ballot(mine);
}

// Activation chunk of token t for lane chunk c: EPC consecutive elements as fp32.
template <int AFMT, int EPC>
__device__ __forceinline__ void load_x_chunk(const void* x, int H, int t, int c, float* v) {
  if constexpr (AFMT == MOE_AFMT_BF16 && EPC == 4) {
    const uint2 q = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(x) + (size_t)t * H + (size_t)c * 4);
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
  } else if constexpr (AFMT == MOE_AFMT_BF16) {
    static_assert(EPC % 8 == 0, "bf16 activation chunks are whole 16-byte loads");
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + (size_t)t * H + (size_t)c * EPC);
#pragma unroll
    for (int i = 0; i < EPC / 8; ++i) {
      const uint4 q = p[i];
      v[8 * i + 0] = bf16_lo(q.x); v[8 * i + 1] = bf16_hi(q.x); v[8 * i + 2] = bf16_lo(q.y); v[8 * i + 3] = bf16_hi(q.y);
      v[8 * i + 4] = bf16_lo(q.z); v[8 * i + 5] = bf16_hi(q.z); v[8 * i + 6] = bf16_lo(q.w); v[8 * i + 7] = bf16_hi(q.w);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + (size_t)t * H + (size_t)c * EPC);
#pragma unroll
    for (int i = 0; i < EPC / 4; ++i) {
      const float4 q = p[i];
      v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
    }
  }
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// 32 e2m1 codes (16 bytes) -> 16 f16 pairs, exact (element 2i in the low nibble).
__device__ __forceinline__ void fp4x32_to_f16x2(const uint4& q, f16x2* o) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[4 * i + 0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 0);
    o[4 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 1);
    o[4 * i + 2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 2);
    o[4 * i + 3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 3);
  }
}

// Raw (unconverted) activation chunk: the loads are issued early and the values are
// converted only where they are used, so nothing waits on them before the weight
// loads have been issued.  Native vectors keep the registers out of memory.
typedef uint32_t u32x4n __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2n __attribute__((ext_vector_type(2)));
typedef float f32x4n __attribute__((ext_vector_type(4)));

template <int AFMT, int EPC>
struct XRaw {
  static constexpr bool kHalf = (AFMT == MOE_AFMT_BF16 && EPC == 4);  // one 8-byte load
  static constexpr int kN = (AFMT == MOE_AFMT_BF16) ? (kHalf ? 1 : EPC / 8) : EPC / 4;
  u32x4n q[kN];
  u32x2n h;
  __device__ __forceinline__ void load(const void* x, int H, int t, int c) {
    if constexpr (kHalf) {
      h = *reinterpret_cast<const u32x2n*>(reinterpret_cast<const uint16_t*>(x) + (size_t)t * H + (size_t)c * 4);
    } else if constexpr (AFMT == MOE_AFMT_BF16) {
      const u32x4n* p = reinterpret_cast<const u32x4n*>(reinterpret_cast<const uint16_t*>(x) + (size_t)t * H + (size_t)c * EPC);
#pragma unroll
      for (int i = 0; i < kN; ++i) q[i] = p[i];
    } else {
      const u32x4n* p = reinterpret_cast<const u32x4n*>(reinterpret_cast<const float*>(x) + (size_t)t * H + (size_t)c * EPC);
#pragma unroll
      for (int i = 0; i < kN; ++i) q[i] = p[i];
    }
  }
  __device__ __forceinline__ void to_f32(float* v) const {
    if constexpr (kHalf) {
      v[0] = bf16_lo(h[0]); v[1] = bf16_hi(h[0]); v[2] = bf16_lo(h[1]); v[3] = bf16_hi(h[1]);
    } else if constexpr (AFMT == MOE_AFMT_BF16) {
#pragma unroll
      for (int i = 0; i < kN; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) { v[8 * i + 2 * j] = bf16_lo(q[i][j]); v[8 * i + 2 * j + 1] = bf16_hi(q[i][j]); }
    } else {
#pragma unroll
      for (int i = 0; i < kN; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) v[4 * i + j] = __uint_as_float(q[i][j]);
    }
  }
};

// ---------------------------------------------------------------------------
// Phase 1, fast path (H a whole number of wavefront-wide chunks, P <= 64): each
// wavefront owns RW consecutive (gate, up) row pairs of one expert; its weight
// chunks and the matching activation chunks are all requested before any is used.
template <int WFMT, int AFMT, int CPL, int RW, int MAXT>
__global__ __launch_bounds__(256) void dec_phase1_fast(DecodeArgs a) {
  const int g = blockIdx.y;
  // both loads issue together (grp_slot has E >= gridDim.y entries, so the read is in
  // bounds even for a group beyond the count, whose value is then unused)
  const int slot = a.grp_slot[g];
  const int H = a.H, I = a.I;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  using RD = RowDot<WFMT>;
  constexpr int EPC = RD::kElems;
  // Loads return in issue order, so whatever a row's dot product needs besides its
  // weights is requested before the weights.  With one token (MAXT == 1) that is
  // token 0's activation chunks, whose address needs no other load; the group's
  // single pair (needed only for the store) comes with the slot.
  float xv[MAXT][CPL][EPC];
  XRaw<AFMT, EPC> xr[CPL];
  int pair0 = 0;
  if constexpr (MAXT == 1) {
    pair0 = a.grp_pair0[g];
#pragma unroll
    for (int c = 0; c < CPL; ++c) xr[c].load(a.x, H, 0, lane + 64 * c);
  }
  if (g >= a.cnt[C_NGRP]) return;
  const int row0 = (blockIdx.x * 4 + wave) * RW;
  if (row0 >= I) return;
  const uint8_t* rec = a.ctrl->arena + (int64_t)slot * a.rec_bytes;
  uint4 qg[RW][CPL], qu[RW][CPL];
  float sg[RW][CPL], su[RW][CPL];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int row = min(row0 + r, I - 1);
    const uint4* gp = reinterpret_cast<const uint4*>(tensor_row<WFMT>(rec, 0, row, H, I));
    const uint4* up = reinterpret_cast<const uint4*>(tensor_row<WFMT>(rec, 1, row, H, I));
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      qg[r][c] = gp[lane + 64 * c];
      qu[r][c] = up[lane + 64 * c];
      sg[r][c] = RD::scale(scale_row<WFMT>(rec, 0, row, H, I), lane + 64 * c);
      su[r][c] = RD::scale(scale_row<WFMT>(rec, 1, row, H, I), lane + 64 * c);
    }
  }
  // the group's pairs (tokens) and their activation chunks
  int pair[MAXT];
  int n = 0;
  if constexpr (MAXT == 1) {
    // every load is in flight; only now consume the first ones (the activations)
    __builtin_amdgcn_sched_barrier(0);
    pair[0] = pair0;
    n = 1;
#pragma unroll
    for (int c = 0; c < CPL; ++c) xr[c].to_f32(xv[0][c]);
  } else {
    uint64_t m = group_mask(a, g);
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      pair[t] = m ? __builtin_ctzll(m) : 0;
      n += (m != 0);
      m &= m - 1;
    }
#pragma unroll
    for (int t = 0; t < MAXT; ++t)
      if (t < n)
#pragma unroll
        for (int c = 0; c < CPL; ++c) load_x_chunk<AFMT, EPC>(a.x, H, pair[t] / a.k, lane + 64 * c, xv[t][c]);
  }
  // FP4: activations as f16 pairs, once per chunk (exact for bf16 inputs inside the
  // f16 range; larger magnitudes overflow to infinity, as the prefill GEMM's f16
  // operands do)
  f16x2 xh[MAXT][CPL][kIsFp4<WFMT> ? 16 : 1];
  if constexpr (kIsFp4<WFMT>) {
#pragma unroll
    for (int t = 0; t < MAXT; ++t)
      if (t < n)
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
          for (int i = 0; i < 16; ++i) xh[t][c][i] = f16x2{(_Float16)xv[t][c][2 * i], (_Float16)xv[t][c][2 * i + 1]};
  }
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int row = row0 + r;
    float accg[MAXT], accu[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; ++t) { accg[t] = 0.f; accu[t] = 0.f; }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      if constexpr (kIsFp4<WFMT>) {
        // codes expand to f16 pairs (exact) and meet the activations in packed dot
        // products with fp32 accumulation: half the VALU work of fp32 FMAs
        f16x2 hg[16], hu[16];
        fp4x32_to_f16x2(qg[r][c], hg);
        fp4x32_to_f16x2(qu[r][c], hu);
#pragma unroll
        for (int t = 0; t < MAXT; ++t) {
          if (t < n) {
            float pg = 0.f, pu = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              pg = __builtin_amdgcn_fdot2(hg[i], xh[t][c][i], pg, false);
              pu = __builtin_amdgcn_fdot2(hu[i], xh[t][c][i], pu, false);
            }
            accg[t] += sg[r][c] * pg;
            accu[t] += su[r][c] * pu;
          }
        }
      } else {
        float vg[EPC], vu[EPC];
        RD::unpack(qg[r][c], vg);
        RD::unpack(qu[r][c], vu);
#pragma unroll
        for (int t = 0; t < MAXT; ++t) {
          if (t < n) {
            float pg = 0.f, pu = 0.f;
#pragma unroll
            for (int i = 0; i < EPC; ++i) {
              pg += vg[i] * xv[t][c][i];
              pu += vu[i] * xv[t][c][i];
            }
            accg[t] += sg[r][c] * pg;
            accu[t] += su[r][c] * pu;
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      if (t < n) {
        const float gs = wave_sum(accg[t]);
        const float us = wave_sum(accu[t]);
        if (lane == 0 && row < I) store_h(a, (int64_t)pair[t] * I + row, silu(gs) * us);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 dot-product paths: bf16 activations against bf16 or FP4 weights.
//
// v_dot2_f32_bf16 multiplies two bf16 pairs exactly and accumulates in fp32, so the
// weights meet the activations as they are stored: bf16 weight words directly, FP4
// codes after the exact scaled convert to bf16 pairs (unit scale), activations as raw
// bf16 words with no conversion.  Per 16-byte weight chunk that is 4 (bf16) or 32 (FP4)
// VALU instructions, against 16 and 34 on the fp32 / f16 paths, which matters because
// the arithmetic of a wavefront's last rows runs after its last bytes arrive.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot_bf16x2(uint32_t w, uint32_t x, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, x), c, false);
}

// Dot product of one 16-byte weight chunk with the matching activation words (bf16
// pairs: 16 for the 32 elements of an e2m1 chunk, 4 for the 8 of a bf16 chunk).  `cs`
// is the convert's scale: 1 for bf16-scaled codes (the block scale multiplies the
// partial sum afterwards), the block's power of two for MXFP4, which the convert
// applies exactly.
template <int WFMT>
__device__ __forceinline__ float chunk_dot_bf16(const u32x4n& q, const uint32_t* xw, float cs = 1.0f) {
  float p = 0.f;
  if constexpr (kIsFp4<WFMT>) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // byte j of word i holds elements 8i + 2j (low nibble) and 8i + 2j + 1
      p = dot_bf16x2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], cs, 0)), xw[4 * i + 0], p);
      p = dot_bf16x2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], cs, 1)), xw[4 * i + 1], p);
      p = dot_bf16x2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], cs, 2)), xw[4 * i + 2], p);
      p = dot_bf16x2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q[i], cs, 3)), xw[4 * i + 3], p);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) p = dot_bf16x2(q[i], xw[i], p);
  }
  return p;
}

// Activation words of token t for lane chunk c (XQ 16-byte loads: the chunk's 32 or 8
// bf16 elements).
template <int XQ>
__device__ __forceinline__ void load_x_words(const void* x, int H, int t, int c, u32x4n* xq) {
  const u32x4n* p = reinterpret_cast<const u32x4n*>(reinterpret_cast<const uint16_t*>(x) + (size_t)t * H) + (size_t)c * XQ;
#pragma unroll
  for (int i = 0; i < XQ; ++i) xq[i] = p[i];
}

// Phase 1, bf16 dot path (H a whole number of wavefront-wide chunks, P <= 64): each
// wavefront owns RW consecutive (gate, up) row pairs of one expert; all its loads are
// issued before any is used, activations first (loads return in issue order), and the
// RW results of a token leave in one store from lanes 0..RW-1.
template <int WFMT, int CPL, int RW, int MAXT, bool ROUTE = false>
__global__ __launch_bounds__(256) void dec_phase1_bf(DecodeArgs a) {
  constexpr int XQ = kIsFp4<WFMT> ? 4 : 1;
  const int g = blockIdx.y;
  const int H = a.H, I = a.I;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  u32x4n xq[MAXT][CPL][XQ];
  int pair[MAXT];
  int n = 0;
  int slot;
  if constexpr (ROUTE) {
    // all resident, one token: wavefront 0 takes the top k from the logits (the selection
    // and gates of the top-k kernel) while the other three stage the token's activation
    // row in LDS, which every wavefront reads back after the barrier.  (Requested by each
    // wavefront ahead of the logits, the row's loads -- one 8 KB row for every wavefront
    // of the launch -- held the logits back, since loads complete in issue order.)  Group g
    // is rank g and its slot is the key.  Workgroup (0, 0) publishes the step.
    static_assert(MAXT == 1, "routed phase 1 is for one token");
    constexpr int NXP = 64 * CPL * XQ;  // 16-byte pieces of the activation row
    __shared__ int s_idx[kSmallLookupPairs];
    __shared__ u32x4n s_x[NXP];
    const bool first = blockIdx.x == 0 && blockIdx.y == 0;
    if (wave == 0) {
      // only workgroup (0, 0) publishes the gates; the others need just the selection
      if (first) topk_wave(a.logits, a.E, a.k, a.renorm, a.topk_out, a.topk_w_out, s_idx);
      else topk_wave_select(a.logits, a.E, a.k, s_idx);
    } else {
      const u32x4n* xp = reinterpret_cast<const u32x4n*>(a.x);
      constexpr int XPT = (NXP + 191) / 192;  // pieces per thread of wavefronts 1..3
      u32x4n xs[XPT];
#pragma unroll
      for (int j = 0; j < XPT; ++j) {
        const int i = threadIdx.x - 64 + 192 * j;
        if (i < NXP) xs[j] = xp[i];
      }
#pragma unroll
      for (int j = 0; j < XPT; ++j) {
        const int i = threadIdx.x - 64 + 192 * j;
        if (i < NXP) s_x[i] = xs[j];
      }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int i = 0; i < XQ; ++i) xq[0][c][i] = s_x[(lane + 64 * c) * XQ + i];
    const int base = a.layer * a.E;
    if (first && wave == 0 && lane < a.k) {
      const int sl = base + s_idx[lane];
      a.grp_slot_out[lane] = sl;
      a.grp_pair0_out[lane] = lane;
      a.pair_grp_out[lane] = lane;
      if (a.slot_out) a.slot_out[lane] = sl;
      if (lane == 0) {
        a.cnt_out[C_NGRP] = a.k;
        a.cnt_out[C_NPAIR_GPU] = a.k;
        a.cnt_out[C_ERR] = 0;
        a.cnt_out[C_T] = 1;
      }
    }
    if (g >= a.k) return;
    slot = base + s_idx[g];
    pair[0] = g;
    n = 1;
  } else {
    // issued with the count (grp_slot has E >= gridDim.y entries, so the read is in bounds
    // even for a group beyond the count, whose value is then unused)
    slot = a.grp_slot[g];
    if constexpr (MAXT == 1) {
      // one token: its activation chunks need no other load, so they go first; the
      // group's single pair (needed only for the store) comes with the slot
      pair[0] = a.grp_pair0[g];
      n = 1;
#pragma unroll
      for (int c = 0; c < CPL; ++c) load_x_words<XQ>(a.x, H, 0, lane + 64 * c, xq[0][c]);
    }
    if (g >= a.cnt[C_NGRP]) return;
  }
  const int row0 = (blockIdx.x * 4 + wave) * RW;
  if (row0 >= I) return;
  const uint8_t* rec = a.ctrl->arena + (int64_t)slot * a.rec_bytes;
  u32x4n qg[RW][CPL], qu[RW][CPL];
  uint16_t sg[RW][CPL], su[RW][CPL];  // block scales (raw bf16 bits or E8M0 bytes)
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const int row = min(row0 + r, I - 1);
    const u32x4n* gp = reinterpret_cast<const u32x4n*>(tensor_row<WFMT>(rec, 0, row, H, I));
    const u32x4n* up = reinterpret_cast<const u32x4n*>(tensor_row<WFMT>(rec, 1, row, H, I));
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      qg[r][c] = gp[lane + 64 * c];
      qu[r][c] = up[lane + 64 * c];
      if constexpr (kIsFp4<WFMT>) {
        sg[r][c] = (uint16_t)scale_raw<WFMT>(scale_row<WFMT>(rec, 0, row, H, I), lane + 64 * c);
        su[r][c] = (uint16_t)scale_raw<WFMT>(scale_row<WFMT>(rec, 1, row, H, I), lane + 64 * c);
      }
    }
  }
  if constexpr (MAXT > 1) {
    uint64_t m = group_mask(a, g);
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      pair[t] = m ? __builtin_ctzll(m) : 0;
      n += (m != 0);
      m &= m - 1;
    }
#pragma unroll
    for (int t = 0; t < MAXT; ++t)
      if (t < n)
#pragma unroll
        for (int c = 0; c < CPL; ++c) load_x_words<XQ>(a.x, H, pair[t] / a.k, lane + 64 * c, xq[t][c]);
  }
  __builtin_amdgcn_sched_barrier(0);  // every load in flight before any use
  float hv[RW][MAXT];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      hv[r][t] = 0.f;
      if (t < n) {
        float accg = 0.f, accu = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          uint32_t xw[4 * XQ];
#pragma unroll
          for (int i = 0; i < 4 * XQ; ++i) xw[i] = xq[t][c][i / 4][i % 4];
          if constexpr (WFMT == MOE_WFMT_MXFP4) {
            accg += chunk_dot_bf16<WFMT>(qg[r][c], xw, e8m0_to_f32(sg[r][c]));
            accu += chunk_dot_bf16<WFMT>(qu[r][c], xw, e8m0_to_f32(su[r][c]));
          } else if constexpr (WFMT == MOE_WFMT_FP4) {
            accg += bf16_to_f32(sg[r][c]) * chunk_dot_bf16<WFMT>(qg[r][c], xw);
            accu += bf16_to_f32(su[r][c]) * chunk_dot_bf16<WFMT>(qu[r][c], xw);
          } else {
            accg += chunk_dot_bf16<WFMT>(qg[r][c], xw);
            accu += chunk_dot_bf16<WFMT>(qu[r][c], xw);
          }
        }
        hv[r][t] = silu(wave_sum(accg)) * wave_sum(accu);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    if (t < n) {
      float v = hv[0][t];
#pragma unroll
      for (int r = 1; r < RW; ++r) v = (lane == r) ? hv[r][t] : v;
      if (lane < RW && row0 + lane < I) store_h(a, (int64_t)pair[t] * I + row0 + lane, v);
    }
  }
}

// Phase 1, generic shapes: one row pair per wavefront, activations staged in LDS.
template <int WFMT, int AFMT>
__global__ __launch_bounds__(256) void dec_phase1(DecodeArgs a) {
  const int g = blockIdx.y;
  if (g >= a.cnt[C_NGRP]) return;
  __shared__ int s_pair[kDecodeMaxTok];
  __shared__ int s_n;
  extern __shared__ float s_x[];  // [n][H]
  const int H = a.H, I = a.I;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  const uint8_t* rec = a.ctrl->arena + (int64_t)a.grp_slot[g] * a.rec_bytes;
  using RD = RowDot<WFMT>;
  constexpr int EPC = RD::kElems;
  const int n = group_pairs(a, g, s_pair, &s_n);
  stage_rows<AFMT>(a.x, s_pair, a.k, n, H, s_x);
  __syncthreads();
  if (row >= I) return;
  float accg[kDecodeMaxTok], accu[kDecodeMaxTok];
#pragma unroll
  for (int t = 0; t < kDecodeMaxTok; ++t) { accg[t] = 0.f; accu[t] = 0.f; }
  for (int c = lane; c < H / EPC; c += 64) {
    float vg[EPC], vu[EPC];
    RD::chunk(tensor_row<WFMT>(rec, 0, row, H, I), c, nullptr, vg);
    RD::chunk(tensor_row<WFMT>(rec, 1, row, H, I), c, nullptr, vu);
    const float scg = RD::scale(scale_row<WFMT>(rec, 0, row, H, I), c);
    const float scu = RD::scale(scale_row<WFMT>(rec, 1, row, H, I), c);
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
        accg[t] += scg * pg;
        accu[t] += scu * pu;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kDecodeMaxTok; ++t) {
    if (t < n) {
      const float gs = wave_sum(accg[t]);
      const float us = wave_sum(accu[t]);
      if (lane == 0) store_h(a, (int64_t)s_pair[t] * I + row, silu(gs) * us);
    }
  }
}

// ---------------------------------------------------------------------------
// Phase 2, fast path (I = 64 chunks per row, P <= 64): each wavefront owns R2 rows
// of W_down of one expert; weight chunks and h slices requested up front.
template <int WFMT, int MAXT>
__global__ __launch_bounds__(256) void dec_phase2_fast(DecodeArgs a) {
  constexpr int R2 = kP2RowsPerWave;
  const int g = blockIdx.y;
  const int slot = a.grp_slot[g];  // issued with the count (see phase 1)
  const int pair0 = (MAXT == 1) ? a.grp_pair0[g] : 0;
  if (g >= a.cnt[C_NGRP]) return;
  const int H = a.H, I = a.I;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r0 = blockIdx.x * kP2Rows + wave * R2;
  if (r0 >= H) return;
  const uint8_t* rec = a.ctrl->arena + (int64_t)slot * a.rec_bytes;
  using RD = RowDot<WFMT>;
  constexpr int EPC = RD::kElems;
  // one token: the group's activated row is requested before the weights (loads
  // return in issue order)
  float hv[MAXT][EPC];
  if constexpr (MAXT == 1) {
    const float4* hp = reinterpret_cast<const float4*>(a.h + (int64_t)pair0 * I + lane * EPC);
#pragma unroll
    for (int i = 0; i < EPC / 4; ++i) {
      const float4 v = hp[i];
      hv[0][4 * i] = v.x; hv[0][4 * i + 1] = v.y; hv[0][4 * i + 2] = v.z; hv[0][4 * i + 3] = v.w;
    }
  }
  uint4 q[R2];
  // the (small) block scales first, kept as raw bits until used: row r then waits
  // only for its own weights
  uint16_t scr[R2];
  if constexpr (kIsFp4<WFMT>) {
#pragma unroll
    for (int r = 0; r < R2; ++r) scr[r] = (uint16_t)scale_raw<WFMT>(scale_row<WFMT>(rec, 2, min(r0 + r, H - 1), H, I), lane);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < R2; ++r)
    q[r] = reinterpret_cast<const uint4*>(tensor_row<WFMT>(rec, 2, min(r0 + r, H - 1), H, I))[lane];
  if constexpr (MAXT == 1) __builtin_amdgcn_sched_barrier(0);  // every load in flight before any use
  int pair[MAXT];
  int n = 0;
  if constexpr (MAXT == 1) {
    pair[0] = pair0;
    n = 1;
  } else {
    uint64_t m = group_mask(a, g);
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      pair[t] = m ? __builtin_ctzll(m) : 0;
      n += (m != 0);
      m &= m - 1;
    }
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      if (t < n) {
        const float4* hp = reinterpret_cast<const float4*>(a.h + (int64_t)pair[t] * I + lane * EPC);
#pragma unroll
        for (int i = 0; i < EPC / 4; ++i) {
          const float4 v = hp[i];
          hv[t][4 * i] = v.x; hv[t][4 * i + 1] = v.y; hv[t][4 * i + 2] = v.z; hv[t][4 * i + 3] = v.w;
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R2; ++r) {
    float v[EPC];
    RD::unpack(q[r], v);
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      if (t < n) {
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < EPC; ++i) p += v[i] * hv[t][i];
        const float scale = kIsFp4<WFMT> ? scale_value<WFMT>(scr[r]) : 1.f;
        const float sum = wave_sum(scale * p);
        const int row = r0 + r;
        if (lane == 0 && row < H) a.d[(int64_t)pair[t] * H + row] = sum;
      }
    }
  }
}

// Phase 2, bf16 dot path (I = 64 chunks per row, P <= 64, bf16 or FP4 weights): each
// wavefront owns R2 rows of W_down of one expert.  The activated rows come as h16, the
// bf16 rounding phase 1 stored (the 16-bit operand rounding the prefill GEMM applies to
// the same values), and meet the weights in v_dot2_f32_bf16.
template <int WFMT, int MAXT>
__global__ __launch_bounds__(256) void dec_phase2_bf(DecodeArgs a) {
  constexpr int R2 = kP2RowsPerWave;
  constexpr int EPC = kIsFp4<WFMT> ? 32 : 8;
  const int g = blockIdx.y;
  const int slot = a.grp_slot[g];  // issued with the count (see phase 1)
  const int pair0 = (MAXT == 1) ? a.grp_pair0[g] : 0;
  if (g >= a.cnt[C_NGRP]) return;
  const int H = a.H, I = a.I;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r0 = blockIdx.x * kP2Rows + wave * R2;
  if (r0 >= H) return;
  const uint8_t* rec = a.ctrl->arena + (int64_t)slot * a.rec_bytes;
  // one token: the group's activated row is requested before the weights
  constexpr int HQ = EPC / 8;  // 16-byte loads of the lane's bf16 h elements
  u32x4n hq[MAXT][HQ];
  if constexpr (MAXT == 1) {
    const u32x4n* hp = reinterpret_cast<const u32x4n*>(a.h16 + (int64_t)pair0 * I + lane * EPC);
#pragma unroll
    for (int i = 0; i < HQ; ++i) hq[0][i] = hp[i];
  }
  uint16_t scr[R2];
  if constexpr (kIsFp4<WFMT>) {
#pragma unroll
    for (int r = 0; r < R2; ++r) scr[r] = (uint16_t)scale_raw<WFMT>(scale_row<WFMT>(rec, 2, min(r0 + r, H - 1), H, I), lane);
  }
  u32x4n q[R2];
#pragma unroll
  for (int r = 0; r < R2; ++r)
    q[r] = reinterpret_cast<const u32x4n*>(tensor_row<WFMT>(rec, 2, min(r0 + r, H - 1), H, I))[lane];
  int pair[MAXT];
  int n = 0;
  if constexpr (MAXT == 1) {
    pair[0] = pair0;
    n = 1;
  } else {
    uint64_t m = group_mask(a, g);
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      pair[t] = m ? __builtin_ctzll(m) : 0;
      n += (m != 0);
      m &= m - 1;
    }
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      if (t < n) {
        const u32x4n* hp = reinterpret_cast<const u32x4n*>(a.h16 + (int64_t)pair[t] * I + lane * EPC);
#pragma unroll
        for (int i = 0; i < HQ; ++i) hq[t][i] = hp[i];
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // every load in flight before any use
  uint32_t hw[MAXT][EPC / 2];  // word i: elements 2i (low half) and 2i + 1
#pragma unroll
  for (int t = 0; t < MAXT; ++t)
    if (t < n)
#pragma unroll
      for (int i = 0; i < EPC / 2; ++i) hw[t][i] = hq[t][i / 4][i % 4];
  float out[R2][MAXT];
#pragma unroll
  for (int r = 0; r < R2; ++r) {
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      out[r][t] = 0.f;
      if (t < n) {
        float p;
        if constexpr (WFMT == MOE_WFMT_MXFP4) p = chunk_dot_bf16<WFMT>(q[r], hw[t], e8m0_to_f32(scr[r]));
        else if constexpr (WFMT == MOE_WFMT_FP4) p = bf16_to_f32(scr[r]) * chunk_dot_bf16<WFMT>(q[r], hw[t]);
        else p = chunk_dot_bf16<WFMT>(q[r], hw[t]);
        out[r][t] = wave_sum(p);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    if (t < n) {
      float v = out[0][t];
#pragma unroll
      for (int r = 1; r < R2; ++r) v = (lane == r) ? out[r][t] : v;
      if (lane < R2 && r0 + lane < H) a.d[(int64_t)pair[t] * H + r0 + lane] = v;
    }
  }
}

// Phase 2 with the combine, one token and no CPU branch (every pair is a GPU pair; pair
// j's expert is found through its slot id, whatever the lookup's group numbering).  A
// workgroup owns R2 rows of the output and has one wavefront per pair: wavefront j
// computes its expert's R2 rows of W_down h_j exactly as dec_phase2_bf does (the same
// loads of the bf16 h_j and dot path), parks them in LDS, and wavefront 0 sums
// w_j * d_j in rank order with one fused multiply-add per pair, the arithmetic of
// dec_combine, so the result is bit-identical to the two separate kernels.
constexpr int kP2cMaxK = 8;
constexpr int kP2cRows = 8;  // output rows per workgroup

template <int WFMT>
__global__ __launch_bounds__(64 * kP2cMaxK) void dec_phase2_combine_bf(DecodeArgs a) {
  constexpr int R2 = kP2cRows;
  constexpr int EPC = kIsFp4<WFMT> ? 32 : 8;  // elements per lane chunk (one 16-byte weight load)
  __shared__ float s_d[kP2cMaxK][R2];
  const int H = a.H, I = a.I, k = a.k;
  const int j = threadIdx.x >> 6, lane = threadIdx.x & 63;  // blockDim.x = 64 * k
  const int r0 = blockIdx.x * R2;
  // a step whose lookup did not place every pair (an expert id out of range: no groups)
  // has stale slot entries, so nothing is read through them and y is 0, as the separate
  // kernels give
  const int ngrp = a.cnt[C_NGRP];
  const int slot = a.slot_idx[j];
  if (ngrp != k) {
    if (j == 0 && lane < R2 && r0 + lane < H) a.y[r0 + lane] = 0.f;
    return;
  }
  const uint8_t* rec = a.ctrl->arena + (int64_t)slot * a.rec_bytes;
  constexpr int HQ = EPC / 8;  // 16-byte loads of the lane's bf16 h elements
  u32x4n hq[HQ];
  const u32x4n* hp = reinterpret_cast<const u32x4n*>(a.h16 + (int64_t)j * I + lane * EPC);
#pragma unroll
  for (int i = 0; i < HQ; ++i) hq[i] = hp[i];
  uint16_t scr[R2];
  if constexpr (kIsFp4<WFMT>) {
#pragma unroll
    for (int r = 0; r < R2; ++r) scr[r] = (uint16_t)scale_raw<WFMT>(scale_row<WFMT>(rec, 2, min(r0 + r, H - 1), H, I), lane);
  }
  u32x4n q[R2];
#pragma unroll
  for (int r = 0; r < R2; ++r)
    q[r] = reinterpret_cast<const u32x4n*>(tensor_row<WFMT>(rec, 2, min(r0 + r, H - 1), H, I))[lane];
  __builtin_amdgcn_sched_barrier(0);  // every load in flight before any use
  uint32_t hw[EPC / 2];
#pragma unroll
  for (int i = 0; i < EPC / 2; ++i) hw[i] = hq[i / 4][i % 4];
  float out[R2];
#pragma unroll
  for (int r = 0; r < R2; ++r) {
    float p;
    if constexpr (WFMT == MOE_WFMT_MXFP4) p = chunk_dot_bf16<WFMT>(q[r], hw, e8m0_to_f32(scr[r]));
    else if constexpr (WFMT == MOE_WFMT_FP4) p = bf16_to_f32(scr[r]) * chunk_dot_bf16<WFMT>(q[r], hw);
    else p = chunk_dot_bf16<WFMT>(q[r], hw);
    out[r] = wave_sum(p);
  }
  float v = out[0];
#pragma unroll
  for (int r = 1; r < R2; ++r) v = (lane == r) ? out[r] : v;
  if (lane < R2) s_d[j][lane] = v;
  __syncthreads();
  if (j == 0 && lane < R2 && r0 + lane < H) {
    float y = 0.f;
    for (int t = 0; t < k; ++t) y = fmaf(a.w[t], s_d[t][lane], y);
    a.y[r0 + lane] = y;
  }
}

// Phase 2, generic shapes.
template <int WFMT, int MAXT>
__global__ __launch_bounds__(256) void dec_phase2(DecodeArgs a) {
  constexpr int R2 = kP2RowsPerWave;
  const int g = blockIdx.y;
  if (g >= a.cnt[C_NGRP]) return;
  const int H = a.H, I = a.I;
  __shared__ int s_pair[kDecodeMaxTok];
  __shared__ int s_n;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint8_t* rec = a.ctrl->arena + (int64_t)a.grp_slot[g] * a.rec_bytes;
  using RD = RowDot<WFMT>;
  constexpr int EPC = RD::kElems;
  const int r0 = blockIdx.x * kP2Rows + wave * R2;
  const int n = min(group_pairs(a, g, s_pair, &s_n), MAXT);
  float acc[R2][MAXT];
#pragma unroll
  for (int r = 0; r < R2; ++r)
#pragma unroll
    for (int t = 0; t < MAXT; ++t) acc[r][t] = 0.f;
  for (int c = lane; c < I / EPC; c += 64) {
    float hv[MAXT][EPC];
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      if (t < n) {
        const float4* hp = reinterpret_cast<const float4*>(a.h + (int64_t)s_pair[t] * I + c * EPC);
#pragma unroll
        for (int i = 0; i < EPC / 4; ++i) {
          const float4 v = hp[i];
          hv[t][4 * i] = v.x; hv[t][4 * i + 1] = v.y; hv[t][4 * i + 2] = v.z; hv[t][4 * i + 3] = v.w;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R2; ++r) {
      const int row = r0 + r;
      if (row >= H) continue;
      float v[EPC];
      RD::chunk(tensor_row<WFMT>(rec, 2, row, H, I), c, nullptr, v);
      const float s = RD::scale(scale_row<WFMT>(rec, 2, row, H, I), c);
#pragma unroll
      for (int t = 0; t < MAXT; ++t) {
        if (t < n) {
          float p = 0.f;
#pragma unroll
          for (int i = 0; i < EPC; ++i) p += v[i] * hv[t][i];
          acc[r][t] += s * p;
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R2; ++r) {
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      if (t < n) {
        const float sum = wave_sum(acc[r][t]);
        const int row = r0 + r;
        if (lane == 0 && row < H) a.d[(int64_t)s_pair[t] * H + row] = sum;
      }
    }
  }
}

// Combine: y[t, r] = sum_{j: GPU pair, rank order} w[t,j] d[(t,j), r]  (+ y_cpu[t, r]),
// one fused multiply-add per pair (the arithmetic dec_phase2_combine_bf repeats).
__global__ void dec_combine(DecodeArgs a, const float* y_cpu) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.T * a.H) return;
  const int t = i / a.H, row = i % a.H;
  float y = 0.f;
  for (int j = 0; j < a.k; ++j) {
    const int p = t * a.k + j;
    if (a.pair_grp[p] >= 0) y = fmaf(a.w[p], a.d[(int64_t)p * a.H + row], y);
  }
  if (y_cpu) y += y_cpu[i];
  a.y[i] = y;
}

// Chunks per lane of a row of `cols` elements, when it is a whole number of
// wavefront-wide 16-byte loads (1, 2, 4, 8); 0 selects the generic kernels.
static int lane_chunks(int wfmt, int cols) {
  const int epc = wfmt == MOE_WFMT_F32 ? 4 : wfmt == MOE_WFMT_BF16 ? 8 : 32;
  if (cols % (64 * epc)) return 0;
  const int c = cols / (64 * epc);
  return (c == 1 || c == 2 || c == 4 || c == 8) ? c : 0;
}

template <int W, int A, int CPL, int MAXT>
static void p1_fast(const DecodeArgs& a, int max_groups, hipStream_t s, Timing tm) {
  if constexpr (A == MOE_AFMT_BF16 && W != MOE_WFMT_F32) {
    // bf16 dot path: 8 KB of weights per wavefront (CPL * RW = 4 lane chunks per tensor)
    constexpr int RW = 4 / CPL;
    dim3 grid((a.I + 4 * RW - 1) / (4 * RW), max_groups);
    launch_timed(dec_phase1_bf<W, CPL, RW, MAXT>, grid, dim3(256), 0, s, tm, a);
  } else {
    // about 16 in-flight 16-byte weight chunks per lane; wide FP4 rows unpack to many registers
    constexpr int RW = (kIsFp4<W> && CPL >= 4) ? 1 : (CPL >= 4) ? 2 : (CPL == 2 ? 4 : 8);
    dim3 grid((a.I + 4 * RW - 1) / (4 * RW), max_groups);
    launch_timed(dec_phase1_fast<W, A, CPL, RW, MAXT>, grid, dim3(256), 0, s, tm, a);
  }
}

template <int W, int CPL>
static void p1_routed(const DecodeArgs& a, hipStream_t s, Timing tm) {
  // every workgroup pays the top-k latency before its loads, so the grid should fit the
  // chip in one round: e2m1 rows take twice the rows per wavefront of the plain kernel
  constexpr int RW = kIsFp4<W> ? 8 / CPL : 4 / CPL;
  dim3 grid((a.I + 4 * RW - 1) / (4 * RW), a.k);
  launch_timed(dec_phase1_bf<W, CPL, RW, 1, true>, grid, dim3(256), 0, s, tm, a);
}

template <int W>
static bool p1_routed_try(const DecodeArgs& a, hipStream_t s, Timing tm) {
  switch (lane_chunks(W, a.H)) {
    case 1: p1_routed<W, 1>(a, s, tm); return true;
    case 2: p1_routed<W, 2>(a, s, tm); return true;
    case 4: p1_routed<W, 4>(a, s, tm); return true;
    default: return false;
  }
}

// All-resident batch-1 phase 1 with the routing taken inside (bf16 activations, bf16 or
// e2m1 weights, rows of 1, 2 or 4 wavefront-wide chunks, k <= 64).
bool decode_phase1_routed_ok(int wfmt, int afmt, int H, int k) {
  if (afmt != MOE_AFMT_BF16 || k > kSmallLookupPairs || wfmt == MOE_WFMT_F32) return false;
  const int c = lane_chunks(wfmt, H);
  return c == 1 || c == 2 || c == 4;
}

bool launch_decode_phase1_routed(int wfmt, int afmt, const DecodeArgs& a, hipStream_t s, Timing tm) {
  if (a.T != 1 || !decode_phase1_routed_ok(wfmt, afmt, a.H, a.k)) return false;
  if (wfmt == MOE_WFMT_BF16) return p1_routed_try<MOE_WFMT_BF16>(a, s, tm);
  if (wfmt == MOE_WFMT_FP4) return p1_routed_try<MOE_WFMT_FP4>(a, s, tm);
  if (wfmt == MOE_WFMT_MXFP4) return p1_routed_try<MOE_WFMT_MXFP4>(a, s, tm);
  return false;
}

template <int W, int A, int MAXT>
static bool p1_try_fast(const DecodeArgs& a, int max_groups, hipStream_t s, Timing tm) {
  switch (lane_chunks(W, a.H)) {
    case 1: p1_fast<W, A, 1, MAXT>(a, max_groups, s, tm); return true;
    case 2: p1_fast<W, A, 2, MAXT>(a, max_groups, s, tm); return true;
    case 4:
      if constexpr (kIsFp4<W> && MAXT > 1) return false;  // 8 KB of activations per token and lane
      else { p1_fast<W, A, 4, MAXT>(a, max_groups, s, tm); return true; }
    default: return false;
  }
}

template <int W, int A>
static void p1_dispatch(const DecodeArgs& a, int max_groups, size_t lds, hipStream_t s, Timing tm) {
  const bool small = a.T * a.k <= 64;
  bool done = false;
  if (small && a.T <= 1) {
    done = p1_try_fast<W, A, 1>(a, max_groups, s, tm);
  } else if constexpr (!kIsFp4<W> || A == MOE_AFMT_BF16) {
    // (FP4 rows with 4 fp32-activation tokens exceed the register file)
    if (small && a.T <= 4) done = p1_try_fast<W, A, 4>(a, max_groups, s, tm);
  }
  if (!done) {
    dim3 grid((a.I + 3) / 4, max_groups);
    launch_timed(dec_phase1<W, A>, grid, dim3(256), (uint32_t)lds, s, tm, a);
  }
}

void launch_decode_phase1(int wfmt, int afmt, const DecodeArgs& a, int max_groups, hipStream_t s, Timing tm) {
  const size_t lds = (size_t)min(a.T, kDecodeMaxTok) * a.H * sizeof(float);
  if (afmt == MOE_AFMT_BF16) {
    if (wfmt == MOE_WFMT_BF16) p1_dispatch<MOE_WFMT_BF16, MOE_AFMT_BF16>(a, max_groups, lds, s, tm);
    else if (wfmt == MOE_WFMT_FP4) p1_dispatch<MOE_WFMT_FP4, MOE_AFMT_BF16>(a, max_groups, lds, s, tm);
    else if (wfmt == MOE_WFMT_MXFP4) p1_dispatch<MOE_WFMT_MXFP4, MOE_AFMT_BF16>(a, max_groups, lds, s, tm);
    else p1_dispatch<MOE_WFMT_F32, MOE_AFMT_BF16>(a, max_groups, lds, s, tm);
  } else {
    if (wfmt == MOE_WFMT_BF16) p1_dispatch<MOE_WFMT_BF16, MOE_AFMT_F32>(a, max_groups, lds, s, tm);
    else if (wfmt == MOE_WFMT_FP4) p1_dispatch<MOE_WFMT_FP4, MOE_AFMT_F32>(a, max_groups, lds, s, tm);
    else if (wfmt == MOE_WFMT_MXFP4) p1_dispatch<MOE_WFMT_MXFP4, MOE_AFMT_F32>(a, max_groups, lds, s, tm);
    else p1_dispatch<MOE_WFMT_F32, MOE_AFMT_F32>(a, max_groups, lds, s, tm);
  }
}

// Whether phase 2 (alone or with the combine) reads the bf16 copy of h: the bf16 dot
// kernels, chosen exactly as in p2_dispatch (T <= 4 takes M <= 4) and by the combine.
bool decode_phase2_reads_h16(int wfmt, int I, int T, int k) {
  return wfmt != MOE_WFMT_F32 && lane_chunks(wfmt, I) == 1 && T * k <= 64 && T <= 4;
}

template <int W, int M>
static void p2_dispatch(const DecodeArgs& a, int max_groups, hipStream_t s, Timing tm) {
  dim3 grid(decode_phase2_rowblocks(a.H), max_groups);
  if (lane_chunks(W, a.I) == 1 && a.T * a.k <= 64) {
    if constexpr (W != MOE_WFMT_F32 && M <= 4) launch_timed(dec_phase2_bf<W, M>, grid, dim3(256), 0, s, tm, a);
    else launch_timed(dec_phase2_fast<W, M>, grid, dim3(256), 0, s, tm, a);
  } else {
    launch_timed(dec_phase2<W, M>, grid, dim3(256), 0, s, tm, a);
  }
}

template <int W>
static void p2_tokens(const DecodeArgs& a, int max_groups, hipStream_t s, Timing tm) {
  if (a.T <= 1) p2_dispatch<W, 1>(a, max_groups, s, tm);
  else if (a.T <= 4) p2_dispatch<W, 4>(a, max_groups, s, tm);
  else p2_dispatch<W, 8>(a, max_groups, s, tm);
}

void launch_decode_phase2(int wfmt, const DecodeArgs& a, int max_groups, hipStream_t s, Timing tm) {
  if (wfmt == MOE_WFMT_BF16) p2_tokens<MOE_WFMT_BF16>(a, max_groups, s, tm);
  else if (wfmt == MOE_WFMT_FP4) p2_tokens<MOE_WFMT_FP4>(a, max_groups, s, tm);
  else if (wfmt == MOE_WFMT_MXFP4) p2_tokens<MOE_WFMT_MXFP4>(a, max_groups, s, tm);
  else p2_tokens<MOE_WFMT_F32>(a, max_groups, s, tm);
}

// Phase 2 and the combine in one launch for one token with no CPU branch (see
// dec_phase2_combine_bf); false: the shape or format needs the separate kernels.
bool launch_decode_phase2_combine(int wfmt, const DecodeArgs& a, hipStream_t s, Timing tm) {
  if (a.T != 1 || a.k < 1 || a.k > kP2cMaxK || wfmt == MOE_WFMT_F32 || lane_chunks(wfmt, a.I) != 1) return false;
  const dim3 grid((a.H + kP2cRows - 1) / kP2cRows), block(64 * a.k);
  if (wfmt == MOE_WFMT_BF16) launch_timed(dec_phase2_combine_bf<MOE_WFMT_BF16>, grid, block, 0, s, tm, a);
  else if (wfmt == MOE_WFMT_FP4) launch_timed(dec_phase2_combine_bf<MOE_WFMT_FP4>, grid, block, 0, s, tm, a);
  else launch_timed(dec_phase2_combine_bf<MOE_WFMT_MXFP4>, grid, block, 0, s, tm, a);
  return true;
}

void launch_decode_combine(const DecodeArgs& a, const float* y_cpu, hipStream_t s) {
  const int n = a.T * a.H;
  hipLaunchKernelGGL(dec_combine, dim3((n + 255) / 256), dim3(256), 0, s, a, y_cpu);
}

}  // namespace rmoe
