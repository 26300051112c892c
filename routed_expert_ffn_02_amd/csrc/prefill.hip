// Prefill: token permutation by expert slot and the grouped SwiGLU GEMMs.
//
// Prefill activates nearly every expert of a layer (FreeToken summary, "prefill"
// challenge section), so the expert FFN is a dense contraction per expert group
// and runs on the MFMA units:
//   GEMM1  [n_g, H] x [H, 2I] -> SwiGLU -> act [n_g, I]   (gate and up tiles of
//          the same output columns are computed by the same wavefront, so the
//          SwiGLU epilogue stays in registers)
//   GEMM2  [n_g, I] x [I, H] -> per-pair outputs ypair[pair, H] (fp32)
//   combine y[t] = sum_j w[t,j] ypair[(t,j)] in rank order (+ CPU partial sum).
// Token rows are gathered through the permutation (stable by (slot, pair)), so
// x is never copied.  Tiles are scheduled (group, n-tile, m-tile) with m-tiles
// of one weight tile adjacent, and the block index is remapped so adjacent
// tiles land on the same XCD (each XCD has its own L2).
//
// BF16 weights use v_mfma_f32_32x32x16_bf16.  FP4 weights (e2m1 codes with a
// bf16 scale per 32 elements) are expanded to f16 with the gfx950 scaled-convert
// instruction at unit scale and multiplied by the scale in f16; e2m1 values have
// at most 2 significant bits and a bf16 scale 8, so the product is exact in f16
// whenever it lies in f16's normal range, and the GEMM uses v_mfma_f32_32x32x16_f16.
// FP32 weights use a plain SIMT path (small shapes; exact fp32 accumulation).
#include "common.hpp"

namespace rmoe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// Native 16-byte vector for register stages: HIP's uint4 is a union-backed struct
// whose copies lower to memcpy and keep the stage out of registers.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 64;   // sorted pair rows per tile
constexpr int BK = 64;   // reduction step (elements)
constexpr int LDSW = BK + 8;  // padded LDS row (elements)

int prefill_bm() { return BM; }


// ---------------------------------------------------------------------------
// Permutation: counting sort of GPU pairs by group (groups are ordered by slot).
constexpr int kChunk = 256;

__global__ __launch_bounds__(kChunk) void perm_hist_kernel(const int32_t* __restrict__ pair_grp, int P, int Gmax,
                                                           int32_t* __restrict__ hist) {
  __shared__ int cnt[kMaxExperts];
  for (int g = threadIdx.x; g < Gmax; g += kChunk) cnt[g] = 0;
  __syncthreads();
  const int p = blockIdx.x * kChunk + threadIdx.x;
  if (p < P) {
    const int g = pair_grp[p];
    if (g >= 0) atomicAdd(&cnt[g], 1);
  }
  __syncthreads();
  for (int g = threadIdx.x; g < Gmax; g += kChunk) hist[(int64_t)blockIdx.x * Gmax + g] = cnt[g];
}

__global__ __launch_bounds__(1024) void perm_scan_kernel(const int32_t* __restrict__ cnt_dev, int nchunks, int Gmax,
                                                         int32_t* __restrict__ hist, int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ tile_base, int bm) {
  __shared__ int s_tmp[64];
  const int ngrp = cnt_dev[C_NGRP];
  const int g = threadIdx.x;
  int tot = 0;
  if (g < ngrp)
    for (int c = 0; c < nchunks; ++c) tot += hist[(int64_t)c * Gmax + g];
  int total;
  const int off = block_excl_scan(tot, s_tmp, &total);
  const int mt = (g < ngrp) ? (tot + bm - 1) / bm : 0;
  int total_tiles;
  const int tb = block_excl_scan(mt, s_tmp, &total_tiles);
  if (g < ngrp) {
    offsets[g] = off;
    tile_base[g] = tb;
    int running = off;
    for (int c = 0; c < nchunks; ++c) {
      const int v = hist[(int64_t)c * Gmax + g];
      hist[(int64_t)c * Gmax + g] = running;
      running += v;
    }
  }
  if (g == 0) {
    offsets[ngrp] = total;
    tile_base[ngrp] = total_tiles;
  }
}

__global__ __launch_bounds__(kChunk) void perm_scatter_kernel(const int32_t* __restrict__ pair_grp, int P, int Gmax,
                                                              const int32_t* __restrict__ hist,
                                                              int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ int s_g[kChunk];
  const int i = threadIdx.x;
  const int p = blockIdx.x * kChunk + i;
  s_g[i] = (p < P) ? pair_grp[p] : -1;
  __syncthreads();
  if (p >= P) return;
  const int g = s_g[i];
  if (g < 0) {
    inv[p] = -1;
    return;
  }
  int r = 0;
  for (int j = 0; j < i; ++j) r += (s_g[j] == g);
  const int pos = hist[(int64_t)blockIdx.x * Gmax + g] + r;
  perm[pos] = p;
  inv[p] = pos;
}

void launch_permute(const int32_t* pair_grp, const int32_t* cnt, int P, int G_max, int32_t* hist, int32_t* perm,
                    int32_t* inv, int32_t* offsets, int32_t* tile_base, int bm, hipStream_t s) {
  const int nchunks = (P + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(perm_hist_kernel, dim3(nchunks), dim3(kChunk), 0, s, pair_grp, P, G_max, hist);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, s, cnt, nchunks, G_max, hist, offsets, tile_base, bm);
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(nchunks), dim3(kChunk), 0, s, pair_grp, P, G_max, hist, perm, inv);
}

// Groups from raw slot ids (the exported moe_permute): distinct slots >= 0, ascending.
// A slot id >= nrange (cnt[C_ERR] = 1) or more than gmax distinct slots (cnt[C_ERR] = 2)
// leaves every pair without a group and no groups, so the permutation kernels that follow
// index nothing out of range; n_groups_out (optional) receives the group count, or -1.
__global__ __launch_bounds__(1024) void groups_from_slots_kernel(const int32_t* __restrict__ slot_idx, int P,
                                                                 int32_t* __restrict__ pair_grp,
                                                                 int32_t* __restrict__ grp_slot,
                                                                 int32_t* __restrict__ cnt, int32_t* flags, int nrange,
                                                                 int gmax, int32_t* n_groups_out) {
  __shared__ int s_tmp[64];
  for (int i = threadIdx.x; i < nrange; i += 1024) flags[i] = 0;
  __syncthreads();
  int bad = 0;
  for (int p = threadIdx.x; p < P; p += 1024) {
    const int sl = slot_idx[p];
    if (sl >= nrange) bad = 1;
    else if (sl >= 0) flags[sl] = 1;
  }
  __threadfence_block();
  __syncthreads();
  const int cpt = (nrange + 1023) / 1024;
  const int i0 = threadIdx.x * cpt, i1 = min(nrange, i0 + cpt);
  int local = 0;
  for (int i = i0; i < i1; ++i) local += flags[i];
  int total;
  int pos = block_excl_scan(local, s_tmp, &total);
  int nbad;
  block_excl_scan(bad, s_tmp, &nbad);
  const int err = nbad ? 1 : (total > gmax ? 2 : 0);
  if (!err) {
    for (int i = i0; i < i1; ++i) {
      if (flags[i]) {
        grp_slot[pos] = i;
        flags[i] = pos + 1;
        ++pos;
      }
    }
  }
  __threadfence_block();
  __syncthreads();
  int npairs = 0;
  for (int p = threadIdx.x; p < P; p += 1024) {
    const int sl = slot_idx[p];
    const int g = (!err && sl >= 0 && sl < nrange) ? flags[sl] - 1 : -1;
    pair_grp[p] = g;
    npairs += (g >= 0);
  }
  int np;
  block_excl_scan(npairs, s_tmp, &np);
  if (threadIdx.x == 0) {
    cnt[C_NGRP] = err ? 0 : total;
    cnt[C_NPAIR_GPU] = np;
    cnt[C_ERR] = err;
    if (n_groups_out) *n_groups_out = err ? -1 : total;
  }
}

void launch_groups_from_slots(const int32_t* slot_idx, int P, int32_t* pair_grp, int32_t* grp_slot, int32_t* cnt,
                              int32_t* scratch_flags, int n_slot_range, int gmax, int32_t* n_groups_out,
                              hipStream_t s) {
  hipLaunchKernelGGL(groups_from_slots_kernel, dim3(1), dim3(1024), 0, s, slot_idx, P, pair_grp, grp_slot, cnt,
                     scratch_flags, n_slot_range, gmax, n_groups_out);
}

// ---------------------------------------------------------------------------
// Tile tables.  A GEMM's tiles are (group, column tile, row tile) in that order, so the row
// tiles of one group's column block (which read the same weights) are adjacent; workgroup b
// runs on XCD b % 8, and XCD x takes a contiguous range of that order, so those tiles share
// one XCD's L2.  The ranges are split by estimated cost rather than by count: in the FP4
// kernels with f16 operands a tile of at most BM / 2 rows (one 32-row fragment per
// wavefront) takes about three quarters of the time of a full one, and with the uneven
// groups of a prompt an equal-count split left one XCD busy 14% longer than another (in
// the bf16 kernels a tile's time follows the weight bytes, which a tile of any height
// reads in full, and in the MX kernels the fragments' MFMAs are too cheap to matter:
// there every tile counts the same).  One small kernel writes, for every
// workgroup of both GEMMs' launches, its tile (or none), so a GEMM workgroup starts with
// one load instead of a binary search over the groups.
struct TileInfo {
  int g, row0, rows, nt;
};

constexpr int kTileCostFull = 4;

int prefill_tile_slots(int max_tiles_m, int nt) {
  // Tiles cost 3 or 4, so an XCD's eighth of the total cost (at most 4 * total / 8) holds
  // at most total / 6 tiles, plus one on each side of its range's boundaries; and
  // total <= max_tiles_m * nt.
  return 8 * (int)(((int64_t)max_tiles_m * nt + 5) / 6 + 2);
}

__device__ void tile_table(int ngrp, const int* s_tb, const int* s_off, const int* s_uc, int bm, int NT, int n,
                           int4* __restrict__ table, int* s_first) {
  const int tid = threadIdx.x;
  const int total = ngrp > 0 ? s_tb[ngrp] * NT : 0;
  // first tile of XCD x: the first whose cost prefix reaches x / 8 of the total cost
  if (tid <= 8) {
    int b = 0;
    if (tid == 8) {
      b = total;
    } else if (tid > 0 && total > 0) {
      const int64_t target = (int64_t)s_uc[ngrp] * NT * tid / 8;
      int lo = 0, hi = ngrp - 1;  // last group whose cost prefix is <= target
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)s_uc[mid] * NT <= target) lo = mid;
        else hi = mid - 1;
      }
      const int mcount = s_tb[lo + 1] - s_tb[lo];
      const int uc = s_uc[lo + 1] - s_uc[lo];  // cost of one column tile of group lo
      const int64_t rem = target - (int64_t)s_uc[lo] * NT;
      int nt = (int)(rem / uc);
      int mt = (int)((rem - (int64_t)nt * uc + kTileCostFull - 1) / kTileCostFull);
      if (mt >= mcount) {
        ++nt;
        mt = 0;
      }
      b = min(total, s_tb[lo] * NT + nt * mcount + mt);
    }
    s_first[tid] = b;
  }
  __syncthreads();
  // a split that would not fit the launch's n / 8 workgroups per XCD falls back to equal
  // counts (which always fit)
  bool fits = true;
  for (int x = 0; x < 8; ++x) fits &= s_first[x + 1] - s_first[x] <= n / 8;
  __syncthreads();
  if (!fits && tid <= 8) s_first[tid] = (int)((int64_t)total * tid / 8);
  __syncthreads();
  for (int e = blockIdx.x * blockDim.x + tid; e < n; e += gridDim.x * blockDim.x) {
    const int x = e & 7, b = s_first[x] + (e >> 3);
    int4 t = {0, 0, 0, 0};
    if (b < s_first[x + 1]) {
      int lo = 0, hi = ngrp - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_tb[mid] * NT <= b) lo = mid;
        else hi = mid - 1;
      }
      const int r = b - s_tb[lo] * NT, mcount = s_tb[lo + 1] - s_tb[lo];
      const int mt = r % mcount;
      const int row0 = s_off[lo] + mt * bm;
      t = int4{lo, row0, min(bm, s_off[lo + 1] - row0), r / mcount};
    }
    table[e] = t;
  }
}

// Workgroups of 1024 threads (groups <= 1024: one per thread in the scan); each computes the
// split from the group counts and writes its slice of both tables.
// Row tiles are bm rows high (a group's last one holds the rest); their count per group
// comes from the group offsets, so a table's bm need not be the permutation's.
__global__ __launch_bounds__(1024) void tile_tables_kernel(const int32_t* __restrict__ cnt,
                                                           const int32_t* __restrict__ offsets, int bm,
                                                           int half_cost, int nt1, int n1, int4* __restrict__ t1,
                                                           int nt2, int n2, int4* __restrict__ t2) {
  __shared__ int s_tb[kMaxExperts + 1], s_off[kMaxExperts + 1], s_uc[kMaxExperts + 1];
  __shared__ int s_tmp[64], s_first[9];
  const int ngrp = min(cnt[C_NGRP], kMaxExperts);
  const int g = threadIdx.x;
  int uc = 0, mcount = 0;  // cost of one column tile of group g (its row tiles), their count
  for (int i = g; i <= ngrp; i += blockDim.x) s_off[i] = offsets[i];
  if (g < ngrp) {
    const int rows = offsets[g + 1] - offsets[g];
    mcount = (rows + bm - 1) / bm;
    if (mcount > 0) {
      const int last = rows - bm * (mcount - 1);
      uc = kTileCostFull * (mcount - 1) + (2 * last <= bm ? half_cost : kTileCostFull);
    }
  }
  int tot, mtot;
  const int pre = block_excl_scan(uc, s_tmp, &tot);
  const int mpre = block_excl_scan(mcount, s_tmp, &mtot);
  if (g < ngrp) {
    s_uc[g] = pre;
    s_tb[g] = mpre;
  }
  if (g == 0 && ngrp >= 0) {
    s_uc[ngrp] = tot;
    s_tb[ngrp] = mtot;
  }
  __syncthreads();
  tile_table(ngrp, s_tb, s_off, s_uc, bm, nt1, n1, t1, s_first);
  __syncthreads();
  tile_table(ngrp, s_tb, s_off, s_uc, bm, nt2, n2, t2, s_first);
}

bool fp4_staged(const PrefillArgs& a);
constexpr int BS_BM = 128;  // row tile of the LDS-staged bf16 kernels

void launch_tile_tables(const PrefillArgs& a, int wfmt, bool mx, int max_tiles_m, hipStream_t s) {
  const bool f16_fp4 = !mx && (wfmt == MOE_WFMT_FP4 || wfmt == MOE_WFMT_MXFP4) && fp4_staged(a);
  // (max_tiles_m counts BM-row tiles, an upper bound for taller ones)
  const int bm = wfmt == MOE_WFMT_BF16 ? BS_BM : BM;
  const int nt1 = a.I / 128, nt2 = a.H / 256;
  const int n1 = prefill_tile_slots(max_tiles_m, nt1), n2 = prefill_tile_slots(max_tiles_m, nt2);
  const int grid = (std::max(n1, n2) + 1023) / 1024;
  hipLaunchKernelGGL(tile_tables_kernel, dim3(grid), dim3(1024), 0, s, a.cnt, a.offsets, bm,
                     f16_fp4 ? 3 : kTileCostFull, nt1, n1, const_cast<int4*>(a.tiles1), nt2, n2,
                     const_cast<int4*>(a.tiles2));
}

// The workgroup's tile from its GEMM's table; false when it has none.  The fields are the
// workgroup's: marked uniform, so addresses built from them (buffer descriptors above all)
// stay in scalar registers.
__device__ __forceinline__ bool decode_tile(const int4* table, TileInfo& ti) {
  const int4 t = table[blockIdx.x];
  if (t.z <= 0) return false;
  ti.g = __builtin_amdgcn_readfirstlane(t.x);
  ti.row0 = __builtin_amdgcn_readfirstlane(t.y);
  ti.rows = __builtin_amdgcn_readfirstlane(t.z);
  ti.nt = __builtin_amdgcn_readfirstlane(t.w);
  return true;
}

// The arena record of tile group g (the same for the whole workgroup).
__device__ __forceinline__ const uint8_t* group_record(const PrefillArgs& a, int g) {
  return a.arena + (int64_t)__builtin_amdgcn_readfirstlane(a.grp_slot[g]) * a.rec_bytes;
}

template <bool F16>
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  if constexpr (F16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                  0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
  }
}

// ---------------------------------------------------------------------------
// Register-streamed grouped GEMMs, for FP4 shapes the LDS-staged kernels below do not take
// (inter % 256 != 0).  Block = 4 wavefronts, 64 sorted rows (2 MFMA row fragments) x
// 4 * 64 weight rows; every wavefront owns 2 weight-row fragments of 32 and computes the
// 2 x 2 fragment product.
//   * B (weights) never touches LDS: each wavefront loads its own weight rows
//     straight into MFMA operand registers and dequantises them there, so every
//     weight byte is read and converted exactly once.
//   * A (activation rows, shared by the 4 wavefronts) goes global -> registers
//     -> LDS, one 64-row x 64-k tile per k-step.
//   * Within a k-step of 64, lane half h (lane >> 5) covers k in [32h, 32h + 32)
//     and MFMA j takes its 8-element slice [32h + 8j, 32h + 8j + 8) from A and B
//     alike: a lane's weight loads are one contiguous 32-element run of a row (one
//     16-byte block of codes with its single scale).
//   * Register stages are indexed by compile-time constants (the k loop is
//     unrolled by the pipeline depth D): D k-steps of loads are in flight while
//     the current step's MFMAs run.

// A: 64 rows x 64 k; thread owns chunks idx = tid + 256 j (row idx / 8, 8-element
// column chunk idx % 8).  f32 sources take two 16-byte loads per chunk.
template <int AFMT>
struct AStage {
  u32x4 v[AFMT == MOE_AFMT_F32 ? 4 : 2];
};

template <int AFMT>
__device__ __forceinline__ void load_a(AStage<AFMT>& st, const void* base, const int64_t* src, int k0) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if constexpr (AFMT == MOE_AFMT_F32) {
      const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(base) + src[j] + k0);
      st.v[2 * j] = p[0];
      st.v[2 * j + 1] = p[1];
    } else {
      st.v[j] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + src[j] + k0);
    }
  }
}

// Chunk j of the stage -> 8 MFMA operand values (bf16, or f16 when TO_F16).
template <int AFMT, bool TO_F16>
__device__ __forceinline__ u32x4 cvt_a8(const AStage<AFMT>& st, int j) {
  if constexpr (AFMT == MOE_AFMT_BF16 && !TO_F16) {
    return st.v[j];
  } else {
    float v[8];
    if constexpr (AFMT == MOE_AFMT_BF16) {
      const u32x4 q = st.v[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_lo(q[i]); v[2 * i + 1] = bf16_hi(q[i]); }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = __uint_as_float(st.v[2 * j][i]);
        v[4 + i] = __uint_as_float(st.v[2 * j + 1][i]);
      }
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t lo, hi;
      if constexpr (TO_F16) {
        lo = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i]);
        hi = __builtin_bit_cast(uint16_t, (_Float16)v[2 * i + 1]);
      } else {
        lo = f32_to_bf16_rne(v[2 * i]);
        hi = f32_to_bf16_rne(v[2 * i + 1]);
      }
      o[i] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    return o;
  }
}

template <int AFMT, bool TO_F16>
__device__ __forceinline__ void store_a(const AStage<AFMT>& st, uint16_t (*sA)[LDSW], int tid) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int idx = tid + 256 * j;
    *reinterpret_cast<u32x4*>(&sA[idx >> 3][(idx & 7) * 8]) = cvt_a8<AFMT, TO_F16>(st, j);
  }
}

// B: this lane's 32-element run of one weight row for one k-step: 16 bytes of FP4 codes at
// row offset (k0 + 32 h) / 2 -- the MFMA slice j of the step is the lane's codes
// 8 j .. 8 j + 7, i.e. k = 32 h + 8 j + [0, 8).  The activation fragments use the same k
// order (a_koff below).
template <int WFMT>
struct BRun;
template <>
struct BRun<MOE_WFMT_FP4> {
  u32x4 v;  // 32 e2m1 codes, element 2i in the low nibble of byte i
};

template <int WFMT>
__device__ __forceinline__ int a_koff(int h, int j) {
  return 32 * h + 8 * j;
}

// Row source of a B run: this lane's row base (FP4: and its scale row).
struct BRow {
  const uint8_t* p;
  const uint16_t* sc;
};

template <int WFMT>
__device__ __forceinline__ BRow b_row(const uint8_t* rec, int H, int I, int tensor, int row, int cols) {
  const int64_t n = (int64_t)H * I;
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(rec + 3 * (n / 2));
  return {rec + tensor * (n / 2) + (int64_t)row * (cols / 2), scales + tensor * (n / 32) + (int64_t)row * (cols / 32)};
}

// Loads of k-step kt (h = lane half).
template <int WFMT>
__device__ __forceinline__ void load_b(BRun<WFMT>& r, const BRow& src, int kt, int h) {
  r.v = *reinterpret_cast<const u32x4*>(src.p + kt * (BK / 2) + 16 * h);
}

// FP4 block scales of a row for the k-step pair (kt, kt + 1), kt even: scales
// [2 kt, 2 kt + 4) in one 8-byte load (aligned: a row holds cols / 32 scales and
// cols % 128 == 0).  Word e holds k-step kt + e; its low half belongs to lane half 0.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x2 load_scales(const BRow& src, int kt) {
  return *reinterpret_cast<const u32x2*>(src.sc + 2 * kt);
}

// MFMA operand j (8 values) of a run of FP4 codes, expanded to f16 and scaled.
template <int WFMT>
struct BOps {
  u32x4 op[4];
};

template <int WFMT>
__device__ __forceinline__ void b_operands(BOps<WFMT>& o, const BRun<WFMT>& r, uint32_t scale_bits) {
  const _Float16 sh = (_Float16)bf16_to_f32((uint16_t)scale_bits);
  const f16x2 s2 = {sh, sh};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = r.v[j];
    const f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
    const f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
    const f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
    const f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
    o.op[j] = u32x4{__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
                    __builtin_bit_cast(uint32_t, v2), __builtin_bit_cast(uint32_t, v3)};
  }
}

// One k-step: 4 MFMA slices j x (2 row fragments) x (2 weight fragments).
template <int WFMT, bool F16>
__device__ __forceinline__ void mfma_step(const uint16_t (*sA)[LDSW], const BOps<WFMT>& b0, const BOps<WFMT>& b1,
                                          int lane, f32x16 (&acc)[2][2]) {
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 a0 = *reinterpret_cast<const u32x4*>(&sA[r][a_koff<WFMT>(h, j)]);
    const u32x4 a1 = *reinterpret_cast<const u32x4*>(&sA[32 + r][a_koff<WFMT>(h, j)]);
    acc[0][0] = mfma32<F16>(a0, b0.op[j], acc[0][0]);
    acc[0][1] = mfma32<F16>(a0, b1.op[j], acc[0][1]);
    acc[1][0] = mfma32<F16>(a1, b0.op[j], acc[1][0]);
    acc[1][1] = mfma32<F16>(a1, b1.op[j], acc[1][1]);
  }
}

// Register stage of one k-step: A chunks and the two B runs.
template <int WFMT>
struct Stage {
  AStage<MOE_AFMT_BF16> a;
  BRun<WFMT> b0, b1;
};

template <int WFMT>
__device__ __forceinline__ void issue(Stage<WFMT>& st, const uint16_t* abase, const int64_t* a_src, const BRow& br0,
                                      const BRow& br1, int kt, int h) {
  load_a<MOE_AFMT_BF16>(st.a, abase, a_src, kt * BK);
  load_b<WFMT>(st.b0, br0, kt, h);
  load_b<WFMT>(st.b1, br1, kt, h);
}

// Prepare a k-step for the MFMAs: its A tile into LDS buffer sAb, its B operands
// into registers (s0, s1: the FP4 scale of each run for this k-step).
template <int WFMT>
__device__ __forceinline__ void prepare(const Stage<WFMT>& st, uint16_t (*sAb)[LDSW], int tid, uint32_t s0,
                                        uint32_t s1, BOps<WFMT>& o0, BOps<WFMT>& o1) {
  store_a<MOE_AFMT_BF16, false>(st.a, sAb, tid);
  b_operands<WFMT>(o0, st.b0, s0);
  b_operands<WFMT>(o1, st.b1, s1);
}

// Software-pipelined k loop over nk k-steps (nk even), two k-steps per iteration.
// Register stages X (even k-steps) and Y (odd) are each refilled two k-steps
// ahead; LDS buffers 0 / 1 hold the A tiles of even / odd k-steps; operand sets
// oX / oY alternate likewise, so nothing is copied at the loop edge.  While the
// MFMAs of k-step s run, the wavefront stores k-step s + 1's A tile and
// dequantises its B operands; one barrier per k-step publishes the A tile.
// Buffer b is rewritten one k-step after it was last read, behind the barrier
// that ended that k-step.  Refills past the end re-read the last k-step (in
// bounds, unused), so the body has no branches and every wait covers exactly one
// stage.  FP4 scales of the pair (s, s + 1) travel with stage X.
template <int WFMT, bool F16>
__device__ __forceinline__ void kloop(int nk, const uint16_t* abase, const int64_t* a_src, const BRow& br0,
                                      const BRow& br1, uint16_t (*sA)[BM][LDSW], int tid, f32x16 (&acc)[2][2]) {
  constexpr bool FP4 = (WFMT == MOE_WFMT_FP4);
  const int lane = tid & 63, h = lane >> 5, hs = 16 * h;
  Stage<WFMT> X, Y;
  BOps<WFMT> oX0, oX1, oY0, oY1;
  u32x2 scX0{}, scX1{};
  issue<WFMT>(X, abase, a_src, br0, br1, 0, h);
  if constexpr (FP4) { scX0 = load_scales(br0, 0); scX1 = load_scales(br1, 0); }
  __builtin_amdgcn_sched_barrier(0);
  issue<WFMT>(Y, abase, a_src, br0, br1, 1, h);
  __builtin_amdgcn_sched_barrier(0);
  uint32_t sY0 = FP4 ? scX0[1] >> hs : 0, sY1 = FP4 ? scX1[1] >> hs : 0;
  prepare<WFMT>(X, sA[0], tid, FP4 ? scX0[0] >> hs : 0, FP4 ? scX1[0] >> hs : 0, oX0, oX1);
  {
    const int kn = min(2, nk - 1);
    issue<WFMT>(X, abase, a_src, br0, br1, kn, h);
    if constexpr (FP4) { scX0 = load_scales(br0, kn & ~1); scX1 = load_scales(br1, kn & ~1); }
  }
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    // even k-step kt: operands oX, A tile in buffer 0; prepare kt + 1 (stage Y)
    prepare<WFMT>(Y, sA[1], tid, sY0, sY1, oY0, oY1);
    issue<WFMT>(Y, abase, a_src, br0, br1, min(kt + 3, nk - 1), h);
    mfma_step<WFMT, F16>(sA[0], oX0, oX1, lane, acc);
    __syncthreads();
    // odd k-step kt + 1: operands oY, A tile in buffer 1; prepare kt + 2 (stage X)
    sY0 = FP4 ? scX0[1] >> hs : 0;
    sY1 = FP4 ? scX1[1] >> hs : 0;
    prepare<WFMT>(X, sA[0], tid, FP4 ? scX0[0] >> hs : 0, FP4 ? scX1[0] >> hs : 0, oX0, oX1);
    {
      const int kn = min(kt + 4, nk - 1);
      issue<WFMT>(X, abase, a_src, br0, br1, kn, h);
      if constexpr (FP4) { scX0 = load_scales(br0, kn & ~1); scX1 = load_scales(br1, kn & ~1); }
    }
    mfma_step<WFMT, F16>(sA[1], oY0, oY1, lane, acc);
    __syncthreads();
  }
}


// Row of output element i (0..15) of a 32x32 MFMA fragment for this lane.
__device__ __forceinline__ int frag_row(int lane, int i) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// ---------------------------------------------------------------------------
// GEMM1: act[sorted row, n0..n0+127] = silu(X W_gate^T) * (X W_up^T) for one group.
// Wavefront w owns act columns n0 + 32 w .. + 31: its two weight fragments are the
// gate and the up rows of those columns, so SwiGLU runs on its own accumulators.
template <int WFMT>
__global__ __launch_bounds__(256, 2) void gemm1_kernel(PrefillArgs a) {
  static_assert(WFMT == MOE_WFMT_FP4, "the register-streamed kernels serve FP4 weights only");
  constexpr bool F16 = true;  // f16 operands and f16 act
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM][LDSW];
  TileInfo ti;
  if (!decode_tile(a.tiles1, ti)) return;
  const int H = a.H, I = a.I;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col0 = ti.nt * 128 + wave * 32;
  const uint8_t* rec = group_record(a, ti.g);

  // A sources: token rows gathered through the permutation.  Rows past the group
  // end read the group's first token; their outputs are never stored.
  int64_t a_src[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int idx = tid + 256 * j, r = idx >> 3;
    const int tok = a.perm[ti.row0 + (r < ti.rows ? r : 0)] / a.k;
    a_src[j] = (int64_t)tok * H + (idx & 7) * 8;
  }
  const BRow bg = b_row<WFMT>(rec, H, I, 0, col0 + (lane & 31), H);
  const BRow bu = b_row<WFMT>(rec, H, I, 1, col0 + (lane & 31), H);

  f32x16 acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][n][i] = 0.f;
  kloop<WFMT, F16>(H / BK, reinterpret_cast<const uint16_t*>(a.xa), a_src, bg, bu, sA, tid, acc);

  // epilogue: SwiGLU in registers, store act (sorted order) as bf16 / f16
  uint16_t* act = reinterpret_cast<uint16_t*>(a.act);
  const int col = col0 + (lane & 31);
#pragma unroll
  for (int m = 0; m < 2; ++m) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * m + frag_row(lane, i);
      if (r < ti.rows) {
        const float g = acc[m][0][i];
        const float v = g * __frcp_rn(1.0f + __expf(-g)) * acc[m][1][i];
        act[(int64_t)(ti.row0 + r) * I + col] = __builtin_bit_cast(uint16_t, (_Float16)v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// GEMM2: ypair[pair, n0..n0+255] = act[sorted rows] W_down^T for one group.
// Wavefront w owns output columns n0 + 64 w .. + 63 (two weight fragments).
template <int WFMT>
__global__ __launch_bounds__(256, 2) void gemm2_kernel(PrefillArgs a) {
  static_assert(WFMT == MOE_WFMT_FP4, "the register-streamed kernels serve FP4 weights only");
  constexpr bool F16 = true;  // f16 operands
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM][LDSW];
  TileInfo ti;
  if (!decode_tile(a.tiles2, ti)) return;
  const int H = a.H, I = a.I;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = ti.nt * 256 + wave * 64;
  const uint8_t* rec = group_record(a, ti.g);

  // A sources: sorted act rows (already in the MFMA operand type).
  int64_t a_src[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int idx = tid + 256 * j, r = idx >> 3;
    a_src[j] = (int64_t)(ti.row0 + (r < ti.rows ? r : 0)) * I + (idx & 7) * 8;
  }
  const BRow b0 = b_row<WFMT>(rec, H, I, 2, c0 + (lane & 31), I);
  const BRow b1 = b_row<WFMT>(rec, H, I, 2, c0 + 32 + (lane & 31), I);

  f32x16 acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][n][i] = 0.f;
  kloop<WFMT, F16>(I / BK, reinterpret_cast<const uint16_t*>(a.act), a_src, b0, b1, sA, tid, acc);

  // pair index of each of the lane's 32 output rows, fetched together (rows past
  // the group end read a valid entry and are not stored)
  int pr[2][16];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * m + frag_row(lane, i);
      pr[m][i] = a.perm[ti.row0 + (r < ti.rows ? r : 0)];
    }
  const int col = c0 + (lane & 31);
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * m + frag_row(lane, i);
      if (r < ti.rows) {
        float* dst = a.ypair + (int64_t)pr[m][i] * H;
        dst[col] = acc[m][0][i];
        dst[col + 32] = acc[m][1][i];
      }
    }
}

// ---------------------------------------------------------------------------
// FP4 grouped GEMMs with the codes staged in LDS.
//
// Fetching MFMA operands lane by lane makes each 1 KB weight load touch 32 rows, i.e.
// 32 cache lines, and the address / L1 path (not the ALUs) then bounds the kernel.
// Here the codes are fetched eight lanes per row, so every load covers whole 128-byte
// lines (a line fetched in two halves at different times reaches HBM twice), written
// to LDS raw (4 bits a weight, a quarter of the bytes of f16), and read back by each
// lane in MFMA layout, where it dequantises them.  A chunk covers 256 k: the
// activation tile (64 x 256, 32 KB) and the block's 256 weight rows x 128 B of codes
// (32 KB), single-buffered in LDS (69 KB, two blocks per CU).  The next chunk waits in
// registers while the current one is multiplied; block scales travel in registers,
// fetched four chunks at a time (see F4Seg).  Refills past the end re-read the last chunk (in
// bounds, unused).  Needs K % 256 == 0.
constexpr int F4_KS = 256;                 // k per chunk
constexpr int F4_AW = F4_KS + 8;           // padded activation row (elements)
constexpr int F4_BP = F4_KS / 2 + 16;      // padded code row (bytes): conflict-free 16-byte reads
constexpr int F4_ROWS = 256;               // weight rows per block

struct F4Chunk {
  u32x4 a[8];  // activation piece i: tile row (tid >> 5) + 8 i, 8 elements at (tid & 31) * 8
  u32x4 b[8];  // code piece j: block row (tid >> 3) + 32 j, 16 bytes at (tid & 7) * 16
};

// Loads go through buffer resources (base and size in scalar registers): a lane's byte
// offset stays in one VGPR for the whole k loop and the chunk's offset is the scalar
// offset, so the register stages share their addressing (no per-piece 64-bit pointers).
struct F4Src {
  __amdgpu_buffer_rsrc_t ra;  // activations
  __amdgpu_buffer_rsrc_t rb;  // expert record
  uint32_t aoff[8];    // byte offset of activation piece i at k = 0
  uint32_t boff[2];    // byte offset of code piece 0 (rows < 128) and piece 4 (rows >= 128) at k = 0
  int32_t bstep;       // bytes from code piece j to piece j + 1 (32 rows)
};

// raw buffer over [p, p + 4 GiB): no size check (every offset here is in bounds by
// construction: records and activation operands stay below 4 GiB, see fp4_staged);
// the last descriptor word is the gfx9 raw-buffer format word
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, -1, 0x00020000);
}

// MR: 32-row activation fragments in the tile (1 for a tile of at most 32 rows, else 2);
// only their rows are fetched and stored.
template <int MR>
__device__ __forceinline__ void f4_issue(F4Chunk& st, const F4Src& src, int c) {
#pragma unroll
  for (int i = 0; i < 4 * MR; ++i)
    st.a[i] = __builtin_amdgcn_raw_buffer_load_b128(src.ra, src.aoff[i], c * (2 * F4_KS), 0);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    st.b[j] = __builtin_amdgcn_raw_buffer_load_b128(src.rb, src.boff[j >> 2], (j & 3) * src.bstep + c * (F4_KS / 2), 0);
}

template <int MR>
__device__ __forceinline__ void f4_store(const F4Chunk& st, uint16_t (*sA)[F4_AW], uint8_t (*sB)[F4_BP], int tid) {
#pragma unroll
  for (int i = 0; i < 4 * MR; ++i) *reinterpret_cast<u32x4*>(&sA[(tid >> 5) + 8 * i][(tid & 31) * 8]) = st.a[i];
#pragma unroll
  for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4*>(&sB[(tid >> 3) + 32 * j][(tid & 7) * 16]) = st.b[j];
}

// Block scales of one weight row.  Chunk c holds blocks [8c, 8c + 8): bf16 scales, 16
// bytes, word w covering k in [64w, 64w + 64) of the chunk with its low half for the lanes
// of half 0 and its high half for half 1; MXFP4 (MX): 8 E8M0 bytes, byte 2w + h for
// sub-step w and lane half h.
//
// They are fetched G chunks at a time (a segment): lane half h loads chunks Gs + hG/2 ..
// Gs + hG/2 + G/2 - 1 of its row, keeps the halves it uses and trades the others with the
// lane 32 away, so a row's scale line is touched once per G chunks.  (Fetched chunk by
// chunk, each 128-byte line was touched eight times, far enough apart for the weight
// stream to evict it in between: it came from memory again every time.)  Pieces past the
// last chunk re-read the last one (in bounds, unused).
template <bool MX, int G>
struct F4Seg {  // the pieces in flight: G / 2 chunks (bf16: one vector each; MX: two per vector)
  u32x4 p[MX ? (G + 3) / 4 : G / 2];
};

template <bool MX, int G>
struct F4SegT {  // this lane's scales of the segment's chunks (c' = chunk - Gs)
  // bf16: t[2c' + (w >> 1)], sub-step w in half w & 1; MX: t[c'], byte w = sub-step w
  uint32_t t[MX ? G : 2 * G];
};

template <bool MX, int G>
__device__ __forceinline__ void f4_seg_load(F4Seg<MX, G>& x, __amdgpu_buffer_rsrc_t rec, uint32_t soff, int s,
                                            int nc, int h) {
  static_assert(G == 2 || G == 4, "segments of two or four chunks");
#pragma unroll
  for (int q = 0; q < G / 2; ++q) {
    // the chunk depends on the lane half, so the whole offset is the lane's (a scalar
    // offset must be the same for every lane)
    const uint32_t c = (uint32_t)min(G * s + (G / 2) * h + q, nc - 1);
    if constexpr (MX) {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rec, soff + 8u * c, 0, 0);
      x.p[q >> 1][2 * (q & 1)] = v[0];
      x.p[q >> 1][2 * (q & 1) + 1] = v[1];
    } else {
      x.p[q] = __builtin_amdgcn_raw_buffer_load_b128(rec, soff + 16u * c, 0, 0);
    }
  }
}

template <bool MX, int G>
__device__ __forceinline__ void f4_seg_build(F4SegT<MX, G>& t, const F4Seg<MX, G>& x, int h) {
  // MX: bytes h and 2 + h of a pair of words (one chunk) -> one word; bf16: the 16-bit
  // halves h of a pair of words (two sub-steps) -> one word
  const uint32_t own = MX ? (h ? 0x07050301u : 0x06040200u) : (h ? 0x07060302u : 0x05040100u);
  const uint32_t other = MX ? (h ? 0x06040200u : 0x07050301u) : (h ? 0x05040100u : 0x07060302u);
  constexpr int NW = MX ? G / 2 : G;  // words this lane builds from its own pieces
  uint32_t keep[NW], give[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t lo = x.p[i >> 1][2 * (i & 1)], hi = x.p[i >> 1][2 * (i & 1) + 1];
    keep[i] = __builtin_amdgcn_perm(hi, lo, own);
    give[i] = __builtin_amdgcn_perm(hi, lo, other);
  }
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t recv = __shfl_xor(give[i], 32);
    t.t[i] = h ? recv : keep[i];
    t.t[NW + i] = h ? keep[i] : recv;
  }
}

// Advance to the next chunk of the segment.
template <bool MX, int G>
__device__ __forceinline__ void f4_seg_next(F4SegT<MX, G>& t) {
  constexpr int W = MX ? 1 : 2, N = MX ? G : 2 * G;
#pragma unroll
  for (int i = 0; i + W < N; ++i) t.t[i] = t.t[i + W];
}

// This lane's scale of sub-step w in the segment's current chunk (low bits).
template <bool MX, int G>
__device__ __forceinline__ uint32_t f4_seg_get(const F4SegT<MX, G>& t, int w) {
  if constexpr (MX) return (t.t[0] >> (8 * w)) & 0xffu;
  else return t.t[w >> 1] >> (16 * (w & 1));
}

// MFMA operands of a run of MXFP4 codes: the convert applies the block's power of
// two 2^(e - 127) itself (exact in f16 inside its range), so no multiply follows.
__device__ __forceinline__ void b_operands_mx(BOps<MOE_WFMT_FP4>& o, const BRun<MOE_WFMT_FP4>& r, uint32_t e) {
  const float sc = __uint_as_float(e << 23);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = r.v[j];
    o.op[j] = u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 0)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 1)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 2)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, sc, 3))};
  }
}

// One chunk: four 64-k sub-steps; lane half h covers k in [32h, 32h + 32) of a
// sub-step (one scale block) and MFMA j its slice [32h + 8j, + 8), in A and B alike.
template <bool MX, int MR>
__device__ __forceinline__ void f4_compute(const uint16_t (*sA)[F4_AW], const uint8_t (*sB)[F4_BP], int rb0, int rb1,
                                           const F4SegT<MX, 4>& t0, const F4SegT<MX, 4>& t1, int lane,
                                           f32x16 (&acc)[MR][2]) {
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    BOps<MOE_WFMT_FP4> o0, o1;
    const BRun<MOE_WFMT_FP4> c0{*reinterpret_cast<const u32x4*>(&sB[rb0 + r][u * 32 + 16 * h])};
    const BRun<MOE_WFMT_FP4> c1{*reinterpret_cast<const u32x4*>(&sB[rb1 + r][u * 32 + 16 * h])};
    if constexpr (MX) {
      b_operands_mx(o0, c0, f4_seg_get<MX, 4>(t0, u));
      b_operands_mx(o1, c1, f4_seg_get<MX, 4>(t1, u));
    } else {
      b_operands<MOE_WFMT_FP4>(o0, c0, f4_seg_get<MX, 4>(t0, u));
      b_operands<MOE_WFMT_FP4>(o1, c1, f4_seg_get<MX, 4>(t1, u));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = u * 64 + 32 * h + 8 * j;
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const u32x4 am = *reinterpret_cast<const u32x4*>(&sA[32 * m + r][k]);
        acc[m][0] = mfma32<true>(am, o0.op[j], acc[m][0]);
        acc[m][1] = mfma32<true>(am, o1.op[j], acc[m][1]);
      }
    }
  }
}

// The k loop over nc = K / 256 chunks.  rb0 / rb1: the wavefront's two 32-row weight
// fragments in the block's LDS rows; sc0 / sc1: byte offsets of their scale rows.  Scale
// segments are four chunks long; segment s is requested with the tiles of chunk 4s and
// unpacked when they are stored.
template <bool MX, int MR>
__device__ __forceinline__ void f4_kloop(int nc, const F4Src& src, uint32_t sc0, uint32_t sc1,
                                         uint16_t (*sA)[F4_AW], uint8_t (*sB)[F4_BP], int rb0, int rb1, int tid,
                                         f32x16 (&acc)[MR][2]) {
  const int lane = tid & 63, h = lane >> 5;
  auto chunk = [&](int c) { return min(c, nc - 1); };
  F4Chunk N;
  F4Seg<MX, 4> x0, x1;
  F4SegT<MX, 4> t0, t1;
  f4_issue<MR>(N, src, chunk(0));
  f4_seg_load<MX, 4>(x0, src.rb, sc0, 0, nc, h);
  f4_seg_load<MX, 4>(x1, src.rb, sc1, 0, nc, h);
  __builtin_amdgcn_sched_barrier(0);
  f4_store<MR>(N, sA, sB, tid);
  f4_seg_build<MX, 4>(t0, x0, h);
  f4_seg_build<MX, 4>(t1, x1, h);
  __syncthreads();
  f4_issue<MR>(N, src, chunk(1));
  __builtin_amdgcn_sched_barrier(0);
  for (int c = 0; c < nc; ++c) {
    f4_compute<MX, MR>(sA, sB, rb0, rb1, t0, t1, lane, acc);
    __syncthreads();  // every wavefront is done with chunk c
    f4_store<MR>(N, sA, sB, tid);
    if (((c + 1) & 3) == 0) {
      f4_seg_build<MX, 4>(t0, x0, h);
      f4_seg_build<MX, 4>(t1, x1, h);
    } else {
      f4_seg_next<MX, 4>(t0);
      f4_seg_next<MX, 4>(t1);
    }
    __syncthreads();
    f4_issue<MR>(N, src, chunk(c + 2));
    if (((c + 2) & 3) == 0) {
      f4_seg_load<MX, 4>(x0, src.rb, sc0, (c + 2) >> 2, nc, h);
      f4_seg_load<MX, 4>(x1, src.rb, sc1, (c + 2) >> 2, nc, h);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// GEMM1 (FP4; MX: MXFP4): act columns n0 .. n0 + 127; block rows 0..127 gate rows n0..,
// 128..255 up.
template <bool MX, int MR>
__device__ __forceinline__ void gemm1_fp4_tile(const PrefillArgs& a, const TileInfo& ti, uint16_t (*sA)[F4_AW],
                                               uint8_t (*sB)[F4_BP]) {
  constexpr uint32_t SB = MX ? 1 : 2;  // bytes per block scale
  const int H = a.H, I = a.I;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = ti.nt * 128;
  const uint8_t* rec = group_record(a, ti.g);
  const int64_t n = (int64_t)H * I;
  // record: gate codes, up codes, down codes (n / 2 bytes each), then bf16 scales

  F4Src src;
  src.ra = buf_rsrc(a.xa);
#pragma unroll
  for (int i = 0; i < 4 * MR; ++i) {
    const int row = (tid >> 5) + 8 * i;
    const uint32_t tok = (uint32_t)(a.perm[ti.row0 + (row < ti.rows ? row : 0)] / a.k);
    src.aoff[i] = 2u * (tok * (uint32_t)H + (uint32_t)(tid & 31) * 8u);
  }
  // block rows 0..127: gate rows n0.., 128..255: up rows n0..
  src.rb = buf_rsrc(rec);
  src.boff[0] = (uint32_t)(n0 + (tid >> 3)) * (uint32_t)(H / 2) + (uint32_t)(tid & 7) * 16u;
  src.boff[1] = src.boff[0] + (uint32_t)(n / 2);
  src.bstep = 32 * (H / 2);
  const int col = n0 + wave * 32 + (lane & 31);
  const uint32_t sc_g = (uint32_t)(3 * (n / 2)) + SB * (uint32_t)col * (uint32_t)(H / 32);
  const uint32_t sc_u = sc_g + SB * (uint32_t)(n / 32);

  f32x16 acc[MR][2];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][q][i] = 0.f;
  f4_kloop<MX, MR>(H / F4_KS, src, sc_g, sc_u, sA, sB, wave * 32, 128 + wave * 32, tid, acc);

  uint16_t* act = reinterpret_cast<uint16_t*>(a.act);
#pragma unroll
  for (int m = 0; m < MR; ++m) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * m + frag_row(lane, i);
      if (r < ti.rows) {
        const float g = acc[m][0][i];
        const float v = g * __frcp_rn(1.0f + __expf(-g)) * acc[m][1][i];
        act[(int64_t)(ti.row0 + r) * I + col] = __builtin_bit_cast(uint16_t, (_Float16)v);
      }
    }
  }
}

// A tile of at most 32 rows runs one 32-row fragment per wavefront (half the MFMAs of
// the padded 64-row tile).
template <bool MX>
__global__ __launch_bounds__(256, 2) void gemm1_fp4_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[64][F4_AW];
  __shared__ __attribute__((aligned(16))) uint8_t sB[F4_ROWS][F4_BP];
  TileInfo ti;
  if (!decode_tile(a.tiles1, ti)) return;
  if (ti.rows <= 32) gemm1_fp4_tile<MX, 1>(a, ti, sA, sB);
  else gemm1_fp4_tile<MX, 2>(a, ti, sA, sB);
}

// GEMM2 (FP4; MX: MXFP4): output columns n0 .. n0 + 255 (down rows); wavefront w owns 64
// of them.
template <bool MX, int MR>
__device__ __forceinline__ void gemm2_fp4_tile(const PrefillArgs& a, const TileInfo& ti, uint16_t (*sA)[F4_AW],
                                               uint8_t (*sB)[F4_BP]) {
  constexpr uint32_t SB = MX ? 1 : 2;  // bytes per block scale
  const int H = a.H, I = a.I;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = ti.nt * 256;
  const uint8_t* rec = group_record(a, ti.g);
  const int64_t n = (int64_t)H * I;
  // record: gate codes, up codes, down codes (n / 2 bytes each), then bf16 scales
  // (gate, up, down: n / 32 each)

  F4Src src;
  src.ra = buf_rsrc(a.act);
#pragma unroll
  for (int i = 0; i < 4 * MR; ++i) {
    const int row = (tid >> 5) + 8 * i;
    src.aoff[i] = 2u * ((uint32_t)(ti.row0 + (row < ti.rows ? row : 0)) * (uint32_t)I + (uint32_t)(tid & 31) * 8u);
  }
  src.rb = buf_rsrc(rec);
  src.boff[0] = (uint32_t)n + (uint32_t)(n0 + (tid >> 3)) * (uint32_t)(I / 2) + (uint32_t)(tid & 7) * 16u;
  src.boff[1] = src.boff[0] + 128u * (uint32_t)(I / 2);
  src.bstep = 32 * (I / 2);
  const int c0 = n0 + wave * 64 + (lane & 31);
  const uint32_t sc0 = (uint32_t)(3 * (n / 2)) + SB * 2u * (uint32_t)(n / 32) + SB * (uint32_t)c0 * (uint32_t)(I / 32);
  const uint32_t sc1 = sc0 + SB * 32u * (uint32_t)(I / 32);

  f32x16 acc[MR][2];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][q][i] = 0.f;
  f4_kloop<MX, MR>(I / F4_KS, src, sc0, sc1, sA, sB, wave * 64, wave * 64 + 32, tid, acc);

  int pr[MR][16];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * m + frag_row(lane, i);
      pr[m][i] = a.perm[ti.row0 + (r < ti.rows ? r : 0)];
    }
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * m + frag_row(lane, i);
      if (r < ti.rows) {
        float* dst = a.ypair + (int64_t)pr[m][i] * H;
        dst[c0] = acc[m][0][i];
        dst[c0 + 32] = acc[m][1][i];
      }
    }
}

template <bool MX>
__global__ __launch_bounds__(256, 2) void gemm2_fp4_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[64][F4_AW];
  __shared__ __attribute__((aligned(16))) uint8_t sB[F4_ROWS][F4_BP];
  TileInfo ti;
  if (!decode_tile(a.tiles2, ti)) return;
  if (ti.rows <= 32) gemm2_fp4_tile<MX, 1>(a, ti, sA, sB);
  else gemm2_fp4_tile<MX, 2>(a, ti, sA, sB);
}

// ---------------------------------------------------------------------------
// bf16 grouped GEMMs with the weights staged in LDS, on the plan of the FP4 kernels above:
// every weight load covers whole 128-byte lines (eight lanes per row), the rows go to LDS
// as they are and each lane reads its MFMA operands back from there.  (The register-direct
// kernels above read 32 bytes of each of 32 rows per load, which bounds them by the
// address path.)  Row tiles are 128 high, so a group of up to 128 rows reads its weights
// once; a tile runs ceil(rows / 32) 32-row fragments per wavefront.  A chunk covers 64 k:
// the activation tile (up to 128 x 64 bf16, 16 KB) and the block's 256 weight rows x 128 B
// (32 KB), single-buffered in LDS (55 KB, two blocks per CU); the next chunk waits in
// registers while the current one is multiplied.  Refills past the end re-read the last
// chunk (in bounds, unused).  Needs K % 64 == 0.
constexpr int BS_KS = 64;          // k per chunk
constexpr int BS_AW = BS_KS + 8;   // padded activation row (elements): conflict-free 16-byte reads

struct BsChunk {
  u32x4 a[4];  // activation piece i: tile row (tid >> 3) + 32 i, 8 elements at (tid & 7) * 8
  u32x4 b[8];  // weight piece j: block row (tid >> 3) + 32 j, 16 bytes at (tid & 7) * 16
};

struct BsSrc {
  __amdgpu_buffer_rsrc_t ra;  // activations
  __amdgpu_buffer_rsrc_t rb;  // expert record
  uint32_t aoff[4];    // byte offset of activation piece i at k = 0
  uint32_t boff[2];    // byte offset of weight piece 0 (rows < 128) and piece 4 (rows >= 128) at k = 0
  int32_t bstep;       // bytes from weight piece j to piece j + 1 (32 rows)
};

template <int MR>
__device__ __forceinline__ void bs_issue(BsChunk& st, const BsSrc& src, int c) {
#pragma unroll
  for (int i = 0; i < MR; ++i) st.a[i] = __builtin_amdgcn_raw_buffer_load_b128(src.ra, src.aoff[i], c * (2 * BS_KS), 0);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    st.b[j] = __builtin_amdgcn_raw_buffer_load_b128(src.rb, src.boff[j >> 2], (j & 3) * src.bstep + c * (2 * BS_KS), 0);
}

template <int MR>
__device__ __forceinline__ void bs_store(const BsChunk& st, uint16_t (*sA)[BS_AW], uint8_t (*sB)[F4_BP], int tid) {
#pragma unroll
  for (int i = 0; i < MR; ++i) *reinterpret_cast<u32x4*>(&sA[(tid >> 3) + 32 * i][(tid & 7) * 8]) = st.a[i];
#pragma unroll
  for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4*>(&sB[(tid >> 3) + 32 * j][(tid & 7) * 16]) = st.b[j];
}

// One chunk: four 16-k MFMA steps; in step j lane half h holds k = 16 j + 8 h + [0, 8)
// of its activation row and of its weight row alike (the operand layout of the 32 x 32 x 16
// bf16 MFMA).
template <int MR>
__device__ __forceinline__ void bs_compute(const uint16_t (*sA)[BS_AW], const uint8_t (*sB)[F4_BP], int rb0, int rb1,
                                           int lane, f32x16 (&acc)[MR][2]) {
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 b0 = *reinterpret_cast<const u32x4*>(&sB[rb0 + r][32 * j + 16 * h]);
    const u32x4 b1 = *reinterpret_cast<const u32x4*>(&sB[rb1 + r][32 * j + 16 * h]);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const u32x4 am = *reinterpret_cast<const u32x4*>(&sA[32 * m + r][16 * j + 8 * h]);
      acc[m][0] = mfma32<false>(am, b0, acc[m][0]);
      acc[m][1] = mfma32<false>(am, b1, acc[m][1]);
    }
  }
}

// The k loop over nc = K / 64 chunks; rb0 / rb1: the wavefront's two 32-row weight
// fragments in the block's LDS rows.
template <int MR>
__device__ __forceinline__ void bs_kloop(int nc, const BsSrc& src, uint16_t (*sA)[BS_AW], uint8_t (*sB)[F4_BP],
                                         int rb0, int rb1, int tid, f32x16 (&acc)[MR][2]) {
  const int lane = tid & 63;
  BsChunk N;
  bs_issue<MR>(N, src, 0);
  __builtin_amdgcn_sched_barrier(0);
  bs_store<MR>(N, sA, sB, tid);
  __syncthreads();
  bs_issue<MR>(N, src, min(1, nc - 1));
  __builtin_amdgcn_sched_barrier(0);
  for (int c = 0; c < nc; ++c) {
    bs_compute<MR>(sA, sB, rb0, rb1, lane, acc);
    __syncthreads();  // every wavefront is done with chunk c
    bs_store<MR>(N, sA, sB, tid);
    __syncthreads();
    bs_issue<MR>(N, src, min(c + 2, nc - 1));
    __builtin_amdgcn_sched_barrier(0);
  }
}

// GEMM1 (bf16 weights): act columns n0 .. n0 + 127; block rows 0..127 gate rows n0..,
// 128..255 up.
template <int MR>
__device__ __forceinline__ void gemm1_bs_tile(const PrefillArgs& a, const TileInfo& ti, uint16_t (*sA)[BS_AW],
                                              uint8_t (*sB)[F4_BP]) {
  const int H = a.H, I = a.I;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = ti.nt * 128;
  const uint8_t* rec = group_record(a, ti.g);
  const int64_t n = (int64_t)H * I;
  // record: gate, up, down weights (n bf16 each)
  BsSrc src;
  src.ra = buf_rsrc(a.xa);
#pragma unroll
  for (int i = 0; i < MR; ++i) {
    const int row = (tid >> 3) + 32 * i;
    const uint32_t tok = (uint32_t)(a.perm[ti.row0 + (row < ti.rows ? row : 0)] / a.k);
    src.aoff[i] = 2u * (tok * (uint32_t)H + (uint32_t)(tid & 7) * 8u);
  }
  src.rb = buf_rsrc(rec);
  src.boff[0] = (uint32_t)(n0 + (tid >> 3)) * (uint32_t)(2 * H) + (uint32_t)(tid & 7) * 16u;
  src.boff[1] = src.boff[0] + (uint32_t)(2 * n);
  src.bstep = 32 * (2 * H);

  f32x16 acc[MR][2];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][q][i] = 0.f;
  bs_kloop<MR>(H / BS_KS, src, sA, sB, wave * 32, 128 + wave * 32, tid, acc);

  uint16_t* act = reinterpret_cast<uint16_t*>(a.act);
  const int col = n0 + wave * 32 + (lane & 31);
#pragma unroll
  for (int m = 0; m < MR; ++m) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * m + frag_row(lane, i);
      if (r < ti.rows) {
        const float g = acc[m][0][i];
        const float v = g * __frcp_rn(1.0f + __expf(-g)) * acc[m][1][i];
        act[(int64_t)(ti.row0 + r) * I + col] = f32_to_bf16_rne(v);
      }
    }
  }
}

__global__ __launch_bounds__(256, 2) void gemm1_bs_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[BS_BM][BS_AW];
  __shared__ __attribute__((aligned(16))) uint8_t sB[F4_ROWS][F4_BP];
  TileInfo ti;
  if (!decode_tile(a.tiles1, ti)) return;
  if (ti.rows <= 32) gemm1_bs_tile<1>(a, ti, sA, sB);
  else if (ti.rows <= 64) gemm1_bs_tile<2>(a, ti, sA, sB);
  else if (ti.rows <= 96) gemm1_bs_tile<3>(a, ti, sA, sB);
  else gemm1_bs_tile<4>(a, ti, sA, sB);
}

// GEMM2 (bf16 weights): output columns n0 .. n0 + 255 (down rows); wavefront w owns 64 of
// them.
template <int MR>
__device__ __forceinline__ void gemm2_bs_tile(const PrefillArgs& a, const TileInfo& ti, uint16_t (*sA)[BS_AW],
                                              uint8_t (*sB)[F4_BP]) {
  const int H = a.H, I = a.I;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = ti.nt * 256;
  const uint8_t* rec = group_record(a, ti.g);
  const int64_t n = (int64_t)H * I;
  BsSrc src;
  src.ra = buf_rsrc(a.act);
#pragma unroll
  for (int i = 0; i < MR; ++i) {
    const int row = (tid >> 3) + 32 * i;
    src.aoff[i] = 2u * ((uint32_t)(ti.row0 + (row < ti.rows ? row : 0)) * (uint32_t)I + (uint32_t)(tid & 7) * 8u);
  }
  src.rb = buf_rsrc(rec);
  src.boff[0] = (uint32_t)(4 * n) + (uint32_t)(n0 + (tid >> 3)) * (uint32_t)(2 * I) + (uint32_t)(tid & 7) * 16u;
  src.boff[1] = src.boff[0] + 128u * (uint32_t)(2 * I);
  src.bstep = 32 * (2 * I);

  f32x16 acc[MR][2];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][q][i] = 0.f;
  bs_kloop<MR>(I / BS_KS, src, sA, sB, wave * 64, wave * 64 + 32, tid, acc);

  const int c0 = n0 + wave * 64 + (lane & 31);
  int pr[MR][16];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * m + frag_row(lane, i);
      pr[m][i] = a.perm[ti.row0 + (r < ti.rows ? r : 0)];
    }
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * m + frag_row(lane, i);
      if (r < ti.rows) {
        float* dst = a.ypair + (int64_t)pr[m][i] * H;
        dst[c0] = acc[m][0][i];
        dst[c0 + 32] = acc[m][1][i];
      }
    }
}

__global__ __launch_bounds__(256, 2) void gemm2_bs_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[BS_BM][BS_AW];
  __shared__ __attribute__((aligned(16))) uint8_t sB[F4_ROWS][F4_BP];
  TileInfo ti;
  if (!decode_tile(a.tiles2, ti)) return;
  if (ti.rows <= 32) gemm2_bs_tile<1>(a, ti, sA, sB);
  else if (ti.rows <= 64) gemm2_bs_tile<2>(a, ti, sA, sB);
  else if (ti.rows <= 96) gemm2_bs_tile<3>(a, ti, sA, sB);
  else gemm2_bs_tile<4>(a, ti, sA, sB);
}

// ---------------------------------------------------------------------------
// MX prefill of MXFP4 experts (opt-in): the activation operand of each GEMM in MXFP8 (E4M3
// elements, one E8M0 scale per 32 along k) meets the weights' e2m1 codes and E8M0 scales as
// stored in v_mfma_scale_f32_32x32x64_f8f6f4 (32 x 32 outputs over 64 k, fp32 accumulation;
// no dequantising instructions).  The instruction's operand layout (measured on gfx950):
// lane l holds row (A) / column (B) l % 32; A bytes 0-15 are k = 16 (l / 32) + j and bytes
// 16-31 are k = 32 + 16 (l / 32) + j; B codes (16 bytes, low nibble first) are
// k = 32 (l / 32) + j; lane l supplies the E8M0 scale of its row / column for the 32-k block
// l / 32.  The accumulator layout is that of the 32 x 32 f16 MFMA (frag_row).
//
// The conversion to MXFP8 (OCP Microscaling v1.0): a block's scale is 2^s with
// s = floor(log2 max|v|) - 8, clamped to [-127, 127] (-127 for a block of zeros or of
// fp32 subnormals); each element v / 2^s goes to the nearest E4M3 value, ties to the even
// code, magnitudes beyond 448 saturating.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  return ef == 0 ? -127 : max(-127, min(127, ef - 127 - 8));
}

// fp32 -> E4M3 code (see above); NaN -> 0x7F
__device__ __forceinline__ uint32_t f32_to_e4m3(float q) {
  const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
  const float a = fabsf(q);
  uint32_t code;
  if (a != a) {
    code = 0x7Fu;
  } else if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {  // below 2^-6: multiples of 2^-9 (8 is the smallest normal, code 0x08)
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;  // -6 .. 8
    uint32_t m = (uint32_t)__builtin_rintf((ldexpf(a, -e) - 1.0f) * 8.0f);
    if (m == 8) {
      m = 0;
      ++e;
    }
    code = ((uint32_t)(e + 7) << 3) | m;
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

// Activations [T, H] (afmt) -> E4M3 codes [T, H] and E8M0 scales [T, H / 32]: one thread
// per 32-element block.
template <int AFMT>
__global__ __launch_bounds__(256) void mx_quant_kernel(const void* __restrict__ x, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales, int64_t nblocks) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  float v[32];
  if constexpr (AFMT == MOE_AFMT_BF16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + 32 * b);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 w = p[q];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * q + 2 * j] = __uint_as_float(w[j] << 16);
        v[8 * q + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + 32 * b);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 w = p[q];
      v[4 * q] = w.x; v[4 * q + 1] = w.y; v[4 * q + 2] = w.z; v[4 * q + 3] = w.w;
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const int s = mx_scale_exp(amax);
  uint32_t w[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    w[q] = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[q] |= f32_to_e4m3(ldexpf(v[4 * q + j], -s)) << (8 * j);
  }
  u32x4* o = reinterpret_cast<u32x4*>(codes + 32 * b);
  o[0] = u32x4{w[0], w[1], w[2], w[3]};
  o[1] = u32x4{w[4], w[5], w[6], w[7]};
  scales[b] = (uint8_t)(s + 127);
}

constexpr int MX_AW = F4_KS + 16;  // padded activation row (bytes): conflict-free 16-byte reads

struct MxChunk {
  u32x4 a[4];   // activation piece i: tile row (tid >> 4) + 16 i, 16 bytes at (tid & 15) * 16
  u32x4 b[8];   // code piece j: block row (tid >> 3) + 32 j, 16 bytes at (tid & 7) * 16
  uint32_t s;   // activation scales (tid < 128): tile row tid >> 1, blocks 4 (tid & 1) .. + 3
};

// Loads go through buffer resources (base and size in scalar registers): a lane's byte
// offset stays in one VGPR for the whole k loop and the chunk's offset is the scalar offset,
// so the two register stages share their addressing (no per-piece 64-bit pointers).
struct MxSrc {
  __amdgpu_buffer_rsrc_t ra;   // activation codes
  __amdgpu_buffer_rsrc_t ras;  // activation scales
  __amdgpu_buffer_rsrc_t rb;   // expert record
  uint32_t aoff[4];    // byte offset of activation piece i at k = 0
  uint32_t asoff;      // byte offset of this thread's scale word at k = 0
  uint32_t boff[2];    // byte offset of code piece 0 (rows < 128) and piece 4 (rows >= 128) at k = 0
  int32_t bstep;       // bytes from code piece j to piece j + 1 (32 rows)
};

template <int MR>
__device__ __forceinline__ void mx_issue(MxChunk& st, const MxSrc& src, int c) {
#pragma unroll
  for (int i = 0; i < 2 * MR; ++i) st.a[i] = __builtin_amdgcn_raw_buffer_load_b128(src.ra, src.aoff[i], c * F4_KS, 0);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    st.b[j] = __builtin_amdgcn_raw_buffer_load_b128(src.rb, src.boff[j >> 2], (j & 3) * src.bstep + c * (F4_KS / 2), 0);
  if (threadIdx.x < 64 * MR) st.s = __builtin_amdgcn_raw_buffer_load_b32(src.ras, src.asoff, c * (F4_KS / 32), 0);
}

template <int MR>
__device__ __forceinline__ void mx_store(const MxChunk& st, uint8_t (*sA)[MX_AW], uint8_t (*sAs)[8],
                                         uint8_t (*sB)[F4_BP], int tid) {
#pragma unroll
  for (int i = 0; i < 2 * MR; ++i) *reinterpret_cast<u32x4*>(&sA[(tid >> 4) + 16 * i][(tid & 15) * 16]) = st.a[i];
#pragma unroll
  for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4*>(&sB[(tid >> 3) + 32 * j][(tid & 7) * 16]) = st.b[j];
  if (tid < 64 * MR) *reinterpret_cast<uint32_t*>(&sAs[tid >> 1][4 * (tid & 1)]) = st.s;
}

__device__ __forceinline__ f32x16 mfma_mx(const u32x4& alo, const u32x4& ahi, const u32x4& b, uint32_t sa,
                                          uint32_t sb, const f32x16& c) {
  typedef int v8i __attribute__((ext_vector_type(8)));
  const v8i av = {(int)alo[0], (int)alo[1], (int)alo[2], (int)alo[3], (int)ahi[0], (int)ahi[1], (int)ahi[2], (int)ahi[3]};
  const v8i bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  // A: E4M3 (format 0), B: e2m1 (format 4); each scale in byte 0 of its operand
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 4, 0, (int)sa, 0, (int)sb);
}

// One 256-k chunk: four 64-k steps; for step u the lane's weight scales are bytes 2u + h of
// the chunk's eight (one E8M0 byte per 32-k block), its activation scales bytes 2u + h of
// its tile row's.
template <int MR>
__device__ __forceinline__ void mx_compute(const uint8_t (*sA)[MX_AW], const uint8_t (*sAs)[8],
                                           const uint8_t (*sB)[F4_BP], int rb0, int rb1, const F4SegT<true, 2>& t0,
                                           const F4SegT<true, 2>& t1, int lane, f32x16 (&acc)[MR][2]) {
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const u32x4 b0 = *reinterpret_cast<const u32x4*>(&sB[rb0 + r][32 * u + 16 * h]);
    const u32x4 b1 = *reinterpret_cast<const u32x4*>(&sB[rb1 + r][32 * u + 16 * h]);
    const uint32_t s0 = f4_seg_get<true, 2>(t0, u), s1 = f4_seg_get<true, 2>(t1, u);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const u32x4 alo = *reinterpret_cast<const u32x4*>(&sA[32 * m + r][64 * u + 16 * h]);
      const u32x4 ahi = *reinterpret_cast<const u32x4*>(&sA[32 * m + r][64 * u + 32 + 16 * h]);
      const uint32_t sa = sAs[32 * m + r][2 * u + h];
      acc[m][0] = mfma_mx(alo, ahi, b0, sa, s0, acc[m][0]);
      acc[m][1] = mfma_mx(alo, ahi, b1, sa, s1, acc[m][1]);
    }
    __builtin_amdgcn_sched_barrier(0);  // one step's LDS operands live at a time
  }
}

// The k loop over nc = K / 256 chunks (the structure of f4_kloop, weight scales fetched
// in two-chunk segments: four would not fit the registers); rb0 / rb1: the wavefront's two 32-row weight fragments
// in the block's LDS rows; sc0 / sc1: byte offsets of their E8M0 scale rows.  Refills past
// the end re-read the last chunk (in bounds, unused).
template <int MR>
__device__ __forceinline__ void mx_kloop(int nc, const MxSrc& src, uint32_t sc0, uint32_t sc1, uint8_t (*sA)[MX_AW],
                                         uint8_t (*sAs)[8], uint8_t (*sB)[F4_BP], int rb0, int rb1, int tid,
                                         f32x16 (&acc)[MR][2]) {
  const int lane = tid & 63, h = lane >> 5;
  MxChunk N;
  F4Seg<true, 2> x0, x1;
  F4SegT<true, 2> t0, t1;
  mx_issue<MR>(N, src, 0);
  f4_seg_load<true, 2>(x0, src.rb, sc0, 0, nc, h);
  f4_seg_load<true, 2>(x1, src.rb, sc1, 0, nc, h);
  __builtin_amdgcn_sched_barrier(0);
  mx_store<MR>(N, sA, sAs, sB, tid);
  f4_seg_build<true, 2>(t0, x0, h);
  f4_seg_build<true, 2>(t1, x1, h);
  __syncthreads();
  mx_issue<MR>(N, src, min(1, nc - 1));
  __builtin_amdgcn_sched_barrier(0);
  for (int c = 0; c < nc; ++c) {
    mx_compute<MR>(sA, sAs, sB, rb0, rb1, t0, t1, lane, acc);
    __syncthreads();  // every wavefront is done with chunk c
    mx_store<MR>(N, sA, sAs, sB, tid);
    if (((c + 1) & 1) == 0) {
      f4_seg_build<true, 2>(t0, x0, h);
      f4_seg_build<true, 2>(t1, x1, h);
    } else {
      f4_seg_next<true, 2>(t0);
      f4_seg_next<true, 2>(t1);
    }
    __syncthreads();
    mx_issue<MR>(N, src, min(c + 2, nc - 1));
    if (((c + 2) & 1) == 0) {
      f4_seg_load<true, 2>(x0, src.rb, sc0, (c + 2) >> 1, nc, h);
      f4_seg_load<true, 2>(x1, src.rb, sc1, (c + 2) >> 1, nc, h);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Activation sources of a tile: piece i of thread tid is tile row (tid >> 4) + 16 i (row 0
// of the tile for rows past its end), the scale word tile row tid >> 1.
template <int MR>
__device__ __forceinline__ void mx_rows(MxSrc& src, const TileInfo& ti, int tid, bool gather, const PrefillArgs& a,
                                        uint32_t K) {
  auto row_of = [&](int r) -> uint32_t {
    const int rr = r < ti.rows ? r : 0;
    return gather ? (uint32_t)(a.perm[ti.row0 + rr] / a.k) : (uint32_t)(ti.row0 + rr);
  };
#pragma unroll
  for (int i = 0; i < 2 * MR; ++i) src.aoff[i] = row_of((tid >> 4) + 16 * i) * K + (uint32_t)(tid & 15) * 16u;
  src.asoff = row_of((tid >> 1) & 63) * (K / 32) + 4u * (uint32_t)(tid & 1);
}

// GEMM1 (MX): act columns n0 .. n0 + 127 of the tile as MXFP8 (codes + one scale per 32
// columns, the wavefront's own 32); block rows 0..127 gate rows n0.., 128..255 up.
template <int MR>
__device__ __forceinline__ void gemm1_mx_tile(const PrefillArgs& a, const TileInfo& ti, uint8_t (*sA)[MX_AW],
                                              uint8_t (*sAs)[8], uint8_t (*sB)[F4_BP]) {
  const int H = a.H, I = a.I;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = ti.nt * 128;
  const uint8_t* rec = group_record(a, ti.g);
  const int64_t n = (int64_t)H * I;
  MxSrc src;
  src.ra = buf_rsrc(a.xa);
  src.ras = buf_rsrc(a.xs);
  mx_rows<MR>(src, ti, tid, true, a, (uint32_t)H);
  src.rb = buf_rsrc(rec);
  src.boff[0] = (uint32_t)(n0 + (tid >> 3)) * (uint32_t)(H / 2) + (uint32_t)(tid & 7) * 16u;
  src.boff[1] = src.boff[0] + (uint32_t)(n / 2);
  src.bstep = 32 * (H / 2);
  const int col = n0 + wave * 32 + (lane & 31);
  // record: gate, up, down codes (n / 2 bytes each), then E8M0 scales (n / 32 each)
  const uint32_t sc_g = (uint32_t)(3 * (n / 2)) + (uint32_t)col * (uint32_t)(H / 32);
  const uint32_t sc_u = sc_g + (uint32_t)(n / 32);
  f32x16 acc[MR][2];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][q][i] = 0.f;
  mx_kloop<MR>(H / F4_KS, src, sc_g, sc_u, sA, sAs, sB, wave * 32, 128 + wave * 32, tid, acc);

  // SwiGLU in fp32, then MXFP8 over each row's 32 columns (held by the 32 lanes of a half)
  uint8_t* act = reinterpret_cast<uint8_t*>(a.act);
#pragma unroll
  for (int m = 0; m < MR; ++m) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * m + frag_row(lane, i);
      const float g = acc[m][0][i];
      const float v = g * __frcp_rn(1.0f + __expf(-g)) * acc[m][1][i];
      float am = fabsf(v);
#pragma unroll
      for (int d = 1; d < 32; d <<= 1) am = fmaxf(am, __shfl_xor(am, d));
      const int s = mx_scale_exp(am);
      const uint32_t code = f32_to_e4m3(ldexpf(v, -s));
      if (r < ti.rows) {
        act[(int64_t)(ti.row0 + r) * I + col] = (uint8_t)code;
        if ((lane & 31) == 0) a.acts[(int64_t)(ti.row0 + r) * (I / 32) + (col >> 5)] = (uint8_t)(s + 127);
      }
    }
  }
}

// GEMM2 (MX): output columns n0 .. n0 + 255 (down rows); wavefront w owns 64 of them.
template <int MR>
__device__ __forceinline__ void gemm2_mx_tile(const PrefillArgs& a, const TileInfo& ti, uint8_t (*sA)[MX_AW],
                                              uint8_t (*sAs)[8], uint8_t (*sB)[F4_BP]) {
  const int H = a.H, I = a.I;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = ti.nt * 256;
  const uint8_t* rec = group_record(a, ti.g);
  const int64_t n = (int64_t)H * I;
  MxSrc src;
  src.ra = buf_rsrc(a.act);
  src.ras = buf_rsrc(a.acts);
  mx_rows<MR>(src, ti, tid, false, a, (uint32_t)I);
  src.rb = buf_rsrc(rec);
  src.boff[0] = (uint32_t)n + (uint32_t)(n0 + (tid >> 3)) * (uint32_t)(I / 2) + (uint32_t)(tid & 7) * 16u;
  src.boff[1] = src.boff[0] + 128u * (uint32_t)(I / 2);
  src.bstep = 32 * (I / 2);
  const int c0 = n0 + wave * 64 + (lane & 31);
  const uint32_t sc0 = (uint32_t)(3 * (n / 2)) + 2u * (uint32_t)(n / 32) + (uint32_t)c0 * (uint32_t)(I / 32);
  const uint32_t sc1 = sc0 + 32u * (uint32_t)(I / 32);
  f32x16 acc[MR][2];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][q][i] = 0.f;
  mx_kloop<MR>(I / F4_KS, src, sc0, sc1, sA, sAs, sB, wave * 64, wave * 64 + 32, tid, acc);

  int pr[MR][16];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * m + frag_row(lane, i);
      pr[m][i] = a.perm[ti.row0 + (r < ti.rows ? r : 0)];
    }
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * m + frag_row(lane, i);
      if (r < ti.rows) {
        float* dst = a.ypair + (int64_t)pr[m][i] * H;
        dst[c0] = acc[m][0][i];
        dst[c0 + 32] = acc[m][1][i];
      }
    }
}

__global__ __launch_bounds__(256, 2) void gemm1_mx_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[64][MX_AW];
  __shared__ __attribute__((aligned(16))) uint8_t sAs[64][8];
  __shared__ __attribute__((aligned(16))) uint8_t sB[F4_ROWS][F4_BP];
  TileInfo ti;
  if (!decode_tile(a.tiles1, ti)) return;
  if (ti.rows <= 32) gemm1_mx_tile<1>(a, ti, sA, sAs, sB);
  else gemm1_mx_tile<2>(a, ti, sA, sAs, sB);
}

__global__ __launch_bounds__(256, 2) void gemm2_mx_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[64][MX_AW];
  __shared__ __attribute__((aligned(16))) uint8_t sAs[64][8];
  __shared__ __attribute__((aligned(16))) uint8_t sB[F4_ROWS][F4_BP];
  TileInfo ti;
  if (!decode_tile(a.tiles2, ti)) return;
  if (ti.rows <= 32) gemm2_mx_tile<1>(a, ti, sA, sAs, sB);
  else gemm2_mx_tile<2>(a, ti, sA, sAs, sB);
}

// ---------------------------------------------------------------------------
// Activations -> 16-bit MFMA operands, once per call (FP4 weights take f16, bf16
// weights bf16).  Same rounding as an in-GEMM conversion (round to nearest even).
template <int AFMT, bool TO_F16>
__global__ __launch_bounds__(256) void act_operands_kernel(const void* __restrict__ x, uint16_t* __restrict__ xo,
                                                            int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  AStage<AFMT> st;
  const int64_t src[2] = {8 * i, 0};
  if constexpr (AFMT == MOE_AFMT_F32) {
    const u32x4* p = reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(x) + src[0]);
    st.v[0] = p[0];
    st.v[1] = p[1];
  } else {
    st.v[0] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(x) + src[0]);
  }
  *reinterpret_cast<u32x4*>(xo + 8 * i) = cvt_a8<AFMT, TO_F16>(st, 0);
}

bool prefill_needs_act_operands(int wfmt, int afmt) {
  return wfmt == MOE_WFMT_FP4 || wfmt == MOE_WFMT_MXFP4 || (wfmt == MOE_WFMT_BF16 && afmt == MOE_AFMT_F32);
}

void launch_act_operands(int wfmt, int afmt, const void* x, void* xo, int64_t n, hipStream_t s) {
  const int64_t n8 = n / 8;
  const dim3 grid((unsigned)((n8 + 255) / 256));
  uint16_t* o = reinterpret_cast<uint16_t*>(xo);
  if (wfmt == MOE_WFMT_FP4 || wfmt == MOE_WFMT_MXFP4) {
    if (afmt == MOE_AFMT_BF16) hipLaunchKernelGGL((act_operands_kernel<MOE_AFMT_BF16, true>), grid, dim3(256), 0, s, x, o, n8);
    else hipLaunchKernelGGL((act_operands_kernel<MOE_AFMT_F32, true>), grid, dim3(256), 0, s, x, o, n8);
  } else {
    hipLaunchKernelGGL((act_operands_kernel<MOE_AFMT_F32, false>), grid, dim3(256), 0, s, x, o, n8);
  }
}

// ---------------------------------------------------------------------------
// FP32 weights: SIMT grouped evaluation (one thread per output element).
__device__ __forceinline__ int group_of_row(const PrefillArgs& a, int row, int ngrp) {
  int lo = 0, hi = ngrp - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.offsets[mid] <= row) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <int AFMT>
__global__ void gemm1_f32_kernel(PrefillArgs a) {
  const int ngrp = a.cnt[C_NGRP];
  if (ngrp <= 0) return;
  const int nrows = a.offsets[ngrp];
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)nrows * a.I) return;
  const int row = (int)(i / a.I), col = (int)(i % a.I);
  const int g = group_of_row(a, row, ngrp);
  const float* W = reinterpret_cast<const float*>(a.arena + (int64_t)a.grp_slot[g] * a.rec_bytes);
  const int64_t n = (int64_t)a.H * a.I;
  const int t = a.perm[row] / a.k;
  float gs = 0.f, us = 0.f;
  for (int h = 0; h < a.H; ++h) {
    const float xv = load_act<AFMT>(a.x, (int64_t)t * a.H + h);
    gs += W[(int64_t)col * a.H + h] * xv;
    us += W[n + (int64_t)col * a.H + h] * xv;
  }
  reinterpret_cast<float*>(a.act)[(int64_t)row * a.I + col] = silu(gs) * us;
}

__global__ void gemm2_f32_kernel(PrefillArgs a) {
  const int ngrp = a.cnt[C_NGRP];
  if (ngrp <= 0) return;
  const int nrows = a.offsets[ngrp];
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)nrows * a.H) return;
  const int row = (int)(i / a.H), col = (int)(i % a.H);
  const int g = group_of_row(a, row, ngrp);
  const float* W = reinterpret_cast<const float*>(a.arena + (int64_t)a.grp_slot[g] * a.rec_bytes);
  const int64_t n = (int64_t)a.H * a.I;
  const float* act = reinterpret_cast<const float*>(a.act) + (int64_t)row * a.I;
  float s = 0.f;
  for (int c = 0; c < a.I; ++c) s += W[2 * n + (int64_t)col * a.I + c] * act[c];
  a.ypair[(int64_t)a.perm[row] * a.H + col] = s;
}

// The LDS-staged FP4 kernels take 256-k chunks and hold byte offsets (activations,
// record) in 32 bits.  MXFP4 contexts are created only for shapes that meet this.
bool fp4_staged(const PrefillArgs& a) {
  return a.H % 256 == 0 && a.I % 256 == 0 && (int64_t)a.T * a.H < (1ll << 31) &&
         (int64_t)a.T * a.k * a.I < (1ll << 31) && a.rec_bytes < (1ll << 32);
}

// The LDS-staged bf16 kernels are the only bf16 path: their 32-bit byte offsets bound
// T * H, T * k * I and the record size, which moe_ffn_prefill checks (64-k chunks; the
// tiles need I % 128 == 0 and H % 256 == 0).


void launch_prefill_gemm1(int wfmt, int afmt, const PrefillArgs& a, int max_tiles_m, hipStream_t s, Timing tm) {
  if (wfmt == MOE_WFMT_F32) {
    const int64_t n = (int64_t)a.T * a.k * a.I;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (afmt == MOE_AFMT_BF16) launch_timed(gemm1_f32_kernel<MOE_AFMT_BF16>, grid, dim3(256), 0, s, tm, a);
    else launch_timed(gemm1_f32_kernel<MOE_AFMT_F32>, grid, dim3(256), 0, s, tm, a);
    return;
  }
  const dim3 grid(prefill_tile_slots(max_tiles_m, a.I / 128));
  if (wfmt == MOE_WFMT_BF16) launch_timed(gemm1_bs_kernel, grid, dim3(256), 0, s, tm, a);
  else if (wfmt == MOE_WFMT_MXFP4) launch_timed(gemm1_fp4_kernel<true>, grid, dim3(256), 0, s, tm, a);
  else if (fp4_staged(a)) launch_timed(gemm1_fp4_kernel<false>, grid, dim3(256), 0, s, tm, a);
  else launch_timed(gemm1_kernel<MOE_WFMT_FP4>, grid, dim3(256), 0, s, tm, a);
}

void launch_mx_quant(int afmt, const void* x, uint8_t* codes, uint8_t* scales, int64_t n, hipStream_t s) {
  const int64_t nb = n / 32;
  const dim3 grid((unsigned)((nb + 255) / 256));
  if (afmt == MOE_AFMT_BF16) hipLaunchKernelGGL(mx_quant_kernel<MOE_AFMT_BF16>, grid, dim3(256), 0, s, x, codes, scales, nb);
  else hipLaunchKernelGGL(mx_quant_kernel<MOE_AFMT_F32>, grid, dim3(256), 0, s, x, codes, scales, nb);
}

void launch_prefill_gemm1_mx(const PrefillArgs& a, int max_tiles_m, hipStream_t s, Timing tm) {
  launch_timed(gemm1_mx_kernel, dim3(prefill_tile_slots(max_tiles_m, a.I / 128)), dim3(256), 0, s, tm, a);
}

void launch_prefill_gemm2_mx(const PrefillArgs& a, int max_tiles_m, hipStream_t s, Timing tm) {
  launch_timed(gemm2_mx_kernel, dim3(prefill_tile_slots(max_tiles_m, a.H / 256)), dim3(256), 0, s, tm, a);
}

void launch_prefill_gemm2(int wfmt, const PrefillArgs& a, int max_tiles_m, hipStream_t s, Timing tm) {
  if (wfmt == MOE_WFMT_F32) {
    const int64_t n = (int64_t)a.T * a.k * a.H;
    launch_timed(gemm2_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, tm, a);
    return;
  }
  const dim3 grid(prefill_tile_slots(max_tiles_m, a.H / 256));
  if (wfmt == MOE_WFMT_BF16) launch_timed(gemm2_bs_kernel, grid, dim3(256), 0, s, tm, a);
  else if (wfmt == MOE_WFMT_MXFP4) launch_timed(gemm2_fp4_kernel<true>, grid, dim3(256), 0, s, tm, a);
  else if (fp4_staged(a)) launch_timed(gemm2_fp4_kernel<false>, grid, dim3(256), 0, s, tm, a);
  else launch_timed(gemm2_kernel<MOE_WFMT_FP4>, grid, dim3(256), 0, s, tm, a);
}

// ---------------------------------------------------------------------------
// Combine: y[t] = sum_j (GPU pairs, rank order) w[t,j] ypair[(t,j)] + y_cpu[t].
// a.pair_gpu marks the GPU pairs (>= 0), or is nullptr when every pair ran on the GPU.
__global__ void prefill_combine_kernel(PrefillArgs a) {
  const int32_t* pair_gpu = a.pair_gpu;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int H4 = a.H / 4;
  if (i >= (int64_t)a.T * H4) return;
  const int t = (int)(i / H4), c = (int)(i % H4) * 4;
  float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < a.k; ++j) {
    const int p = t * a.k + j;
    if (pair_gpu && pair_gpu[p] < 0) continue;
    const float w = a.w[p];
    const float4 v = *reinterpret_cast<const float4*>(a.ypair + (int64_t)p * a.H + c);
    y.x += w * v.x; y.y += w * v.y; y.z += w * v.z; y.w += w * v.w;
  }
  if (a.y_cpu) {
    const float4 v = *reinterpret_cast<const float4*>(a.y_cpu + (int64_t)t * a.H + c);
    y.x += v.x; y.y += v.y; y.z += v.z; y.w += v.w;
  }
  *reinterpret_cast<float4*>(a.y + (int64_t)t * a.H + c) = y;
}

void launch_prefill_combine(const PrefillArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.T * (a.H / 4);
  hipLaunchKernelGGL(prefill_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
}

// ---------------------------------------------------------------------------
// The permutation with no allocation: moe_permute_noalloc keeps the scratch its kernels
// use (slot flags, group ids per pair, the inverse permutation, per-chunk group
// histograms, tile bases, counters) in one file-scope device array instead of context
// memory, for callers that cannot allocate.  Each device holds its own copy; its device
// address is looked up once per device (hipGetSymbolAddress) and every call on that
// device shares it.
constexpr int kNoAllocMaxPairs = 1 << 16;   // P = T * k
constexpr int kNoAllocMaxSlots = 1 << 16;   // n_slot_range
constexpr size_t kNaFlags = 0;
constexpr size_t kNaPairGrp = kNaFlags + kNoAllocMaxSlots;
constexpr size_t kNaInv = kNaPairGrp + kNoAllocMaxPairs;
constexpr size_t kNaHist = kNaInv + kNoAllocMaxPairs;
constexpr size_t kNaTileBase = kNaHist + (size_t)(kNoAllocMaxPairs / kChunk) * kMaxExperts;
constexpr size_t kNaCnt = kNaTileBase + kMaxExperts + 64;
constexpr size_t kNaInts = kNaCnt + C_COUNT;   // 524,368 ints: 2 MiB

static __device__ __align__(256) int32_t scratch[kNaInts];

namespace {
constexpr int kNaMaxDevices = 64;
std::mutex g_na_mu;
int32_t* g_na_ptr[kNaMaxDevices] = {};  // device address of `scratch` on each device

moe_status noalloc_scratch(int32_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNaMaxDevices) return MOE_EHIP;
  std::lock_guard<std::mutex> lock(g_na_mu);
  if (!g_na_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_EHIP;
    g_na_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_na_ptr[dev];
  return MOE_OK;
}
}  // namespace

}  // namespace rmoe

extern "C" MOE_API moe_status moe_permute_noalloc(const int32_t* slot_idx, int32_t P, int32_t n_slot_range,
                                                  int32_t* perm, int32_t* offsets, int32_t* group_slot,
                                                  int32_t* n_groups, moe_stream_t stream) {
  using namespace rmoe;
  if (!slot_idx || !perm || !offsets || !group_slot || !n_groups) return MOE_EINVAL;
  if (P < 1 || P > kNoAllocMaxPairs || n_slot_range < 1 || n_slot_range > kNoAllocMaxSlots) return MOE_EINVAL;
  int32_t* base = nullptr;
  const moe_status st = noalloc_scratch(&base);
  if (st != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int gmax = std::min(P, kMaxExperts);
  // every scratch word a kernel reads is written earlier in the same call: the flags are
  // cleared first, each chunk's histogram row and the tile bases are written in full
  launch_groups_from_slots(slot_idx, P, base + kNaPairGrp, group_slot, base + kNaCnt, base + kNaFlags, n_slot_range,
                           gmax, n_groups, s);
  launch_permute(base + kNaPairGrp, base + kNaCnt, P, gmax, base + kNaHist, perm, base + kNaInv, offsets,
                 base + kNaTileBase, prefill_bm(), s);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}
