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

__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int per = nblocks >> 3;
  return (bid & 7) * per + (bid >> 3);
}

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
__global__ __launch_bounds__(1024) void groups_from_slots_kernel(const int32_t* __restrict__ slot_idx, int P,
                                                                 int32_t* __restrict__ pair_grp,
                                                                 int32_t* __restrict__ grp_slot,
                                                                 int32_t* __restrict__ cnt, int32_t* flags, int nrange) {
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
  __syncthreads();
  for (int i = i0; i < i1; ++i) {
    if (flags[i]) {
      grp_slot[pos] = i;
      flags[i] = pos + 1;
      ++pos;
    }
  }
  __threadfence_block();
  __syncthreads();
  int npairs = 0;
  for (int p = threadIdx.x; p < P; p += 1024) {
    const int sl = slot_idx[p];
    const int g = (sl >= 0 && sl < nrange) ? flags[sl] - 1 : -1;
    pair_grp[p] = g;
    npairs += (g >= 0);
  }
  int np;
  block_excl_scan(npairs, s_tmp, &np);
  int nbad;
  block_excl_scan(bad, s_tmp, &nbad);
  if (threadIdx.x == 0) {
    cnt[C_NGRP] = total;
    cnt[C_NPAIR_GPU] = np;
    cnt[C_ERR] = nbad ? 1 : 0;
  }
}

void launch_groups_from_slots(const int32_t* slot_idx, int P, int32_t* pair_grp, int32_t* grp_slot, int32_t* cnt,
                              int32_t* scratch_flags, int n_slot_range, hipStream_t s) {
  hipLaunchKernelGGL(groups_from_slots_kernel, dim3(1), dim3(1024), 0, s, slot_idx, P, pair_grp, grp_slot, cnt,
                     scratch_flags, n_slot_range);
}

// ---------------------------------------------------------------------------
// Record addressing (same layout as the decode kernels).
template <int WFMT>
__device__ __forceinline__ int64_t tbytes(int H, int I) {
  const int64_t n = (int64_t)H * I;
  if constexpr (WFMT == MOE_WFMT_F32) return n * 4;
  else if constexpr (WFMT == MOE_WFMT_BF16) return n * 2;
  else return n / 2;
}

// Tile decode shared by both GEMMs: returns false when the block has no tile.
struct TileInfo {
  int g, row0, rows, nt;
};

__device__ __forceinline__ bool decode_tile(const PrefillArgs& a, int NT, TileInfo& ti) {
  const int ngrp = a.cnt[C_NGRP];
  if (ngrp <= 0) return false;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int total = a.tile_base[ngrp] * NT;
  if (bid >= total) return false;
  int lo = 0, hi = ngrp - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.tile_base[mid] * NT <= bid) lo = mid;
    else hi = mid - 1;
  }
  const int r = bid - a.tile_base[lo] * NT;
  const int mcount = a.tile_base[lo + 1] - a.tile_base[lo];
  ti.g = lo;
  ti.nt = r / mcount;
  const int mt = r % mcount;
  ti.row0 = a.offsets[lo] + mt * BM;
  ti.rows = min(BM, a.offsets[lo + 1] - ti.row0);
  return true;
}

// 8 activation values (bf16 or f32 source) -> 16 bytes of bf16 or f16 for the MFMA A operand.
template <int AFMT, bool TO_F16>
__device__ __forceinline__ u32x4 load_x8(const void* x, int64_t off) {
  float v[8];
  if constexpr (AFMT == MOE_AFMT_BF16) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(x) + off);
    if constexpr (!TO_F16) return q;
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint16_t lo, hi;
    if constexpr (TO_F16) {
      _Float16 l = (_Float16)v[2 * i], h = (_Float16)v[2 * i + 1];
      lo = __builtin_bit_cast(uint16_t, l);
      hi = __builtin_bit_cast(uint16_t, h);
    } else {
      lo = f32_to_bf16_rne(v[2 * i]);
      hi = f32_to_bf16_rne(v[2 * i + 1]);
    }
    w[i] = (uint32_t)lo | ((uint32_t)hi << 16);
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// 32 e2m1 codes (16 bytes) times one bf16 scale -> 32 f16 (64 bytes), exact in range.
__device__ __forceinline__ void fp4x32_to_f16(const u32x4& q, uint16_t scale_bits, u32x4* out) {
  const _Float16 sh = (_Float16)bf16_to_f32(scale_bits);
  const f16x2 s2 = {sh, sh};
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  uint32_t o[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 0) * s2;
    f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 1) * s2;
    f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 2) * s2;
    f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 3) * s2;
    o[4 * i + 0] = __builtin_bit_cast(uint32_t, v0);
    o[4 * i + 1] = __builtin_bit_cast(uint32_t, v1);
    o[4 * i + 2] = __builtin_bit_cast(uint32_t, v2);
    o[4 * i + 3] = __builtin_bit_cast(uint32_t, v3);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = u32x4{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
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
// Tile loaders.  Register stages are plain unrolled arrays (no captures), so they
// stay in VGPRs and the next k-step's loads overlap the current step's MFMAs.

// A: 64 rows x 64 k of activations (2 16-byte chunks per thread), rows gathered
// through the permutation (GEMM1) or contiguous sorted rows (GEMM2).
struct AStage {
  u32x4 v[2];
};
// B (bf16): 128 weight rows x 64 k (4 chunks per thread); (fp4): 128 rows x 32 bytes of
// codes (1 chunk per thread) and that chunk's bf16 block scale.
template <int WFMT>
struct BStage {
  u32x4 v[WFMT == MOE_WFMT_BF16 ? 4 : 1];
  uint16_t sc;
};

template <int WFMT>
__device__ __forceinline__ void load_b(BStage<WFMT>& st, const uint8_t* const* rowp, const uint16_t* const* scp,
                                       int k0, int tid) {
  if constexpr (WFMT == MOE_WFMT_BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) st.v[j] = *reinterpret_cast<const u32x4*>(rowp[j] + (int64_t)k0 * 2 + (tid & 7) * 16);
  } else {
    st.v[0] = *reinterpret_cast<const u32x4*>(rowp[0] + k0 / 2 + (tid & 1) * 16);
    st.sc = scp[0][k0 / 32 + (tid & 1)];
  }
}

template <int WFMT>
__device__ __forceinline__ void store_b(const BStage<WFMT>& st, uint16_t (*sB)[LDSW], int tid) {
  if constexpr (WFMT == MOE_WFMT_BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = tid + 256 * j;
      *reinterpret_cast<u32x4*>(&sB[idx >> 3][(idx & 7) * 8]) = st.v[j];
    }
  } else {
    u32x4 o[4];
    fp4x32_to_f16(st.v[0], st.sc, o);
    const int wr = tid >> 1, half = tid & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(&sB[wr][half * 32 + i * 8]) = o[i];
  }
}

__device__ __forceinline__ void store_a(const AStage& st, uint16_t (*sA)[LDSW], int tid) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int idx = tid + 256 * j;
    *reinterpret_cast<u32x4*>(&sA[idx >> 3][(idx & 7) * 8]) = st.v[j];
  }
}

// Per-thread source rows of the B tile: bf16 threads own rows idx >> 3 for idx = tid + 256 j;
// fp4 threads own row tid >> 1.  wrow(i) maps tile row i (0..127) to a tensor row.
template <int WFMT, typename RowFn>
__device__ __forceinline__ void b_rows(const uint8_t* rec, int H, int I, int t_base, RowFn wrow, int cols, int tid,
                                       const uint8_t** rowp, const uint16_t** scp) {
  const int64_t tb = tbytes<WFMT>(H, I);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(rec + 3 * ((int64_t)H * I / 2));
  if constexpr (WFMT == MOE_WFMT_BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int t, r;
      wrow((tid + 256 * j) >> 3, t, r);
      rowp[j] = rec + (int64_t)t * tb + (int64_t)r * cols * 2;
    }
  } else {
    int t, r;
    wrow(tid >> 1, t, r);
    rowp[0] = rec + (int64_t)t * tb + (int64_t)r * (cols / 2);
    scp[0] = scales + (int64_t)t * ((int64_t)H * I / 32) + (int64_t)r * (cols / 32);
  }
  (void)t_base;
}

// ---------------------------------------------------------------------------
// GEMM1: act[sorted row, n0..n0+63] = silu(X W_gate^T) * (X W_up^T) for one group.
// Block: 256 threads = 4 wavefronts in a 2 (rows) x 2 (act columns) grid of
// 32x32 output blocks; each wavefront owns the gate and the up accumulators of
// the same 32x32 block.
template <int WFMT, int AFMT>
__global__ __launch_bounds__(256, 2) void gemm1_kernel(PrefillArgs a) {
  constexpr bool F16 = (WFMT == MOE_WFMT_FP4);
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM][LDSW];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][128][LDSW];
  TileInfo ti;
  if (!decode_tile(a, a.I / 64, ti)) return;
  const int H = a.H, I = a.I;
  const int n0 = ti.nt * 64;
  const uint8_t* rec = a.arena + (int64_t)a.grp_slot[ti.g] * a.rec_bytes;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // A sources: 2 chunks per thread (row = idx / 8, 16-byte column chunk = idx % 8)
  int64_t a_src[2];
  bool a_ok[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int idx = tid + 256 * j, r = idx >> 3;
    a_ok[j] = r < ti.rows;
    const int tok = a_ok[j] ? a.perm[ti.row0 + r] / a.k : 0;
    a_src[j] = (int64_t)tok * H + (idx & 7) * 8;
  }
  // B sources: tile rows 0..63 are gate rows n0.., 64..127 the up rows n0..
  const uint8_t* rowp[WFMT == MOE_WFMT_BF16 ? 4 : 1];
  const uint16_t* scp[1] = {nullptr};
  b_rows<WFMT>(rec, H, I, 0, [&](int i, int& t, int& r) { t = i >> 6; r = n0 + (i & 63); }, H, tid, rowp, scp);

  AStage ra;
  BStage<WFMT> rb;
#pragma unroll
  for (int j = 0; j < 2; ++j) ra.v[j] = a_ok[j] ? load_x8<AFMT, F16>(a.x, a_src[j]) : u32x4{0, 0, 0, 0};
  load_b<WFMT>(rb, rowp, scp, 0, tid);

  f32x16 accg, accu;
#pragma unroll
  for (int i = 0; i < 16; ++i) { accg[i] = 0.f; accu[i] = 0.f; }
  const int nk = H / BK;
  const int arow = wm * 32 + (lane & 31);
  const int bg = wn * 32 + (lane & 31), bu = 64 + wn * 32 + (lane & 31);
  const int koff = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    store_a(ra, sA[buf], tid);
    store_b<WFMT>(rb, sB[buf], tid);
    __syncthreads();
    if (kt + 1 < nk) {
      const int k0 = (kt + 1) * BK;
#pragma unroll
      for (int j = 0; j < 2; ++j) ra.v[j] = a_ok[j] ? load_x8<AFMT, F16>(a.x, a_src[j] + k0) : u32x4{0, 0, 0, 0};
      load_b<WFMT>(rb, rowp, scp, k0, tid);
    }
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      const u32x4 av = *reinterpret_cast<const u32x4*>(&sA[buf][arow][kk + koff]);
      const u32x4 gv = *reinterpret_cast<const u32x4*>(&sB[buf][bg][kk + koff]);
      const u32x4 uv = *reinterpret_cast<const u32x4*>(&sB[buf][bu][kk + koff]);
      accg = mfma32<F16>(av, gv, accg);
      accu = mfma32<F16>(av, uv, accu);
    }
  }
  // epilogue: SwiGLU in registers, store act (sorted order) as bf16 / f16
  uint16_t* act = reinterpret_cast<uint16_t*>(a.act);
  const int col = n0 + wn * 32 + (lane & 31);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = wm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
    if (r < ti.rows) {
      const float g = accg[i];
      const float v = g * __frcp_rn(1.0f + __expf(-g)) * accu[i];
      uint16_t bits;
      if constexpr (F16) bits = __builtin_bit_cast(uint16_t, (_Float16)v);
      else bits = f32_to_bf16_rne(v);
      act[(int64_t)(ti.row0 + r) * I + col] = bits;
    }
  }
}

// ---------------------------------------------------------------------------
// GEMM2: ypair[pair, n0..n0+127] = act[sorted rows] W_down^T for one group.
template <int WFMT>
__global__ __launch_bounds__(256, 2) void gemm2_kernel(PrefillArgs a) {
  constexpr bool F16 = (WFMT == MOE_WFMT_FP4);
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM][LDSW];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][128][LDSW];
  TileInfo ti;
  if (!decode_tile(a, a.H / 128, ti)) return;
  const int H = a.H, I = a.I;
  const int n0 = ti.nt * 128;
  const uint8_t* rec = a.arena + (int64_t)a.grp_slot[ti.g] * a.rec_bytes;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const uint16_t* act = reinterpret_cast<const uint16_t*>(a.act);

  const uint16_t* a_src[2];
  bool a_ok[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int idx = tid + 256 * j, r = idx >> 3;
    a_ok[j] = r < ti.rows;
    a_src[j] = act + (int64_t)(ti.row0 + (a_ok[j] ? r : 0)) * I + (idx & 7) * 8;
  }
  const uint8_t* rowp[WFMT == MOE_WFMT_BF16 ? 4 : 1];
  const uint16_t* scp[1] = {nullptr};
  b_rows<WFMT>(rec, H, I, 0, [&](int i, int& t, int& r) { t = 2; r = n0 + i; }, I, tid, rowp, scp);

  AStage ra;
  BStage<WFMT> rb;
#pragma unroll
  for (int j = 0; j < 2; ++j) ra.v[j] = a_ok[j] ? *reinterpret_cast<const u32x4*>(a_src[j]) : u32x4{0, 0, 0, 0};
  load_b<WFMT>(rb, rowp, scp, 0, tid);

  f32x16 acc0, acc1;
#pragma unroll
  for (int i = 0; i < 16; ++i) { acc0[i] = 0.f; acc1[i] = 0.f; }
  const int nk = I / BK;
  const int arow = wm * 32 + (lane & 31);
  const int b0 = wn * 64 + (lane & 31), b1 = b0 + 32;
  const int koff = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    store_a(ra, sA[buf], tid);
    store_b<WFMT>(rb, sB[buf], tid);
    __syncthreads();
    if (kt + 1 < nk) {
      const int k0 = (kt + 1) * BK;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        ra.v[j] = a_ok[j] ? *reinterpret_cast<const u32x4*>(a_src[j] + k0) : u32x4{0, 0, 0, 0};
      load_b<WFMT>(rb, rowp, scp, k0, tid);
    }
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      const u32x4 av = *reinterpret_cast<const u32x4*>(&sA[buf][arow][kk + koff]);
      const u32x4 w0 = *reinterpret_cast<const u32x4*>(&sB[buf][b0][kk + koff]);
      const u32x4 w1 = *reinterpret_cast<const u32x4*>(&sB[buf][b1][kk + koff]);
      acc0 = mfma32<F16>(av, w0, acc0);
      acc1 = mfma32<F16>(av, w1, acc1);
    }
  }
  const int c0 = n0 + wn * 64 + (lane & 31);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = wm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
    if (r < ti.rows) {
      const int p = a.perm[ti.row0 + r];
      float* dst = a.ypair + (int64_t)p * H;
      dst[c0] = acc0[i];
      dst[c0 + 32] = acc1[i];
    }
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

static int padded_grid(int tiles_m, int nt) {
  int n = tiles_m * nt;
  return ((n + 7) / 8) * 8;
}

void launch_prefill_gemm1(int wfmt, int afmt, const PrefillArgs& a, int max_tiles_m, hipStream_t s, Timing tm) {
  if (wfmt == MOE_WFMT_F32) {
    const int64_t n = (int64_t)a.T * a.k * a.I;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (afmt == MOE_AFMT_BF16) launch_timed(gemm1_f32_kernel<MOE_AFMT_BF16>, grid, dim3(256), 0, s, tm, a);
    else launch_timed(gemm1_f32_kernel<MOE_AFMT_F32>, grid, dim3(256), 0, s, tm, a);
    return;
  }
  const dim3 grid(padded_grid(max_tiles_m, a.I / 64));
#define G1(W, A) launch_timed(gemm1_kernel<W, A>, grid, dim3(256), 0, s, tm, a)
  if (wfmt == MOE_WFMT_BF16) {
    if (afmt == MOE_AFMT_BF16) G1(MOE_WFMT_BF16, MOE_AFMT_BF16); else G1(MOE_WFMT_BF16, MOE_AFMT_F32);
  } else {
    if (afmt == MOE_AFMT_BF16) G1(MOE_WFMT_FP4, MOE_AFMT_BF16); else G1(MOE_WFMT_FP4, MOE_AFMT_F32);
  }
#undef G1
}

void launch_prefill_gemm2(int wfmt, const PrefillArgs& a, int max_tiles_m, hipStream_t s, Timing tm) {
  if (wfmt == MOE_WFMT_F32) {
    const int64_t n = (int64_t)a.T * a.k * a.H;
    launch_timed(gemm2_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, tm, a);
    return;
  }
  const dim3 grid(padded_grid(max_tiles_m, a.H / 128));
  if (wfmt == MOE_WFMT_BF16) launch_timed(gemm2_kernel<MOE_WFMT_BF16>, grid, dim3(256), 0, s, tm, a);
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

}  // namespace rmoe
