// Router logits and top-k / softmax gates.
//
// The router and the cache lookup run on the GPU and pick k of E experts per
// token (FreeToken summary, "decode co-design" section: router and cache lookup
// on the GPU; "MoE" section: k << E).  Gates are the softmax over all E logits
// taken at the chosen experts (renorm = 1: renormalised over the k chosen).
#include <algorithm>

#include "common.hpp"

namespace rmoe {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Decode-sized batches: one workgroup per expert row, of up to sixteen wavefronts (one
// 16-byte weight chunk per lane at H = 4096); thread i takes the row's chunks i, i + n,
// ... (n threads, loads coalesced across the block) with the matching activations, so the
// whole 4 MB of an E = 256, H = 4096 router is in flight at once over E workgroups (one
// memory round trip).  Wavefront sums meet in LDS and are added in wavefront order.
constexpr int kRouteWaves = 16;  // wavefronts per workgroup at most

template <int AFMT>
__device__ __forceinline__ float4 route_x4(const void* x, size_t i) {  // 4 activations at element i
  if constexpr (AFMT == MOE_AFMT_BF16) {
    const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + i);
    return make_float4(bf16_lo(q.x), bf16_hi(q.x), bf16_lo(q.y), bf16_hi(q.y));
  } else {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(x) + i);
  }
}

template <int AFMT>
__global__ __launch_bounds__(64 * kRouteWaves) void route_gemv(const void* __restrict__ x, const float* __restrict__ wr,
                                                               const float* __restrict__ bias,
                                                               float* __restrict__ logits, int T, int E, int H) {
  __shared__ float s_part[kRouteWaves][kDecodeMaxTok];
  const int e = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const int nc = H / 4;  // 16-byte chunks in a row
  const float4* row = reinterpret_cast<const float4*>(wr + (size_t)e * H);
  float acc[kDecodeMaxTok];
#pragma unroll
  for (int t = 0; t < kDecodeMaxTok; ++t) acc[t] = 0.f;
  for (int c = threadIdx.x; c < nc; c += blockDim.x) {
    const float4 w4 = row[c];
    float4 x4[kDecodeMaxTok];
#pragma unroll
    for (int t = 0; t < kDecodeMaxTok; ++t)
      if (t < T) x4[t] = route_x4<AFMT>(x, (size_t)t * H + 4 * c);
#pragma unroll
    for (int t = 0; t < kDecodeMaxTok; ++t)
      if (t < T) acc[t] += w4.x * x4[t].x + w4.y * x4[t].y + w4.z * x4[t].z + w4.w * x4[t].w;
  }
#pragma unroll
  for (int t = 0; t < kDecodeMaxTok; ++t) {
    if (t < T) {
      const float v = wave_sum(acc[t]);
      if (lane == 0) s_part[wave][t] = v;
    }
  }
  __syncthreads();
  if (threadIdx.x < T) {
    const int t = threadIdx.x;
    float z = 0.f;
    for (int w = 0; w < nw; ++w) z += s_part[w][t];
    logits[(size_t)t * E + e] = z + (bias ? bias[(size_t)t * E + e] : 0.f);
  }
}

// ---------------------------------------------------------------------------
// Long prompts: fp32 MFMA (v_mfma_f32_16x16x4_f32: exact fp32 products, fp32
// accumulation).  A block owns 32 tokens x 64 experts; wavefront (wm, wn) of the
// 2 x 2 grid owns 16 tokens x 32 experts (two 16x16 accumulators).  K runs in
// chunks of 32 through double-buffered LDS; the next chunk is loaded into
// registers while the current one is multiplied.
constexpr int kRgT = 32, kRgE = 64, kRgK = 32, kRgP = kRgK + 4;  // padded LDS row (floats)

template <int AFMT>
__global__ __launch_bounds__(256) void route_gemm(const void* __restrict__ x, const float* __restrict__ wr,
                                                   const float* __restrict__ bias, float* __restrict__ logits,
                                                   int T, int E, int H) {
  __shared__ __attribute__((aligned(16))) float sX[2][kRgT][kRgP];
  __shared__ __attribute__((aligned(16))) float sW[2][kRgE][kRgP];
  const int t0 = blockIdx.x * kRgT, e0 = blockIdx.y * kRgE;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // loader roles: x piece = token tid / 8, k (tid % 8) * 4 (4 values); W pieces = expert
  // tid / 4, k (tid % 4) * 8 (8 values).  Rows past T / E read row 0 and are never stored.
  const int xt = tid >> 3, xk = (tid & 7) * 4;
  const int we = tid >> 2, wk = (tid & 3) * 8;
  const size_t xrow = (size_t)(t0 + xt < T ? t0 + xt : 0) * H;
  const float* wrow = wr + (size_t)(e0 + we < E ? e0 + we : 0) * H;
  float4 px, pw0, pw1;
  auto load = [&](int k0) {
    px = route_x4<AFMT>(x, xrow + k0 + xk);
    pw0 = *reinterpret_cast<const float4*>(wrow + k0 + wk);
    pw1 = *reinterpret_cast<const float4*>(wrow + k0 + wk + 4);
  };
  auto store = [&](int buf) {
    *reinterpret_cast<float4*>(&sX[buf][xt][xk]) = px;
    *reinterpret_cast<float4*>(&sW[buf][we][wk]) = pw0;
    *reinterpret_cast<float4*>(&sW[buf][we][wk + 4]) = pw1;
  };
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const int r = lane & 15, kq = lane >> 4;
  load(0);
  store(0);
  __syncthreads();
  const int nk = H / kRgK;
  for (int c = 0; c < nk; ++c) {
    const int buf = c & 1;
    if (c + 1 < nk) load((c + 1) * kRgK);
#pragma unroll
    for (int kk = 0; kk < kRgK; kk += 4) {
      const float a = sX[buf][wm * 16 + r][kk + kq];
      const float b0 = sW[buf][wn * 32 + r][kk + kq];
      const float b1 = sW[buf][wn * 32 + 16 + r][kk + kq];
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b1, acc1, 0, 0, 0);
    }
    if (c + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }
  // accumulator element i of lane l: token 4 (l / 16) + i, expert l % 16 (of the 16x16 tile)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + wm * 16 + 4 * kq + i;
    if (t >= T) continue;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = e0 + wn * 32 + 16 * h + r;
      if (e < E) logits[(size_t)t * E + e] = (h ? acc1[i] : acc0[i]) + (bias ? bias[(size_t)t * E + e] : 0.f);
    }
  }
}

void launch_route_logits(const void* x, int afmt, const float* wr, const float* bias, float* logits, int T, int E,
                         int H, hipStream_t s) {
  if (T <= kDecodeMaxTok && T * H <= kDecodeMaxTH) {
    // one chunk per lane where the row allows (H = 4096: sixteen wavefronts)
    const int nw = std::min(kRouteWaves, std::max(1, (H / 4 + 63) / 64));
    if (afmt == MOE_AFMT_BF16)
      hipLaunchKernelGGL(route_gemv<MOE_AFMT_BF16>, dim3(E), dim3(64 * nw), 0, s, x, wr, bias, logits, T, E, H);
    else
      hipLaunchKernelGGL(route_gemv<MOE_AFMT_F32>, dim3(E), dim3(64 * nw), 0, s, x, wr, bias, logits, T, E, H);
  } else {
    dim3 grid((T + kRgT - 1) / kRgT, (E + kRgE - 1) / kRgE);
    if (afmt == MOE_AFMT_BF16)
      hipLaunchKernelGGL(route_gemm<MOE_AFMT_BF16>, grid, dim3(256), 0, s, x, wr, bias, logits, T, E, H);
    else
      hipLaunchKernelGGL(route_gemm<MOE_AFMT_F32>, grid, dim3(256), 0, s, x, wr, bias, logits, T, E, H);
  }
}

// ---------------------------------------------------------------------------
// Top-k + gates: one wavefront per token.  Each lane holds E/64 logits; k rounds
// of a wave arg-max under the total order (value descending, index ascending).
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k, int renorm,
                                                   int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_wave(logits + (size_t)t * E, E, k, renorm, idx_out + (size_t)t * k, w_out + (size_t)t * k);
}

void launch_topk(const float* logits, int T, int E, int k, int renorm, int32_t* idx, float* w, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, renorm, idx, w);
}

}  // namespace rmoe
