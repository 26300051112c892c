// Router logits and top-k / softmax gates.
//
// The router and the cache lookup run on the GPU and pick k of E experts per
// token (FreeToken summary, "decode co-design" section: router and cache lookup
// on the GPU; "MoE" section: k << E).  Gates are the softmax over all E logits
// taken at the chosen experts (renorm = 1: renormalised over the k chosen).
#include "common.hpp"

namespace rmoe {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Decode-sized batches: one wavefront per expert row, activations staged in LDS
// as fp32.  W_r rows are read with 16-byte lane loads (fully coalesced), eight
// per lane requested before any is used, so a 16 KB row takes two memory round
// trips rather than sixteen.
constexpr int kRouteWaves = 4;
constexpr int kRouteBatch = 8;  // 16-byte row chunks per lane in flight

template <int AFMT>
__global__ __launch_bounds__(256) void route_gemv(const void* __restrict__ x, const float* __restrict__ wr,
                                                   const float* __restrict__ bias, float* __restrict__ logits,
                                                   int T, int E, int H) {
  extern __shared__ float s_x[];  // [T][H]
  constexpr int EV = (AFMT == MOE_AFMT_BF16) ? 8 : 4;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = min(blockIdx.x * kRouteWaves + wave, E - 1);  // rows past E recompute the last one, unstored
  const float4* row = reinterpret_cast<const float4*>(wr + (size_t)e * H);
  const int nc = H / 4;  // 16-byte chunks of a row; lanes past the row's end load nothing
  // the first batch of the row is requested before the activations are staged; chunk
  // indices past the row's end are clamped (in bounds) and their products skipped
  float4 w4[kRouteBatch];
#pragma unroll
  for (int b = 0; b < kRouteBatch; ++b) w4[b] = row[min(lane + 64 * b, nc - 1)];
  for (int i = threadIdx.x; i < T * H / EV; i += blockDim.x) {
    const uint4 q = reinterpret_cast<const uint4*>(x)[i];
    float* dst = s_x + i * EV;
    if constexpr (AFMT == MOE_AFMT_BF16) {
      *reinterpret_cast<float4*>(dst) = make_float4(bf16_lo(q.x), bf16_hi(q.x), bf16_lo(q.y), bf16_hi(q.y));
      *reinterpret_cast<float4*>(dst + 4) = make_float4(bf16_lo(q.z), bf16_hi(q.z), bf16_lo(q.w), bf16_hi(q.w));
    } else {
      *reinterpret_cast<float4*>(dst) = make_float4(__uint_as_float(q.x), __uint_as_float(q.y),
                                                    __uint_as_float(q.z), __uint_as_float(q.w));
    }
  }
  __syncthreads();
  float acc[kDecodeMaxTok];
#pragma unroll
  for (int t = 0; t < kDecodeMaxTok; ++t) acc[t] = 0.f;
  for (int c0 = 0; c0 < nc; c0 += 64 * kRouteBatch) {
#pragma unroll
    for (int b = 0; b < kRouteBatch; ++b) {
      const int c = c0 + lane + 64 * b;
      if (c < nc) {
#pragma unroll
        for (int t = 0; t < kDecodeMaxTok; ++t) {
          if (t < T) {
            const float4 x4 = *reinterpret_cast<const float4*>(&s_x[t * H + 4 * c]);
            acc[t] += w4[b].x * x4.x + w4[b].y * x4.y + w4[b].z * x4.z + w4[b].w * x4.w;
          }
        }
      }
    }
    const int c1 = c0 + 64 * kRouteBatch;
    if (c1 < nc) {
#pragma unroll
      for (int b = 0; b < kRouteBatch; ++b) w4[b] = row[min(c1 + lane + 64 * b, nc - 1)];
    }
  }
  if (blockIdx.x * kRouteWaves + wave >= E) return;
#pragma unroll
  for (int t = 0; t < kDecodeMaxTok; ++t) {
    if (t < T) {
      float s = wave_sum(acc[t]);
      if (lane == 0) logits[(size_t)t * E + e] = s + (bias ? bias[(size_t)t * E + e] : 0.f);
    }
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
__device__ __forceinline__ float4 route_x4(const void* x, size_t i) {  // 4 activations at element i
  if constexpr (AFMT == MOE_AFMT_BF16) {
    const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + i);
    return make_float4(bf16_lo(q.x), bf16_hi(q.x), bf16_lo(q.y), bf16_hi(q.y));
  } else {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(x) + i);
  }
}

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
    dim3 grid((E + kRouteWaves - 1) / kRouteWaves);
    size_t lds = (size_t)T * H * sizeof(float);
    if (afmt == MOE_AFMT_BF16)
      hipLaunchKernelGGL(route_gemv<MOE_AFMT_BF16>, grid, dim3(256), lds, s, x, wr, bias, logits, T, E, H);
    else
      hipLaunchKernelGGL(route_gemv<MOE_AFMT_F32>, grid, dim3(256), lds, s, x, wr, bias, logits, T, E, H);
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
