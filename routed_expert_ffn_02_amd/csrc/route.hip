// Router logits and top-k / softmax gates.
//
// The router and the cache lookup run on the GPU and pick k of E experts per
// token (FreeToken summary, "decode co-design" section: router and cache lookup
// on the GPU; "MoE" section: k << E).  Gates are the softmax over all E logits
// taken at the chosen experts (renorm = 1: renormalised over the k chosen).
#include "common.hpp"

namespace rmoe {

// ---------------------------------------------------------------------------
// Decode-sized batches: one wavefront per expert row, activations staged in LDS
// as fp32.  W_r rows are read with 16-byte lane loads (fully coalesced).
constexpr int kRouteWaves = 4;

template <int AFMT>
__global__ __launch_bounds__(256) void route_gemv(const void* __restrict__ x, const float* __restrict__ wr,
                                                   const float* __restrict__ bias, float* __restrict__ logits,
                                                   int T, int E, int H) {
  extern __shared__ float s_x[];  // [T][H]
  constexpr int EV = (AFMT == MOE_AFMT_BF16) ? 8 : 4;
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
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * kRouteWaves + wave;
  if (e >= E) return;
  float acc[kDecodeMaxTok];
#pragma unroll
  for (int t = 0; t < kDecodeMaxTok; ++t) acc[t] = 0.f;
  const float4* row = reinterpret_cast<const float4*>(wr + (size_t)e * H);
  for (int c = lane; c < H / 4; c += 64) {
    float4 w4 = row[c];
#pragma unroll
    for (int t = 0; t < kDecodeMaxTok; ++t) {
      if (t < T) {
        const float4 x4 = *reinterpret_cast<const float4*>(&s_x[t * H + 4 * c]);
        acc[t] += w4.x * x4.x + w4.y * x4.y + w4.z * x4.z + w4.w * x4.w;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kDecodeMaxTok; ++t) {
    if (t < T) {
      float s = wave_sum(acc[t]);
      if (lane == 0) logits[(size_t)t * E + e] = s + (bias ? bias[(size_t)t * E + e] : 0.f);
    }
  }
}

// ---------------------------------------------------------------------------
// Long prompts: LDS-tiled fp32 GEMM, 64 tokens x 64 experts per block, K step 16,
// each thread 4x4 outputs.
template <int AFMT>
__global__ __launch_bounds__(256) void route_gemm(const void* __restrict__ x, const float* __restrict__ wr,
                                                   const float* __restrict__ bias, float* __restrict__ logits,
                                                   int T, int E, int H) {
  __shared__ float sA[16][64 + 4];
  __shared__ float sB[16][64 + 4];
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < H; k0 += 16) {
    for (int i = threadIdx.x; i < 64 * 16; i += 256) {
      int r = i / 16, kk = i % 16;
      int t = t0 + r, e = e0 + r;
      sA[kk][r] = (t < T) ? load_act<AFMT>(x, (size_t)t * H + k0 + kk) : 0.f;
      sB[kk][r] = (e < E) ? wr[(size_t)e * H + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int e = e0 + tx * 4 + j;
      if (e < E) logits[(size_t)t * E + e] = acc[i][j] + (bias ? bias[(size_t)t * E + e] : 0.f);
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
    dim3 grid((T + 63) / 64, (E + 63) / 64);
    if (afmt == MOE_AFMT_BF16)
      hipLaunchKernelGGL(route_gemm<MOE_AFMT_BF16>, grid, dim3(256), 0, s, x, wr, bias, logits, T, E, H);
    else
      hipLaunchKernelGGL(route_gemm<MOE_AFMT_F32>, grid, dim3(256), 0, s, x, wr, bias, logits, T, E, H);
  }
}

// ---------------------------------------------------------------------------
// Top-k + gates: one wavefront per token.  Each lane holds E/64 logits; k rounds
// of a wave arg-max under the total order (value descending, index ascending).
constexpr int kTopkPerLane = kMaxExperts / 64;

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k, int renorm,
                                                   int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const float* z = logits + (size_t)t * E;
  float v[kTopkPerLane];
  bool taken[kTopkPerLane];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kTopkPerLane; ++i) {
    int e = lane + 64 * i;
    v[i] = (e < E) ? z[e] : -INFINITY;
    taken[i] = (e >= E);
    mx = fmaxf(mx, v[i]);
  }
  mx = wave_max(mx);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kTopkPerLane; ++i)
    if (lane + 64 * i < E) sum += __expf(v[i] - mx);
  sum = wave_sum(sum);
  float sel_sum = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kTopkPerLane; ++i) {
      int e = lane + 64 * i;
      if (!taken[i] && better(v[i], e, bv, bi)) { bv = v[i]; bi = e; }
    }
    // wave arg-max under the same order: the largest value, then the lowest index
    // among the lanes holding it (-0 and +0 compare equal, as in `better`)
    const float wv = wave_max(bv);
    bi = wave_min_i32(bv == wv ? bi : 0x7fffffff);
    bv = wv;
    // bi is the same on every lane; mark it taken
#pragma unroll
    for (int i = 0; i < kTopkPerLane; ++i)
      if (lane + 64 * i == bi) taken[i] = true;
    float p = __expf(bv - mx) / sum;
    sel_sum += p;
    if (lane == 0) {
      idx_out[(size_t)t * k + j] = bi;
      w_out[(size_t)t * k + j] = p;
    }
  }
  if (renorm && lane == 0) {
    for (int j = 0; j < k; ++j) w_out[(size_t)t * k + j] = w_out[(size_t)t * k + j] / sel_sum;
  }
}

void launch_topk(const float* logits, int T, int E, int k, int renorm, int32_t* idx, float* w, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, renorm, idx, w);
}

}  // namespace rmoe
