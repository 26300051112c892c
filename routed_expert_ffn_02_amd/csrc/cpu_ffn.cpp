// Host CPU branch: SwiGLU over the experts the q* split sends to the CPU.
//
// The CPU executes misses directly from the host expert pool without changing
// residency; its workers form a persistent pool pinned to cores and consume
// expert weights with SIMD and in-kernel dequantisation so the branch stays
// bandwidth bound; it returns gate-weighted per-token partial outputs
// (FreeToken summary, "측정된 대역폭이 분할을 결정합니다" and "CUDA Graph와
// 공존하는 LRU 캐시"; reading notes, 05 Implementation).
//
// Phase A: h[pair, i] = silu(W_gate[i] . x_t) * (W_up[i] . x_t), tasks over
//          (CPU expert, 64-row block of I).
// Phase B: y[t, r] = sum_{j in C, rank order} w[t,j] (W_down[r] . h[(t,j)]),
//          tasks over 64-row blocks of H.
#include <immintrin.h>
#include <pthread.h>
#include <sched.h>

#include <cmath>
#include <cstring>

#include "internal.hpp"

namespace rmoe {

// ---------------------------------------------------------------- pool
CpuPool::CpuPool(int threads) : nthreads_(threads < 1 ? 1 : threads) {
  cpu_set_t allowed;
  CPU_ZERO(&allowed);
  std::vector<int> cpus;
  if (sched_getaffinity(0, sizeof(allowed), &allowed) == 0)
    for (int c = 0; c < CPU_SETSIZE; ++c)
      if (CPU_ISSET(c, &allowed)) cpus.push_back(c);
  for (int i = 1; i < nthreads_; ++i) {
    threads_.emplace_back([this, i] { worker(i); });
    if (!cpus.empty()) {
      cpu_set_t one;
      CPU_ZERO(&one);
      CPU_SET(cpus[i % cpus.size()], &one);
      pthread_setaffinity_np(threads_.back().native_handle(), sizeof(one), &one);
    }
  }
}

CpuPool::~CpuPool() {
  stop_.store(true);
  {
    std::lock_guard<std::mutex> lk(mu_);
    gen_.fetch_add(1);
  }
  cv_.notify_all();
  for (auto& t : threads_) t.join();
}

constexpr int kIdxBits = 22;
constexpr uint64_t kIdxMask = (1ull << kIdxBits) - 1;

// Claim the next task of whatever generation the claim word currently holds.
static inline bool claim(std::atomic<uint64_t>& word, int* out) {
  uint64_t v = word.load(std::memory_order_acquire);
  for (;;) {
    const uint64_t next = v & kIdxMask, n = (v >> kIdxBits) & kIdxMask;
    if (next >= n) return false;
    if (word.compare_exchange_weak(v, v + 1, std::memory_order_acq_rel, std::memory_order_acquire)) {
      *out = (int)next;
      return true;
    }
  }
}

void CpuPool::worker(int) {
  // Start from the constructor's generation (0), not from whatever gen_ holds when
  // this thread first runs: a run() or the destructor may already have bumped it,
  // and a worker that took that value as "seen" would wait for a change that never
  // comes (the destructor's join would then block forever).
  uint64_t seen = 0;
  for (;;) {
    uint64_t g;
    int spins = 0;
    while ((g = gen_.load(std::memory_order_acquire)) == seen) {
      if (++spins < 20000) {
        _mm_pause();
      } else {
        std::unique_lock<std::mutex> lk(mu_);
        cv_.wait(lk, [&] { return gen_.load() != seen; });
      }
    }
    seen = g;
    if (stop_.load()) return;
    int i;
    // A successful claim means run() of that generation is still waiting for this
    // task, so fn_ (published before the claim word) is that generation's function.
    while (claim(claim_, &i)) {
      (*fn_.load(std::memory_order_acquire))(i);
      done_.fetch_add(1, std::memory_order_acq_rel);
    }
  }
}

void CpuPool::run(int n, const std::function<void(int)>& fn) {
  if (n <= 0) return;
  fn_.store(&fn, std::memory_order_release);
  done_.store(0, std::memory_order_release);
  {
    std::lock_guard<std::mutex> lk(mu_);
    const uint64_t g = gen_.load() + 1;
    claim_.store(((g & 0xfffffull) << (2 * kIdxBits)) | ((uint64_t)n << kIdxBits), std::memory_order_release);
    gen_.store(g, std::memory_order_release);
  }
  cv_.notify_all();
  int i;
  while (claim(claim_, &i)) {
    fn(i);
    done_.fetch_add(1, std::memory_order_acq_rel);
  }
  while (done_.load(std::memory_order_acquire) < n) _mm_pause();
}

// ---------------------------------------------------------------- dot kernels
static const float kE2M1[16] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f,
                                -0.f, -0.5f, -1.f, -1.5f, -2.f, -3.f, -4.f, -6.f};

static inline float bf16f(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Generic (any x86-64) dot products.
static float dot_f32_generic(const float* w, const float* x, int n) {
  float s = 0.f;
  for (int i = 0; i < n; ++i) s += w[i] * x[i];
  return s;
}
static float dot_bf16_generic(const uint16_t* w, const float* x, int n) {
  float s = 0.f;
  for (int i = 0; i < n; ++i) s += bf16f(w[i]) * x[i];
  return s;
}
// FP4 with de-interleaved activations: xe[i] = x[2i], xo[i] = x[2i+1].
static float dot_fp4_generic(const uint8_t* codes, const uint16_t* scales, const float* xe, const float* xo, int n) {
  float s = 0.f;
  for (int b = 0; b < n / 32; ++b) {
    float p = 0.f;
    for (int i = 0; i < 16; ++i) {
      const uint8_t c = codes[b * 16 + i];
      p += kE2M1[c & 15] * xe[b * 16 + i] + kE2M1[c >> 4] * xo[b * 16 + i];
    }
    s += bf16f(scales[b]) * p;
  }
  return s;
}

__attribute__((target("avx512f,avx512bw"))) static float dot_f32_avx512(const float* w, const float* x, int n) {
  __m512 a0 = _mm512_setzero_ps(), a1 = _mm512_setzero_ps();
  int i = 0;
  for (; i + 32 <= n; i += 32) {
    a0 = _mm512_fmadd_ps(_mm512_loadu_ps(w + i), _mm512_loadu_ps(x + i), a0);
    a1 = _mm512_fmadd_ps(_mm512_loadu_ps(w + i + 16), _mm512_loadu_ps(x + i + 16), a1);
  }
  float s = _mm512_reduce_add_ps(_mm512_add_ps(a0, a1));
  for (; i < n; ++i) s += w[i] * x[i];
  return s;
}

__attribute__((target("avx512f,avx512bw"))) static float dot_bf16_avx512(const uint16_t* w, const float* x, int n) {
  __m512 a0 = _mm512_setzero_ps(), a1 = _mm512_setzero_ps();
  int i = 0;
  for (; i + 32 <= n; i += 32) {
    __m512i q = _mm512_loadu_si512(w + i);
    __m512 lo = _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(_mm512_castsi512_si256(q)), 16));
    __m512 hi = _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(_mm512_extracti64x4_epi64(q, 1)), 16));
    a0 = _mm512_fmadd_ps(lo, _mm512_loadu_ps(x + i), a0);
    a1 = _mm512_fmadd_ps(hi, _mm512_loadu_ps(x + i + 16), a1);
  }
  float s = _mm512_reduce_add_ps(_mm512_add_ps(a0, a1));
  for (; i < n; ++i) s += bf16f(w[i]) * x[i];
  return s;
}

__attribute__((target("avx512f,avx512bw"))) static float dot_fp4_avx512(const uint8_t* codes, const uint16_t* scales,
                                                                         const float* xe, const float* xo, int n) {
  const __m512 lut = _mm512_loadu_ps(kE2M1);
  const __m512i m4 = _mm512_set1_epi32(15);
  __m512 acc = _mm512_setzero_ps();
  for (int b = 0; b < n / 32; ++b) {
    const __m512i d = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(codes + b * 16)));
    const __m512 vlo = _mm512_permutexvar_ps(_mm512_and_si512(d, m4), lut);
    const __m512 vhi = _mm512_permutexvar_ps(_mm512_srli_epi32(d, 4), lut);
    __m512 p = _mm512_mul_ps(vlo, _mm512_loadu_ps(xe + b * 16));
    p = _mm512_fmadd_ps(vhi, _mm512_loadu_ps(xo + b * 16), p);
    acc = _mm512_fmadd_ps(_mm512_set1_ps(bf16f(scales[b])), p, acc);
  }
  return _mm512_reduce_add_ps(acc);
}

struct Dots {
  float (*f32)(const float*, const float*, int);
  float (*bf16)(const uint16_t*, const float*, int);
  float (*fp4)(const uint8_t*, const uint16_t*, const float*, const float*, int);
};

static Dots pick_dots() {
  __builtin_cpu_init();
  if (__builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw"))
    return Dots{dot_f32_avx512, dot_bf16_avx512, dot_fp4_avx512};
  return Dots{dot_f32_generic, dot_bf16_generic, dot_fp4_generic};
}

// MXFP4 block scales of one row as bf16 bits: the E8M0 byte e (1..254) is the exponent
// field of 2^(e - 127), so the bf16 pattern is e << 7 (bf16 shares fp32's exponent).
static inline const uint16_t* mx_row_scales(const uint8_t* src, int nb, uint16_t* dst) {
  for (int b = 0; b < nb; ++b) dst[b] = (uint16_t)(src[b] << 7);
  return dst;
}

// ---------------------------------------------------------------- the branch
void cpu_ffn(CpuPool& pool, const CpuFfnJob& job) {
  static const Dots D = pick_dots();
  const int H = job.H, I = job.I, T = job.T, k = job.k, P = T * k;
  const int ncpu = (int)job.rec.size();
  if (ncpu == 0) return;
  const int64_t n = (int64_t)H * I;
  // pairs of each CPU expert
  std::vector<std::vector<int>> pairs(ncpu);
  for (int p = 0; p < P; ++p) {
    const int s = job.slot_idx[p];
    if (s < 0 && s != INT32_MIN) {
      const int c = -1 - s;
      if (c < ncpu) pairs[c].push_back(p);
    }
  }
  // FP4 dots read de-interleaved activations
  const bool fp4 = job.wfmt == MOE_WFMT_FP4 || job.wfmt == MOE_WFMT_MXFP4;
  const bool mx = job.wfmt == MOE_WFMT_MXFP4;
  std::vector<float> xe, xo, he, ho;
  if (fp4) {
    xe.resize((size_t)T * H / 2);
    xo.resize((size_t)T * H / 2);
    for (int t = 0; t < T; ++t)
      for (int i = 0; i < H / 2; ++i) {
        xe[(size_t)t * H / 2 + i] = job.x[(size_t)t * H + 2 * i];
        xo[(size_t)t * H / 2 + i] = job.x[(size_t)t * H + 2 * i + 1];
      }
  }
  const int RB = 64;
  const int nrb_i = (I + RB - 1) / RB;  // task counts stay far below 2^22
  pool.run(ncpu * nrb_i, [&](int task) {
    const int c = task / nrb_i, i0 = (task % nrb_i) * RB, i1 = std::min(I, i0 + RB);
    const uint8_t* rec = job.rec[c];
    std::vector<uint16_t> mg(mx ? H / 32 : 0), mu(mx ? H / 32 : 0);
    for (int p : pairs[c]) {
      const int t = p / k;
      const float* x = job.x + (size_t)t * H;
      for (int i = i0; i < i1; ++i) {
        float g, u;
        if (job.wfmt == MOE_WFMT_F32) {
          const float* W = reinterpret_cast<const float*>(rec);
          g = D.f32(W + (int64_t)i * H, x, H);
          u = D.f32(W + n + (int64_t)i * H, x, H);
        } else if (job.wfmt == MOE_WFMT_BF16) {
          const uint16_t* W = reinterpret_cast<const uint16_t*>(rec);
          g = D.bf16(W + (int64_t)i * H, x, H);
          u = D.bf16(W + n + (int64_t)i * H, x, H);
        } else {
          const float* e = xe.data() + (size_t)t * H / 2;
          const float* o = xo.data() + (size_t)t * H / 2;
          const uint16_t *sg, *su;
          if (mx) {
            const uint8_t* sb = rec + 3 * (n / 2);
            sg = mx_row_scales(sb + (int64_t)i * (H / 32), H / 32, mg.data());
            su = mx_row_scales(sb + n / 32 + (int64_t)i * (H / 32), H / 32, mu.data());
          } else {
            const uint16_t* sc = reinterpret_cast<const uint16_t*>(rec + 3 * (n / 2));
            sg = sc + (int64_t)i * (H / 32);
            su = sc + n / 32 + (int64_t)i * (H / 32);
          }
          g = D.fp4(rec + (int64_t)i * (H / 2), sg, e, o, H);
          u = D.fp4(rec + n / 2 + (int64_t)i * (H / 2), su, e, o, H);
        }
        job.h[(size_t)p * I + i] = (g / (1.0f + std::exp(-g))) * u;
      }
    }
  });
  if (fp4) {
    he.resize((size_t)P * I / 2);
    ho.resize((size_t)P * I / 2);
    for (int c = 0; c < ncpu; ++c)
      for (int p : pairs[c])
        for (int i = 0; i < I / 2; ++i) {
          he[(size_t)p * I / 2 + i] = job.h[(size_t)p * I + 2 * i];
          ho[(size_t)p * I / 2 + i] = job.h[(size_t)p * I + 2 * i + 1];
        }
  }
  std::vector<int> cpu_of_pair(P, -1);
  for (int c = 0; c < ncpu; ++c)
    for (int p : pairs[c]) cpu_of_pair[p] = c;
  const int nrb_h = (H + RB - 1) / RB;
  pool.run(nrb_h, [&](int task) {
    const int r0 = task * RB, r1 = std::min(H, r0 + RB);
    std::vector<uint16_t> md(mx ? I / 32 : 0);
    for (int r = r0; r < r1; ++r) {
      for (int t = 0; t < T; ++t) {
        float acc = 0.f;
        for (int j = 0; j < k; ++j) {
          const int p = t * k + j;
          const int c = cpu_of_pair[p];
          if (c < 0) continue;
          const uint8_t* rec = job.rec[c];
          const float* h = job.h + (size_t)p * I;
          float d;
          if (job.wfmt == MOE_WFMT_F32) {
            d = D.f32(reinterpret_cast<const float*>(rec) + 2 * n + (int64_t)r * I, h, I);
          } else if (job.wfmt == MOE_WFMT_BF16) {
            d = D.bf16(reinterpret_cast<const uint16_t*>(rec) + 2 * n + (int64_t)r * I, h, I);
          } else {
            const uint16_t* sd =
                mx ? mx_row_scales(rec + 3 * (n / 2) + 2 * (n / 32) + (int64_t)r * (I / 32), I / 32, md.data())
                   : reinterpret_cast<const uint16_t*>(rec + 3 * (n / 2)) + 2 * (n / 32) + (int64_t)r * (I / 32);
            d = D.fp4(rec + n + (int64_t)r * (I / 2), sd, he.data() + (size_t)p * I / 2, ho.data() + (size_t)p * I / 2, I);
          }
          acc += job.w[p] * d;
        }
        job.y[(size_t)t * H + r] = acc;
      }
    }
  });
}

}  // namespace rmoe
