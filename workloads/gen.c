/*
 * Seeded synthetic input generator for the routed-MoE workloads.
 *
 * Holds none of the method's arithmetic: it only turns (seed, stream, counter)
 * into numbers and writes them into caller buffers.  Both the CPU oracle (for
 * single experts, activations and router weights) and the GPU benchmark (to fill
 * the pinned host expert pool) call this one implementation, so every value is
 * produced by the same code on both sides.
 *
 * Generator: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014).  Its n-th output from seed k is
 * mix(k + n*gamma), so it can be evaluated at any counter position.
 *
 * Approximately normal values: the sum of the four 16-bit fields of one 64-bit
 * output (Irwin-Hall with n = 4), centred and scaled to the requested standard
 * deviation.  Integer sum -> float conversion is exact and the scaling is one
 * IEEE single multiply, so the value is the same on every IEEE machine.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <math.h>
#include <pthread.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Per-stream key: a SplitMix64 output of the seed, perturbed by the stream id. */
static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(seed * GOLDEN + mix64(stream + GOLDEN));
}

static inline uint64_t draw(uint64_t key, uint64_t ctr) { return mix64(key + ctr * GOLDEN); }

uint64_t wl_hash(uint64_t seed, uint64_t stream, uint64_t ctr) {
  return draw(stream_key(seed, stream), ctr);
}

/* Irwin-Hall(4) of 16-bit uniforms: sum in [0, 4*65535], centred. */
static inline int32_t ih4(uint64_t r) {
  int32_t s = (int32_t)(r & 0xFFFF) + (int32_t)((r >> 16) & 0xFFFF) +
              (int32_t)((r >> 32) & 0xFFFF) + (int32_t)(r >> 48);
  return s - 131070;
}

static float ih4_scale(float sigma) {
  /* standard deviation of the centred sum of four uniforms on {0..65535} */
  double sd = sqrt(4.0 * (65536.0 * 65536.0 - 1.0) / 12.0);
  return (float)((double)sigma / sd);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

void wl_normal_f32(float* out, int64_t n, uint64_t seed, uint64_t stream, uint64_t ctr0, float sigma) {
  uint64_t k = stream_key(seed, stream);
  float c = ih4_scale(sigma);
  for (int64_t i = 0; i < n; ++i) out[i] = (float)ih4(draw(k, ctr0 + (uint64_t)i)) * c;
}

void wl_normal_bf16(uint16_t* out, int64_t n, uint64_t seed, uint64_t stream, uint64_t ctr0, float sigma) {
  uint64_t k = stream_key(seed, stream);
  float c = ih4_scale(sigma);
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne((float)ih4(draw(k, ctr0 + (uint64_t)i)) * c);
}

/* Byte i of the output is byte (i % 8) of draw(ctr0 + i / 8); n need not be a multiple of 8. */
void wl_bytes(uint8_t* out, int64_t n, uint64_t seed, uint64_t stream, uint64_t ctr0) {
  uint64_t k = stream_key(seed, stream);
  int64_t i = 0;
  for (; i + 8 <= n; i += 8) {
    uint64_t r = draw(k, ctr0 + (uint64_t)(i / 8));
    memcpy(out + i, &r, 8);
  }
  if (i < n) {
    uint64_t r = draw(k, ctr0 + (uint64_t)(i / 8));
    memcpy(out + i, &r, (size_t)(n - i));
  }
}

/* lo + (top 32 bits of the draw) % (hi - lo + 1): integers in [lo, hi] (bytes). */
void wl_uniform_u8(uint8_t* out, int64_t n, uint64_t seed, uint64_t stream, uint64_t ctr0, int32_t lo, int32_t hi) {
  uint64_t k = stream_key(seed, stream);
  uint64_t span = (uint64_t)(hi - lo + 1);
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)(lo + (int32_t)((draw(k, ctr0 + (uint64_t)i) >> 32) % span));
}

/* bf16(lo + (hi - lo) * u) with u = (top 16 bits of the draw) / 65536. */
void wl_uniform_bf16(uint16_t* out, int64_t n, uint64_t seed, uint64_t stream, uint64_t ctr0, float lo, float hi) {
  uint64_t k = stream_key(seed, stream);
  float span = hi - lo;
  for (int64_t i = 0; i < n; ++i) {
    float u = (float)(draw(k, ctr0 + (uint64_t)i) >> 48) * (1.0f / 65536.0f);
    out[i] = f32_to_bf16_rne(lo + span * u);
  }
}

void wl_uniform_f64(double* out, int64_t n, uint64_t seed, uint64_t stream, uint64_t ctr0) {
  uint64_t k = stream_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = (double)(draw(k, ctr0 + (uint64_t)i) >> 11) * (1.0 / 9007199254740992.0);
}

/* ------------------------------------------------------------------------ */
/* Expert weights.  Stream ids: one per (backing key, tensor).               */

#define DOMAIN_EXPERT (1ULL << 56)
#define DOMAIN_SCALE  (2ULL << 56)

enum { WL_F32 = 0, WL_BF16 = 1, WL_FP4 = 2, WL_MXFP4 = 3 };

typedef struct {
  int32_t n_layers, n_experts, hidden, inter;
  int32_t wfmt;        /* WL_F32, WL_BF16, WL_FP4 (e2m1 codes + bf16 scale per 32),
                          WL_MXFP4 (e2m1 codes + E8M0 scale byte per 32) */
  int32_t exact;       /* 0: dense random values; 1: the sparse few-bit values of
                          wl_exact_tensor (every sum of products exact in fp32) */
  uint64_t seed;
  int64_t alias_records;  /* 0: every key has its own values; R > 0: key -> key % R */
  float sigma;            /* weight standard deviation (F32/BF16) */
  float fp4_scale_lo, fp4_scale_hi;  /* FP4 block scales ~ U[lo, hi] */
  float pad2;
  int32_t mx_exp_lo, mx_exp_hi;      /* MXFP4 block scale bytes ~ uniform integers in [lo, hi] */
} wl_cfg;

static inline int64_t backing(const wl_cfg* c, int64_t key) {
  return c->alias_records > 0 ? key % c->alias_records : key;
}

/* rows x cols of tensor t (0 gate [I,H], 1 up [I,H], 2 down [H,I]) */
static inline void tensor_shape(const wl_cfg* c, int t, int64_t* rows, int64_t* cols) {
  if (t < 2) { *rows = c->inter; *cols = c->hidden; }
  else { *rows = c->hidden; *cols = c->inter; }
}

/*
 * Exact-arithmetic expert tensors (exact = 1).  Sparse rows of few-bit values whose
 * products with the exact activations below, and every partial sum of those products,
 * are representable in fp32, so any summation order gives the same result:
 *   gate rows  one nonzero (1 row in 8 all zero): a positive code 1..7, block scale
 *              2^6 or 2^7;
 *   up rows    one nonzero: a code of either sign, block scale 2^-3 or 2^-2;
 *   down rows  four nonzeros (positions may coincide; the last drawn wins): codes of
 *              either sign, block scale 2^-4 or 2^-3.
 * Every 32-element block of a row has its own power-of-two scale (drawn per block, also
 * for all-zero blocks).  FP4 stores the 4-bit code and the scale (bf16 bits of the power
 * of two); MXFP4 stores the code and the E8M0 byte 127 + exponent; F32 / BF16 store the
 * value itself, from the magnitudes {0.5, 1, 1.5, 2, 3, 4, 6} (indexed by the code's low
 * three bits minus one; bit 3 is the sign) times the block's power of two.
 */
static const float kMag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

static int exact_tensor(const wl_cfg* c, int64_t key, int t, void* values, void* scales) {
  int64_t rows, cols;
  tensor_shape(c, t, &rows, &cols);
  if (cols % 32) return -1;
  const int64_t nb = cols / 32;
  const uint64_t sid = ((uint64_t)backing(c, key) << 2) | (uint64_t)t;
  const uint64_t kv = stream_key(c->seed, DOMAIN_EXPERT | sid), ks = stream_key(c->seed, DOMAIN_SCALE | sid);
  const int base = t == 0 ? 6 : (t == 1 ? -3 : -4);
  const int fp4 = c->wfmt == WL_FP4 || c->wfmt == WL_MXFP4;
  if (fp4) memset(values, 0, (size_t)(rows * cols / 2));
  else memset(values, 0, (size_t)(rows * cols * (c->wfmt == WL_F32 ? 4 : 2)));
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const int e = base + (int)(draw(ks, (uint64_t)(r * nb + b)) & 1);
      if (c->wfmt == WL_FP4) ((uint16_t*)scales)[r * nb + b] = (uint16_t)((uint32_t)(127 + e) << 7);
      else if (c->wfmt == WL_MXFP4) ((uint8_t*)scales)[r * nb + b] = (uint8_t)(127 + e);
    }
    const int nnz = t == 2 ? 4 : 1;
    for (int i = 0; i < nnz; ++i) {
      const uint64_t d = draw(kv, (uint64_t)(r * 4 + i));
      if (t == 0 && (d & 7) == 0) break;  /* an all-zero gate row */
      const int64_t p = (int64_t)((d >> 3) % (uint64_t)cols);
      const uint32_t mag = 1u + (uint32_t)((d >> 40) % 7u);
      const uint32_t code = mag | (t == 0 ? 0u : (uint32_t)((d >> 47) & 1u) << 3);
      if (fp4) {
        uint8_t* byte = (uint8_t*)values + r * (cols / 2) + p / 2;
        *byte = (p & 1) ? (uint8_t)((*byte & 0x0F) | (code << 4)) : (uint8_t)((*byte & 0xF0) | code);
      } else {
        const int e = base + (int)(draw(ks, (uint64_t)(r * nb + p / 32)) & 1);
        const float v = (code & 8u ? -kMag[mag] : kMag[mag]) * ldexpf(1.0f, e);
        if (c->wfmt == WL_F32) ((float*)values)[r * cols + p] = v;
        else ((uint16_t*)values)[r * cols + p] = f32_to_bf16_rne(v);  /* exact: at most 2 significant bits */
      }
    }
  }
  return 0;
}

/* Exact-arithmetic activations: 0 with probability 1/8, else 1 or 2 (fp32, or bf16 bits). */
void wl_exact_act(void* out, int64_t n, int bf16, uint64_t seed, uint64_t stream, uint64_t ctr0) {
  uint64_t k = stream_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) {
    const uint64_t d = draw(k, ctr0 + (uint64_t)i);
    const float v = (d & 7) == 0 ? 0.0f : (float)(1 + ((d >> 3) & 1));
    if (bf16) ((uint16_t*)out)[i] = f32_to_bf16_rne(v);
    else ((float*)out)[i] = v;
  }
}

/* Exact-arithmetic router weights [rows, cols]: eight nonzeros per row (positions may
 * coincide), values +-{1, 2, 4} * 2^-6. */
void wl_exact_router(float* out, int64_t rows, int64_t cols, uint64_t seed, uint64_t stream) {
  uint64_t k = stream_key(seed, stream);
  memset(out, 0, (size_t)(rows * cols) * sizeof(float));
  for (int64_t r = 0; r < rows; ++r)
    for (int i = 0; i < 8; ++i) {
      const uint64_t d = draw(k, (uint64_t)(r * 8 + i));
      const float v = ldexpf((float)(1u << ((d >> 40) % 3u)), -6);
      out[r * cols + (int64_t)((d >> 3) % (uint64_t)cols)] = (d >> 47) & 1 ? -v : v;
    }
}

/*
 * Logical values of one expert tensor.
 *  F32:  values = float[rows*cols]
 *  BF16: values = uint16 bf16 bits [rows*cols]
 *  FP4:  values = uint8 codes [rows*cols/2], element 2i in the low nibble of byte i
 *        (elements run along a row, i.e. along the reduction dimension);
 *        scales = uint16 bf16 bits [rows*cols/32], one per 32 consecutive elements of a row.
 *  MXFP4: codes as FP4; scales = uint8 E8M0 exponents [rows*cols/32] (scale 2^(e - 127)).
 */
int wl_expert_tensor(const wl_cfg* c, int64_t key, int t, void* values, void* scales) {
  if (!c || t < 0 || t > 2 || key < 0 || key >= (int64_t)c->n_layers * c->n_experts) return -1;
  int64_t rows, cols;
  tensor_shape(c, t, &rows, &cols);
  int64_t n = rows * cols;
  uint64_t sid = ((uint64_t)backing(c, key) << 2) | (uint64_t)t;
  if (c->exact) return (c->wfmt == WL_FP4 || c->wfmt == WL_MXFP4) && !scales ? -1 : exact_tensor(c, key, t, values, scales);
  switch (c->wfmt) {
    case WL_F32: wl_normal_f32((float*)values, n, c->seed, DOMAIN_EXPERT | sid, 0, c->sigma); return 0;
    case WL_BF16: wl_normal_bf16((uint16_t*)values, n, c->seed, DOMAIN_EXPERT | sid, 0, c->sigma); return 0;
    case WL_FP4:
      if (cols % 32) return -1;
      wl_bytes((uint8_t*)values, n / 2, c->seed, DOMAIN_EXPERT | sid, 0);
      if (scales)
        wl_uniform_bf16((uint16_t*)scales, n / 32, c->seed, DOMAIN_SCALE | sid, 0, c->fp4_scale_lo, c->fp4_scale_hi);
      return 0;
    case WL_MXFP4:
      if (cols % 32 || c->mx_exp_lo < 0 || c->mx_exp_hi > 255 || c->mx_exp_lo > c->mx_exp_hi) return -1;
      wl_bytes((uint8_t*)values, n / 2, c->seed, DOMAIN_EXPERT | sid, 0);
      if (scales) wl_uniform_u8((uint8_t*)scales, n / 32, c->seed, DOMAIN_SCALE | sid, 0, c->mx_exp_lo, c->mx_exp_hi);
      return 0;
  }
  return -1;
}

/*
 * Bytes of one packed expert record in the pool format the library reads:
 *  F32 / BF16: [gate I*H | up I*H | down H*I], each row-major, element size 4 / 2;
 *  FP4:        [gate codes I*H/2 | up codes | down codes H*I/2 |
 *               gate scales I*H/32 bf16 | up scales | down scales];
 *  MXFP4:      as FP4 with one scale byte (E8M0) per 32 elements.
 */
int64_t wl_record_bytes(const wl_cfg* c) {
  int64_t n = (int64_t)c->hidden * c->inter;
  switch (c->wfmt) {
    case WL_F32: return 3 * n * 4;
    case WL_BF16: return 3 * n * 2;
    case WL_FP4: return 3 * (n / 2) + 3 * (n / 32) * 2;
    case WL_MXFP4: return 3 * (n / 2) + 3 * (n / 32);
  }
  return -1;
}

int wl_pack_record(const wl_cfg* c, int64_t key, void* dst) {
  int64_t n = (int64_t)c->hidden * c->inter;
  uint8_t* p = (uint8_t*)dst;
  int rc = 0;
  for (int t = 0; t < 3 && rc == 0; ++t) {
    switch (c->wfmt) {
      case WL_F32: rc = wl_expert_tensor(c, key, t, p + (size_t)t * n * 4, NULL); break;
      case WL_BF16: rc = wl_expert_tensor(c, key, t, p + (size_t)t * n * 2, NULL); break;
      case WL_FP4:
        rc = wl_expert_tensor(c, key, t, p + (size_t)t * (n / 2), p + 3 * (size_t)(n / 2) + (size_t)t * (n / 32) * 2);
        break;
      case WL_MXFP4:
        rc = wl_expert_tensor(c, key, t, p + (size_t)t * (n / 2), p + 3 * (size_t)(n / 2) + (size_t)t * (n / 32));
        break;
      default: rc = -1;
    }
  }
  return rc;
}

typedef struct {
  const wl_cfg* c;
  uint8_t* pool;
  int64_t rec;
  int64_t first, count, tid, nthreads;
  int rc;
} fill_job;

static void* fill_worker(void* arg) {
  fill_job* j = (fill_job*)arg;
  for (int64_t i = j->tid; i < j->count; i += j->nthreads) {
    int rc = wl_pack_record(j->c, j->first + i, j->pool + (size_t)i * (size_t)j->rec);
    if (rc) { j->rc = rc; break; }
  }
  return NULL;
}

/* Pack records for keys [first, first+count) into pool[0 .. count*record_bytes). */
int wl_fill_pool(const wl_cfg* c, void* pool, int64_t first, int64_t count, int threads) {
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  int64_t rec = wl_record_bytes(c);
  if (rec <= 0) return -1;
  pthread_t th[256];
  fill_job jobs[256];
  for (int i = 0; i < threads; ++i) {
    jobs[i] = (fill_job){c, (uint8_t*)pool, rec, first, count, i, threads, 0};
    if (pthread_create(&th[i], NULL, fill_worker, &jobs[i])) { threads = i; break; }
  }
  int rc = 0;
  for (int i = 0; i < threads; ++i) { pthread_join(th[i], NULL); if (jobs[i].rc) rc = jobs[i].rc; }
  return rc;
}
