// Expert bank file: the host pool stored in its runtime layout, loaded with parallel
// direct I/O.
//
// The FreeToken summary ("전문가 뱅크와 FTW 포맷"; "탄력적 메모리 관리", engine
// bootstrap) and the reading notes (05 Implementation) describe a weight format whose
// experts are pre-merged in the runtime bank layout, indexed by the flattened id
// l*E + e, so that start-up skips tensor discovery and repacking and reads aligned
// chunks with parallel direct I/O straight into exactly sized host banks; serving then
// starts from a cold cache, which the ordinary miss path fills.
//
// Here one bank holds whole expert records (one record per key, the layout
// moe_record_bytes defines), so the file is a 4 KiB header followed by the records in
// key order.  Records are multiples of 4 KiB for every supported shape, so a page-aligned
// pool is read with O_DIRECT in large aligned chunks by several threads.  Memory that the
// kernel cannot do direct I/O into (page-locked memory the GPU driver maps, here) takes
// O_DIRECT reads into per-thread bounce buffers and a copy; a file system without
// O_DIRECT takes buffered pread.
#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <cerrno>
#include <chrono>
#include <cstring>
#include <thread>
#include <vector>

#include "internal.hpp"

namespace rmoe {
namespace {

constexpr char kMagic[8] = {'R', 'M', 'O', 'E', 'B', 'N', 'K', '1'};
constexpr int64_t kHeaderBytes = 4096;
constexpr int64_t kAlign = 4096;
constexpr int64_t kChunk = 64ll << 20;  // bytes per read request

struct Header {
  char magic[8];
  uint32_t version;
  int32_t n_layers, n_experts, hidden, inter, wfmt;
  int64_t record_bytes, n_records, data_offset;
};
static_assert(sizeof(Header) <= kHeaderBytes, "header fits its block");

bool read_header(int fd, Header* h) {
  if (pread(fd, h, sizeof(Header), 0) != (ssize_t)sizeof(Header)) return false;
  return std::memcmp(h->magic, kMagic, 8) == 0 && h->version == 1 && h->record_bytes > 0 && h->n_records > 0 &&
         h->data_offset == kHeaderBytes;
}

// Read [off, off + n) of the file into dst with `threads` workers over kChunk pieces.
// Mode kDirect: O_DIRECT straight into dst (every piece a multiple of kAlign at an aligned
// file offset and address).  kBounce: O_DIRECT into a page-aligned buffer per worker, then
// a copy into dst (for destinations the kernel cannot do direct I/O into, e.g. memory the
// GPU driver mapped).  kBuffered: plain pread through the page cache.  *err receives the
// first errno seen.
enum ReadMode { kDirect = 0, kBounce = 1, kBuffered = 2 };

bool parallel_read(const char* path, ReadMode mode, int64_t off, uint8_t* dst, int64_t n, int threads, int* err) {
  const int64_t pieces = (n + kChunk - 1) / kChunk;
  std::atomic<int64_t> next{0};
  std::atomic<bool> ok{true};
  std::atomic<int> first_err{0};
  auto fail = [&](int e) {
    int zero = 0;
    first_err.compare_exchange_strong(zero, e ? e : EIO);
    ok = false;
  };
  auto worker = [&] {
    const int fd = open(path, O_RDONLY | (mode == kBuffered ? 0 : O_DIRECT));
    if (fd < 0) return fail(errno);
    void* bounce = nullptr;
    if (mode == kBounce && posix_memalign(&bounce, kAlign, kChunk) != 0) {
      close(fd);
      return fail(ENOMEM);
    }
    for (int64_t p; ok && (p = next.fetch_add(1)) < pieces;) {
      const int64_t b = p * kChunk, len = std::min(kChunk, n - b);
      uint8_t* to = mode == kBounce ? static_cast<uint8_t*>(bounce) : dst + b;
      for (int64_t done = 0; done < len;) {
        const ssize_t r = pread(fd, to + done, (size_t)(len - done), off + b + done);
        if (r <= 0) {
          if (r < 0 && errno == EINTR) continue;
          fail(r < 0 ? errno : EIO);
          break;
        }
        done += r;
      }
      if (ok && mode == kBounce) std::memcpy(dst + b, bounce, (size_t)len);
    }
    free(bounce);
    close(fd);
  };
  std::vector<std::thread> ts;
  for (int i = 1; i < threads; ++i) ts.emplace_back(worker);
  worker();
  for (auto& t : ts) t.join();
  if (err && !*err) *err = first_err.load();
  return ok;
}

// Whether one block scale keeps every nonzero weight e2m1(code) * scale of its block in
// f16's normal range [2^-14, 65504] (|code| in 0.5 .. 6).  bf16 scale bits: zero passes; a
// nonzero |s| needs 2^-13 <= |s| (biased exponent >= 114) and 6 |s| <= 65504 (exponent
// 140 with at most 42 of 128 mantissa steps, or below 140); inf / NaN / subnormals fail.
// E8M0 byte e (2^(e - 127)): 114 <= e <= 140.
bool scale_ok_bf16(uint16_t b) {
  const int e = (b >> 7) & 0xff, m = b & 0x7f;
  if (e == 0) return m == 0;
  return (e >= 114 && e < 140) || (e == 140 && m <= 42);
}
bool scale_ok_e8m0(uint8_t e) { return e >= 114 && e <= 140; }

}  // namespace
}  // namespace rmoe

using namespace rmoe;

extern "C" MOE_API moe_status moe_pool_check_f16(const moe_config* cfg, const void* pool, int64_t n_records,
                                                 int64_t* first_bad) {
  if (!cfg || !pool || n_records < 0 || !first_bad) return MOE_EINVAL;
  const int64_t S = moe_record_bytes(cfg);
  if (S <= 0) return MOE_EINVAL;
  *first_bad = -1;
  if (cfg->wfmt != MOE_WFMT_FP4 && cfg->wfmt != MOE_WFMT_MXFP4) return MOE_OK;  // no block scales
  const int64_t n = (int64_t)cfg->hidden * cfg->inter;
  const int64_t scales = 3 * (n / 32), off = 3 * (n / 2);  // after the three tensors' codes
  const bool mx = cfg->wfmt == MOE_WFMT_MXFP4;
  const int nt = (int)std::max<int64_t>(1, std::min<int64_t>({16, n_records, (int64_t)std::thread::hardware_concurrency()}));
  std::atomic<int64_t> bad{INT64_MAX};
  std::vector<std::thread> ts;
  for (int t = 0; t < nt; ++t)
    ts.emplace_back([&, t] {
      for (int64_t r = t; r < n_records && r < bad.load(std::memory_order_relaxed); r += nt) {
        const uint8_t* sc = static_cast<const uint8_t*>(pool) + r * S + off;
        bool ok = true;
        if (mx) {
          for (int64_t i = 0; i < scales && ok; ++i) ok = scale_ok_e8m0(sc[i]);
        } else {
          for (int64_t i = 0; i < scales && ok; ++i) {
            uint16_t b;
            std::memcpy(&b, sc + 2 * i, 2);
            ok = scale_ok_bf16(b);
          }
        }
        if (!ok) {
          int64_t cur = bad.load();
          while (r < cur && !bad.compare_exchange_weak(cur, r)) {
          }
          return;
        }
      }
    });
  for (auto& th : ts) th.join();
  if (bad.load() != INT64_MAX) {
    *first_bad = bad.load();
    return MOE_EINVAL;
  }
  return MOE_OK;
}

extern "C" MOE_API moe_status moe_bank_write(const char* path, const moe_config* cfg, const void* pool,
                                             int64_t n_records) {
  if (!path || !cfg || !pool || n_records < 1) return MOE_EINVAL;
  const int64_t S = moe_record_bytes(cfg);
  if (S <= 0 || n_records > (int64_t)cfg->n_layers * cfg->n_experts) return MOE_EINVAL;
  Header h{};
  std::memcpy(h.magic, kMagic, 8);
  h.version = 1;
  h.n_layers = cfg->n_layers;
  h.n_experts = cfg->n_experts;
  h.hidden = cfg->hidden;
  h.inter = cfg->inter;
  h.wfmt = cfg->wfmt;
  h.record_bytes = S;
  h.n_records = n_records;
  h.data_offset = kHeaderBytes;
  const int fd = open(path, O_WRONLY | O_CREAT | O_TRUNC, 0644);
  if (fd < 0) return MOE_EINVAL;
  std::vector<uint8_t> block(kHeaderBytes, 0);
  std::memcpy(block.data(), &h, sizeof(h));
  bool ok = pwrite(fd, block.data(), kHeaderBytes, 0) == kHeaderBytes;
  const uint8_t* src = static_cast<const uint8_t*>(pool);
  const int64_t total = n_records * S;
  for (int64_t done = 0; ok && done < total;) {
    const ssize_t w = pwrite(fd, src + done, (size_t)std::min<int64_t>(kChunk, total - done), kHeaderBytes + done);
    if (w <= 0) {
      if (w < 0 && errno == EINTR) continue;
      ok = false;
      break;
    }
    done += w;
  }
  ok = ok && fsync(fd) == 0;
  close(fd);
  return ok ? MOE_OK : MOE_EHIP;
}

extern "C" MOE_API moe_status moe_bank_info(const char* path, moe_bank_header* out) {
  if (!path || !out) return MOE_EINVAL;
  const int fd = open(path, O_RDONLY);
  if (fd < 0) return MOE_EINVAL;
  Header h;
  const bool ok = read_header(fd, &h);
  struct stat st;
  const bool sized = ok && fstat(fd, &st) == 0 && st.st_size >= h.data_offset + h.record_bytes * h.n_records;
  close(fd);
  if (!ok || !sized) return MOE_EINVAL;
  *out = moe_bank_header{h.n_layers, h.n_experts, h.hidden, h.inter, h.wfmt, 0, h.record_bytes, h.n_records};
  return MOE_OK;
}

extern "C" MOE_API moe_status moe_bank_read(const char* path, const moe_config* cfg, void* dst, int64_t dst_bytes,
                                            int32_t threads, moe_bank_stats* out) {
  moe_bank_header h;
  if (!dst || threads < 1 || threads > 256 || moe_bank_info(path, &h) != MOE_OK) return MOE_EINVAL;
  if (cfg && (cfg->n_layers != h.n_layers || cfg->n_experts != h.n_experts || cfg->hidden != h.hidden ||
              cfg->inter != h.inter || cfg->wfmt != h.wfmt || moe_record_bytes(cfg) != h.record_bytes))
    return MOE_EINVAL;
  const int64_t n = h.record_bytes * h.n_records;
  if (dst_bytes < n) return MOE_EINVAL;
  uint8_t* d = static_cast<uint8_t*>(dst);
  const bool aligned = n % kAlign == 0;
  const bool dst_aligned = aligned && reinterpret_cast<uintptr_t>(d) % kAlign == 0;
  const auto t0 = std::chrono::steady_clock::now();
  int err = 0;
  ReadMode used = kBuffered;
  if (dst_aligned && parallel_read(path, kDirect, kHeaderBytes, d, n, threads, &err)) used = kDirect;
  else if (aligned && parallel_read(path, kBounce, kHeaderBytes, d, n, threads, &err)) used = kBounce;
  else if (!parallel_read(path, kBuffered, kHeaderBytes, d, n, threads, &err)) return MOE_EHIP;
  if (out) {
    out->bytes = (uint64_t)n;
    out->seconds = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    out->mode = used;
    out->threads = threads;
    out->direct_errno = err;
    out->pad = 0;
  }
  return MOE_OK;
}

extern "C" MOE_API moe_status moe_pool_load(moe_ctx* ctx, const char* path, int32_t threads, void** host_pool,
                                            moe_bank_stats* out) {
  if (!ctx || !host_pool) return MOE_EINVAL;
  moe_bank_header h;
  if (moe_bank_info(path, &h) != MOE_OK) {
    ctx->err = "bank file missing, malformed or truncated";
    return MOE_EINVAL;
  }
  void* p = nullptr;
  moe_status st = moe_pool_alloc(ctx, h.n_records, &p);
  if (st != MOE_OK) return st;
  st = moe_bank_read(path, &ctx->cfg, p, h.n_records * ctx->S, threads, out);
  if (st != MOE_OK) {  // release the unfilled pool: the context holds none again
    ctx->err = st == MOE_EINVAL ? "bank file does not match the context's shape and format" : "bank read failed";
    hipHostFree(p);
    ctx->pool = nullptr;
    ctx->pool_dev = nullptr;
    ctx->pool_records = 0;
    ctx->pool_owned = ctx->pool_pinned = false;
    return st;
  }
  *host_pool = p;
  return MOE_OK;
}
