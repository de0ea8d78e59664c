// C-ABI entry points of libcpthd: host-side validation, then stream-ordered
// launches.  Validation order: scalar arguments and NULL checks first (no HIP
// call), then device membership of every pointer, then byte-range overlap of
// outputs against inputs and each other, then the launches.  Nothing is
// launched when any check fails ("Add stream-ordered CP gradient return
// primitive", author's reply: a fail-closed validation boundary; section
// "Description": device guards on every tensor and self-alias assertions).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "cpthd.h"
#include "cpthd_internal.h"

namespace cpthd {
namespace {

struct Range {
  uintptr_t lo, hi;
};

// What the host knows of the metadata it built, by buffer address.  It only
// picks the permutation engine's tile shape: every kernel reads and validates
// the metadata itself on the device, so a stale record (a buffer rebuilt by
// other means, or memory reused) can cost speed but never change a result.
struct MetaRecord {
  int32_t policy, num_docs, cp_size;
  int64_t total_tokens;
  bool row_maps;
};
std::mutex g_records_mu;
std::unordered_map<const void*, MetaRecord> g_records;
constexpr size_t kMaxRecords = 4096;

void remember_meta(const void* meta, const MetaRecord& r) {
  std::lock_guard<std::mutex> lock(g_records_mu);
  if (g_records.size() >= kMaxRecords && g_records.find(meta) == g_records.end()) g_records.clear();
  g_records[meta] = r;
}

// Fill the hints of `a` (tile shape, and the shape the unit-tile kernels start
// their lookups from) from the record of `meta` when it matches
// the call's token count (and CP size, when the call has one).
void hint_from_record(const void* meta, int64_t total_tokens, int32_t cp_size, PermuteArgs* a) {
  a->hint_policy = -1;
  a->hint_docs = -1;
  a->hint_cp_size = 0;
  a->hint_local_tokens = 0;
  a->hint_row_maps = false;
  std::lock_guard<std::mutex> lock(g_records_mu);
  auto it = g_records.find(meta);
  if (it == g_records.end()) return;
  const MetaRecord& r = it->second;
  if (r.total_tokens != total_tokens || (cp_size > 0 && r.cp_size != cp_size)) return;
  a->hint_policy = r.policy;
  a->hint_docs = r.num_docs;
  a->hint_cp_size = r.cp_size;
  a->hint_local_tokens = r.total_tokens / r.cp_size;
  a->hint_row_maps = r.row_maps;
}

Range range_of(const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

// NULL, or not 16-byte aligned (the kernels read the header in one scalar load).
bool bad_meta_ptr(const void* meta) {
  return meta == nullptr || (reinterpret_cast<uintptr_t>(meta) & 15) != 0;
}

// Byte ranges of a metadata buffer for one call's checks.  The kernels write
// the 64-byte header (sticky call flags, the epoch wait's timeout mask), so it
// is an output of the call; the tables after it are only read, an input.  The
// tables' extent is known when the call names B and W (num_docs >= 0), or when
// the host built the metadata at this address for the call's token count (and
// CP size, when the call has one); otherwise the header alone is covered.
struct MetaSpan {
  int64_t bytes;  // extent checked against the allocation
  Range header;
  Range tables;   // empty when unknown
};

MetaSpan meta_span(const void* meta, int64_t total_tokens, int32_t cp_size, int32_t num_docs) {
  int64_t bytes = (int64_t)sizeof(cp_meta_header);
  if (num_docs >= 0 && cp_size > 0) {
    bytes = (int64_t)cp_meta_bytes(num_docs, cp_size);
  } else {
    std::lock_guard<std::mutex> lock(g_records_mu);
    auto it = g_records.find(meta);
    if (it != g_records.end() && it->second.total_tokens == total_tokens &&
        (cp_size <= 0 || it->second.cp_size == cp_size))
      bytes = (int64_t)(it->second.row_maps
                            ? cp_meta_bytes_row_maps(it->second.num_docs, it->second.cp_size, total_tokens)
                            : cp_meta_bytes(it->second.num_docs, it->second.cp_size));
  }
  if (bytes < (int64_t)sizeof(cp_meta_header)) bytes = (int64_t)sizeof(cp_meta_header);
  const uintptr_t a = reinterpret_cast<uintptr_t>(meta);
  return MetaSpan{bytes, Range{a, a + sizeof(cp_meta_header)}, Range{a + sizeof(cp_meta_header), a + (uintptr_t)bytes}};
}

bool overlap(const Range& a, const Range& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

// Every output against every input and every other output.
int check_alias(const std::vector<Range>& outs, const std::vector<Range>& ins) {
  for (size_t i = 0; i < outs.size(); ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return CP_ERR_ALIAS;
    for (size_t j = i + 1; j < outs.size(); ++j)
      if (overlap(outs[i], outs[j])) return CP_ERR_ALIAS;
  }
  return CP_OK;
}

int current_device(int* dev) {
  if (hipGetDevice(dev) != hipSuccess) {
    (void)hipGetLastError();
    return CP_ERR_HIP;
  }
  return CP_OK;
}

// [p, p + bytes) must be device memory of device `dev` (CP_ERR_DEVICE) and lie
// inside one allocation (CP_ERR_SHAPE: the buffer is smaller than the call's
// sizes say), so that no kernel can touch memory outside what the caller
// passed.  When the runtime cannot report the allocation's extent, the
// membership check alone applies.
//
// Buffers of one call often lie in one allocation (rank slices of one tensor,
// small tensors that the caching allocator put in one segment), and the two
// runtime lookups per buffer are most of a small call's host time; `cache`
// keeps the allocations already checked during the current call, so a buffer
// inside one of them is checked against its extent without a lookup.  A cache
// lives for one call only (an allocation can be freed between calls).
struct AllocCache {
  static constexpr int kCap = 16;
  uintptr_t base[kCap];
  uintptr_t end[kCap];
  int n = 0;
};

int check_device_buf(const void* p, int64_t bytes, int dev, AllocCache* cache) {
  if (p == nullptr) return CP_ERR_ARG;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if (cache != nullptr) {
    for (int i = 0; i < cache->n; ++i)
      if (a >= cache->base[i] && a < cache->end[i])
        return bytes >= 0 && (uint64_t)bytes <= cache->end[i] - a ? CP_OK : CP_ERR_SHAPE;
  }
  hipPointerAttribute_t attr;
  memset(&attr, 0, sizeof(attr));
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return CP_ERR_DEVICE;
  }
  if (attr.type != hipMemoryTypeDevice || attr.device != dev) return CP_ERR_DEVICE;
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
    (void)hipGetLastError();
    return CP_OK;
  }
  const uintptr_t end = reinterpret_cast<uintptr_t>(base) + size;
  if (a < reinterpret_cast<uintptr_t>(base) || bytes < 0 || (uint64_t)bytes > end - a) return CP_ERR_SHAPE;
  if (cache != nullptr && cache->n < AllocCache::kCap) {
    cache->base[cache->n] = reinterpret_cast<uintptr_t>(base);
    cache->end[cache->n] = end;
    ++cache->n;
  }
  return CP_OK;
}

// rows * row_bytes, or -1 when it would exceed 2^62 bytes.
int64_t checked_bytes(int64_t rows, int64_t row_bytes) {
  if (rows < 0 || row_bytes < 0) return -1;
  if (row_bytes != 0 && rows > (int64_t(1) << 62) / row_bytes) return -1;
  return rows * row_bytes;
}

bool valid_layout_dtype(int32_t dt) { return dt == CP_F32 || dt == CP_BF16 || dt == CP_F16; }
bool is_fp8(int32_t dt) { return dt == CP_FP8_E4M3 || dt == CP_FP8_E5M2; }

// (in, out) pairs of the gradient return and the slot sum.
int check_sum_dtypes(int32_t in, int32_t out) {
  if (is_fp8(in) || is_fp8(out)) return CP_ERR_UNSUPPORTED;
  if (in == CP_F32 && out == CP_F32) return CP_OK;
  if (in == CP_F32 && out == CP_BF16) return CP_OK;
  if (in == CP_BF16 && out == CP_BF16) return CP_OK;
  if (in == CP_BF16 && out == CP_F32) return CP_OK;
  if (valid_layout_dtype(in) && valid_layout_dtype(out)) return CP_ERR_UNSUPPORTED;
  return CP_ERR_ARG;
}

int hip_status(hipError_t e) { return e == hipSuccess ? CP_OK : CP_ERR_HIP; }

// A wait limit in device wall-clock ticks: wait_timeout_us <= 0 means 2 s;
// limits above one hour are held at one hour (no overflow in the conversion).
int64_t wait_ticks(int dev, int64_t wait_timeout_us) {
  int rate_khz = 0;
  if (hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || rate_khz <= 0) {
    (void)hipGetLastError();
    rate_khz = 100000;
  }
  int64_t us = wait_timeout_us > 0 ? wait_timeout_us : 2000000;
  if (us > int64_t(3600) * 1000000) us = int64_t(3600) * 1000000;
  return us * (int64_t)rate_khz / 1000;
}

// ---------------------------------------------------------------- timing hooks
struct ProfileRecord {
  std::string name;
  hipEvent_t start, stop;
};
std::mutex g_prof_mutex;
bool g_prof_enabled = false;
std::string g_prof_only;  // record only this kernel name ("" = every kernel)
std::vector<ProfileRecord> g_prof_records;
std::vector<hipEvent_t> g_prof_free;
std::string g_prof_pending_name;
hipEvent_t g_prof_pending_start = nullptr;
constexpr size_t kProfCapacity = 1 << 16;

hipEvent_t take_event() {
  if (!g_prof_free.empty()) {
    hipEvent_t e = g_prof_free.back();
    g_prof_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return e;
}


}  // namespace

void profile_before(const char* name, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_prof_mutex);
  if (!g_prof_enabled || g_prof_records.size() >= kProfCapacity) return;
  if (!g_prof_only.empty() && g_prof_only != name) return;
  hipEvent_t e = take_event();
  if (e == nullptr) return;
  if (hipEventRecord(e, stream) != hipSuccess) {
    (void)hipGetLastError();
    g_prof_free.push_back(e);
    return;
  }
  g_prof_pending_name = name;
  g_prof_pending_start = e;
}

void profile_after(hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_prof_mutex);
  if (g_prof_pending_start == nullptr) return;
  hipEvent_t e = take_event();
  if (e != nullptr && hipEventRecord(e, stream) == hipSuccess) {
    g_prof_records.push_back(ProfileRecord{g_prof_pending_name, g_prof_pending_start, e});
  } else {
    (void)hipGetLastError();
    g_prof_free.push_back(g_prof_pending_start);
    if (e != nullptr) g_prof_free.push_back(e);
  }
  g_prof_pending_start = nullptr;
}


}  // namespace cpthd

using namespace cpthd;

extern "C" {

size_t cp_meta_bytes(int32_t num_docs, int32_t cp_size) {
  if (num_docs < 0 || num_docs >= INT32_MAX || cp_size < 1 || cp_size > CP_MAX_CP_SIZE) return 0;
  return (size_t)meta_tables_bytes(num_docs, cp_size);
}

size_t cp_meta_bytes_row_maps(int32_t num_docs, int32_t cp_size, int64_t total_tokens) {
  const size_t tables = cp_meta_bytes(num_docs, cp_size);
  if (tables == 0 || total_tokens < 0 || total_tokens > INT32_MAX) return 0;
  return tables + (((size_t)total_tokens * 8 + 255) & ~(size_t)255);
}

int cp_build_meta(const int32_t* cu_seqlens, int32_t num_docs, int64_t total_tokens,
                  int32_t cp_size, int32_t policy, void* meta, size_t meta_bytes,
                  cp_stream_t stream) {
  if (cu_seqlens == nullptr || bad_meta_ptr(meta)) return CP_ERR_ARG;
  if (num_docs < 0 || num_docs >= INT32_MAX || cp_size < 1 || cp_size > CP_MAX_CP_SIZE) return CP_ERR_ARG;
  if (total_tokens < 0 || total_tokens > INT32_MAX) return CP_ERR_ARG;
  if (policy != CP_POLICY_DUAL_CHUNK_SWAP && policy != CP_POLICY_PACKED_CONTIGUOUS) return CP_ERR_ARG;
  if (policy == CP_POLICY_PACKED_CONTIGUOUS && total_tokens % cp_size != 0) return CP_ERR_SHAPE;
  if (meta_bytes < cp_meta_bytes(num_docs, cp_size)) return CP_ERR_SHAPE;
  // Row maps when the buffer holds them, under dual-chunk-swap (packed-
  // contiguous rows follow from arithmetic).
  const bool row_maps = policy == CP_POLICY_DUAL_CHUNK_SWAP && total_tokens > 0 &&
                        meta_bytes >= cp_meta_bytes_row_maps(num_docs, cp_size, total_tokens);
  const int64_t used = (int64_t)(row_maps ? cp_meta_bytes_row_maps(num_docs, cp_size, total_tokens)
                                          : cp_meta_bytes(num_docs, cp_size));
  int dev, st;
  if ((st = current_device(&dev)) != CP_OK) return st;
  AllocCache cache;
  if ((st = check_device_buf(cu_seqlens, 4 * ((int64_t)num_docs + 1), dev, &cache)) != CP_OK) return st;
  if ((st = check_device_buf(meta, used, dev, &cache)) != CP_OK) return st;
  if ((st = check_alias({range_of(meta, (int64_t)meta_bytes)},
                        {range_of(cu_seqlens, 4 * ((int64_t)num_docs + 1))})) != CP_OK)
    return st;
  if ((st = hip_status(launch_build_meta(cu_seqlens, num_docs, total_tokens, cp_size, policy, row_maps, meta,
                                         reinterpret_cast<hipStream_t>(stream)))) != CP_OK)
    return st;
  remember_meta(meta, MetaRecord{policy, num_docs, cp_size, total_tokens, row_maps});
  return CP_OK;
}

size_t cp_attn_meta_bytes(int32_t num_docs, int32_t cp_size) {
  if (num_docs < 0 || num_docs >= INT32_MAX || cp_size < 1 || cp_size > CP_MAX_CP_SIZE) return 0;
  const size_t bytes = 64 + 2 * (size_t)cp_size * (size_t)attn_record_bytes(num_docs);
  return (bytes + 255) & ~(size_t)255;
}

int cp_build_attn_meta(void* meta, int32_t num_docs, int32_t cp_size, void* attn,
                       size_t attn_bytes, cp_stream_t stream) {
  if (bad_meta_ptr(meta) || attn == nullptr) return CP_ERR_ARG;
  if (num_docs < 0 || num_docs >= INT32_MAX || cp_size < 1 || cp_size > CP_MAX_CP_SIZE) return CP_ERR_ARG;
  if (attn_bytes < cp_attn_meta_bytes(num_docs, cp_size)) return CP_ERR_SHAPE;
  int dev, st;
  if ((st = current_device(&dev)) != CP_OK) return st;
  AllocCache cache;
  const MetaSpan ms = meta_span(meta, -1, cp_size, num_docs);
  if ((st = check_device_buf(meta, ms.bytes, dev, &cache)) != CP_OK) return st;
  if ((st = check_device_buf(attn, (int64_t)cp_attn_meta_bytes(num_docs, cp_size), dev, &cache)) != CP_OK) return st;
  if ((st = check_alias({range_of(attn, (int64_t)attn_bytes), ms.header}, {ms.tables})) != CP_OK)
    return st;
  return hip_status(launch_build_attn_meta(static_cast<cp_meta_header*>(meta), num_docs, cp_size, attn,
                                           reinterpret_cast<hipStream_t>(stream)));
}

int cp_meta_status(const void* meta, cp_stream_t stream, int32_t* flags_out,
                   uint64_t* timeouts_out) {
  if (bad_meta_ptr(meta)) return CP_ERR_ARG;
  int dev, st;
  if ((st = current_device(&dev)) != CP_OK) return st;
  AllocCache cache;
  if ((st = check_device_buf(meta, (int64_t)sizeof(cp_meta_header), dev, &cache)) != CP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(s) != hipSuccess) {
    (void)hipGetLastError();
    return CP_ERR_HIP;
  }
  cp_meta_header h;
  if (hipMemcpy(&h, meta, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) {
    (void)hipGetLastError();
    return CP_ERR_HIP;
  }
  int32_t flags = h.flags;
  if (h.magic != CP_META_MAGIC) flags |= CP_CALL_BAD_MAGIC;
  if (flags_out) *flags_out = flags;
  if (timeouts_out) *timeouts_out = h.wait_timeout_ranks;
  if (flags != 0) return CP_ERR_META;
  if (h.wait_timeout_ranks != 0) return CP_ERR_TIMEOUT;
  return CP_OK;
}

static int layout_call(int32_t n_tensors, const void* const* ins, void* const* outs,
                       int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t dtype,
                       void* meta, cp_stream_t stream, bool to_local) {
  if (is_fp8(dtype)) return CP_ERR_UNSUPPORTED;
  if (!valid_layout_dtype(dtype)) return CP_ERR_ARG;
  if (n_tensors < 1 || n_tensors > kMaxLayoutTensors) return CP_ERR_ARG;
  if (total_tokens < 0 || total_tokens > INT32_MAX || heads < 1 || head_dim < 1) return CP_ERR_ARG;
  if (total_tokens == 0) return CP_OK;  // nothing to move; empty tensors may have NULL data
  if (ins == nullptr || outs == nullptr || bad_meta_ptr(meta)) return CP_ERR_ARG;
  for (int t = 0; t < n_tensors; ++t)
    if (ins[t] == nullptr || outs[t] == nullptr) return CP_ERR_ARG;
  const int64_t row_bytes = checked_bytes((int64_t)heads * head_dim, dtype_bytes(dtype));
  const int64_t bytes = checked_bytes(total_tokens, row_bytes);
  if (row_bytes < 0 || bytes < 0) return CP_ERR_ARG;
  int dev, st;
  if ((st = current_device(&dev)) != CP_OK) return st;
  AllocCache cache;
  const MetaSpan ms = meta_span(meta, total_tokens, -1, -1);
  if ((st = check_device_buf(meta, ms.bytes, dev, &cache)) != CP_OK) return st;
  std::vector<Range> in_ranges{ms.tables}, out_ranges{ms.header};
  for (int t = 0; t < n_tensors; ++t) {
    if ((st = check_device_buf(ins[t], bytes, dev, &cache)) != CP_OK) return st;
    if ((st = check_device_buf(outs[t], bytes, dev, &cache)) != CP_OK) return st;
    in_ranges.push_back(range_of(ins[t], bytes));
    out_ranges.push_back(range_of(outs[t], bytes));
  }
  if ((st = check_alias(out_ranges, in_ranges)) != CP_OK) return st;
  PermuteArgs a;
  memset(&a, 0, sizeof(a));
  a.meta = static_cast<cp_meta_header*>(meta);
  a.n_tensors = n_tensors;
  for (int t = 0; t < n_tensors; ++t) {
    a.global[t] = static_cast<char*>(to_local ? const_cast<void*>(ins[t]) : outs[t]);
    a.local[t] = static_cast<char*>(to_local ? outs[t] : const_cast<void*>(ins[t]));
  }
  a.local_table = false;
  a.to_local = to_local;
  a.total_tokens = total_tokens;
  a.row_bytes = row_bytes;
  a.expect_cp_size = -1;
  a.expect_policy = -1;
  hint_from_record(meta, total_tokens, -1, &a);
  return hip_status(launch_permute(a, reinterpret_cast<hipStream_t>(stream)));
}

int cp_partition_thd(const void* x, void* parts, int64_t total_tokens, int32_t heads,
                     int32_t head_dim, int32_t dtype, void* meta, cp_stream_t stream) {
  return layout_call(1, &x, &parts, total_tokens, heads, head_dim, dtype, meta, stream, true);
}

int cp_gather_thd(const void* parts, void* x, int64_t total_tokens, int32_t heads,
                  int32_t head_dim, int32_t dtype, void* meta, cp_stream_t stream) {
  return layout_call(1, &parts, &x, total_tokens, heads, head_dim, dtype, meta, stream, false);
}

int cp_partition_thd_multi(int32_t n_tensors, const void* const* xs, void* const* parts,
                           int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t dtype,
                           void* meta, cp_stream_t stream) {
  return layout_call(n_tensors, xs, parts, total_tokens, heads, head_dim, dtype, meta, stream, true);
}

int cp_gather_thd_multi(int32_t n_tensors, const void* const* parts, void* const* xs,
                        int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t dtype,
                        void* meta, cp_stream_t stream) {
  return layout_call(n_tensors, parts, xs, total_tokens, heads, head_dim, dtype, meta, stream, false);
}

// Common scalar checks of the gradient-return family.
static int grad_scalar_checks(int32_t rank, int32_t cp_size, int32_t n_tensors, int64_t total_tokens,
                              int32_t heads, int32_t head_dim, int32_t in_dtype, int32_t out_dtype,
                              const void* meta) {
  int st;
  if ((st = check_sum_dtypes(in_dtype, out_dtype)) != CP_OK) return st;
  if (cp_size < 1 || cp_size > CP_MAX_CP_SIZE) return CP_ERR_ARG;
  if (rank != CP_ALL_RANKS && (rank < 0 || rank >= cp_size)) return CP_ERR_ARG;
  if (n_tensors < 1) return CP_ERR_ARG;
  if (total_tokens < 0 || total_tokens > INT32_MAX || heads < 1 || head_dim < 1) return CP_ERR_ARG;
  // T % W under either policy; dual-chunk-swap metadata also guarantees T % 2W
  // (every document is a multiple of 2W), which the kernels check on the device.
  if (total_tokens % (int64_t)cp_size != 0) return CP_ERR_SHAPE;
  if (total_tokens > 0 && bad_meta_ptr(meta)) return CP_ERR_ARG;
  // every buffer size fits comfortably in 64 bits
  const int64_t row_elems = (int64_t)heads * head_dim;
  if (checked_bytes(total_tokens, checked_bytes(row_elems, 4)) < 0) return CP_ERR_ARG;
  return CP_OK;
}

// The launches of the gradient return after validation: scatter (writers of
// this call into every owner's slot), epoch publish and wait, owner sums.
// rank < 0: every rank in stream order.  out[t][o] and grads[t][w] are
// flattened host tables as in cp_grad_return; S(t, o, w) gives the device
// address of slot [t][o][w].
extern "C++" {
template <typename SlotFn>
static int grad_return_launches(int rank, int W, int n_tensors, const void* const* grads,
                                 SlotFn S, void* const* out, int64_t total_tokens,
                                 int64_t in_row, int64_t row_elems, int32_t in_dtype, int32_t out_dtype,
                                 cp_meta_header* h, uint32_t* epochs, uint32_t epoch, int64_t ticks,
                                 int32_t phases, hipStream_t s) {
  const bool all = rank < 0;
  const int64_t n = total_tokens / W;
  const int w_lo = all ? 0 : rank, w_hi = all ? W : rank + 1;  // writers this call acts for
  const int o_lo = w_lo, o_hi = w_hi;                           // owners this call sums for
  auto G = [&](int t, int w) { return grads[(size_t)t * W + w]; };
  auto O = [&](int t, int o) { return out[(size_t)t * W + o]; };
  int st;
  // 1. scatter: writer w's global gradient -> slot [o][w] of every owner o
  for (int t = 0; t < n_tensors && (phases & CP_PHASE_SCATTER); ++t) {
    for (int w = w_lo; w < w_hi; ++w) {
      PermuteArgs a;
      memset(&a, 0, sizeof(a));
      a.meta = h;
      a.n_tensors = 1;
      a.global[0] = static_cast<char*>(const_cast<void*>(G(t, w)));
      for (int o = 0; o < W; ++o) a.table.p[o] = static_cast<char*>(S(t, o, w));
      a.local_table = true;
      a.to_local = true;
      a.total_tokens = total_tokens;
      a.row_bytes = in_row;
      a.expect_cp_size = W;
      a.expect_policy = -1;  // the owner's rows follow the metadata's policy
      hint_from_record(h, total_tokens, W, &a);
      if ((st = hip_status(launch_permute(a, s))) != CP_OK) return st;
    }
  }
  // 2-3. publish this call's writer epochs, wait for this call's owners
  if (epochs && (phases & (CP_PHASE_PUBLISH | CP_PHASE_WAIT))) {
    if ((phases & CP_PHASE_PUBLISH) &&
        (st = hip_status(launch_epoch_publish(epochs, W, all ? -1 : rank, epoch, s))) != CP_OK)
      return st;
    if ((phases & CP_PHASE_WAIT) &&
        (st = hip_status(launch_epoch_wait(epochs, W, all ? -1 : rank, epoch, ticks, h, s))) != CP_OK)
      return st;
  }
  // 4. owner o: out = slot 0 + slot 1 + ... + slot W-1 (after out itself when accumulating)
  for (int t = 0; t < n_tensors && (phases & CP_PHASE_SUM); ++t) {
    for (int o = o_lo; o < o_hi; ++o) {
      SlotSumArgs a;
      memset(&a, 0, sizeof(a));
      for (int w = 0; w < W; ++w) a.in.p[w] = static_cast<const char*>(S(t, o, w));
      a.out = static_cast<char*>(O(t, o));
      a.num_slots = W;
      a.n_elems = n * row_elems;
      a.in_dtype = in_dtype;
      a.out_dtype = out_dtype;
      a.gate_meta = h;
      a.gate_T = total_tokens;
      a.owner = epochs ? o : -1;
      a.accumulate = (phases & CP_SUM_ACCUMULATE) != 0;
      if ((st = hip_status(launch_slot_sum(a, s))) != CP_OK) return st;
    }
  }
  return CP_OK;
}
}  // extern "C++"

int cp_grad_return(int32_t rank, int32_t cp_size, int32_t n_tensors, const void* const* grads,
                   void* const* slots, void* const* out, int64_t total_tokens, int32_t heads,
                   int32_t head_dim, int32_t in_dtype, int32_t out_dtype, void* meta,
                   uint32_t* epochs, uint32_t epoch, int64_t wait_timeout_us,
                   int32_t phases, cp_stream_t stream) {
  int st;
  if ((st = grad_scalar_checks(rank, cp_size, n_tensors, total_tokens, heads, head_dim, in_dtype,
                               out_dtype, meta)) != CP_OK)
    return st;
  if ((phases & CP_PHASE_ALL) == 0 || (phases & ~(CP_PHASE_ALL | CP_SUM_ACCUMULATE)) != 0) return CP_ERR_ARG;
  const bool all = rank == CP_ALL_RANKS;
  if (!all && epochs == nullptr) return CP_ERR_ARG;
  if (total_tokens == 0) return CP_OK;  // nothing to move; empty tensors may have NULL data
  if (grads == nullptr || slots == nullptr || out == nullptr) return CP_ERR_ARG;
  const int W = cp_size;
  const int64_t n = total_tokens / W;
  const int64_t row_elems = (int64_t)heads * head_dim;
  const int64_t in_row = row_elems * dtype_bytes(in_dtype);
  const int64_t out_row = row_elems * dtype_bytes(out_dtype);
  auto G = [&](int t, int w) { return grads[(size_t)t * W + w]; };
  auto S = [&](int t, int o, int w) { return slots[((size_t)t * W + o) * W + w]; };
  auto O = [&](int t, int o) { return out[(size_t)t * W + o]; };
  const int w_lo = all ? 0 : rank, w_hi = all ? W : rank + 1;  // writers this call acts for
  const int o_lo = w_lo, o_hi = w_hi;                           // owners this call sums for

  // NULL checks on every table entry this call touches.
  for (int t = 0; t < n_tensors; ++t) {
    for (int w = w_lo; w < w_hi; ++w) {
      if (G(t, w) == nullptr) return CP_ERR_ARG;
      for (int o = 0; o < W; ++o)
        if (S(t, o, w) == nullptr) return CP_ERR_ARG;
    }
    for (int o = o_lo; o < o_hi; ++o) {
      if (O(t, o) == nullptr) return CP_ERR_ARG;
      for (int w = 0; w < W; ++w)
        if (S(t, o, w) == nullptr) return CP_ERR_ARG;
    }
  }
  int dev;
  if ((st = current_device(&dev)) != CP_OK) return st;
  AllocCache cache;
  const MetaSpan ms = meta_span(meta, total_tokens, W, -1);
  if ((st = check_device_buf(meta, ms.bytes, dev, &cache)) != CP_OK) return st;
  if (epochs && (st = check_device_buf(epochs, 4 * (int64_t)W * W, dev, &cache)) != CP_OK) return st;
  std::vector<Range> ins{ms.tables}, outs{ms.header};
  for (int t = 0; t < n_tensors; ++t) {
    for (int w = w_lo; w < w_hi; ++w) {
      if ((st = check_device_buf(G(t, w), total_tokens * in_row, dev, &cache)) != CP_OK) return st;
      ins.push_back(range_of(G(t, w), total_tokens * in_row));
      for (int o = 0; o < W; ++o) {
        if ((st = check_device_buf(S(t, o, w), n * in_row, dev, &cache)) != CP_OK) return st;
        outs.push_back(range_of(S(t, o, w), n * in_row));
      }
    }
    for (int o = o_lo; o < o_hi; ++o) {
      if ((st = check_device_buf(O(t, o), n * out_row, dev, &cache)) != CP_OK) return st;
      outs.push_back(range_of(O(t, o), n * out_row));
      for (int w = 0; w < W; ++w) {
        if (w >= w_lo && w < w_hi) continue;  // already listed as an output of this call
        if ((st = check_device_buf(S(t, o, w), n * in_row, dev, &cache)) != CP_OK) return st;
        ins.push_back(range_of(S(t, o, w), n * in_row));
      }
    }
  }
  if (epochs) {
    outs.push_back(range_of(epochs, 4 * (int64_t)W * W));
  }
  if ((st = check_alias(outs, ins)) != CP_OK) return st;

  return grad_return_launches(all ? -1 : rank, W, n_tensors, grads, S, out, total_tokens, in_row,
                              row_elems, in_dtype, out_dtype, static_cast<cp_meta_header*>(meta), epochs, epoch,
                              epochs && (phases & (CP_PHASE_PUBLISH | CP_PHASE_WAIT)) ? wait_ticks(dev, wait_timeout_us) : 0,
                              phases, reinterpret_cast<hipStream_t>(stream));
}

int cp_grad_return_noalloc(int32_t cp_size, int32_t n_tensors, const void* const* grads,
                           void* const* out, int64_t total_tokens, int32_t heads, int32_t head_dim,
                           int32_t in_dtype, int32_t out_dtype, void* meta, int32_t flags,
                           cp_stream_t stream) {
  int st;
  if ((st = grad_scalar_checks(CP_ALL_RANKS, cp_size, n_tensors, total_tokens, heads, head_dim, in_dtype,
                               out_dtype, meta)) != CP_OK)
    return st;
  if ((flags & ~CP_SUM_ACCUMULATE) != 0) return CP_ERR_ARG;
  if (total_tokens == 0) return CP_OK;  // nothing to move; empty tensors may have NULL data
  if (grads == nullptr || out == nullptr) return CP_ERR_ARG;
  const int W = cp_size;
  const int64_t n = total_tokens / W;
  const int64_t row_elems = (int64_t)heads * head_dim;
  const int64_t in_row = row_elems * dtype_bytes(in_dtype);
  const int64_t out_row = row_elems * dtype_bytes(out_dtype);
  // Slot [t][o][w] at ((t W + o) W + w) * stride in the static workspace; every
  // slot starts 256-byte aligned.  Sizes beyond the workspace are refused.
  const int64_t slot_bytes = checked_bytes(n, in_row);
  if (slot_bytes < 0 || slot_bytes > kNoallocScratchBytes) return CP_ERR_TOO_LARGE;
  const int64_t stride = (slot_bytes + 255) / 256 * 256;
  const int64_t slots_per_tensor = (int64_t)W * W;
  if ((int64_t)n_tensors > kNoallocScratchBytes / (slots_per_tensor * stride)) return CP_ERR_TOO_LARGE;
  for (int t = 0; t < n_tensors; ++t)
    for (int w = 0; w < W; ++w)
      if (grads[(size_t)t * W + w] == nullptr || out[(size_t)t * W + w] == nullptr) return CP_ERR_ARG;
  int dev;
  if ((st = current_device(&dev)) != CP_OK) return st;
  AllocCache cache;
  const MetaSpan ms = meta_span(meta, total_tokens, W, -1);
  if ((st = check_device_buf(meta, ms.bytes, dev, &cache)) != CP_OK) return st;
  std::vector<Range> ins{ms.tables}, outs{ms.header};
  for (int t = 0; t < n_tensors; ++t) {
    for (int w = 0; w < W; ++w) {
      const void* g = grads[(size_t)t * W + w];
      if ((st = check_device_buf(g, total_tokens * in_row, dev, &cache)) != CP_OK) return st;
      ins.push_back(range_of(g, total_tokens * in_row));
      void* p = out[(size_t)t * W + w];
      if ((st = check_device_buf(p, n * out_row, dev, &cache)) != CP_OK) return st;
      outs.push_back(range_of(p, n * out_row));
    }
  }
  if ((st = check_alias(outs, ins)) != CP_OK) return st;
  // The workspace's device address on this device (never the host-side name).
  void* base = nullptr;
  if ((st = hip_status(noalloc_scratch(&base))) != CP_OK) return st;
  char* const ws = static_cast<char*>(base);
  auto S = [&](int t, int o, int w) -> void* {
    return ws + (((int64_t)t * W + o) * W + w) * stride;
  };
  return grad_return_launches(-1, W, n_tensors, grads, S, out, total_tokens, in_row, row_elems, in_dtype,
                              out_dtype, static_cast<cp_meta_header*>(meta), nullptr, 0, 0,
                              CP_PHASE_SCATTER | CP_PHASE_SUM | (flags & CP_SUM_ACCUMULATE),
                              reinterpret_cast<hipStream_t>(stream));
}

int cp_grad_return_fused(int32_t rank, int32_t cp_size, int32_t n_tensors,
                         const void* const* grads, void* const* out, int64_t total_tokens,
                         int32_t heads, int32_t head_dim, int32_t in_dtype, int32_t out_dtype,
                         void* meta, int32_t flags, cp_stream_t stream) {
  int st;
  if ((st = grad_scalar_checks(rank, cp_size, n_tensors, total_tokens, heads, head_dim, in_dtype,
                               out_dtype, meta)) != CP_OK)
    return st;
  if ((flags & ~CP_SUM_ACCUMULATE) != 0) return CP_ERR_ARG;
  if (total_tokens == 0) return CP_OK;  // nothing to move; empty tensors may have NULL data
  if (grads == nullptr || out == nullptr) return CP_ERR_ARG;
  const int W = cp_size;
  const bool all = rank == CP_ALL_RANKS;
  const int o_lo = all ? 0 : rank, o_hi = all ? W : rank + 1;
  const int64_t n = total_tokens / W;
  const int64_t row_elems = (int64_t)heads * head_dim;
  const int64_t in_row = row_elems * dtype_bytes(in_dtype);
  const int64_t out_row = row_elems * dtype_bytes(out_dtype);
  for (int t = 0; t < n_tensors; ++t) {
    for (int w = 0; w < W; ++w)
      if (grads[(size_t)t * W + w] == nullptr) return CP_ERR_ARG;
    for (int o = o_lo; o < o_hi; ++o)
      if (out[(size_t)t * W + o] == nullptr) return CP_ERR_ARG;
  }
  int dev;
  if ((st = current_device(&dev)) != CP_OK) return st;
  AllocCache cache;
  const MetaSpan ms = meta_span(meta, total_tokens, W, -1);
  if ((st = check_device_buf(meta, ms.bytes, dev, &cache)) != CP_OK) return st;
  std::vector<Range> ins{ms.tables}, outs{ms.header};
  for (int t = 0; t < n_tensors; ++t) {
    for (int w = 0; w < W; ++w) {
      const void* g = grads[(size_t)t * W + w];
      if ((st = check_device_buf(g, total_tokens * in_row, dev, &cache)) != CP_OK) return st;
      ins.push_back(range_of(g, total_tokens * in_row));
    }
    for (int o = o_lo; o < o_hi; ++o) {
      void* p = out[(size_t)t * W + o];
      if ((st = check_device_buf(p, n * out_row, dev, &cache)) != CP_OK) return st;
      outs.push_back(range_of(p, n * out_row));
    }
  }
  if ((st = check_alias(outs, ins)) != CP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (int t = 0; t < n_tensors; ++t) {
    FusedArgs a;
    memset(&a, 0, sizeof(a));
    a.meta = static_cast<cp_meta_header*>(meta);
    for (int w = 0; w < W; ++w) a.grads.p[w] = static_cast<const char*>(grads[(size_t)t * W + w]);
    for (int o = o_lo; o < o_hi; ++o) a.out.p[o] = static_cast<char*>(out[(size_t)t * W + o]);
    a.cp_size = W;
    a.owner_begin = o_lo;
    a.owner_end = o_hi;
    a.total_tokens = total_tokens;
    a.row_elems = row_elems;
    a.in_dtype = in_dtype;
    a.out_dtype = out_dtype;
    a.accumulate = (flags & CP_SUM_ACCUMULATE) != 0;
    if ((st = hip_status(launch_fused(a, s))) != CP_OK) return st;
  }
  return CP_OK;
}

int cp_slot_sum(int32_t num_slots, const void* const* slots, void* out, int64_t n_elems,
                int32_t in_dtype, int32_t out_dtype, int32_t flags, cp_stream_t stream) {
  int st;
  if ((st = check_sum_dtypes(in_dtype, out_dtype)) != CP_OK) return st;
  if (num_slots < 1 || num_slots > CP_MAX_CP_SIZE || n_elems < 0) return CP_ERR_ARG;
  if (checked_bytes(n_elems, 4) < 0) return CP_ERR_ARG;
  if ((flags & ~CP_SUM_ACCUMULATE) != 0) return CP_ERR_ARG;
  if (n_elems == 0) return CP_OK;
  if (slots == nullptr || out == nullptr) return CP_ERR_ARG;
  for (int w = 0; w < num_slots; ++w)
    if (slots[w] == nullptr) return CP_ERR_ARG;
  int dev;
  if ((st = current_device(&dev)) != CP_OK) return st;
  AllocCache cache;
  std::vector<Range> ins;
  for (int w = 0; w < num_slots; ++w) {
    if ((st = check_device_buf(slots[w], n_elems * dtype_bytes(in_dtype), dev, &cache)) != CP_OK) return st;
    ins.push_back(range_of(slots[w], n_elems * dtype_bytes(in_dtype)));
  }
  if ((st = check_device_buf(out, n_elems * dtype_bytes(out_dtype), dev, &cache)) != CP_OK) return st;
  if ((st = check_alias({range_of(out, n_elems * dtype_bytes(out_dtype))}, ins)) != CP_OK) return st;
  SlotSumArgs a;
  memset(&a, 0, sizeof(a));
  for (int w = 0; w < num_slots; ++w) a.in.p[w] = static_cast<const char*>(slots[w]);
  a.out = static_cast<char*>(out);
  a.num_slots = num_slots;
  a.n_elems = n_elems;
  a.in_dtype = in_dtype;
  a.out_dtype = out_dtype;
  a.gate_meta = nullptr;
  a.owner = -1;
  a.accumulate = (flags & CP_SUM_ACCUMULATE) != 0;
  return hip_status(launch_slot_sum(a, reinterpret_cast<hipStream_t>(stream)));
}

int cp_allreduce(int32_t algo, int32_t cp_size, const void* const* in, void* const* out,
                 int64_t n_elems, int32_t dtype, cp_stream_t stream) {
  if (algo != CP_ALLREDUCE_ONE_SHOT && algo != CP_ALLREDUCE_RING && algo != CP_ALLREDUCE_TWO_SHOT)
    return CP_ERR_ARG;
  if (is_fp8(dtype) || dtype == CP_F16) return CP_ERR_UNSUPPORTED;
  if (dtype != CP_F32 && dtype != CP_BF16) return CP_ERR_ARG;
  if (cp_size < 1 || cp_size > CP_MAX_CP_SIZE || n_elems < 0) return CP_ERR_ARG;
  const int64_t bytes = checked_bytes(n_elems, dtype_bytes(dtype));
  if (bytes < 0) return CP_ERR_ARG;
  if (n_elems == 0) return CP_OK;
  if (in == nullptr || out == nullptr) return CP_ERR_ARG;
  for (int r = 0; r < cp_size; ++r)
    if (in[r] == nullptr || out[r] == nullptr) return CP_ERR_ARG;
  int dev, st;
  if ((st = current_device(&dev)) != CP_OK) return st;
  AllocCache cache;
  std::vector<Range> ins, outs;
  for (int r = 0; r < cp_size; ++r) {
    if ((st = check_device_buf(in[r], bytes, dev, &cache)) != CP_OK) return st;
    if ((st = check_device_buf(out[r], bytes, dev, &cache)) != CP_OK) return st;
    ins.push_back(range_of(in[r], bytes));
    outs.push_back(range_of(out[r], bytes));
  }
  if ((st = check_alias(outs, ins)) != CP_OK) return st;
  AllreduceArgs a;
  memset(&a, 0, sizeof(a));
  for (int r = 0; r < cp_size; ++r) {
    a.in.p[r] = static_cast<const char*>(in[r]);
    a.out.p[r] = static_cast<char*>(out[r]);
  }
  a.cp_size = cp_size;
  a.n_elems = n_elems;
  a.dtype = dtype;
  a.chunk = (n_elems + cp_size - 1) / cp_size;  // the ring's chunks: ceil(n / W) elements
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (algo == CP_ALLREDUCE_ONE_SHOT) return hip_status(launch_allreduce_one_shot(a, s));
  if (algo == CP_ALLREDUCE_TWO_SHOT) return hip_status(launch_allreduce_two_shot(a, s));
  if (cp_size == 1) return hip_status(launch_ring_gather_step(a, 0, true, s));
  for (int step = 0; step < cp_size - 1; ++step)
    if ((st = hip_status(launch_ring_reduce_step(a, step, s))) != CP_OK) return st;
  for (int step = 0; step < cp_size - 1; ++step)
    if ((st = hip_status(launch_ring_gather_step(a, step, false, s))) != CP_OK) return st;
  return CP_OK;
}

size_t cp_allreduce_signal_bytes(int32_t cp_size) {
  if (cp_size < 1 || cp_size > CP_MAX_CP_SIZE) return 0;
  const size_t bytes = 8 * (size_t)signal_words(cp_size);
  return (bytes + 255) & ~(size_t)255;
}

int cp_allreduce_signal(int32_t cp_size, const void* const* in, void* const* out, int64_t n_elems,
                        int32_t dtype, void* signals, size_t signals_bytes, uint64_t epoch,
                        int64_t wait_timeout_us, cp_stream_t stream) {
  if (is_fp8(dtype) || dtype == CP_F16) return CP_ERR_UNSUPPORTED;
  if (dtype != CP_F32 && dtype != CP_BF16) return CP_ERR_ARG;
  if (cp_size < 1 || cp_size > CP_MAX_CP_SIZE || n_elems < 0) return CP_ERR_ARG;
  if (epoch == 0 || epoch >= (uint64_t(1) << 55)) return CP_ERR_ARG;
  const int64_t bytes = checked_bytes(n_elems, dtype_bytes(dtype));
  if (bytes < 0) return CP_ERR_ARG;
  if (n_elems == 0) return CP_OK;
  if (in == nullptr || out == nullptr || signals == nullptr) return CP_ERR_ARG;
  for (int r = 0; r < cp_size; ++r)
    if (in[r] == nullptr || out[r] == nullptr) return CP_ERR_ARG;
  const size_t sig_bytes = cp_allreduce_signal_bytes(cp_size);
  if (signals_bytes < sig_bytes) return CP_ERR_SHAPE;
  int dev, st;
  if ((st = current_device(&dev)) != CP_OK) return st;
  AllocCache cache;
  std::vector<Range> ins, outs;
  for (int r = 0; r < cp_size; ++r) {
    if ((st = check_device_buf(in[r], bytes, dev, &cache)) != CP_OK) return st;
    if ((st = check_device_buf(out[r], bytes, dev, &cache)) != CP_OK) return st;
    ins.push_back(range_of(in[r], bytes));
    outs.push_back(range_of(out[r], bytes));
  }
  if ((st = check_device_buf(signals, (int64_t)sig_bytes, dev, &cache)) != CP_OK) return st;
  outs.push_back(range_of(signals, (int64_t)sig_bytes));
  if ((st = check_alias(outs, ins)) != CP_OK) return st;
  AllreduceArgs a;
  memset(&a, 0, sizeof(a));
  for (int r = 0; r < cp_size; ++r) {
    a.in.p[r] = static_cast<const char*>(in[r]);
    a.out.p[r] = static_cast<char*>(out[r]);
  }
  a.cp_size = cp_size;
  a.n_elems = n_elems;
  a.dtype = dtype;
  a.chunk = (n_elems + cp_size - 1) / cp_size;  // the ring's chunks: ceil(n / W) elements
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (cp_size == 1) return hip_status(launch_ring_gather_step(a, 0, true, s));
  RingSignalArgs g;
  memset(&g, 0, sizeof(g));
  const int tiles = ring_signal_tiles(a, &g.tile_elems);
  if (tiles < 1) return CP_ERR_UNSUPPORTED;  // not even one workgroup per rank can be resident
  g.signals = static_cast<uint64_t*>(signals);
  g.epoch = epoch;
  g.timeout_ticks = wait_ticks(dev, wait_timeout_us);
  return hip_status(launch_ring_signal(a, g, tiles, s));
}

int cp_allreduce_signal_status(const void* signals, int32_t cp_size, uint64_t epoch, cp_stream_t stream) {
  if (signals == nullptr || cp_size < 1 || cp_size > CP_MAX_CP_SIZE || epoch == 0) return CP_ERR_ARG;
  int dev, st;
  if ((st = current_device(&dev)) != CP_OK) return st;
  AllocCache cache;
  if ((st = check_device_buf(signals, (int64_t)cp_allreduce_signal_bytes(cp_size), dev, &cache)) != CP_OK)
    return st;
  if (hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream)) != hipSuccess) {
    (void)hipGetLastError();
    return CP_ERR_HIP;
  }
  uint64_t words[2] = {0, 0};
  if (hipMemcpy(words, signals, sizeof(words), hipMemcpyDeviceToHost) != hipSuccess) {
    (void)hipGetLastError();
    return CP_ERR_HIP;
  }
  if (words[1] >= epoch) return CP_ERR_ARG;
  if (words[0] >= epoch) return CP_ERR_TIMEOUT;
  return CP_OK;
}

const char* cp_status_string(int status) {
  switch (status) {
    case CP_OK: return "ok";
    case CP_ERR_ARG: return "invalid argument";
    case CP_ERR_UNSUPPORTED: return "unsupported dtype or mode";
    case CP_ERR_SHAPE: return "inconsistent sizes";
    case CP_ERR_DEVICE: return "pointer is not device memory of the current device";
    case CP_ERR_ALIAS: return "output overlaps an input or another output";
    case CP_ERR_HIP: return "HIP runtime error";
    case CP_ERR_TIMEOUT: return "epoch wait timed out";
    case CP_ERR_META: return "invalid metadata or call/metadata mismatch";
    case CP_ERR_TOO_LARGE: return "the call needs more than the static workspace holds";
    default: return "unknown status";
  }
}

int cp_version(void) { return 300; }

int cp_profile_enable(int enable) {
  std::lock_guard<std::mutex> lock(g_prof_mutex);
  g_prof_enabled = enable != 0;
  return CP_OK;
}

int cp_profile_select(const char* name) {
  if (name != nullptr && strnlen(name, 128) > 127) return CP_ERR_ARG;
  std::lock_guard<std::mutex> lock(g_prof_mutex);
  g_prof_only = name != nullptr ? name : "";
  return CP_OK;
}

int cp_profile_read(char* names, int64_t* counts, double* total_ms, int capacity) {
  std::vector<ProfileRecord> recs;
  {
    std::lock_guard<std::mutex> lock(g_prof_mutex);
    recs.swap(g_prof_records);
  }
  std::vector<std::string> order;
  std::map<std::string, std::pair<int64_t, double>> agg;
  int status = CP_OK;
  for (ProfileRecord& r : recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
      (void)hipGetLastError();
      status = CP_ERR_HIP;
    }
    if (agg.find(r.name) == agg.end()) order.push_back(r.name);
    auto& slot = agg[r.name];
    slot.first += 1;
    slot.second += ms;
  }
  {
    std::lock_guard<std::mutex> lock(g_prof_mutex);
    for (ProfileRecord& r : recs) {
      g_prof_free.push_back(r.start);
      g_prof_free.push_back(r.stop);
    }
  }
  if (status != CP_OK) return -status;
  int k = 0;
  for (const std::string& nm : order) {
    if (k >= capacity) break;
    if (names) {
      strncpy(names + (size_t)k * 128, nm.c_str(), 127);
      names[(size_t)k * 128 + 127] = '\0';
    }
    if (counts) counts[k] = agg[nm].first;
    if (total_ms) total_ms[k] = agg[nm].second;
    ++k;
  }
  return (int)order.size();
}

}  // extern "C"
