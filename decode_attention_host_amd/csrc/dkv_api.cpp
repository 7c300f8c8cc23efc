// dkv_api.cpp - the C ABI of libdkv: argument validation, plan cache, pinned
// host allocation, bandwidth probe and kernel launches.
//
// Validation happens on the host before anything is enqueued; a failing call
// launches nothing and leaves its message in dkv_last_error().
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <list>
#include <memory>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "dkv.h"
#include "dkv_internal.h"

namespace {

thread_local std::string g_last_error;

dkv_status set_err(dkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

dkv_status ok() {
  g_last_error.clear();
  return DKV_OK;
}

dkv_status hip_err(hipError_t e, const char* what) {
  return set_err(DKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

// The thread's last-error message, shared with the other translation units.
dkv_status dkv::error(dkv_status st, const char* msg) { return set_err(st, "%s", msg); }
dkv_status dkv::success() { return ok(); }

namespace {

constexpr int kMaxCopyDevices = 64;

bool debug_validate() {
  static const bool on = [] {
    const char* v = getenv("DKV_DEBUG_VALIDATE");
    return v && v[0] && v[0] != '0';
  }();
  return on;
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int64_t x) {
  int s = 0;
  while ((int64_t(1) << s) < x) ++s;
  return s;
}

// ---------------------------------------------------------------- tuning
std::mutex g_tune_mu;
dkv_tuning g_tune{};
uint64_t g_tune_gen = 1;

dkv_tuning tuning_snapshot(uint64_t* gen) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  if (gen) *gen = g_tune_gen;
  return g_tune;
}

int device_cus(int* dev_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  if (dev_out) *dev_out = dev;
  return cus;
}

// ---------------------------------------------------------------- plan cache
// A prefill plan: its device image in pinned host memory, the source of every
// upload.  The image is freed with the last reference; uploads from it may
// still be queued then, so the device is synchronised first (this happens
// only on eviction, never on a cache hit).
struct PlanEntry {
  dkv::PlanLayout lay;
  void* pinned = nullptr;
  size_t bytes = 0;
  bool captured = false;   // referenced by a captured graph: never evicted
  PlanEntry() = default;
  PlanEntry(const PlanEntry&) = delete;
  PlanEntry& operator=(const PlanEntry&) = delete;
  ~PlanEntry() {
    if (pinned) {
      (void)hipDeviceSynchronize();
      (void)hipHostFree(pinned);
    }
  }
};

// True while `s` is capturing a graph (its work is recorded, not run).
bool stream_capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) return false;
  return st == hipStreamCaptureStatusActive;
}

struct PlanCache {
  std::mutex mu;
  std::list<std::string> lru;
  std::unordered_map<std::string, std::pair<std::shared_ptr<PlanEntry>, std::list<std::string>::iterator>>
      map;
  static constexpr size_t kCap = 64;
};

PlanCache& cache() {
  static PlanCache* c = new PlanCache();  // never destroyed: entries may be in flight at exit
  return *c;
}

template <class T>
void put(std::string& k, const T& v) {
  k.append(reinterpret_cast<const char*>(&v), sizeof(T));
}

uint64_t fnv1a(const void* data, size_t n, uint64_t h = 1469598103934665603ull) {
  const uint8_t* p = static_cast<const uint8_t*>(data);
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 1099511628211ull;
  }
  return h;
}

dkv_status validate_desc(const dkv_kv_desc* kv) {
  if (!kv) return set_err(DKV_ERR_INVALID, "kv descriptor is NULL");
  if (kv->num_kv_heads < 1) return set_err(DKV_ERR_INVALID, "num_kv_heads must be >= 1");
  if (kv->head_dim != 64 && kv->head_dim != 128)
    return set_err(DKV_ERR_UNSUPPORTED, "head_dim %d not built (64 or 128)", kv->head_dim);
  if (kv->page_size < 0 || (kv->page_size > 0 && (!is_pow2(kv->page_size) || kv->page_size > 1024)))
    return set_err(DKV_ERR_INVALID, "page_size must be 0 or a power of two <= 1024 (got %d)",
                   kv->page_size);
  if (kv->host_rows < 0 || kv->dev_rows < 0)
    return set_err(DKV_ERR_INVALID, "pool capacities must be >= 0");
  if (kv->host_rows > 0 && (!kv->host_k || !kv->host_v))
    return set_err(DKV_ERR_INVALID, "host_rows > 0 but host_k/host_v is NULL");
  if (kv->dev_rows > 0 && (!kv->dev_k || !kv->dev_v))
    return set_err(DKV_ERR_INVALID, "dev_rows > 0 but dev_k/dev_v is NULL");
  if (kv->page_size == 0) {
    if (kv->host_stride < 0 || kv->dev_stride < 0)
      return set_err(DKV_ERR_INVALID, "strides must be >= 0");
  } else {
    if (kv->max_pages < 1) return set_err(DKV_ERR_INVALID, "paged layout needs max_pages >= 1");
    if (!kv->page_table) return set_err(DKV_ERR_INVALID, "paged layout needs page_table");
  }
  const uintptr_t al = 16;
  if ((uintptr_t)kv->host_k % al || (uintptr_t)kv->host_v % al || (uintptr_t)kv->dev_k % al ||
      (uintptr_t)kv->dev_v % al)
    return set_err(DKV_ERR_INVALID, "KV pools must be 16-byte aligned");
  return DKV_OK;
}

dkv_status validate_ratio(double r) {
  if (!(r >= 0.0 && r <= 1.0)) return set_err(DKV_ERR_INVALID, "offload_ratio must be in [0, 1]");
  return DKV_OK;
}

std::shared_ptr<PlanEntry> cache_insert(const std::string& key, std::shared_ptr<PlanEntry> e);
std::shared_ptr<PlanEntry> cache_find(const std::string& key);

// Drops the least recently used entries not held by a captured graph until
// the cache is within its capacity (caller holds c.mu); the dropped entries
// go to *evicted, to be released outside the lock.
void cache_trim(PlanCache& c, std::vector<std::shared_ptr<PlanEntry>>* evicted) {
  auto lit = c.lru.end();
  while (c.map.size() > PlanCache::kCap && lit != c.lru.begin()) {
    --lit;
    auto mit = c.map.find(*lit);
    if (mit->second.first->captured) continue;
    evicted->push_back(mit->second.first);
    c.map.erase(mit);
    lit = c.lru.erase(lit);
  }
}

// Stores a freshly built plan in the cache (or returns the entry another
// thread stored first) and evicts unreferenced old entries.
std::shared_ptr<PlanEntry> cache_insert(const std::string& key, std::shared_ptr<PlanEntry> e) {
  PlanCache& c = cache();
  std::vector<std::shared_ptr<PlanEntry>> evicted;
  {
    std::lock_guard<std::mutex> lk(c.mu);
    auto it = c.map.find(key);
    if (it != c.map.end()) {
      evicted.push_back(e);
      e = it->second.first;
    } else {
      c.lru.push_front(key);
      c.map.emplace(key, std::make_pair(e, c.lru.begin()));
      cache_trim(c, &evicted);
    }
  }
  // evicted images are freed (after a device synchronisation) by the last
  // reference: here, or at the end of a call that still holds one
  evicted.clear();
  return e;
}

std::shared_ptr<PlanEntry> cache_find(const std::string& key) {
  PlanCache& c = cache();
  std::lock_guard<std::mutex> lk(c.mu);
  auto it = c.map.find(key);
  if (it == c.map.end()) return nullptr;
  c.lru.splice(c.lru.begin(), c.lru, it->second.second);
  return it->second.first;
}

// Builds or fetches the plan of a prefill call.
dkv_status get_prefill_plan(const dkv_kv_desc* kv, int32_t batch, int32_t hq, const int32_t* q_start,
                            const int32_t* q_pos0, const int32_t* seq_lens, double ratio,
                            std::shared_ptr<PlanEntry>* out, bool fresh = false) {
  if (batch < 1) return set_err(DKV_ERR_INVALID, "batch must be >= 1");
  if (!seq_lens || !q_start || !q_pos0) return set_err(DKV_ERR_INVALID, "seq_lens, q_start and q_pos0 are required");
  if (hq < 1 || hq % kv->num_kv_heads)
    return set_err(DKV_ERR_INVALID, "num_q_heads %d must be a positive multiple of num_kv_heads %d", hq,
                   kv->num_kv_heads);
  const int g = hq / kv->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return set_err(DKV_ERR_UNSUPPORTED, "query group size %d not built (1, 2, 4, 8)", g);
  if (kv->page_size > 0 && !kv->page_table_host)
    return set_err(DKV_ERR_INVALID, "paged layout needs page_table_host to plan");
  uint64_t gen = 0;
  const dkv_tuning t = tuning_snapshot(&gen);
  int dev = 0;
  int cus = t.num_cus;
  if (cus <= 0) {
    cus = device_cus(&dev);
    if (cus <= 0) return set_err(DKV_ERR_HIP, "cannot query the current device's CU count");
  }
  std::string key(fresh ? "prefill-fused" : "prefill");
  put(key, dev); put(key, cus); put(key, gen); put(key, batch); put(key, hq);
  put(key, kv->num_kv_heads); put(key, kv->head_dim); put(key, kv->page_size); put(key, kv->max_pages);
  put(key, kv->host_stride); put(key, kv->dev_stride); put(key, kv->host_rows); put(key, kv->dev_rows);
  put(key, ratio);
  key.append(reinterpret_cast<const char*>(seq_lens), sizeof(int32_t) * (size_t)batch);
  key.append(reinterpret_cast<const char*>(q_start), sizeof(int32_t) * (size_t)(batch + 1));
  key.append(reinterpret_cast<const char*>(q_pos0), sizeof(int32_t) * (size_t)batch);
  if (kv->page_size > 0) {
    uint64_t h = 1469598103934665603ull;
    for (int b = 0; b < batch; ++b) {
      const int64_t L = std::max(0, seq_lens[b]);
      const int64_t npg = std::min<int64_t>((L + kv->page_size - 1) / kv->page_size, kv->max_pages);
      h = fnv1a(kv->page_table_host + (int64_t)b * kv->max_pages, sizeof(int32_t) * npg, h);
    }
    put(key, h);
  }
  if (auto hit = cache_find(key)) {
    *out = hit;
    return DKV_OK;
  }
  dkv::PlanInput in{};
  in.batch = batch; in.hq = hq; in.hkv = kv->num_kv_heads; in.head_dim = kv->head_dim;
  in.page_size = kv->page_size; in.max_pages = kv->max_pages;
  in.host_stride = kv->host_stride; in.dev_stride = kv->dev_stride;
  in.host_rows = kv->host_rows; in.dev_rows = kv->dev_rows;
  in.seq_lens = seq_lens; in.page_table_host = kv->page_table_host; in.ratio = ratio;
  in.num_cus = cus; in.host_wgs = t.host_wgs; in.dev_wgs = t.dev_wgs;
  in.host_chunk = t.host_chunk; in.dev_chunk = t.dev_chunk;
  in.host_bw = t.host_bw_gbs; in.dev_bw = t.dev_bw_gbs;
  in.stage_max_bytes = t.stage_max_mib < 0 ? 0 : (int64_t)(t.stage_max_mib == 0 ? 4096 : t.stage_max_mib) << 20;
  in.prefill_fresh = fresh ? 1 : 0;
  auto e = std::make_shared<PlanEntry>();
  std::vector<uint8_t> blob;
  std::string err;
  if (!dkv::build_prefill_plan(in, q_start, q_pos0, &e->lay, &blob, &err))
    return set_err(DKV_ERR_INVALID, "%s", err.c_str());
  e->bytes = blob.size();
  hipError_t he = hipHostMalloc(&e->pinned, e->bytes, hipHostMallocDefault);
  if (he != hipSuccess) return set_err(DKV_ERR_NOMEM, "plan staging: %s", hipGetErrorString(he));
  memcpy(e->pinned, blob.data(), e->bytes);
  *out = cache_insert(key, e);
  return DKV_OK;
}

// Prefill workspace: plan image, the rows' rotation table ((cos, sin) fp64
// per row and pair), then the HBM staging pool (K rows, then V rows).
size_t rope_table_bytes(int32_t n_rows, int d) { return (size_t)n_rows * (d / 2) * 16; }
size_t prefill_stage_off(const dkv::PlanLayout& L, int hq, int d) {
  return (L.blob_bytes + rope_table_bytes(L.n_rows, d) + 255) / 256 * 256;
}
size_t prefill_ws_bytes(const dkv::PlanLayout& L, int hq, int hkv, int d) {
  return prefill_stage_off(L, hq, d) + (size_t)L.stage_rows * hkv * d * 2 * 2;
}

// Fused prefill workspace: the prefill workspace, then the fresh rows (K, V),
// the partials, the split offsets and the projection scratch.
struct FusedLayout {
  size_t fresh_off, part_o_off, part_lse_off, offsets_off, proj_off, total;
};
FusedLayout fused_layout(const dkv::PlanLayout& L, int hq, int hkv, int d, int hidden) {
  auto up = [](size_t a) { return (a + 255) / 256 * 256; };
  FusedLayout f{};
  const size_t rowb = (size_t)hkv * d * 2;
  f.fresh_off = up(prefill_ws_bytes(L, hq, hkv, d));
  f.part_o_off = up(f.fresh_off + 2 * rowb * (size_t)L.n_rows);
  f.part_lse_off = up(f.part_o_off + (size_t)L.num_splits * hq * d * 4);
  f.offsets_off = up(f.part_lse_off + (size_t)L.num_splits * hq * 4);
  f.proj_off = up(f.offsets_off + ((size_t)L.n_rows + 1) * 4);
  f.total = f.proj_off + (hidden > 0 ? dkv_append_workspace_bytes(L.n_rows, hidden, hkv * d) : 0);
  return f;
}

void fill_info(const dkv::PlanLayout& L, size_t ws, dkv_plan_info* info) {
  info->workspace_bytes = (int64_t)ws;
  info->num_splits = L.num_splits;
  info->host_items = L.n_host_items;
  info->dev_items = L.n_dev_items;
  info->host_wgs = L.host_wgs;
  info->dev_wgs = L.dev_wgs;
  info->host_chunk = L.host_chunk;
  info->dev_chunk = L.dev_chunk;
  info->host_bytes = L.host_bytes;
  info->dev_bytes = L.dev_bytes;
  info->staged_bytes = L.staged_bytes;
}

// f_i = theta^(-2i/D) in IEEE double, the exponent formed as (-2 i) / D.
dkv::RopeFreq rope_freq(double theta, int d) {
  dkv::RopeFreq r{};
  for (int i = 0; i < d / 2 && i < 64; ++i) r.f[i] = std::pow(theta, -2.0 * (double)i / (double)d);
  return r;
}

// ---------------------------------------------------------------- workgroup trace
std::mutex g_trace_mu;
uint64_t* g_trace_buf = nullptr;
int32_t g_trace_cap = 0;

// ---------------------------------------------------------------- kernel timing
struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> rec[8];
};

Timing& timing() {
  static Timing* t = new Timing();
  return *t;
}

hipEvent_t take_event(Timing& t) {
  if (!t.pool.empty()) {
    hipEvent_t e = t.pool.back();
    t.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Brackets one kernel launch with an event pair when timing is on.
struct TimedLaunch {
  int kernel;
  hipStream_t stream;
  hipEvent_t e0 = nullptr;
  TimedLaunch(int k, hipStream_t s) : kernel(k), stream(s) {
    if (stream_capturing(s)) return;  // graphs replay without the event pair
    Timing& t = timing();
    std::lock_guard<std::mutex> lk(t.mu);
    if (!t.on) return;
    e0 = take_event(t);
    if (e0 && hipEventRecord(e0, s) != hipSuccess) {
      t.pool.push_back(e0);
      e0 = nullptr;
    }
  }
  void done() {
    if (!e0) return;
    Timing& t = timing();
    std::lock_guard<std::mutex> lk(t.mu);
    hipEvent_t e1 = take_event(t);
    if (e1 && hipEventRecord(e1, stream) == hipSuccess) {
      t.rec[kernel].push_back({e0, e1});
    } else {
      t.pool.push_back(e0);
      if (e1) t.pool.push_back(e1);
    }
    e0 = nullptr;
  }
};

// Offloaded-linear planner input: tuning fields as for decode.
dkv::PlanInput linear_input(double ratio, int32_t cus, const dkv_tuning& t) {
  dkv::PlanInput in{};
  in.ratio = ratio;
  in.num_cus = cus;
  in.host_wgs = t.host_wgs; in.dev_wgs = t.dev_wgs;
  in.host_chunk = t.host_chunk; in.dev_chunk = t.dev_chunk;
  in.host_bw = t.host_bw_gbs; in.dev_bw = t.dev_bw_gbs;
  return in;
}

dkv_status validate_linear(int32_t m, int32_t n, int32_t k, double ratio) {
  if (m < 1 || n < 1 || k < 1) return set_err(DKV_ERR_INVALID, "m, out_features and in_features must be >= 1");
  if (k % 8) return set_err(DKV_ERR_INVALID, "in_features must be a multiple of 8 (got %d)", k);
  if ((int64_t)m * n > ((int64_t)1 << 40)) return set_err(DKV_ERR_INVALID, "m * out_features too large");
  return validate_ratio(ratio);
}

// The linear call's shape: no plan image, the kernel derives its items.
dkv_status get_linear_shape(int32_t n, int32_t k, double ratio, int32_t cus_override, dkv::LinearShape* z) {
  const dkv_tuning t = tuning_snapshot(nullptr);
  int cus = cus_override > 0 ? cus_override : t.num_cus;
  if (cus <= 0) {
    int dev = 0;
    cus = device_cus(&dev);
    if (cus <= 0) return set_err(DKV_ERR_HIP, "cannot query the current device's CU count");
  }
  std::string err;
  if (!dkv::linear_shape(linear_input(ratio, cus, t), n, k, z, &err)) return set_err(DKV_ERR_INVALID, "%s", err.c_str());
  return DKV_OK;
}

void fill_linear_info(const dkv::LinearShape& z, dkv_plan_info* info) {
  *info = dkv_plan_info{};
  info->workspace_bytes = (int64_t)z.ws_bytes;
  info->num_splits = z.num_splits;
  info->host_items = z.n_host_items;
  info->dev_items = z.n_dev_items;
  info->host_wgs = z.host_wgs;
  info->dev_wgs = z.dev_wgs;
  info->host_chunk = z.n_host_items ? z.kc_host : 0;
  info->dev_chunk = z.n_dev_items ? z.kc_dev : 0;
  info->host_bytes = z.host_bytes;
  info->dev_bytes = z.dev_bytes;
}

// ---------------------------------------------------------------- decode shape
//
// A decode call has no host plan: the launch shape (workgroups per tier and KV
// head, item-length rules) follows from its arguments, and the kernel derives
// the items from the lengths in device memory.  The workspace holds the unit
// queues and counters (zero between calls: every call leaves them zeroed),
// the paged layout's tier lists, and the fused form's partials (one slot per
// item and one per appended token of each sequence) with their merge counts.
struct DecodeShape {
  dkv::DecodeTemplate t{};
  int32_t g = 0;
  int32_t max_slots = 0;   // fused: partial slots in the workspace
  int64_t max_splits = 0;  // split bound over any lengths that fit the pools
  size_t counters_off = 0, group_off = 0, tiers_off = 0, lists_off = 0, part_o_off = 0, part_lse_off = 0,
         proj_off = 0, total = 0;
};

dkv::PlanInput decode_input(const dkv_kv_desc* kv, int32_t batch, int32_t hq, double ratio, int32_t cus,
                            const dkv_tuning& t) {
  dkv::PlanInput in{};
  in.batch = batch; in.hq = hq; in.hkv = kv->num_kv_heads; in.head_dim = kv->head_dim;
  in.page_size = kv->page_size; in.max_pages = kv->max_pages;
  in.host_stride = kv->host_stride; in.dev_stride = kv->dev_stride;
  in.host_rows = kv->host_rows; in.dev_rows = kv->dev_rows;
  in.page_table_host = kv->page_table_host; in.ratio = ratio;
  in.num_cus = cus; in.host_wgs = t.host_wgs; in.dev_wgs = t.dev_wgs;
  in.host_chunk = t.host_chunk; in.dev_chunk = t.dev_chunk;
  in.host_bw = t.host_bw_gbs; in.dev_bw = t.dev_bw_gbs;
  return in;
}

dkv_status decode_shape(const dkv_kv_desc* kv, int32_t batch, int32_t hq, double ratio, bool fused, int32_t hidden,
                        int32_t num_cus, DecodeShape* out, bool static_layout = false) {
  if (batch < 1 || batch > dkv::kDecodeMaxBatch)
    return set_err(DKV_ERR_UNSUPPORTED, "batch %d outside 1..%d", batch, dkv::kDecodeMaxBatch);
  if (hq < 1 || hq % kv->num_kv_heads)
    return set_err(DKV_ERR_INVALID, "num_q_heads %d must be a positive multiple of num_kv_heads %d", hq,
                   kv->num_kv_heads);
  const int g = hq / kv->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return set_err(DKV_ERR_UNSUPPORTED, "query group size %d not built (1, 2, 4, 8)", g);
  if (kv->page_size == 0 && validate_ratio(ratio) != DKV_OK) return DKV_ERR_INVALID;
  const dkv_tuning tu = tuning_snapshot(nullptr);
  int cus = num_cus > 0 ? num_cus : tu.num_cus;
  if (cus <= 0) {
    cus = device_cus(nullptr);
    if (cus <= 0) return set_err(DKV_ERR_HIP, "cannot query the current device's CU count");
  }
  const bool paged = kv->page_size > 0;
  const bool host_tier = kv->host_rows > 0 && (paged || ratio > 0.0);
  const bool dev_tier = kv->dev_rows > 0 && (paged || ratio < 1.0);
  if (!host_tier && !dev_tier) return set_err(DKV_ERR_INVALID, "no tier can hold tokens (pool rows and ratio)");
  const double frac = paged ? (double)kv->host_rows / (double)(kv->host_rows + kv->dev_rows) : ratio;
  DecodeShape d;
  d.t = dkv::decode_template(decode_input(kv, batch, hq, ratio, cus, tu), host_tier, dev_tier, frac);
  d.g = g;
  d.max_splits = dkv::decode_max_splits(d.t, batch, kv->host_rows, kv->dev_rows);
  const int64_t slots = d.max_splits + batch;
  // the kernel addresses the fused partials with 31-bit byte offsets
  if (fused && slots * hq * (int64_t)kv->head_dim * 4 > INT32_MAX)
    return set_err(DKV_ERR_UNSUPPORTED, "fused step: %lld partial slots x %d heads x %d dims exceed 2 GiB",
                   (long long)slots, hq, kv->head_dim);
  d.max_slots = fused ? (int32_t)slots : 0;
  auto up = [](size_t a) { return (a + 255) / 256 * 256; };
  const size_t hkv = (size_t)kv->num_kv_heads, D = (size_t)kv->head_dim, B = (size_t)batch;
  const size_t S = (size_t)d.max_slots;
  d.counters_off = 0;
  d.group_off = up((size_t)dkv::decode_counter_words() * 4);
  d.tiers_off = up(d.group_off + (fused ? (S + B) * hkv * 4 : 0));
  if (static_layout) {  // counters in the static scratch's fixed counter area
    if (d.tiers_off > dkv::kDecodeStaticCounterBytes)
      return set_err(DKV_ERR_UNSUPPORTED, "this shape needs %zu bytes of counters, beyond the static %zu bytes",
                     d.tiers_off, dkv::kDecodeStaticCounterBytes);
    d.tiers_off = dkv::kDecodeStaticCounterBytes;
  }
  d.lists_off = up(d.tiers_off + (paged ? B * 4 * 4 : 0));
  d.part_o_off = up(d.lists_off + (paged ? 2 * B * (size_t)kv->max_pages * 4 : 0));
  d.part_lse_off = up(d.part_o_off + (fused ? S * (size_t)hq * D * 4 : 0));
  d.proj_off = up(d.part_lse_off + (fused ? S * (size_t)hq * 4 : 0));
  d.total = d.proj_off +
            (fused && hidden > 0 ? dkv_append_workspace_bytes(batch, hidden, kv->num_kv_heads * kv->head_dim) : 0);
  *out = d;
  return DKV_OK;
}

dkv::DecodeArgs decode_args(const dkv_kv_desc* kv, const DecodeShape& d, int32_t batch, int32_t hq, const void* q,
                            const int32_t* q_pos, const int32_t* seq_lens, double ratio, float scale,
                            double rope_theta, void* workspace) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  dkv::DecodeArgs a{};
  a.host_k = static_cast<uint16_t*>(kv->host_k);
  a.host_v = static_cast<uint16_t*>(kv->host_v);
  a.dev_k = static_cast<uint16_t*>(kv->dev_k);
  a.dev_v = static_cast<uint16_t*>(kv->dev_v);
  a.host_rows = kv->host_rows;
  a.dev_rows = kv->dev_rows;
  a.host_stride = kv->host_stride;
  a.dev_stride = kv->dev_stride;
  a.page_table = kv->page_size > 0 ? kv->page_table : nullptr;
  a.max_pages = kv->max_pages;
  a.page_shift = kv->page_size > 0 ? log2i(kv->page_size) : -1;
  a.q = static_cast<const uint16_t*>(q);
  a.q_pos = q_pos;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.hq = hq;
  a.hkv = kv->num_kv_heads;
  a.head_dim = kv->head_dim;
  a.ratio = kv->page_size > 0 ? 0.0 : ratio;
  a.scale_log2 = scale * 1.44269504088896340736f;
  a.tmpl = d.t;
  a.counters = reinterpret_cast<int32_t*>(ws + d.counters_off);
  a.group_cnt = reinterpret_cast<int32_t*>(ws + d.group_off);
  a.tier_counts = reinterpret_cast<const int32_t*>(ws + d.tiers_off);
  a.tier_pages = reinterpret_cast<const int32_t*>(ws + d.lists_off);
  a.part_o = reinterpret_cast<float*>(ws + d.part_o_off);
  a.part_lse = reinterpret_cast<float*>(ws + d.part_lse_off);
  a.max_slots = d.max_slots;
  a.freq = rope_freq(rope_theta, kv->head_dim);
  std::lock_guard<std::mutex> lk(g_trace_mu);
  a.wg_trace = g_trace_buf;
  a.wg_trace_cap = g_trace_cap;
  return a;
}

// DKV_DEBUG_VALIDATE: the lengths (and the page table) read back and checked
// against the layout before anything is launched.
dkv_status decode_debug_check(const dkv_kv_desc* kv, int32_t batch, const int32_t* seq_lens, double ratio,
                              int new_tokens, hipStream_t s) {
  std::vector<int32_t> sl(batch);
  hipError_t he = hipStreamSynchronize(s);
  if (he == hipSuccess) he = hipMemcpy(sl.data(), seq_lens, 4 * (size_t)batch, hipMemcpyDeviceToHost);
  if (he != hipSuccess) return hip_err(he, "debug copy of seq_lens");
  std::vector<int32_t> pt;
  if (kv->page_size > 0) {
    pt.resize((size_t)batch * kv->max_pages);
    he = hipMemcpy(pt.data(), kv->page_table, pt.size() * 4, hipMemcpyDeviceToHost);
    if (he != hipSuccess) return hip_err(he, "debug copy of page_table");
  }
  for (int b = 0; b < batch; ++b) {
    const int64_t L = sl[b];
    if (L < 0) return set_err(DKV_ERR_INVALID, "seq_lens[%d] = %lld is negative", b, (long long)L);
    const int64_t placed = L + new_tokens;
    if (kv->page_size == 0) {
      int64_t nh, nd, ph;
      dkv::contig_tiers(ratio, L, placed, &nh, &nd, &ph);
      if (ph > 0 && (ph > kv->host_stride || (int64_t)b * kv->host_stride + ph > kv->host_rows))
        return set_err(DKV_ERR_INVALID, "sequence %d: host rows needed beyond host_stride/host_rows", b);
      if (placed - ph > 0 &&
          (placed - ph > kv->dev_stride || (int64_t)b * kv->dev_stride + (placed - ph) > kv->dev_rows))
        return set_err(DKV_ERR_INVALID, "sequence %d: device rows needed beyond dev_stride/dev_rows", b);
    } else {
      const int64_t npg = (placed + kv->page_size - 1) / kv->page_size;
      if (npg > kv->max_pages) return set_err(DKV_ERR_INVALID, "sequence %d needs %lld pages > max_pages", b,
                                              (long long)npg);
      for (int64_t j = 0; j < npg; ++j) {
        const int32_t e = pt[(size_t)b * kv->max_pages + j];
        const bool host = (e & 1) != 0;
        if (e < 0 || ((int64_t)(e >> 1) + 1) * kv->page_size > (host ? kv->host_rows : kv->dev_rows))
          return set_err(DKV_ERR_INVALID, "page_table[%d][%lld] = %d: unmapped or beyond its pool", b,
                         (long long)j, e);
      }
    }
  }
  return DKV_OK;
}

dkv_status validate_decode_common(const dkv_kv_desc* kv, const void* q, const int32_t* q_pos,
                                  const int32_t* seq_lens, float scale, double rope_theta, const void* workspace) {
  dkv_status st = validate_desc(kv);
  if (st != DKV_OK) return st;
  if (!q || !q_pos || !seq_lens || !workspace)
    return set_err(DKV_ERR_INVALID, "q, q_pos, seq_lens and workspace are required");
  if (!(std::isfinite(scale)) || !(std::isfinite(rope_theta)) || rope_theta <= 0.0)
    return set_err(DKV_ERR_INVALID, "scale must be finite and rope_theta > 0");
  if ((uintptr_t)workspace % 256) return set_err(DKV_ERR_INVALID, "workspace must be 256-byte aligned");
  return DKV_OK;
}

// ---------------------------------------------------------------- staged prefetch
//
// The conventional design the zero-copy path is compared with (SplitKernel
// README, Overview: prefetching offloaded data into GPU memory costs HBM
// traffic and capacity and leaves pipeline bubbles): the host tier is copied
// by the DMA engine, chunk by chunk, into a two-slot HBM ring on a copy
// stream; each staged chunk is attended from HBM (one launch of the fused
// decode kernel, no new token) while the next chunk is copied; the HBM tier is
// attended alongside; the per-chunk results are merged by log-sum-exp.

struct StagedLayout {
  int64_t nh = 0, nd = 0;        // host / HBM tokens of the sequence
  int32_t chunk = 0, n_chunks = 0, n_rows = 0;
  DecodeShape step;              // workspace of the per-chunk decode launches
  size_t ring_off = 0, ring_slot_bytes = 0, part_o_off = 0, part_lse_off = 0, ints_off = 0, total = 0;
};

dkv_status staged_layout(const dkv_kv_desc* kv, int32_t hq, int64_t seq_len, double ratio, int32_t chunk,
                         StagedLayout* out) {
  if (kv->page_size != 0) return set_err(DKV_ERR_UNSUPPORTED, "the staged comparator takes the contiguous layout");
  if (seq_len < 1 || seq_len > INT32_MAX) return set_err(DKV_ERR_INVALID, "seq_len must be in [1, 2^31)");
  if (chunk < 64 || chunk % 64) return set_err(DKV_ERR_INVALID, "chunk_tokens must be a positive multiple of 64");
  if (validate_ratio(ratio) != DKV_OK) return DKV_ERR_INVALID;
  StagedLayout L;
  int64_t ph;
  dkv::contig_tiers(ratio, seq_len, seq_len, &L.nh, &L.nd, &ph);
  if (L.nh > kv->host_stride || L.nh > kv->host_rows || L.nd > kv->dev_stride || L.nd > kv->dev_rows)
    return set_err(DKV_ERR_INVALID, "the sequence's rows exceed the layout");
  L.chunk = chunk;
  L.n_chunks = (int32_t)((L.nh + chunk - 1) / chunk);
  L.n_rows = L.n_chunks + (L.nd > 0 ? 1 : 0);
  // every per-chunk launch reads an HBM-only view of `chunk` rows
  dkv_kv_desc view = *kv;
  view.host_k = view.host_v = nullptr;
  view.host_rows = view.host_stride = 0;
  view.dev_rows = view.dev_stride = std::max<int64_t>(chunk, L.nd);
  view.dev_k = view.dev_v = reinterpret_cast<void*>(256);  // shape only
  dkv_status st = decode_shape(&view, 1, hq, 0.0, true, 0, 0, &L.step);
  if (st != DKV_OK) return st;
  auto up = [](size_t a) { return (a + 255) / 256 * 256; };
  const size_t row_bytes = (size_t)kv->num_kv_heads * kv->head_dim * 2;
  L.ring_slot_bytes = up((size_t)chunk * row_bytes);
  L.ring_off = up(L.step.total);
  L.part_o_off = L.ring_off + 4 * L.ring_slot_bytes;  // two slots of K and of V
  L.part_lse_off = up(L.part_o_off + (size_t)std::max(1, L.n_rows) * hq * kv->head_dim * 4);
  L.ints_off = up(L.part_lse_off + (size_t)std::max(1, L.n_rows) * hq * 4);
  L.total = up(L.ints_off + (size_t)(L.n_rows + 3) * 4);
  *out = L;
  return DKV_OK;
}

struct CopyEngine {
  std::mutex mu;
  hipStream_t stream[kMaxCopyDevices] = {};
  hipEvent_t ev[kMaxCopyDevices][4] = {};
};
CopyEngine& copy_engine() {
  static CopyEngine* c = new CopyEngine();
  return *c;
}

}  // namespace

extern "C" {

const char* dkv_last_error(void) { return g_last_error.c_str(); }

int32_t dkv_version(void) { return 1 * 10000 + 0 * 100 + 0; }

dkv_status dkv_plan_cache_release_captured(void) {
  PlanCache& c = cache();
  std::vector<std::shared_ptr<PlanEntry>> evicted;
  {
    std::lock_guard<std::mutex> lk(c.mu);
    for (auto& kv : c.map) kv.second.first->captured = false;
    cache_trim(c, &evicted);
  }
  evicted.clear();  // images freed by their last reference (after a device synchronisation)
  return ok();
}

dkv_status dkv_plan_cache_stats(int32_t* entries, int32_t* captured, int64_t* pinned_bytes) {
  if (!entries || !captured || !pinned_bytes) return set_err(DKV_ERR_INVALID, "entries, captured and pinned_bytes are required");
  PlanCache& c = cache();
  std::lock_guard<std::mutex> lk(c.mu);
  int32_t n = 0, k = 0;
  int64_t bytes = 0;
  for (const auto& kv : c.map) {
    ++n;
    if (kv.second.first->captured) ++k;
    bytes += (int64_t)kv.second.first->bytes;
  }
  *entries = n;
  *captured = k;
  *pinned_bytes = bytes;
  return ok();
}

dkv_status dkv_split_point(double ratio, int64_t length, int64_t* n_host) {
  if (!n_host) return set_err(DKV_ERR_INVALID, "n_host is NULL");
  if (validate_ratio(ratio) != DKV_OK) return DKV_ERR_INVALID;
  if (length < 0) return set_err(DKV_ERR_INVALID, "length must be >= 0");
  *n_host = (int64_t)std::floor(ratio * (double)length);
  return ok();
}

dkv_status dkv_set_tuning(const dkv_tuning* t) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  if (t) {
    if (t->num_cus < 0 || t->host_wgs < 0 || t->dev_wgs < 0 || t->host_chunk < 0 ||
        t->dev_chunk < 0 || !(t->host_bw_gbs >= 0) || !(t->dev_bw_gbs >= 0) || t->writer_wgs < 0)
      return set_err(DKV_ERR_INVALID, "tuning fields must be >= 0");
    if (t->reserved != 0) return set_err(DKV_ERR_INVALID, "tuning.reserved must be 0");
    if (t->host_wgs > 65535 || t->dev_wgs > 65535 || t->writer_wgs > 65535)
      return set_err(DKV_ERR_INVALID, "workgroup counts must be <= 65535");
    g_tune = *t;
  } else {
    g_tune = dkv_tuning{};
  }
  ++g_tune_gen;
  return ok();
}

dkv_status dkv_get_tuning(dkv_tuning* t) {
  if (!t) return set_err(DKV_ERR_INVALID, "tuning is NULL");
  *t = tuning_snapshot(nullptr);
  return ok();
}

dkv_status dkv_decode_plan(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads,
                           const int32_t* seq_lens, double offload_ratio, dkv_plan_info* info) {
  if (!info) return set_err(DKV_ERR_INVALID, "info is NULL");
  dkv_status st = validate_desc(kv);
  if (st != DKV_OK) return st;
  DecodeShape d;
  st = decode_shape(kv, batch, num_q_heads, offload_ratio, false, 0, 0, &d);
  if (st != DKV_OK) return st;
  *info = dkv_plan_info{};
  info->workspace_bytes = (int64_t)d.total;
  info->num_splits = (int32_t)std::min<int64_t>(d.max_splits, INT32_MAX);
  info->host_wgs = d.t.team_h * kv->num_kv_heads;
  info->dev_wgs = d.t.team_d * kv->num_kv_heads;
  if (seq_lens) {
    dkv_plan_info exact{};
    st = dkv_plan_inspect(kv, batch, num_q_heads, seq_lens, offload_ratio, 0, nullptr, 0, nullptr, 0, nullptr,
                          &exact);
    if (st != DKV_OK) return st;
    info->host_items = exact.host_items;
    info->dev_items = exact.dev_items;
    info->host_chunk = exact.host_chunk;
    info->dev_chunk = exact.dev_chunk;
    info->host_bytes = exact.host_bytes;
    info->dev_bytes = exact.dev_bytes;
  }
  return ok();
}

dkv_status dkv_plan_inspect(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads,
                            const int32_t* seq_lens, double offload_ratio, int32_t num_cus,
                            int64_t* items, int32_t items_cap, int32_t* page_list,
                            int32_t page_cap, int32_t* split_offsets, dkv_plan_info* info) {
  dkv_status st = validate_desc(kv);
  if (st != DKV_OK) return st;
  if (!seq_lens) return set_err(DKV_ERR_INVALID, "seq_lens is required");
  if (num_cus < 0) return set_err(DKV_ERR_INVALID, "num_cus must be >= 0");
  if (kv->page_size > 0 && !kv->page_table_host)
    return set_err(DKV_ERR_INVALID, "paged layout needs page_table_host to inspect");
  DecodeShape d;
  st = decode_shape(kv, batch, num_q_heads, offload_ratio, false, 0, num_cus, &d);
  if (st != DKV_OK) return st;
  const dkv::PlanInput in = decode_input(kv, batch, num_q_heads, offload_ratio, 1, tuning_snapshot(nullptr));
  std::vector<int64_t> nh(batch), nd(batch);
  std::vector<std::vector<int32_t>> hp(batch), dp(batch);
  for (int b = 0; b < batch; ++b) {
    if (seq_lens[b] < 0) return set_err(DKV_ERR_INVALID, "seq_lens[%d] is negative", b);
    if (kv->page_size == 0) {
      int64_t ph;
      dkv::contig_tiers(offload_ratio, seq_lens[b], seq_lens[b], &nh[b], &nd[b], &ph);
      if (ph > 0 && (ph > kv->host_stride || (int64_t)b * kv->host_stride + ph > kv->host_rows))
        return set_err(DKV_ERR_INVALID, "sequence %d: host rows needed beyond host_stride/host_rows", b);
      if (seq_lens[b] - ph > 0 && (seq_lens[b] - ph > kv->dev_stride ||
                                   (int64_t)b * kv->dev_stride + (seq_lens[b] - ph) > kv->dev_rows))
        return set_err(DKV_ERR_INVALID, "sequence %d: device rows needed beyond dev_stride/dev_rows", b);
    } else if (!dkv::decode_tiers_host(in, b, seq_lens[b], &hp[b], &dp[b], &nh[b], &nd[b])) {
      return set_err(DKV_ERR_INVALID, "sequence %d: page table entry unmapped or beyond its pool", b);
    }
  }
  std::vector<dkv::DecodeHostItem> list;
  std::vector<int32_t> offs;
  dkv::DecodeSizes z{};
  dkv::decode_enumerate(d.t, batch, nh.data(), nd.data(), &list, &offs, &z);
  int32_t n_host = 0, n_page = 0;
  int64_t host_tok = 0, dev_tok = 0;
  for (int b = 0; b < batch; ++b) {
    host_tok += nh[b];
    dev_tok += nd[b];
  }
  for (size_t i = 0; i < list.size(); ++i) {
    const dkv::DecodeHostItem& it = list[i];
    n_host += it.host;
    int64_t first;
    if (kv->page_size == 0) {
      first = (int64_t)it.b * (it.host ? kv->host_stride : kv->dev_stride) + it.k0;
    } else {
      // logical pages of the item, appended to page_list
      const std::vector<int32_t>& pg = it.host ? hp[it.b] : dp[it.b];
      first = n_page;
      const int64_t p0 = it.k0 / kv->page_size, p1 = (it.k0 + it.n_tok + kv->page_size - 1) / kv->page_size;
      for (int64_t k = p0; k < p1; ++k, ++n_page)
        if (page_list && n_page < page_cap) page_list[n_page] = pg[k];
    }
    if (items && (int64_t)i < items_cap) {
      int64_t* o = items + 5 * i;
      o[0] = it.host; o[1] = it.b; o[2] = it.slot; o[3] = it.n_tok; o[4] = first;
    }
  }
  if (split_offsets) memcpy(split_offsets, offs.data(), sizeof(int32_t) * (batch + 1));
  if (info) {
    const int64_t row_bytes = (int64_t)kv->num_kv_heads * kv->head_dim * 2;
    *info = dkv_plan_info{};
    info->workspace_bytes = (int64_t)d.total;
    info->num_splits = offs[batch];
    info->host_items = n_host;
    info->dev_items = (int32_t)list.size() - n_host;
    info->host_wgs = d.t.team_h * kv->num_kv_heads;
    info->dev_wgs = d.t.team_d * kv->num_kv_heads;
    info->host_chunk = n_host ? z.ch : 0;
    info->dev_chunk = (int32_t)list.size() > n_host ? z.cd : 0;
    info->host_bytes = host_tok * row_bytes * 2;
    info->dev_bytes = dev_tok * row_bytes * 2;
  }
  return ok();
}
dkv_status dkv_prefill_plan_inspect(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads,
                                    const int32_t* q_start, const int32_t* q_pos0, const int32_t* seq_lens,
                                    double offload_ratio, int32_t fused, int32_t num_cus, int64_t* items, int32_t items_cap,
                                    int32_t* pages, int32_t pages_cap, int64_t* tiles, int32_t tiles_cap,
                                    int32_t* split_offsets, int32_t offsets_cap, dkv_plan_info* info) {
  dkv_status st = validate_desc(kv);
  if (st != DKV_OK) return st;
  if (kv->page_size == 0 && validate_ratio(offload_ratio) != DKV_OK) return DKV_ERR_INVALID;
  if (num_cus < 1) return set_err(DKV_ERR_INVALID, "num_cus must be >= 1");
  if (num_q_heads < 1 || num_q_heads % kv->num_kv_heads)
    return set_err(DKV_ERR_INVALID, "num_q_heads must be a positive multiple of num_kv_heads");
  const dkv_tuning t = tuning_snapshot(nullptr);
  dkv::PlanInput in{};
  in.batch = batch; in.hq = num_q_heads; in.hkv = kv->num_kv_heads; in.head_dim = kv->head_dim;
  in.page_size = kv->page_size; in.max_pages = kv->max_pages;
  in.host_stride = kv->host_stride; in.dev_stride = kv->dev_stride;
  in.host_rows = kv->host_rows; in.dev_rows = kv->dev_rows;
  in.seq_lens = seq_lens; in.page_table_host = kv->page_table_host;
  in.ratio = kv->page_size == 0 ? offload_ratio : 0.0;
  in.num_cus = num_cus; in.host_wgs = t.host_wgs; in.dev_wgs = t.dev_wgs;
  in.host_chunk = t.host_chunk; in.dev_chunk = t.dev_chunk;
  in.host_bw = t.host_bw_gbs; in.dev_bw = t.dev_bw_gbs;
  in.stage_max_bytes = t.stage_max_mib < 0 ? 0 : (int64_t)(t.stage_max_mib == 0 ? 4096 : t.stage_max_mib) << 20;
  in.prefill_fresh = fused ? 1 : 0;
  dkv::PlanLayout L;
  std::vector<uint8_t> blob;
  std::string err;
  if (!dkv::build_prefill_plan(in, q_start, q_pos0, &L, &blob, &err))
    return set_err(DKV_ERR_INVALID, "%s", err.c_str());
  const dkv::PrefillItem* it = reinterpret_cast<const dkv::PrefillItem*>(blob.data() + L.items_off);
  const int n_items = L.n_host_items + L.n_dev_items;
  if (items)
    for (int i = 0; i < n_items && i < items_cap; ++i) {
      int64_t* o = items + 11 * (size_t)i;
      o[0] = it[i].pool; o[1] = it[i].b; o[2] = it[i].row0; o[3] = it[i].n_rows; o[4] = it[i].pos0;
      o[5] = it[i].n_tok;
      o[6] = kv->page_size > 0 && it[i].pool != dkv::kPoolFresh ? it[i].plist : it[i].row_pool;
      o[7] = it[i].tok0;
      o[8] = it[i].split_idx; o[9] = it[i].n_splits; o[10] = it[i].base;
    }
  if (pages)
    memcpy(pages, blob.data() + L.plist_off, sizeof(int32_t) * std::min(2 * L.n_plist, pages_cap));
  if (tiles) {
    const dkv::StageTile* tl = reinterpret_cast<const dkv::StageTile*>(blob.data() + L.stage_tiles_off);
    for (int i = 0; i < L.n_stage_tiles && i < tiles_cap; ++i) {
      tiles[3 * (size_t)i] = tl[i].src_row;
      tiles[3 * (size_t)i + 1] = tl[i].dst_row;
      tiles[3 * (size_t)i + 2] = tl[i].n_rows;
    }
  }
  if (split_offsets)
    memcpy(split_offsets, blob.data() + L.offsets_off, sizeof(int32_t) * std::min(L.n_rows + 1, offsets_cap));
  if (info)
    fill_info(L, fused ? fused_layout(L, num_q_heads, kv->num_kv_heads, kv->head_dim, 0).total
                       : prefill_ws_bytes(L, num_q_heads, kv->num_kv_heads, kv->head_dim), info);
  return ok();
}

dkv_status dkv_decode_attn_split(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads,
                                 const void* q, const int32_t* q_pos, const int32_t* seq_lens,
                                 double offload_ratio, float scale, double rope_theta,
                                 void* workspace, size_t workspace_bytes, float* part_o,
                                 float* part_lse, int32_t* split_offsets, int32_t num_splits_cap,
                                 void* stream) {
  dkv_status st = validate_decode_common(kv, q, q_pos, seq_lens, scale, rope_theta, workspace);
  if (st != DKV_OK) return st;
  if (!part_o || !part_lse || !split_offsets)
    return set_err(DKV_ERR_INVALID, "part_o, part_lse and split_offsets are required");
  DecodeShape d;
  st = decode_shape(kv, batch, num_q_heads, offload_ratio, false, 0, 0, &d);
  if (st != DKV_OK) return st;
  if (workspace_bytes < d.total)
    return set_err(DKV_ERR_INVALID, "workspace too small: %zu < %zu bytes", workspace_bytes, d.total);
  if ((int64_t)num_splits_cap < d.max_splits)
    return set_err(DKV_ERR_INVALID, "num_splits_cap %d < %lld (the split bound of this shape)", num_splits_cap,
                   (long long)d.max_splits);
  hipStream_t s = (hipStream_t)stream;
  if (debug_validate()) {
    st = decode_debug_check(kv, batch, seq_lens, offload_ratio, 0, s);
    if (st != DKV_OK) return st;
  }
  dkv::DecodeArgs a = decode_args(kv, d, batch, num_q_heads, q, q_pos, seq_lens, offload_ratio, scale, rope_theta,
                                  workspace);
  a.fused = 0;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.split_offsets = split_offsets;
  a.max_slots = num_splits_cap;
  hipError_t he;
  if (kv->page_size > 0) {
    TimedLaunch t_tiers(DKV_KERNEL_TIERS, s);
    he = (hipError_t)dkv::launch_decode_tiers(a, const_cast<int32_t*>(a.tier_counts),
                                              const_cast<int32_t*>(a.tier_pages), stream);
    t_tiers.done();
    if (he != hipSuccess) return hip_err(he, "tier lists launch");
  }
  TimedLaunch t_attn(DKV_KERNEL_ATTN, s);
  he = (hipError_t)dkv::launch_decode(a, stream);
  t_attn.done();
  if (he != hipSuccess) return hip_err(he, "attention launch");
  return ok();
}

dkv_status dkv_decode_step_plan(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads, double offload_ratio,
                                int32_t hidden, dkv_plan_info* info) {
  if (!info) return set_err(DKV_ERR_INVALID, "info is NULL");
  dkv_status st = validate_desc(kv);
  if (st != DKV_OK) return st;
  if (hidden < 0) return set_err(DKV_ERR_INVALID, "hidden must be >= 0");
  DecodeShape d;
  st = decode_shape(kv, batch, num_q_heads, offload_ratio, true, hidden, 0, &d);
  if (st != DKV_OK) return st;
  *info = dkv_plan_info{};
  info->workspace_bytes = (int64_t)d.total;
  info->num_splits = d.max_slots;
  info->host_wgs = d.t.team_h * kv->num_kv_heads;
  info->dev_wgs = d.t.team_d * kv->num_kv_heads;
  return ok();
}

// The fused decode step on a given workspace (the caller's, or the static
// scratch for the allocation-free entry point).
static dkv_status decode_step_impl(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads, const void* q,
                                   const int32_t* q_pos, const int32_t* seq_lens, const int32_t* pos_new,
                                   const void* x, int32_t hidden, const void* wk, const void* wv,
                                   const void* k_new, const void* v_new, double offload_ratio, float scale,
                                   double rope_theta, void* workspace, size_t workspace_bytes, float* out_o,
                                   float* out_lse, void* stream, bool static_scratch = false) {
  dkv_status st = validate_decode_common(kv, q, q_pos, seq_lens, scale, rope_theta, workspace);
  if (st != DKV_OK) return st;
  if (!out_o) return set_err(DKV_ERR_INVALID, "out_o is required");
  const bool proj = x != nullptr;
  const bool append = proj || k_new != nullptr || v_new != nullptr;
  const int32_t kvd = kv->num_kv_heads * kv->head_dim;
  if (proj) {
    if (!wk || !wv) return set_err(DKV_ERR_INVALID, "projection mode needs wk and wv");
    if (hidden < 256 || hidden % 256)
      return set_err(DKV_ERR_UNSUPPORTED, "hidden %d must be a positive multiple of 256", hidden);
    if ((2 * kvd) % 64) return set_err(DKV_ERR_UNSUPPORTED, "2*Hkv*D must be a multiple of 64");
    if ((uintptr_t)x % 16 || (uintptr_t)wk % 16 || (uintptr_t)wv % 16)
      return set_err(DKV_ERR_INVALID, "x, wk, wv must be 16-byte aligned");
  } else if (append && (!k_new || !v_new)) {
    return set_err(DKV_ERR_INVALID, "appending needs both k_new and v_new (or x with wk and wv)");
  }
  DecodeShape d;
  st = decode_shape(kv, batch, num_q_heads, offload_ratio, true, proj ? hidden : 0, 0, &d, static_scratch);
  if (st != DKV_OK) return st;
  if (workspace_bytes < d.total) {
    if (static_scratch)
      return set_err(DKV_ERR_UNSUPPORTED, "this shape needs %zu bytes of scratch, beyond the static %zu bytes",
                     d.total, workspace_bytes);
    return set_err(DKV_ERR_INVALID, "workspace too small: %zu < %zu bytes", workspace_bytes, d.total);
  }
  hipStream_t s = (hipStream_t)stream;
  if (debug_validate()) {
    st = decode_debug_check(kv, batch, seq_lens, offload_ratio, append ? 1 : 0, s);
    if (st != DKV_OK) return st;
  }
  dkv::DecodeArgs a = decode_args(kv, d, batch, num_q_heads, q, q_pos, seq_lens, offload_ratio, scale, rope_theta,
                                  workspace);
  a.fused = 1;
  a.new_tokens = append ? 1 : 0;
  a.out_o = out_o;
  a.out_lse = out_lse;
  a.pos_new = pos_new;
  hipError_t he;
  if (proj) {
    uint8_t* ws = static_cast<uint8_t*>(workspace) + d.proj_off;
    dkv::ProjArgs p{};
    p.x = static_cast<const uint16_t*>(x);
    p.wk = static_cast<const uint16_t*>(wk);
    p.wv = static_cast<const uint16_t*>(wv);
    p.n_new = batch;
    p.n_pad = (batch + 15) / 16 * 16;
    p.hidden = hidden;
    p.kv_dim = kvd;
    p.ksplit = hidden / 256;
    p.kslice = 256;
    const int64_t part = (int64_t)p.ksplit * p.n_pad * 2 * kvd * 4;
    p.partial = reinterpret_cast<float*>(ws);
    p.out = reinterpret_cast<float*>(ws + ((part + 255) / 256) * 256);
    TimedLaunch t_proj(DKV_KERNEL_APPEND, s);
    he = (hipError_t)dkv::launch_project(p, stream);
    t_proj.done();
    if (he != hipSuccess) return hip_err(he, "projection launch");
    a.kv_proj = p.out;
  } else if (append) {
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
  }
  if (kv->page_size > 0) {
    TimedLaunch t_tiers(DKV_KERNEL_TIERS, s);
    he = (hipError_t)dkv::launch_decode_tiers(a, const_cast<int32_t*>(a.tier_counts),
                                              const_cast<int32_t*>(a.tier_pages), stream);
    t_tiers.done();
    if (he != hipSuccess) return hip_err(he, "tier lists launch");
  }
  TimedLaunch t_attn(DKV_KERNEL_ATTN, s);
  he = (hipError_t)dkv::launch_decode(a, stream);
  t_attn.done();
  if (he != hipSuccess) return hip_err(he, "decode step launch");
  return ok();
}

dkv_status dkv_decode_step(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads, const void* q,
                           const int32_t* q_pos, const int32_t* seq_lens, const int32_t* pos_new, const void* x,
                           int32_t hidden, const void* wk, const void* wv, const void* k_new, const void* v_new,
                           double offload_ratio, float scale, double rope_theta, void* workspace,
                           size_t workspace_bytes, float* out_o, float* out_lse, void* stream) {
  return decode_step_impl(kv, batch, num_q_heads, q, q_pos, seq_lens, pos_new, x, hidden, wk, wv, k_new, v_new,
                          offload_ratio, scale, rope_theta, workspace, workspace_bytes, out_o, out_lse, stream);
}

dkv_status dkv_decode_step_static(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads, const void* q,
                                  const int32_t* q_pos, const int32_t* seq_lens, const int32_t* pos_new,
                                  const void* x, int32_t hidden, const void* wk, const void* wv, const void* k_new,
                                  const void* v_new, double offload_ratio, float scale, double rope_theta,
                                  float* out_o, float* out_lse, void* stream) {
  void* scratch = nullptr;
  size_t bytes = 0;
  hipError_t he = (hipError_t)dkv::decode_static_scratch(&scratch, &bytes);
  if (he != hipSuccess) return hip_err(he, "address of the static decode scratch");
  return decode_step_impl(kv, batch, num_q_heads, q, q_pos, seq_lens, pos_new, x, hidden, wk, wv, k_new, v_new,
                          offload_ratio, scale, rope_theta, scratch, bytes, out_o, out_lse, stream, true);
}

dkv_status dkv_decode_errors(const dkv_kv_desc* kv, const void* workspace, int32_t clear, int32_t* flags) {
  if (!kv || !workspace || !flags) return set_err(DKV_ERR_INVALID, "kv, workspace and flags are required");
  hipError_t he = hipDeviceSynchronize();
  const int32_t* w = static_cast<const int32_t*>(workspace) + dkv::decode_error_word();
  if (he == hipSuccess) he = hipMemcpy(flags, w, 4, hipMemcpyDeviceToHost);
  if (he == hipSuccess && clear) he = hipMemset(const_cast<int32_t*>(w), 0, 4);
  if (he == hipSuccess) he = hipDeviceSynchronize();
  if (he != hipSuccess) return hip_err(he, "reading the decode error word");
  return ok();
}

dkv_status dkv_decode_staged_plan(const dkv_kv_desc* kv, int32_t num_q_heads, int64_t seq_len, double offload_ratio,
                                  int32_t chunk_tokens, dkv_plan_info* info) {
  if (!info) return set_err(DKV_ERR_INVALID, "info is NULL");
  dkv_status st = validate_desc(kv);
  if (st != DKV_OK) return st;
  StagedLayout L;
  st = staged_layout(kv, num_q_heads, seq_len, offload_ratio, chunk_tokens, &L);
  if (st != DKV_OK) return st;
  const int64_t row_bytes = (int64_t)kv->num_kv_heads * kv->head_dim * 2;
  *info = dkv_plan_info{};
  info->workspace_bytes = (int64_t)L.total;
  info->num_splits = L.n_rows;
  info->host_items = L.n_chunks;
  info->host_chunk = L.chunk;
  info->host_bytes = L.nh * row_bytes * 2;
  info->dev_bytes = L.nd * row_bytes * 2;
  info->staged_bytes = L.nh * row_bytes * 2;
  return ok();
}

dkv_status dkv_decode_staged(const dkv_kv_desc* kv, int32_t num_q_heads, const void* q, const int32_t* q_pos,
                             int64_t seq_len, double offload_ratio, float scale, double rope_theta,
                             int32_t chunk_tokens, void* workspace, size_t workspace_bytes, float* out_o,
                             float* out_lse, void* stream) {
  dkv_status st = validate_desc(kv);
  if (st != DKV_OK) return st;
  if (!q || !q_pos || !workspace || !out_o)
    return set_err(DKV_ERR_INVALID, "q, q_pos, workspace and out_o are required");
  if ((uintptr_t)workspace % 256) return set_err(DKV_ERR_INVALID, "workspace must be 256-byte aligned");
  StagedLayout L;
  st = staged_layout(kv, num_q_heads, seq_len, offload_ratio, chunk_tokens, &L);
  if (st != DKV_OK) return st;
  if (workspace_bytes < L.total)
    return set_err(DKV_ERR_INVALID, "workspace too small: %zu < %zu bytes", workspace_bytes, L.total);
  int dev = 0;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return hip_err(he, "current device");
  if (dev < 0 || dev >= kMaxCopyDevices) return set_err(DKV_ERR_UNSUPPORTED, "device index %d", dev);
  hipStream_t s = (hipStream_t)stream;
  CopyEngine& ce = copy_engine();
  std::lock_guard<std::mutex> lk(ce.mu);
  if (!ce.stream[dev]) {  // the copy stream and its events, once per device (default priority)
    he = hipStreamCreateWithFlags(&ce.stream[dev], hipStreamNonBlocking);
    for (int k = 0; k < 4 && he == hipSuccess; ++k) he = hipEventCreateWithFlags(&ce.ev[dev][k], hipEventDisableTiming);
    if (he != hipSuccess) return hip_err(he, "copy stream");
  }
  hipStream_t cs = ce.stream[dev];
  hipEvent_t* copied = &ce.ev[dev][0];  // [2]
  hipEvent_t* freed = &ce.ev[dev][2];   // [2]
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const int hq = num_q_heads, D = kv->head_dim;
  const size_t row_bytes = (size_t)kv->num_kv_heads * D * 2;
  float* part_o = reinterpret_cast<float*>(ws + L.part_o_off);
  float* part_lse = reinterpret_cast<float*>(ws + L.part_lse_off);
  int32_t* ints = reinterpret_cast<int32_t*>(ws + L.ints_off);  // [n_rows] lengths, then offsets {0, n_rows}
  std::vector<int32_t> host_ints(L.n_rows + 2);
  for (int i = 0; i < L.n_chunks; ++i)
    host_ints[i] = (int32_t)std::min<int64_t>(L.chunk, L.nh - (int64_t)i * L.chunk);
  if (L.nd > 0) host_ints[L.n_chunks] = (int32_t)L.nd;
  host_ints[L.n_rows] = 0;
  host_ints[L.n_rows + 1] = L.n_rows;
  he = hipMemcpyAsync(ints, host_ints.data(), host_ints.size() * 4, hipMemcpyHostToDevice, s);
  if (he != hipSuccess) return hip_err(he, "chunk lengths upload");
  // the ring is free once earlier work on the stream is done
  he = hipEventRecord(freed[0], s);
  if (he == hipSuccess) he = hipEventRecord(freed[1], s);
  if (he != hipSuccess) return hip_err(he, "ring events");
  auto view_of = [&](void* k, void* v, int64_t rows, int64_t stride) {
    dkv_kv_desc w = *kv;
    w.host_k = w.host_v = nullptr;
    w.host_rows = w.host_stride = 0;
    w.dev_k = k;
    w.dev_v = v;
    w.dev_rows = rows;
    w.dev_stride = stride;
    return w;
  };
  // the HBM tier, on the compute stream, while the first chunk is copied
  if (L.nd > 0) {
    const dkv_kv_desc w = view_of(kv->dev_k, kv->dev_v, L.nd, L.nd);
    st = dkv_decode_step(&w, 1, hq, q, q_pos, ints + L.n_chunks, nullptr, nullptr, 0, nullptr, nullptr, nullptr,
                         nullptr, 0.0, scale, rope_theta, ws, L.ring_off, part_o + (size_t)L.n_chunks * hq * D,
                         part_lse + (size_t)L.n_chunks * hq, stream);
    if (st != DKV_OK) return st;
  }
  for (int i = 0; i < L.n_chunks; ++i) {
    const int slot = i & 1;
    uint8_t* rk = ws + L.ring_off + (size_t)(2 * slot) * L.ring_slot_bytes;
    uint8_t* rv = rk + L.ring_slot_bytes;
    const size_t bytes = (size_t)host_ints[i] * row_bytes;
    const size_t src_off = (size_t)i * L.chunk * row_bytes;
    he = hipStreamWaitEvent(cs, freed[slot], 0);
    if (he == hipSuccess)
      he = hipMemcpyAsync(rk, static_cast<const uint8_t*>(kv->host_k) + src_off, bytes, hipMemcpyDefault, cs);
    if (he == hipSuccess)
      he = hipMemcpyAsync(rv, static_cast<const uint8_t*>(kv->host_v) + src_off, bytes, hipMemcpyDefault, cs);
    if (he == hipSuccess) he = hipEventRecord(copied[slot], cs);
    if (he == hipSuccess) he = hipStreamWaitEvent(s, copied[slot], 0);
    if (he != hipSuccess) return hip_err(he, "staging copy");
    const dkv_kv_desc w = view_of(rk, rv, L.chunk, L.chunk);
    st = dkv_decode_step(&w, 1, hq, q, q_pos, ints + i, nullptr, nullptr, 0, nullptr, nullptr, nullptr, nullptr, 0.0,
                         scale, rope_theta, ws, L.ring_off, part_o + (size_t)i * hq * D, part_lse + (size_t)i * hq,
                         stream);
    if (st != DKV_OK) return st;
    he = hipEventRecord(freed[slot], s);
    if (he != hipSuccess) return hip_err(he, "ring events");
  }
  return dkv_merge_lse(part_o, part_lse, ints + L.n_rows, 1, hq, D, out_o, out_lse, stream);
}

dkv_status dkv_merge_lse(const float* part_o, const float* part_lse, const int32_t* split_offsets,
                         int32_t batch, int32_t num_q_heads, int32_t head_dim, float* out_o,
                         float* out_lse, void* stream) {
  if (!part_o || !part_lse || !split_offsets || !out_o)
    return set_err(DKV_ERR_INVALID, "part_o, part_lse, split_offsets and out_o are required");
  if (batch < 1 || num_q_heads < 1) return set_err(DKV_ERR_INVALID, "batch and num_q_heads must be >= 1");
  if (head_dim != 64 && head_dim != 128)
    return set_err(DKV_ERR_UNSUPPORTED, "head_dim %d not built (64 or 128)", head_dim);
  if ((int64_t)batch * num_q_heads > 0x7fffffff) return set_err(DKV_ERR_INVALID, "batch * heads too large");
  dkv::MergeArgs a{};
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.split_offsets = split_offsets;
  a.batch = batch;
  a.hq = num_q_heads;
  a.head_dim = head_dim;
  a.out_o = out_o;
  a.out_lse = out_lse;
  TimedLaunch tl(DKV_KERNEL_MERGE, (hipStream_t)stream);
  hipError_t he = (hipError_t)dkv::launch_merge(a, stream);
  tl.done();
  if (he != hipSuccess) return hip_err(he, "merge launch");
  return ok();
}

dkv_status dkv_linear_plan(int32_t m, int32_t out_features, int32_t in_features, double offload_ratio,
                           dkv_plan_info* info) {
  if (!info) return set_err(DKV_ERR_INVALID, "info is NULL");
  dkv_status st = validate_linear(m, out_features, in_features, offload_ratio);
  if (st != DKV_OK) return st;
  dkv::LinearShape z;
  st = get_linear_shape(out_features, in_features, offload_ratio, 0, &z);
  if (st != DKV_OK) return st;
  fill_linear_info(z, info);
  return ok();
}

dkv_status dkv_linear_plan_inspect(int32_t out_features, int32_t in_features, double offload_ratio,
                                   int32_t num_cus, int32_t* items, int32_t items_cap, dkv_plan_info* info) {
  dkv_status st = validate_linear(1, out_features, in_features, offload_ratio);
  if (st != DKV_OK) return st;
  if (num_cus < 1) return set_err(DKV_ERR_INVALID, "num_cus must be >= 1");
  dkv::LinearShape z;
  st = get_linear_shape(out_features, in_features, offload_ratio, num_cus, &z);
  if (st != DKV_OK) return st;
  std::vector<dkv::LinearItem> it;
  dkv::linear_items(z, out_features, in_features, &it);
  for (int i = 0; items && i < (int)it.size() && i < items_cap; ++i) {
    int32_t* o = items + 6 * (size_t)i;
    o[0] = it[i].pool; o[1] = it[i].row0; o[2] = it[i].n_rows; o[3] = it[i].k0; o[4] = it[i].k1; o[5] = it[i].slot;
  }
  if (info) fill_linear_info(z, info);
  return ok();
}

dkv_status dkv_linear_split(const void* host_w, const void* dev_w, int32_t out_features, int32_t in_features,
                            double offload_ratio, const void* x, int32_t m, float* y, void* workspace,
                            size_t workspace_bytes, void* stream) {
  dkv_status st = validate_linear(m, out_features, in_features, offload_ratio);
  if (st != DKV_OK) return st;
  if (!x || !y || !workspace) return set_err(DKV_ERR_INVALID, "x, y and workspace are required");
  if ((uintptr_t)workspace % 256) return set_err(DKV_ERR_INVALID, "workspace must be 256-byte aligned");
  if (((uintptr_t)x | (uintptr_t)host_w | (uintptr_t)dev_w) % 16)
    return set_err(DKV_ERR_INVALID, "x and the weights must be 16-byte aligned");
  dkv::LinearShape z;
  st = get_linear_shape(out_features, in_features, offload_ratio, 0, &z);
  if (st != DKV_OK) return st;
  if (z.n_host_items > 0 && !host_w) return set_err(DKV_ERR_INVALID, "host_w is required for offload_ratio > 0");
  if (z.n_dev_items > 0 && !dev_w) return set_err(DKV_ERR_INVALID, "dev_w is required for offload_ratio < 1");
  if (workspace_bytes < z.ws_bytes)
    return set_err(DKV_ERR_INVALID, "workspace too small: %zu < %zu bytes", workspace_bytes, z.ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  dkv::LinearArgs a{};
  a.counters = reinterpret_cast<int32_t*>(ws);
  a.n_host_items = z.n_host_items;
  a.n_dev_items = z.n_dev_items;
  a.host_wgs = z.host_wgs;
  a.dev_wgs = z.dev_wgs;
  a.n = out_features;
  a.k = in_features;
  a.n_host = z.n_host;
  a.bh = z.bh;
  a.kc_host = z.kc_host;
  a.kc_dev = z.kc_dev;
  a.sp_host = z.sp_host;
  a.sp_dev = z.sp_dev;
  a.p_host = z.sp_host > 1 ? z.n_host_items : 0;
  a.host_w = static_cast<const uint16_t*>(host_w);
  a.dev_w = static_cast<const uint16_t*>(dev_w);
  a.part = z.num_splits > 0 ? reinterpret_cast<float*>(ws + z.part_off) : nullptr;
  // tokens in launches of up to 64, one launch each (every launch leaves the
  // workspace counters at zero)
  for (int32_t m0 = 0; m0 < m; m0 += dkv::kLinMaxTokens) {
    a.m = std::min(dkv::kLinMaxTokens, m - m0);
    a.x = static_cast<const uint16_t*>(x) + (size_t)m0 * in_features;
    a.y = y + (size_t)m0 * out_features;
    TimedLaunch tl(DKV_KERNEL_LINEAR, s);
    hipError_t he = (hipError_t)dkv::launch_linear(a, stream);
    tl.done();
    if (he != hipSuccess) return hip_err(he, "linear launch");
  }
  return ok();
}

size_t dkv_append_workspace_bytes(int32_t n_new, int32_t hidden, int32_t kv_dim) {
  if (n_new <= 0 || hidden <= 0 || kv_dim <= 0) return 0;
  const int64_t n_pad = ((int64_t)n_new + 15) / 16 * 16;
  const int64_t ksplit = hidden / 256;
  const int64_t part = ksplit * n_pad * 2 * kv_dim * 4;
  const int64_t out = (int64_t)n_new * 2 * kv_dim * 4;
  return (size_t)(((part + 255) / 256) * 256 + out);
}

dkv_status dkv_project_rope_append(const dkv_kv_desc* kv, int32_t batch, const int32_t* seq_lens,
                                   double offload_ratio, int32_t n_new, const int32_t* seq_idx,
                                   const int32_t* pos, const void* x, int32_t hidden,
                                   const void* wk, const void* wv, const void* k_new,
                                   const void* v_new, double rope_theta, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  dkv_status st = validate_desc(kv);
  if (st != DKV_OK) return st;
  if (batch < 1) return set_err(DKV_ERR_INVALID, "batch must be >= 1");
  if (n_new < 0) return set_err(DKV_ERR_INVALID, "n_new must be >= 0");
  if (n_new == 0) return ok();
  if (!seq_idx || !pos) return set_err(DKV_ERR_INVALID, "seq_idx and pos are required");
  if (kv->page_size == 0) {
    if (!seq_lens) return set_err(DKV_ERR_INVALID, "contiguous placement needs seq_lens");
    if (validate_ratio(offload_ratio) != DKV_OK) return DKV_ERR_INVALID;
  }
  if (!(std::isfinite(rope_theta)) || rope_theta <= 0.0)
    return set_err(DKV_ERR_INVALID, "rope_theta must be > 0");
  const int32_t kvd = kv->num_kv_heads * kv->head_dim;
  const bool proj = x != nullptr;
  if (proj) {
    if (!wk || !wv) return set_err(DKV_ERR_INVALID, "projection mode needs wk and wv");
    if (hidden < 256 || hidden % 256)
      return set_err(DKV_ERR_UNSUPPORTED, "hidden %d must be a positive multiple of 256", hidden);
    if ((2 * kvd) % 64) return set_err(DKV_ERR_UNSUPPORTED, "2*Hkv*D must be a multiple of 64");
    const size_t need = dkv_append_workspace_bytes(n_new, hidden, kvd);
    if (!workspace || workspace_bytes < need)
      return set_err(DKV_ERR_INVALID, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
    if ((uintptr_t)workspace % 256) return set_err(DKV_ERR_INVALID, "workspace must be 256-byte aligned");
    if ((uintptr_t)x % 16 || (uintptr_t)wk % 16 || (uintptr_t)wv % 16)
      return set_err(DKV_ERR_INVALID, "x, wk, wv must be 16-byte aligned");
  } else {
    if (!k_new || !v_new) return set_err(DKV_ERR_INVALID, "no-projection mode needs k_new and v_new");
    if ((uintptr_t)k_new % 16 || (uintptr_t)v_new % 16)
      return set_err(DKV_ERR_INVALID, "k_new, v_new must be 16-byte aligned");
  }
  hipStream_t s = (hipStream_t)stream;
  if (debug_validate()) {
    std::vector<int32_t> si(n_new), ps(n_new), sl(kv->page_size == 0 ? batch : 0);
    hipError_t he = hipStreamSynchronize(s);
    if (he == hipSuccess) he = hipMemcpy(si.data(), seq_idx, 4 * (size_t)n_new, hipMemcpyDeviceToHost);
    if (he == hipSuccess) he = hipMemcpy(ps.data(), pos, 4 * (size_t)n_new, hipMemcpyDeviceToHost);
    if (he == hipSuccess && !sl.empty())
      he = hipMemcpy(sl.data(), seq_lens, 4 * (size_t)batch, hipMemcpyDeviceToHost);
    if (he != hipSuccess) return hip_err(he, "debug copy of append metadata");
    std::vector<int32_t> pt;
    if (kv->page_size > 0) {
      pt.resize((size_t)batch * kv->max_pages);
      he = hipMemcpy(pt.data(), kv->page_table, pt.size() * 4, hipMemcpyDeviceToHost);
      if (he != hipSuccess) return hip_err(he, "debug copy of page_table");
    }
    for (int i = 0; i < n_new; ++i) {
      const int b = si[i], p = ps[i];
      if (b < 0 || b >= batch || p < 0) return set_err(DKV_ERR_INVALID, "token %d: bad sequence/position", i);
      int64_t row;
      bool host;
      if (kv->page_size == 0) {
        const int L = sl[b];
        if (p >= L) return set_err(DKV_ERR_INVALID, "token %d: position %d >= seq_len %d", i, p, L);
        const int64_t nh = (int64_t)std::floor(offload_ratio * (double)L);
        host = p < nh;
        if (host && nh > kv->host_stride) return set_err(DKV_ERR_INVALID, "token %d: host_stride too small", i);
        if (!host && L - nh > kv->dev_stride) return set_err(DKV_ERR_INVALID, "token %d: dev_stride too small", i);
        row = host ? (int64_t)b * kv->host_stride + p : (int64_t)b * kv->dev_stride + (p - nh);
      } else {
        const int lp = p / kv->page_size;
        if (lp >= kv->max_pages) return set_err(DKV_ERR_INVALID, "token %d: page index beyond max_pages", i);
        const int32_t e = pt[(size_t)b * kv->max_pages + lp];
        if (e < 0) return set_err(DKV_ERR_INVALID, "token %d: unmapped page", i);
        host = (e & 1) != 0;
        row = (int64_t)(e >> 1) * kv->page_size + p % kv->page_size;
      }
      if (row >= (host ? kv->host_rows : kv->dev_rows))
        return set_err(DKV_ERR_INVALID, "token %d: row %lld beyond the pool", i, (long long)row);
    }
  }
  dkv::AppendArgs a{};
  a.batch = batch;
  a.n_new = n_new;
  a.seq_lens = seq_lens;
  a.ratio = offload_ratio;
  a.seq_idx = seq_idx;
  a.pos = pos;
  a.host_k = static_cast<uint16_t*>(kv->host_k);
  a.host_v = static_cast<uint16_t*>(kv->host_v);
  a.dev_k = static_cast<uint16_t*>(kv->dev_k);
  a.dev_v = static_cast<uint16_t*>(kv->dev_v);
  a.host_rows = kv->host_rows;
  a.dev_rows = kv->dev_rows;
  a.host_stride = kv->host_stride;
  a.dev_stride = kv->dev_stride;
  a.page_table = kv->page_table;
  a.max_pages = kv->max_pages;
  a.page_size = kv->page_size;
  a.hkv = kv->num_kv_heads;
  a.head_dim = kv->head_dim;
  a.freq = rope_freq(rope_theta, kv->head_dim);
  if (proj) {
    dkv::ProjArgs p{};
    p.x = static_cast<const uint16_t*>(x);
    p.wk = static_cast<const uint16_t*>(wk);
    p.wv = static_cast<const uint16_t*>(wv);
    p.n_new = n_new;
    p.n_pad = (n_new + 15) / 16 * 16;
    p.hidden = hidden;
    p.kv_dim = kvd;
    p.ksplit = hidden / 256;
    p.kslice = 256;
    const int64_t part = (int64_t)p.ksplit * p.n_pad * 2 * kvd * 4;
    p.partial = static_cast<float*>(workspace);
    p.out = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + ((part + 255) / 256) * 256);
    hipError_t he = (hipError_t)dkv::launch_project(p, stream);
    if (he != hipSuccess) return hip_err(he, "projection launch");
    a.kv_proj = p.out;
  } else {
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
  }
  TimedLaunch tl(DKV_KERNEL_APPEND, s);
  hipError_t he = (hipError_t)dkv::launch_append(a, stream);
  tl.done();
  if (he != hipSuccess) return hip_err(he, "append launch");
  return ok();
}

dkv_status dkv_host_alloc(size_t bytes, uint32_t flags, void** host_ptr, void** dev_ptr) {
  if (!host_ptr || !dev_ptr) return set_err(DKV_ERR_INVALID, "host_ptr and dev_ptr are required");
  if (bytes == 0) return set_err(DKV_ERR_INVALID, "bytes must be > 0");
  if (flags > DKV_HOST_NONCOHERENT) return set_err(DKV_ERR_INVALID, "unknown flags %u", flags);
  *host_ptr = nullptr;
  *dev_ptr = nullptr;
  unsigned hf = hipHostMallocMapped | hipHostMallocPortable |
                (flags == DKV_HOST_NONCOHERENT ? hipHostMallocNonCoherent : hipHostMallocCoherent);
  void* h = nullptr;
  hipError_t e = hipHostMalloc(&h, bytes, hf);
  if (e != hipSuccess || !h)
    return set_err(DKV_ERR_NOMEM, "hipHostMalloc(%zu): %s", bytes, hipGetErrorString(e));
  void* d = nullptr;
  e = hipHostGetDevicePointer(&d, h, 0);
  if (e != hipSuccess) {
    (void)hipHostFree(h);
    return hip_err(e, "hipHostGetDevicePointer");
  }
  *host_ptr = h;
  *dev_ptr = d;
  return ok();
}

dkv_status dkv_host_free(void* host_ptr) {
  if (!host_ptr) return ok();
  // kernels queued on any stream may still read the block
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_err(e, "hipDeviceSynchronize before hipHostFree");
  e = hipHostFree(host_ptr);
  if (e != hipSuccess) return hip_err(e, "hipHostFree");
  return ok();
}

dkv_status dkv_probe_read(const void* src, const void* src2, size_t bytes, int32_t nwg, int32_t mode,
                          int32_t iters, void* dma_dst, const void* dma_src_host,
                          dkv_bw_result* out, void* stream) {
  if (!src || !out) return set_err(DKV_ERR_INVALID, "src and out are required");
  if (bytes < 16 || bytes % 16) return set_err(DKV_ERR_INVALID, "bytes must be a positive multiple of 16");
  if (nwg < 1 || nwg > 65535 || iters < 1 || iters > 1000)
    return set_err(DKV_ERR_INVALID, "nwg in [1,65535], iters in [1,1000]");
  if (mode < 0 || mode > 7 || (mode & 6) == 6) return set_err(DKV_ERR_INVALID, "mode: bit 0, and bit 1 or bit 2");
  if ((mode & 4) && (bytes % 2048 || nwg % ((src2 ? 2 : 1) * 8)))
    return set_err(DKV_ERR_INVALID, "segment mode needs 2 KiB rows and 8 workgroups per buffer");
  if ((uintptr_t)src % 16 || (uintptr_t)src2 % 16) return set_err(DKV_ERR_INVALID, "sources must be 16-byte aligned");
  if (src2 && nwg % 2) return set_err(DKV_ERR_INVALID, "two buffers need an even workgroup count");
  const double total_bytes = (double)bytes * (src2 ? 2 : 1);
  hipStream_t s = (hipStream_t)stream;
  float* sink = nullptr;
  hipError_t e = hipMalloc(&sink, 256);
  if (e != hipSuccess) return hip_err(e, "probe sink");
  std::vector<hipEvent_t> ev(2 * (size_t)iters, nullptr);
  for (auto& x : ev)
    if (e == hipSuccess) e = hipEventCreate(&x);
  dkv_status st = DKV_OK;
  // best of `iters` timed passes, each bracketed by its own events
  auto timed = [&](auto launch, double* best_ms, double* avg_ms) -> hipError_t {
    hipError_t r = launch();  // warm-up
    for (int i = 0; i < iters && r == hipSuccess; ++i) {
      r = hipEventRecord(ev[2 * i], s);
      if (r == hipSuccess) r = launch();
      if (r == hipSuccess) r = hipEventRecord(ev[2 * i + 1], s);
    }
    if (r == hipSuccess) r = hipEventSynchronize(ev[2 * iters - 1]);
    double best = 1e30, sum = 0.0;
    for (int i = 0; i < iters && r == hipSuccess; ++i) {
      float ms = 0.f;
      r = hipEventElapsedTime(&ms, ev[2 * i], ev[2 * i + 1]);
      best = std::min(best, (double)ms);
      sum += ms;
    }
    *best_ms = best;
    *avg_ms = sum / iters;
    return r;
  };
  double best = 0.0, avg = 0.0;
  if (e == hipSuccess)
    e = timed([&] { return (hipError_t)dkv::launch_probe_read(src, src2, bytes, nwg, mode, sink, stream); }, &best,
              &avg);
  if (e != hipSuccess) {
    st = hip_err(e, "probe kernel");
  } else {
    out->read_ms = best;
    out->read_gbs = total_bytes / (best * 1e6);
    out->dma_gbs = 0.0;
    if (dma_dst && dma_src_host) {
      e = timed([&] { return hipMemcpyAsync(dma_dst, dma_src_host, bytes, hipMemcpyHostToDevice, s); }, &best, &avg);
      if (e != hipSuccess)
        st = hip_err(e, "probe DMA");
      else
        out->dma_gbs = (double)bytes / (best * 1e6);
    }
  }
  for (auto& x : ev)
    if (x) (void)hipEventDestroy(x);
  (void)hipFree(sink);
  if (st != DKV_OK) return st;
  return ok();
}

dkv_status dkv_kernel_timing(int32_t enable) {
  Timing& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  t.on = enable != 0;
  return ok();
}

dkv_status dkv_kernel_timing_read(int32_t kernel, int32_t* count, double* total_ms) {
  if (kernel < 0 || kernel > DKV_KERNEL_TIERS || !count || !total_ms)
    return set_err(DKV_ERR_INVALID, "kernel id in [0,4] and outputs required");
  Timing& t = timing();
  std::vector<std::pair<hipEvent_t, hipEvent_t>> rec;
  {
    std::lock_guard<std::mutex> lk(t.mu);
    rec.swap(t.rec[kernel]);
  }
  double tot = 0.0;
  hipError_t err = hipSuccess;
  for (auto& p : rec) {
    float ms = 0.f;
    if (err == hipSuccess) err = hipEventSynchronize(p.second);
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, p.first, p.second);
    tot += ms;
  }
  {
    std::lock_guard<std::mutex> lk(t.mu);
    for (auto& p : rec) {
      t.pool.push_back(p.first);
      t.pool.push_back(p.second);
    }
  }
  if (err != hipSuccess) return hip_err(err, "kernel timing");
  *count = (int32_t)rec.size();
  *total_ms = tot;
  return ok();
}

dkv_status dkv_attn_trace(void* dev_buffer, int32_t capacity_wgs) {
  if (capacity_wgs < 0 || (capacity_wgs > 0 && !dev_buffer))
    return set_err(DKV_ERR_INVALID, "trace buffer required for a positive capacity");
  std::lock_guard<std::mutex> lk(g_trace_mu);
  g_trace_buf = capacity_wgs > 0 ? static_cast<uint64_t*>(dev_buffer) : nullptr;
  g_trace_cap = capacity_wgs;
  return ok();
}

dkv_status dkv_prefill_plan(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads,
                            const int32_t* q_start, const int32_t* q_pos0, const int32_t* seq_lens,
                            double offload_ratio, dkv_plan_info* info) {
  if (!info) return set_err(DKV_ERR_INVALID, "info is NULL");
  dkv_status st = validate_desc(kv);
  if (st != DKV_OK) return st;
  if (kv->page_size == 0 && validate_ratio(offload_ratio) != DKV_OK) return DKV_ERR_INVALID;
  std::shared_ptr<PlanEntry> e;
  st = get_prefill_plan(kv, batch, num_q_heads, q_start, q_pos0, seq_lens,
                        kv->page_size == 0 ? offload_ratio : 0.0, &e);
  if (st != DKV_OK) return st;
  fill_info(e->lay, prefill_ws_bytes(e->lay, num_q_heads, kv->num_kv_heads, kv->head_dim), info);
  return ok();
}

// Staging copy, query rotation and the prefill kernel, after the plan image is
// in the workspace.  fresh_k/fresh_v: the new rows (fused step) or NULL.
// rope_table_ready: the rotation table (and the split offsets) were written
// earlier in the call.
static dkv_status prefill_stages(const dkv_kv_desc* kv, int32_t num_q_heads, const void* q,
                                 const dkv::PlanLayout& L, uint8_t* ws, float scale, double rope_theta,
                                 const uint16_t* fresh_k, const uint16_t* fresh_v, float* part_o,
                                 float* part_lse, int32_t* split_offsets, void* stream,
                                 const dkv::AppendArgs* writers = nullptr, bool rope_table_ready = false) {
  hipStream_t s = (hipStream_t)stream;
  double* rope_cs = reinterpret_cast<double*>(ws + L.blob_bytes);
  const size_t pool_elems = (size_t)L.stage_rows * kv->num_kv_heads * kv->head_dim;
  uint16_t* stage_k = reinterpret_cast<uint16_t*>(ws + prefill_stage_off(L, num_q_heads, kv->head_dim));
  uint16_t* stage_v = stage_k + pool_elems;
  hipError_t he;
  if (L.n_stage_tiles > 0) {
    dkv::StageArgs sa{};
    sa.tiles = reinterpret_cast<const dkv::StageTile*>(ws + L.stage_tiles_off);
    sa.n_tiles = L.n_stage_tiles;
    sa.row_chunks = kv->num_kv_heads * kv->head_dim / 8;
    sa.src_k = static_cast<const uint16_t*>(kv->host_k);
    sa.src_v = static_cast<const uint16_t*>(kv->host_v);
    sa.dst_k = stage_k;
    sa.dst_v = stage_v;
    int cus = tuning_snapshot(nullptr).num_cus;
    if (cus <= 0) cus = device_cus(nullptr);
    TimedLaunch t_stage(DKV_KERNEL_STAGE, s);
    he = (hipError_t)dkv::launch_stage(sa, std::max(64, std::max(cus, 1) / 2), stream);
    t_stage.done();
    if (he != hipSuccess) return hip_err(he, "stage launch");
  }
  const float scale_log2 = scale * 1.44269504088896340736f;
  if (!rope_table_ready) {
    TimedLaunch t_rope(DKV_KERNEL_ROPE_Q, s);
    he = (hipError_t)dkv::launch_rope_table(reinterpret_cast<const int32_t*>(ws + L.rowpos_off), L.n_rows,
                                            kv->head_dim, rope_freq(rope_theta, kv->head_dim), rope_cs,
                                            reinterpret_cast<const int32_t*>(ws + L.offsets_off),
                                            split_offsets, stream);
    t_rope.done();
    if (he != hipSuccess) return hip_err(he, "rope table launch");
  }
  dkv::PrefillArgs a{};
  a.host_items = reinterpret_cast<const dkv::PrefillItem*>(ws + L.items_off);
  a.dev_items = a.host_items + L.n_host_items;
  a.pages = kv->page_size > 0 ? reinterpret_cast<const int32_t*>(ws + L.plist_off) : nullptr;
  a.unit_counters = reinterpret_cast<int32_t*>(ws + L.counters_off);
  a.n_host_items = L.n_host_items;
  a.n_dev_items = L.n_dev_items;
  a.host_wgs = L.host_wgs;
  a.dev_wgs = L.dev_wgs;
  a.dev_queues = L.dev_queues;
  a.host_k = static_cast<const uint16_t*>(kv->host_k);
  a.host_v = static_cast<const uint16_t*>(kv->host_v);
  a.dev_k = static_cast<const uint16_t*>(kv->dev_k);
  a.dev_v = static_cast<const uint16_t*>(kv->dev_v);
  a.stage_k = stage_k;
  a.stage_v = stage_v;
  a.fresh_k = fresh_k;
  a.fresh_v = fresh_v;
  a.page_shift = kv->page_size > 0 ? log2i(kv->page_size) : 0;
  a.hq = num_q_heads;
  a.hkv = kv->num_kv_heads;
  a.head_dim = kv->head_dim;
  a.part_o = part_o;
  a.part_lse = part_lse;
  if (writers) {
    // a few workgroups keep the host link busy with the slot writes
    a.app = *writers;
    const int32_t tuned = tuning_snapshot(nullptr).writer_wgs;
    a.writer_wgs = tuned > 0 ? std::min<int32_t>(tuned, std::max<int32_t>(1, writers->n_new))
                             : (int32_t)std::min<int64_t>(64, std::max<int64_t>(1, writers->n_new / 8));
  }
  a.q = static_cast<const uint16_t*>(q);
  a.rope_cs = rope_cs;
  a.scale_log2 = scale_log2;
  TimedLaunch t_attn(DKV_KERNEL_PREFILL, s);
  he = (hipError_t)dkv::launch_prefill(a, stream);
  t_attn.done();
  if (he != hipSuccess) return hip_err(he, "prefill launch");
  return DKV_OK;
}

dkv_status dkv_prefill_attn_split(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads,
                                  const void* q, const int32_t* q_start, const int32_t* q_pos0,
                                  const int32_t* seq_lens, double offload_ratio, float scale,
                                  double rope_theta, void* workspace, size_t workspace_bytes,
                                  float* part_o, float* part_lse, int32_t* split_offsets,
                                  int32_t num_splits_cap, void* stream) {
  dkv_status st = validate_desc(kv);
  if (st != DKV_OK) return st;
  if (kv->page_size == 0 && validate_ratio(offload_ratio) != DKV_OK) return DKV_ERR_INVALID;
  if (batch < 1 || !q_start) return set_err(DKV_ERR_INVALID, "batch >= 1 and q_start are required");
  if (q_start[batch] == 0) return ok();  // no query rows: nothing is read or written
  if (!q || !part_o || !part_lse || !split_offsets || !workspace)
    return set_err(DKV_ERR_INVALID, "q, part_o, part_lse, split_offsets and workspace are required");
  if ((uintptr_t)q % 16) return set_err(DKV_ERR_INVALID, "q must be 16-byte aligned");
  if (!(std::isfinite(scale)) || !(std::isfinite(rope_theta)) || rope_theta <= 0.0)
    return set_err(DKV_ERR_INVALID, "scale must be finite and rope_theta > 0");
  if ((uintptr_t)workspace % 256) return set_err(DKV_ERR_INVALID, "workspace must be 256-byte aligned");
  std::shared_ptr<PlanEntry> e;
  st = get_prefill_plan(kv, batch, num_q_heads, q_start, q_pos0, seq_lens,
                        kv->page_size == 0 ? offload_ratio : 0.0, &e);
  if (st != DKV_OK) return st;
  const dkv::PlanLayout& L = e->lay;
  if (L.n_rows == 0) return ok();  // no query rows
  const size_t need = prefill_ws_bytes(L, num_q_heads, kv->num_kv_heads, kv->head_dim);
  if (workspace_bytes < need)
    return set_err(DKV_ERR_INVALID, "workspace too small: %zu < %zu bytes", workspace_bytes, need);
  if (num_splits_cap < L.num_splits)
    return set_err(DKV_ERR_INVALID, "num_splits_cap %d < %d splits", num_splits_cap, L.num_splits);
  hipStream_t s = (hipStream_t)stream;
  if (stream_capturing(s)) {
    std::lock_guard<std::mutex> lk(cache().mu);
    e->captured = true;
  }
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipError_t he = hipMemcpyAsync(ws, e->pinned, e->bytes, hipMemcpyHostToDevice, s);
  if (he != hipSuccess) return hip_err(he, "plan upload");
  st = prefill_stages(kv, num_q_heads, q, L, ws, scale, rope_theta, nullptr, nullptr, part_o, part_lse,
                      split_offsets, stream);
  return st == DKV_OK ? ok() : st;
}

dkv_status dkv_prefill_fused_plan(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads,
                                  const int32_t* q_start, const int32_t* q_pos0, const int32_t* seq_lens,
                                  double offload_ratio, int32_t hidden, dkv_plan_info* info) {
  if (!info) return set_err(DKV_ERR_INVALID, "info is NULL");
  dkv_status st = validate_desc(kv);
  if (st != DKV_OK) return st;
  if (kv->page_size == 0 && validate_ratio(offload_ratio) != DKV_OK) return DKV_ERR_INVALID;
  std::shared_ptr<PlanEntry> e;
  st = get_prefill_plan(kv, batch, num_q_heads, q_start, q_pos0, seq_lens,
                        kv->page_size == 0 ? offload_ratio : 0.0, &e, true);
  if (st != DKV_OK) return st;
  fill_info(e->lay, fused_layout(e->lay, num_q_heads, kv->num_kv_heads, kv->head_dim, hidden).total, info);
  return ok();
}

dkv_status dkv_prefill_fused(const dkv_kv_desc* kv, int32_t batch, int32_t num_q_heads, const void* q,
                             const int32_t* q_start, const int32_t* q_pos0, const int32_t* seq_lens,
                             double offload_ratio, float scale, double rope_theta, const void* x,
                             int32_t hidden, const void* wk, const void* wv, const void* k_new,
                             const void* v_new, void* workspace, size_t workspace_bytes, float* out_o,
                             float* out_lse, void* stream) {
  dkv_status st = validate_desc(kv);
  if (st != DKV_OK) return st;
  if (kv->page_size == 0 && validate_ratio(offload_ratio) != DKV_OK) return DKV_ERR_INVALID;
  if (batch < 1 || !q_start) return set_err(DKV_ERR_INVALID, "batch >= 1 and q_start are required");
  if (q_start[batch] == 0) return ok();  // no new rows: nothing is read or written
  if (!q || !out_o || !workspace) return set_err(DKV_ERR_INVALID, "q, out_o and workspace are required");
  if ((uintptr_t)q % 16) return set_err(DKV_ERR_INVALID, "q must be 16-byte aligned");
  if (!(std::isfinite(scale)) || !(std::isfinite(rope_theta)) || rope_theta <= 0.0)
    return set_err(DKV_ERR_INVALID, "scale must be finite and rope_theta > 0");
  if ((uintptr_t)workspace % 256) return set_err(DKV_ERR_INVALID, "workspace must be 256-byte aligned");
  const int32_t kvd = kv->num_kv_heads * kv->head_dim;
  const bool proj = x != nullptr;
  if (proj) {
    if (!wk || !wv) return set_err(DKV_ERR_INVALID, "projection mode needs wk and wv");
    if (hidden < 256 || hidden % 256)
      return set_err(DKV_ERR_UNSUPPORTED, "hidden %d must be a positive multiple of 256", hidden);
    if ((2 * kvd) % 64) return set_err(DKV_ERR_UNSUPPORTED, "2*Hkv*D must be a multiple of 64");
    if ((uintptr_t)x % 16 || (uintptr_t)wk % 16 || (uintptr_t)wv % 16)
      return set_err(DKV_ERR_INVALID, "x, wk, wv must be 16-byte aligned");
  } else {
    if (!k_new || !v_new) return set_err(DKV_ERR_INVALID, "no-projection mode needs k_new and v_new");
    if ((uintptr_t)k_new % 16 || (uintptr_t)v_new % 16)
      return set_err(DKV_ERR_INVALID, "k_new, v_new must be 16-byte aligned");
  }
  std::shared_ptr<PlanEntry> e;
  st = get_prefill_plan(kv, batch, num_q_heads, q_start, q_pos0, seq_lens,
                        kv->page_size == 0 ? offload_ratio : 0.0, &e, true);
  if (st != DKV_OK) return st;
  const dkv::PlanLayout& L = e->lay;
  if (L.n_rows == 0) return ok();
  const FusedLayout F = fused_layout(L, num_q_heads, kv->num_kv_heads, kv->head_dim, proj ? hidden : 0);
  if (workspace_bytes < F.total)
    return set_err(DKV_ERR_INVALID, "workspace too small: %zu < %zu bytes", workspace_bytes, F.total);
  hipStream_t s = (hipStream_t)stream;
  if (stream_capturing(s)) {
    std::lock_guard<std::mutex> lk(cache().mu);
    e->captured = true;
  }
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hipError_t he = hipMemcpyAsync(ws, e->pinned, e->bytes, hipMemcpyHostToDevice, s);
  if (he != hipSuccess) return hip_err(he, "plan upload");
  uint16_t* fresh_k = reinterpret_cast<uint16_t*>(ws + F.fresh_off);
  uint16_t* fresh_v = fresh_k + (size_t)L.n_rows * kvd;
  const bool direct = L.num_splits == L.n_rows && out_lse != nullptr;
  int32_t* offs = reinterpret_cast<int32_t*>(ws + F.offsets_off);
  double* rope_cs = reinterpret_cast<double*>(ws + L.blob_bytes);
  // 1. new K/V (projection) -> cache slots and the fresh rows
  dkv::AppendArgs a{};
  a.batch = batch;
  a.n_new = L.n_rows;
  a.seq_lens = reinterpret_cast<const int32_t*>(ws + L.seqlens_off);
  a.ratio = kv->page_size == 0 ? offload_ratio : 0.0;
  a.seq_idx = reinterpret_cast<const int32_t*>(ws + L.rowseq_off);
  a.pos = reinterpret_cast<const int32_t*>(ws + L.rowpos_off);
  a.host_k = static_cast<uint16_t*>(kv->host_k);
  a.host_v = static_cast<uint16_t*>(kv->host_v);
  a.dev_k = static_cast<uint16_t*>(kv->dev_k);
  a.dev_v = static_cast<uint16_t*>(kv->dev_v);
  a.host_rows = kv->host_rows;
  a.dev_rows = kv->dev_rows;
  a.host_stride = kv->host_stride;
  a.dev_stride = kv->dev_stride;
  a.page_table = kv->page_table;
  a.max_pages = kv->max_pages;
  a.page_size = kv->page_size;
  a.hkv = kv->num_kv_heads;
  a.head_dim = kv->head_dim;
  a.freq = rope_freq(rope_theta, kv->head_dim);
  a.fresh_k = fresh_k;
  a.fresh_v = fresh_v;
  if (proj) {
    dkv::ProjArgs p{};
    p.x = static_cast<const uint16_t*>(x);
    p.wk = static_cast<const uint16_t*>(wk);
    p.wv = static_cast<const uint16_t*>(wv);
    p.n_new = L.n_rows;
    p.n_pad = (L.n_rows + 15) / 16 * 16;
    p.hidden = hidden;
    p.kv_dim = kvd;
    p.ksplit = hidden / 256;
    p.kslice = 256;
    const int64_t part = (int64_t)p.ksplit * p.n_pad * 2 * kvd * 4;
    p.partial = reinterpret_cast<float*>(ws + F.proj_off);
    p.out = reinterpret_cast<float*>(ws + F.proj_off + ((part + 255) / 256) * 256);
    he = (hipError_t)dkv::launch_project(p, stream);
    if (he != hipSuccess) return hip_err(he, "projection launch");
    a.kv_proj = p.out;
  } else {
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
  }
  // Does any new row land in a host slot?  Those writes cross the link and
  // are done by writer workgroups of the prefill launch, concurrently with
  // attention; when every slot is in HBM the append writes them itself.
  bool host_slots = false;
  for (int b = 0; b < batch && !host_slots; ++b) {
    const int64_t p0 = q_pos0[b], p1 = p0 + (q_start[b + 1] - q_start[b]);
    if (p1 <= p0) continue;
    if (kv->page_size == 0) {
      host_slots = p0 < (int64_t)std::floor(a.ratio * (double)seq_lens[b]);
    } else {
      for (int64_t pg = p0 / kv->page_size; pg <= (p1 - 1) / kv->page_size && !host_slots; ++pg) {
        const int32_t e = pg < kv->max_pages ? kv->page_table_host[(int64_t)b * kv->max_pages + pg] : -1;
        host_slots = e >= 0 && (e & 1);
      }
    }
  }
  // the HBM copy of the new rows first (attention reads it), with the rows'
  // rotation table (the queries use it)
  {
    dkv::AppendArgs af = a;
    af.skip_slots = host_slots ? 1 : 0;
    TimedLaunch tl(DKV_KERNEL_APPEND, s);
    he = (hipError_t)dkv::launch_append_rows(af, rope_cs, reinterpret_cast<const int32_t*>(ws + L.offsets_off),
                                             offs, stream);
    tl.done();
    if (he != hipSuccess) return hip_err(he, "append launch");
  }
  // 2. staging of re-read prefix rows, query rotation, prefill attention.
  // With one split per row the split slot of row r is r and its normalised
  // partial is the result: it is written to the output and no merge runs.
  float* part_o = direct ? out_o : reinterpret_cast<float*>(ws + F.part_o_off);
  float* part_lse = direct ? out_lse : reinterpret_cast<float*>(ws + F.part_lse_off);
  st = prefill_stages(kv, num_q_heads, q, L, ws, scale, rope_theta, fresh_k, fresh_v, part_o, part_lse, offs,
                      stream, host_slots ? &a : nullptr, true);
  if (st != DKV_OK) return st;
  if (direct) return ok();
  // 3. merge of each row's splits
  dkv::MergeArgs m{};
  m.part_o = part_o;
  m.part_lse = part_lse;
  m.split_offsets = offs;
  m.batch = L.n_rows;
  m.hq = num_q_heads;
  m.head_dim = kv->head_dim;
  m.out_o = out_o;
  m.out_lse = out_lse;
  TimedLaunch tm(DKV_KERNEL_MERGE, s);
  he = (hipError_t)dkv::launch_merge(m, stream);
  tm.done();
  if (he != hipSuccess) return hip_err(he, "merge launch");
  return ok();
}

}  // extern "C"
