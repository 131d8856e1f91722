// C ABI of the block-sparse attention library: request validation, the
// online request path (mask state -> statistics transfer -> regime lookup and
// ranked fallback -> launch preparation), plan lifetime and kernel dispatch.
//
// Tessera paper, section 3 "Online request path" and section 5.2 "Online
// Plan Selection": the runtime builds the shared mask state on the GPU,
// transfers only its scalar statistics to the host, selects the first
// eligible plan of the regime's ranking (the key's base plan on a lookup
// miss), derives only that plan's metadata from the block-CSR, binds the
// temporary workspace and invokes the plan's kernels.
#include <algorithm>
#include <chrono>
#include <new>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/bsa.h"
#include "bsa_internal.h"
#include "catalog.h"

using namespace bsa;

namespace {

thread_local std::string g_err;

bsa_status fail(bsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define HIP_TRY(expr)                                                                        \
  do {                                                                                       \
    hipError_t e_ = (expr);                                                                  \
    if (e_ != hipSuccess)                                                                    \
      return fail(BSA_ERR_HIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_), __FILE__, \
                  __LINE__);                                                                 \
  } while (0)

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- device memory cache ------------------------------------------------------
// Plans come and go once per request; the cache keeps freed device blocks per
// (device, size class) so steady-state requests make no hipMalloc calls.
struct Pool {
  std::mutex mu;
  std::map<std::pair<int, size_t>, std::vector<void*>> free;
  size_t idle = 0;
  static constexpr size_t kIdleCap = size_t(16) << 30;
};
Pool g_pool;

size_t size_class(size_t bytes) {
  if (bytes <= 65536) return 65536;
  size_t p = 65536;
  while (p < bytes) p <<= 1;
  // eight classes per octave
  const size_t step = p / 16;
  return ((bytes + step - 1) / step) * step;
}

struct DevBuf {
  void* ptr = nullptr;
  size_t cap = 0;
  int dev = -1;
  bool pooled = false;  // from the cache (returned to it on release)
};

hipError_t pool_alloc(int dev, size_t bytes, DevBuf* b) {
  const size_t cap = size_class(bytes ? bytes : 1);
  {
    std::lock_guard<std::mutex> lk(g_pool.mu);
    auto it = g_pool.free.find({dev, cap});
    if (it != g_pool.free.end() && !it->second.empty()) {
      b->ptr = it->second.back();
      it->second.pop_back();
      g_pool.idle -= cap;
      b->cap = cap;
      b->dev = dev;
      b->pooled = true;
      return hipSuccess;
    }
  }
  hipError_t e = hipMalloc(&b->ptr, cap);
  if (e != hipSuccess) return e;
  b->cap = cap;
  b->dev = dev;
  b->pooled = true;
  return hipSuccess;
}

void pool_release(DevBuf* b) {
  if (!b->ptr) return;
  if (!b->pooled) {  // carved from the static scratch: nothing to return
    b->ptr = nullptr;
    return;
  }
  std::lock_guard<std::mutex> lk(g_pool.mu);
  if (g_pool.idle + b->cap > Pool::kIdleCap) {
    (void)hipFree(b->ptr);
  } else {
    g_pool.free[{b->dev, b->cap}].push_back(b->ptr);
    g_pool.idle += b->cap;
  }
  b->ptr = nullptr;
}

// Bump allocator over the library's fixed per-device scratch array, for the
// entry point that allocates nothing: buffers are carved 256-byte aligned and
// are never returned one by one (the next call starts over).
struct Arena {
  char* base = nullptr;
  size_t cap = 0;
  size_t used = 0;
  size_t left() const { return cap - std::min(cap, (used + 255) & ~size_t(255)); }
};

hipError_t arena_alloc(Arena* a, int dev, size_t bytes, DevBuf* b) {
  const size_t off = (a->used + 255) & ~size_t(255);
  const size_t n = bytes ? bytes : 1;
  if (off > a->cap || n > a->cap - off) return hipErrorOutOfMemory;
  b->ptr = a->base + off;
  b->cap = n;
  b->dev = dev;
  b->pooled = false;
  a->used = off + n;
  return hipSuccess;
}

// 256-byte aligned size of a buffer carved from the arena
size_t arena_size(size_t bytes) { return ((bytes ? bytes : 1) + 255) & ~size_t(255); }

// Largest column array (sized for every mask block) that is allocated before
// the statistics are known, so that the compaction can be queued ahead of the
// host's selection and overlap it.  1 GiB covers masks of 2.7e8 blocks (the
// largest benchmark masks need 0.2-0.3 GB); the array comes from the device
// memory cache and holds only the active blocks' columns.
constexpr size_t kEarlyCompactBytes = size_t(1) << 30;

// Fine-grained (coherent) pinned host memory, one per thread, that the mask
// state kernels write the statistics into directly: the single device-to-host
// crossing of the request path needs no separate copy.
MaskStats* pinned_stats() {
  thread_local MaskStats* p = nullptr;
  if (!p) {
    if (hipHostMalloc((void**)&p, sizeof(MaskStats), hipHostMallocCoherent | hipHostMallocPortable) !=
        hipSuccess)
      p = nullptr;
    else
      std::memset(p, 0, sizeof(MaskStats));  // sequence numbers start at 1
  }
  return p;
}

CompareResult* pinned_compare() {
  thread_local CompareResult* p = nullptr;
  if (!p) {
    if (hipHostMalloc((void**)&p, sizeof(CompareResult), hipHostMallocCoherent | hipHostMallocPortable) !=
        hipSuccess)
      p = nullptr;
    else
      std::memset(p, 0, sizeof(CompareResult));
  }
  return p;
}

// Spins until the GPU has stored `seq` into *flag (a system-scope release
// after the record's other fields), checking the stream now and then so that
// a failed or finished stream ends the wait.
bsa_status wait_host_seq(const unsigned long long* flag, unsigned long long seq, hipStream_t s,
                         const char* what) {
  for (unsigned spin = 1;; ++spin) {
    if (__atomic_load_n(flag, __ATOMIC_ACQUIRE) == seq) return BSA_OK;
    if ((spin & 255) == 0) {
      const hipError_t q = hipStreamQuery(s);
      if (q == hipSuccess) {
        if (__atomic_load_n(flag, __ATOMIC_ACQUIRE) == seq) return BSA_OK;
        return fail(BSA_ERR_HIP, "%s were not delivered", what);
      }
      if (q != hipErrorNotReady) return fail(BSA_ERR_HIP, "waiting for the %s: %s", what, hipGetErrorString(q));
    }
  }
}

int device_cus(int dev) {
  static std::mutex mu;
  static std::map<int, int> cache;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  cache[dev] = n;
  return n;
}

int wg_per_cu_cached(int tq, int tkv, int d, bool stream = false) {
  static std::mutex mu;
  static std::map<int, int> cache;
  const int key = (tq << 20) | (tkv << 8) | d | (stream ? 1 << 30 : 0);
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int n = attn_wg_per_cu(tq, tkv, d, stream);
  if (n <= 0) n = 1;
  cache[key] = n;
  return n;
}

// Split-K rule of the "balance" organizations: a query tile's traversal is cut
// when it holds more entries than 2/split of the even share of all entries
// over the resident workgroup slots of the device (at least 4 entries per
// partition).
struct PlanShape {
  DimMap mq, mk;
  int split = 0;           // entries per partition, 0 = never split
  int split_min = 0;       // rows of more entries are split
  int groups = 0;          // > 0: stream organization over this many workgroups
  int64_t tasks_upper = 0;
  int64_t slots_upper = 0;
  int64_t ws_bytes = 0;
  int64_t nqt = 0;
  int nqt_head = 0;
};

PlanShape shape_plan(const CatalogEntry& e, const bsa_request& r, const MaskStats& st, int dev) {
  PlanShape p;
  p.mq = map_dim(r.block_q, e.tq, kMinCoarsenBlockQ);
  p.mk = map_dim(r.block_kv, e.tkv, 1);
  p.nqt_head = (int)cdiv(r.N, e.tq);
  p.nqt = (int64_t)r.H * p.nqt_head;
  // entries visited over all query tiles (upper bound for coarsened lists)
  const int64_t W = (int64_t)p.mq.refine * (int64_t)st.nnz;
  const int64_t row_max = (int64_t)p.mq.coarsen * st.max_row_nnz;
  int split = 0, split_min = 0;
  if (r.force_split == BSA_SPLIT_STREAM) {
    // one equal range of entries per resident workgroup slot
    const int64_t slots = (int64_t)device_cus(dev) * wg_per_cu_cached(e.tq, e.tkv, e.d, true);
    p.groups = (int)std::max<int64_t>(1, std::min<int64_t>(slots, kMaxStreamGroups));
    p.tasks_upper = p.nqt + p.groups;
    p.slots_upper = 2 * (int64_t)p.groups;
    p.ws_bytes = p.slots_upper * (int64_t)e.tq * (2 * 4 + e.d * 4);
    return p;
  }
  if (r.force_split > 0) {
    split = split_min = r.force_split;
  } else if (r.force_split < 0 && e.split) {
    const int64_t slots = (int64_t)device_cus(dev) * wg_per_cu_cached(e.tq, e.tkv, e.d);
    split = (int)std::max<int64_t>(4, cdiv(2 * std::max<int64_t>(W, 1), slots * e.split));
    // rows up to kSplitRowFactor times the mean row length stay whole
    const int64_t mean = cdiv(std::max<int64_t>(W, 1), p.nqt);
    split_min = (int)std::min<int64_t>(std::max<int64_t>(split, kSplitRowFactor * mean), 1 << 30);
    if (row_max <= split_min) split = split_min = 0;
  }
  p.split = split;
  p.split_min = split_min;
  if (split > 0) {
    p.tasks_upper = p.nqt + W / split + 1;
    p.slots_upper = 2 * W / split + 1;
  } else {
    p.tasks_upper = p.nqt;
    p.slots_upper = 0;
  }
  // per slot and query row: fp32 m and l, then d fp32 partial outputs
  p.ws_bytes = p.slots_upper * (int64_t)e.tq * (2 * 4 + e.d * 4);
  return p;
}

}  // namespace

// Per-device cache of HIP events (timing and non-timing), so that creating
// and destroying a plan per request creates no events in steady state.
namespace {
std::mutex g_ev_mu;
std::map<std::pair<int, bool>, std::vector<hipEvent_t>> g_ev_cache;

hipError_t event_get(int dev, bool timing, hipEvent_t* e) {
  {
    std::lock_guard<std::mutex> lk(g_ev_mu);
    auto& v = g_ev_cache[{dev, timing}];
    if (!v.empty()) {
      *e = v.back();
      v.pop_back();
      return hipSuccess;
    }
  }
  return hipEventCreateWithFlags(e, timing ? hipEventDefault : hipEventDisableTiming);
}

void event_put(int dev, bool timing, hipEvent_t e) {
  if (!e) return;
  std::lock_guard<std::mutex> lk(g_ev_mu);
  g_ev_cache[{dev, timing}].push_back(e);
}
}  // namespace

struct bsa_plan {
  Arena* arena = nullptr;  // non-null: every buffer comes from the static scratch
  bsa_request req{};    // batch folded into H (req.H = batch * heads, req.batch = 1)
  int32_t heads = 0;    // heads per batch entry, as requested
  int dev = 0;
  int nqb = 0, nkb = 0;
  const CatalogEntry* entry = nullptr;
  PlanShape shape;
  int ntr = 0;  // tile-list rows per head
  int64_t grid = 0;
  bool coarse = false;
  MaskStats stats{};
  bsa_plan_info info{};
  DevBuf stats_dev, row_cnt, row_ptr, row_part, cols, rsig, trow_cnt, trow_ptr_buf, tcol_buf, tbits_buf, tsig_buf,
      parts, slot_off, tasks, ws, seg_ptr, spec_parts, spec_slot, spec_tasks, split_tiles, spec_split, xq;
  const int32_t* trow_ptr = nullptr;
  const int32_t* tcol = nullptr;
  const int32_t* tsig = nullptr;  // per tile-list row: the column of its median entry
  const uint32_t* tbits = nullptr;
  // stream-order bookkeeping, updated by runs of a const plan
  mutable hipEvent_t ev[3] = {nullptr, nullptr, nullptr};  // timing events of bsa_run_timed (created on first use)
  hipEvent_t done = nullptr;          // recorded after plan creation and after untimed runs
  mutable hipEvent_t last = nullptr;  // recorded after the plan's latest stream work (done or ev[2])

  hipError_t alloc(size_t bytes, DevBuf* b) {
    return arena ? arena_alloc(arena, dev, bytes, b) : pool_alloc(dev, bytes, b);
  }

  ~bsa_plan() {
    for (DevBuf* b : {&stats_dev, &row_cnt, &row_ptr, &row_part, &cols, &rsig, &trow_cnt, &trow_ptr_buf, &tcol_buf,
                      &tbits_buf, &tsig_buf, &parts, &slot_off, &tasks, &ws, &seg_ptr, &spec_parts, &spec_slot,
                      &spec_tasks, &split_tiles, &spec_split, &xq})
      pool_release(b);
    for (auto& e : ev) event_put(dev, true, e);
    event_put(dev, false, done);
  }
};

namespace {

// The request with its batch entries folded into the head count: every
// (batch entry, head) pair is an independent head of the mask and the tasks.
bsa_request folded(const bsa_request& r) {
  bsa_request f = r;
  if (r.batch > 1) f.H = (int32_t)((int64_t)r.H * r.batch);
  f.batch = 1;
  return f;
}

bsa_status validate_request(const bsa_request* rq) {
  if (!rq) return fail(BSA_ERR_INVALID_ARG, "request is NULL");
  if (rq->H < 1 || rq->N < 1) return fail(BSA_ERR_INVALID_ARG, "H and N must be >= 1 (H=%d N=%d)", rq->H, rq->N);
  if (rq->batch < 0) return fail(BSA_ERR_INVALID_ARG, "batch %d < 0", rq->batch);
  if ((int64_t)rq->H * std::max(rq->batch, 1) >= (int64_t(1) << 31))
    return fail(BSA_ERR_UNSUPPORTED, "batch * H too large");
  if (!rq->mask) return fail(BSA_ERR_INVALID_ARG, "mask pointer is NULL");
  if (rq->dtype != BSA_DTYPE_BF16) return fail(BSA_ERR_UNSUPPORTED, "dtype %d unsupported (bf16 only)", rq->dtype);
  if (rq->layout != BSA_LAYOUT_HND && rq->layout != BSA_LAYOUT_NHD)
    return fail(BSA_ERR_UNSUPPORTED, "layout %d unsupported", rq->layout);
  // the kernels address one head's rows through 32-bit byte offsets
  const int64_t row_bytes = (int64_t)rq->d * 2 * (rq->layout == BSA_LAYOUT_NHD ? rq->H : 1);
  if ((int64_t)rq->N * row_bytes >= (int64_t(1) << 31))
    return fail(BSA_ERR_UNSUPPORTED, "N * row stride too large for layout %d", rq->layout);
  const bsa_request fr = folded(*rq);
  const bsa_request* r = &fr;
  if (r->d != 32 && r->d != 64 && r->d != 128 && r->d != 256)
    return fail(BSA_ERR_UNSUPPORTED, "head dim %d unsupported (32, 64, 128, 256)", r->d);
  if (!pow2(r->block_q) || r->block_q < 16 || r->block_q > 256)
    return fail(BSA_ERR_UNSUPPORTED, "block_q %d unsupported (power of two in [16, 256])", r->block_q);
  if (!pow2(r->block_kv) || r->block_kv < 16 || r->block_kv > 256)
    return fail(BSA_ERR_UNSUPPORTED, "block_kv %d unsupported (power of two in [16, 256])", r->block_kv);
  const int64_t nqb = cdiv(r->N, r->block_q), nkb = cdiv(r->N, r->block_kv);
  if ((int64_t)r->H * nqb * nkb >= (int64_t(1) << 31))
    return fail(BSA_ERR_UNSUPPORTED, "mask has %lld blocks (limit 2^31)", (long long)((int64_t)r->H * nqb * nkb));
  if ((int64_t)r->H * r->N >= (int64_t(1) << 31))
    return fail(BSA_ERR_UNSUPPORTED, "H*N too large");
  if (r->force_plan >= (int)catalog().size() || r->force_plan < -1)
    return fail(BSA_ERR_INVALID_ARG, "force_plan %d out of range", r->force_plan);
  if (r->force_split < -1 && r->force_split != BSA_SPLIT_STREAM)
    return fail(BSA_ERR_INVALID_ARG, "force_split %d invalid", r->force_split);
  if (r->workspace_limit < 0) return fail(BSA_ERR_INVALID_ARG, "negative workspace limit");
  return BSA_OK;
}

}  // namespace

// ---- plan cache (warm exact repeats) -------------------------------------------
struct bsa_plan_cache {
  struct Entry {
    bsa_request key{};  // mask pointer cleared
    int dev = 0;
    DevBuf mask_copy;
    int64_t bytes = 0;
    hipEvent_t copied = nullptr;  // recorded after the mask copy
    bsa_plan* plan = nullptr;
    DevBuf guard;  // task-count word of this plan's speculative runs
    uint64_t last_use = 0;
  };
  int capacity = 4;
  int64_t max_bytes = 0;
  std::vector<Entry> entries;
  std::map<int, DevBuf> flags;  // per device: int32[kMaxCompare], zero between checks
  uint64_t tick = 0;
  std::mutex mu;
};

namespace {

bool same_request(const bsa_request& a, const bsa_request& b) {
  return a.H == b.H && std::max(a.batch, 1) == std::max(b.batch, 1) && a.N == b.N && a.d == b.d &&
         a.block_q == b.block_q && a.block_kv == b.block_kv && a.dtype == b.dtype && a.layout == b.layout && a.force_plan == b.force_plan &&
         a.force_split == b.force_split && a.workspace_limit == b.workspace_limit;
}

void drop_entry(bsa_plan_cache::Entry& e);

struct RunIO {
  const void *q, *k, *v;
  void* o;
};

}  // namespace

static bsa_status run_impl(const bsa_plan* p, const void* q, const void* k, const void* v, void* o,
                           hipStream_t s, bool timed, float* attn_ms, float* merge_ms,
                           const unsigned long long* guard);

namespace {

// Looks the request up in the cache (candidates: same request on this device,
// most recently used first, compared with the request mask on the GPU) and
// returns a cached plan on an exact repeat, else plans, caches and returns a
// new one.  With io: also runs the returned plan on io.  The most recently
// used candidate then runs speculatively right behind the comparison, guarded
// by its verdict, so the host's wait for the verdict overlaps that run.
bsa_status cache_acquire(bsa_plan_cache* c, const bsa_request* req, hipStream_t s, const RunIO* io,
                         bsa_plan** out, int32_t* hit) {
  if (!c || !out || !hit) return fail(BSA_ERR_INVALID_ARG, "NULL argument");
  const bsa_status vs = validate_request(req);
  if (vs != BSA_OK) return vs;
  if (io && (!io->q || !io->k || !io->v || !io->o)) return fail(BSA_ERR_INVALID_ARG, "NULL tensor pointer");
  std::lock_guard<std::mutex> lk(c->mu);
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  const int64_t bytes = (int64_t)folded(*req).H * cdiv(req->N, req->block_q) * cdiv(req->N, req->block_kv);
  *hit = 0;
  *out = nullptr;
  std::vector<int> cand;
  for (int i = 0; i < (int)c->entries.size(); ++i)
    if (c->entries[i].dev == dev && same_request(c->entries[i].key, *req)) cand.push_back(i);
  std::sort(cand.begin(), cand.end(),
            [&](int a, int b) { return c->entries[a].last_use > c->entries[b].last_use; });
  if ((int)cand.size() > kMaxCompare) cand.resize(kMaxCompare);
  if (!cand.empty()) {
    CompareResult* host = pinned_compare();
    if (!host) return fail(BSA_ERR_NO_MEMORY, "pinned host allocation failed");
    DevBuf& fl = c->flags[dev];
    if (!fl.ptr) {
      HIP_TRY(pool_alloc(dev, sizeof(int32_t) * kMaxCompare, &fl));
      HIP_TRY(hipMemset(fl.ptr, 0, sizeof(int32_t) * kMaxCompare));
    }
    CompareArgs a{};
    a.mask = req->mask;
    a.ncand = (int32_t)cand.size();
    for (int k = 0; k < a.ncand; ++k) {
      a.cand[k] = (const uint8_t*)c->entries[cand[k]].mask_copy.ptr;
      HIP_TRY(hipStreamWaitEvent(s, c->entries[cand[k]].copied, 0));  // copy made on another stream
    }
    a.bytes = bytes;
    a.flags = (int32_t*)fl.ptr;
    // the guard word belongs to the speculated plan, so a run of it still
    // queued on another stream never sees another request's verdict
    bsa_plan* spec = c->entries[cand[0]].plan;
    if (io) {
      a.spec_ntasks = &((const MaskStats*)spec->stats_dev.ptr)->n_tasks;
      a.guard = (unsigned long long*)c->entries[cand[0]].guard.ptr;
    }
    thread_local unsigned long long seq = 0;  // the host record is per thread
    ++seq;
    HIP_TRY(launch_mask_compare(a, host, seq, s));
    if (io) {
      const bsa_status rs = run_impl(spec, io->q, io->k, io->v, io->o, s, false, nullptr, nullptr, a.guard);
      if (rs != BSA_OK) return rs;
    }
    const bsa_status ws = wait_host_seq(&host->seq, seq, s, "mask comparison results");
    if (ws != BSA_OK) return ws;
    for (int k = 0; k < a.ncand; ++k) {
      if (!host->differs[k]) {
        bsa_plan_cache::Entry& e = c->entries[cand[k]];
        e.last_use = ++c->tick;
        *out = e.plan;
        *hit = 1;
        if (io && k > 0) return run_impl(e.plan, io->q, io->k, io->v, io->o, s, false, nullptr, nullptr, nullptr);
        return BSA_OK;
      }
    }
  }
  // miss: plan, keep a copy of the mask, evict the least recently used
  bsa_plan* p = nullptr;
  const bsa_status st = bsa_plan_create(req, s, &p);
  if (st != BSA_OK) return st;
  bsa_plan_cache::Entry e;
  e.key = *req;
  e.key.mask = nullptr;
  e.dev = dev;
  e.bytes = bytes;
  e.plan = p;
  e.last_use = ++c->tick;
  hipError_t he = pool_alloc(dev, (size_t)bytes, &e.mask_copy);
  if (he == hipSuccess) he = pool_alloc(dev, sizeof(unsigned long long), &e.guard);
  if (he == hipSuccess) he = hipMemcpyAsync(e.mask_copy.ptr, req->mask, (size_t)bytes, hipMemcpyDeviceToDevice, s);
  if (he == hipSuccess) he = event_get(dev, false, &e.copied);
  if (he == hipSuccess) he = hipEventRecord(e.copied, s);
  if (he != hipSuccess) {
    drop_entry(e);
    return fail(BSA_ERR_HIP, "caching the mask: %s", hipGetErrorString(he));
  }
  c->entries.push_back(e);
  auto total = [&]() {
    int64_t t = 0;
    for (auto& x : c->entries) t += x.bytes;
    return t;
  };
  while ((int)c->entries.size() > c->capacity ||
         (c->max_bytes > 0 && total() > c->max_bytes && c->entries.size() > 1)) {
    int lru = -1;
    for (int i = 0; i < (int)c->entries.size(); ++i)
      if (c->entries[i].plan != p && (lru < 0 || c->entries[i].last_use < c->entries[lru].last_use)) lru = i;
    if (lru < 0) break;
    drop_entry(c->entries[lru]);
    c->entries.erase(c->entries.begin() + lru);
  }
  *out = p;
  if (io) return run_impl(p, io->q, io->k, io->v, io->o, s, false, nullptr, nullptr, nullptr);
  return BSA_OK;
}

}  // namespace

namespace {

// Task-list prediction for repeated request keys: the catalog entry the last
// request of the same key (device, geometry, options) selected.  When that
// entry maps both dimensions without coarsening, its task builder can be
// queued right behind the mask-state kernels, before the host has read the
// statistics, deriving its split size on the device; if the host's selection
// agrees, the plan takes that task list and launches no builder of its own.
struct PredKey {
  int dev, H, N, d, bq, bkv, dtype, layout, force_plan, force_split;
  int64_t ws_limit;
  bool operator<(const PredKey& o) const {
    return std::tie(dev, H, N, d, bq, bkv, dtype, layout, force_plan, force_split, ws_limit) <
           std::tie(o.dev, o.H, o.N, o.d, o.bq, o.bkv, o.dtype, o.layout, o.force_plan, o.force_split, o.ws_limit);
  }
};
std::mutex g_pred_mu;
std::map<PredKey, int> g_pred;
constexpr size_t kMaxPredKeys = 256;

PredKey pred_key(int dev, const bsa_request& r) {
  return PredKey{dev, r.H, r.N, r.d, r.block_q, r.block_kv, (int)r.dtype, r.layout, r.force_plan, r.force_split,
                 r.workspace_limit};
}

// The entry can be predicted: uncoarsened in both dimensions and organized
// by k_tasks with the plan's own split rule or none, in an order that needs
// no column list (the speculative builder runs before the compaction).
bool predictable(const CatalogEntry& e, const bsa_request& r) {
  if (r.force_split != -1 && r.force_split != 0) return false;
  if (e.order == 2) return false;
  const DimMap mq = map_dim(r.block_q, e.tq, kMinCoarsenBlockQ), mk = map_dim(r.block_kv, e.tkv, 1);
  return mq.ok && mk.ok && mq.coarsen == 1 && mk.coarsen == 1;
}

int pred_lookup(const PredKey& k) {
  std::lock_guard<std::mutex> lk(g_pred_mu);
  auto it = g_pred.find(k);
  return it == g_pred.end() ? -1 : it->second;
}

void pred_store(const PredKey& k, int id) {
  std::lock_guard<std::mutex> lk(g_pred_mu);
  if (id < 0) {
    g_pred.erase(k);
    return;
  }
  if (g_pred.size() >= kMaxPredKeys && !g_pred.count(k)) g_pred.clear();
  g_pred[k] = id;
}

}  // namespace

extern "C" {

const char* bsa_status_string(int32_t s) {
  switch (s) {
    case BSA_OK: return "BSA_OK";
    case BSA_ERR_INVALID_ARG: return "BSA_ERR_INVALID_ARG";
    case BSA_ERR_UNSUPPORTED: return "BSA_ERR_UNSUPPORTED";
    case BSA_ERR_NO_MEMORY: return "BSA_ERR_NO_MEMORY";
    case BSA_ERR_HIP: return "BSA_ERR_HIP";
    case BSA_ERR_TABLE: return "BSA_ERR_TABLE";
    default: return "BSA_ERR_UNKNOWN";
  }
}

const char* bsa_last_error(void) { return g_err.c_str(); }

int32_t bsa_catalog_size(void) { return (int32_t)catalog().size(); }

bsa_status bsa_catalog_get(int32_t id, bsa_catalog_entry* out) {
  if (!out || id < 0 || id >= (int)catalog().size()) return fail(BSA_ERR_INVALID_ARG, "bad catalog id %d", id);
  const CatalogEntry& e = catalog()[id];
  std::memset(out, 0, sizeof *out);
  out->id = e.id;
  out->tile_q = e.tq;
  out->tile_kv = e.tkv;
  out->d = e.d;
  out->split = e.split;
  out->xcd_remap = e.xcd_remap;
  out->order = e.order;
  std::snprintf(out->name, sizeof out->name, "%s", e.name.c_str());
  return BSA_OK;
}

const char* bsa_catalog_hash(void) {
  static std::string s = [] {
    char buf[32];
    std::snprintf(buf, sizeof buf, "%016llx", (unsigned long long)catalog_hash_value());
    return std::string(buf);
  }();
  return s.c_str();
}

const char* bsa_table_version(void) {
  thread_local std::string v;
  v = table_version();
  return v.c_str();
}

bsa_status bsa_table_load(const char* path) {
  std::string err;
  bsa_status st = table_load_file(path, &err);
  if (st != BSA_OK) return fail(st, "%s", err.c_str());
  return BSA_OK;
}

bsa_status bsa_plan_eligible(int32_t id, const bsa_request* req, int32_t* out) {
  if (!req || !out || id < 0 || id >= (int)catalog().size())
    return fail(BSA_ERR_INVALID_ARG, "bad arguments to bsa_plan_eligible");
  std::string why;
  *out = eligible(catalog()[id], folded(*req), -1, &why) ? 1 : 0;
  return BSA_OK;
}

bsa_status bsa_select(const bsa_request* req, double density, double run_coverage, double row_skew,
                      int32_t* plan_id, int32_t* regime) {
  if (!req || !plan_id || !regime) return fail(BSA_ERR_INVALID_ARG, "NULL argument to bsa_select");
  const bsa_request fr = folded(*req);
  Selection s = lookup(fr, density, run_coverage, row_skew);
  *regime = s.regime;
  for (int c : s.candidates) {
    if (eligible(catalog()[c], fr, -1, nullptr)) {
      *plan_id = c;
      return BSA_OK;
    }
  }
  *plan_id = -1;
  return fail(BSA_ERR_UNSUPPORTED, "no eligible plan for B=(%d,%d) d=%d", req->block_q, req->block_kv, req->d);
}

bsa_status bsa_base_plan(const bsa_request* req, int32_t* plan_id) {
  if (!req || !plan_id) return fail(BSA_ERR_INVALID_ARG, "NULL argument to bsa_base_plan");
  *plan_id = base_plan(folded(*req));
  if (*plan_id < 0)
    return fail(BSA_ERR_UNSUPPORTED, "no eligible base plan for B=(%d,%d) d=%d", req->block_q, req->block_kv,
                req->d);
  return BSA_OK;
}

// Device bytes a candidate plan adds to the shared mask state when its
// buffers are carved from the arena (tile list of a coarsened mapping, task
// list, split bookkeeping, split-K workspace), each rounded as the arena does.
static size_t plan_bytes(const CatalogEntry& e, const bsa_request& r, const PlanShape& sh, const MaskStats& st,
                         int nqb, int nkb) {
  (void)nkb;
  const size_t nnz = std::max<size_t>((size_t)st.nnz, 1);
  const size_t nqt = (size_t)sh.nqt;
  size_t b = 0;
  if (sh.mq.coarsen > 1 || sh.mk.coarsen > 1) {
    const size_t ntrows = (size_t)r.H * (size_t)cdiv(nqb, sh.mq.coarsen);
    b += 2 * arena_size(sizeof(int32_t) * ntrows) + arena_size(sizeof(int32_t) * (ntrows + 1)) +
         arena_size(sizeof(int32_t) * nnz) + arena_size(sizeof(uint32_t) * nnz);
  }
  b += 2 * arena_size(sizeof(int32_t) * nqt) + arena_size(sizeof(Task) * (size_t)std::max<int64_t>(sh.tasks_upper, 1));
  if (sh.groups > 0) b += arena_size(sizeof(int32_t) * (size_t)(sh.groups + 1));
  else if (sh.split > 0) b += arena_size(sizeof(int32_t) * nqt);
  if (sh.slots_upper > 0) b += arena_size((size_t)sh.ws_bytes);
  if (sh.groups == 0 && e.xcd_remap > 0) b += arena_size(8 * sizeof(unsigned long long));  // XCD queues
  return b;
}

// Plan creation.  arena == nullptr: buffers from the device memory cache,
// statistics through the thread's coherent host record.  Otherwise every
// buffer is carved from the arena (the static scratch), the statistics come
// back by one stream-ordered copy, no task list is built speculatively, and
// candidate plans whose buffers do not fit the arena's remaining space are
// ineligible (the workspace condition of section 4.4).
static bsa_status plan_create_impl(const bsa_request* req, hipStream_t s, std::unique_ptr<bsa_plan>& p,
                                   Arena* arena) {
  bsa_status vs = validate_request(req);
  if (vs != BSA_OK) return vs;
  const int32_t heads = req->H;
  const bsa_request fr = folded(*req);
  req = &fr;
  p.reset(new bsa_plan());
  p->arena = arena;
  p->heads = heads;
  // On an error return, kernels already queued may still use the plan's
  // buffers: wait for the stream before they go back to the cache.
  struct DrainOnError {
    std::unique_ptr<bsa_plan>& plan;
    hipStream_t stream;
    bool ok = false;
    ~DrainOnError() {
      if (plan && !ok) (void)hipStreamSynchronize(stream);
    }
  } drain{p, s};
  p->req = *req;
  p->req.mask = nullptr;  // not retained
  HIP_TRY(hipGetDevice(&p->dev));
  const bsa_request& r = *req;
  p->nqb = (int)cdiv(r.N, r.block_q);
  p->nkb = (int)cdiv(r.N, r.block_kv);
  const int nrows = r.H * p->nqb;

  // ---- shared mask state: counts, offsets, columns, statistics ---------------
  MaskStats* host = nullptr;
  if (arena) {
    // the mask state's own buffers must fit before anything is launched
    const size_t need = arena_size(sizeof(MaskStats)) + 2 * arena_size(sizeof(int32_t) * ((size_t)nrows + 1)) +
                        (mask_small_ok(r.mask, nrows, p->nkb)
                             ? arena_size(sizeof(int32_t) * (size_t)nrows * (size_t)p->nkb)
                             : arena_size(sizeof(int32_t) * (size_t)nrows) +
                                   arena_size(sizeof(RowPartial) * (size_t)row_count_blocks(nrows)));
    if (need > arena->left())
      return fail(BSA_ERR_UNSUPPORTED, "request needs %zu bytes of mask state, the static scratch holds %zu",
                  need, arena->cap);
  } else {
    host = pinned_stats();
    if (!host) return fail(BSA_ERR_NO_MEMORY, "pinned host allocation failed");
  }
  HIP_TRY(p->alloc(sizeof(MaskStats), &p->stats_dev));
  HIP_TRY(p->alloc(sizeof(int32_t) * ((size_t)nrows + 1), &p->row_ptr));
  HIP_TRY(p->alloc(sizeof(int32_t) * ((size_t)nrows + 1), &p->rsig));
  MaskStats* dst = (MaskStats*)p->stats_dev.ptr;
  // speculative task list of the entry this request key selected last time
  // (not with the static scratch: its space goes to the selected plan)
  const PredKey pkey = pred_key(p->dev, r);
  const int pred_id = arena ? -1 : pred_lookup(pkey);
  bool spec_launched = false;
  // Allocates the speculative buffers and fills `ts` (ts.enabled stays 0
  // when there is no usable prediction).
  auto prepare_spec = [&](TaskSpec& ts) -> hipError_t {
    ts = TaskSpec{};
    if (pred_id < 0 || pred_id >= (int)catalog().size()) return hipSuccess;
    const CatalogEntry& e = catalog()[pred_id];
    if (!predictable(e, r) || !attn_launcher(e.tq, e.tkv, e.d)) return hipSuccess;
    const DimMap mq = map_dim(r.block_q, e.tq, kMinCoarsenBlockQ);
    const int nqt_head = (int)cdiv(r.N, e.tq);
    const int64_t nqt = (int64_t)r.H * nqt_head;
    const int dev_split = r.force_split == 0 ? 0 : e.split;
    const int64_t slots = (int64_t)device_cus(p->dev) * wg_per_cu_cached(e.tq, e.tkv, e.d);
    // W / split <= slots * split share / 2 for the balance rule
    const int64_t cap = nqt + (dev_split > 0 ? slots * dev_split / 2 + 2 : 0);
    hipError_t err;
    if ((err = p->alloc(sizeof(int32_t) * (size_t)nqt, &p->spec_parts)) != hipSuccess) return err;
    if ((err = p->alloc(sizeof(int32_t) * (size_t)nqt, &p->spec_slot)) != hipSuccess) return err;
    if ((err = p->alloc(sizeof(Task) * (size_t)std::max<int64_t>(cap, 1), &p->spec_tasks)) != hipSuccess)
      return err;
    if (dev_split > 0 && (err = p->alloc(sizeof(int32_t) * (size_t)nqt, &p->spec_split)) != hipSuccess)
      return err;
    ts.enabled = 1;
    ts.H = r.H;
    ts.nqt_head = nqt_head;
    ts.ntr = p->nqb;
    ts.refine_q = mq.refine;
    ts.order = e.order;
    ts.dev_split = dev_split;
    ts.slots = (int32_t)slots;
    ts.parts = (int32_t*)p->spec_parts.ptr;
    ts.slot_base = (int32_t*)p->spec_slot.ptr;
    ts.tasks = (Task*)p->spec_tasks.ptr;
    ts.split_tiles = (int32_t*)p->spec_split.ptr;
    return hipSuccess;
  };
  thread_local unsigned long long seq = 0;  // the host statistics buffer is per thread
  ++seq;
  const size_t cols_bound = sizeof(int32_t) * (size_t)nrows * (size_t)p->nkb;
  bool early_compact;
  if (mask_small_ok(r.mask, nrows, p->nkb)) {
    // small mask: counts, statistics, scan and compaction in one launch
    early_compact = true;
    HIP_TRY(p->alloc(cols_bound, &p->cols));
    // (with a prediction, the same kernel also builds the speculative list)
    TaskSpec ts;
    HIP_TRY(prepare_spec(ts));
    HIP_TRY(launch_mask_small(r.mask, nrows, p->nkb, (int32_t*)p->row_ptr.ptr, (int32_t*)p->cols.ptr,
                              (int32_t*)p->rsig.ptr, dst, host, seq, s, ts));
    spec_launched = ts.enabled != 0;
  } else {
    HIP_TRY(p->alloc(sizeof(int32_t) * (size_t)nrows, &p->row_cnt));
    const int npart = row_count_blocks(nrows);
    HIP_TRY(p->alloc(sizeof(RowPartial) * (size_t)npart, &p->row_part));
    RowPartial* part = (RowPartial*)p->row_part.ptr;
    HIP_TRY(launch_row_count(r.mask, nrows, p->nkb, (int32_t*)p->row_cnt.ptr, part, s));
    HIP_TRY(launch_scan((int32_t*)p->row_cnt.ptr, (int32_t*)p->row_ptr.ptr, nrows, part, npart, dst, host, seq,
                        s));
    TaskSpec ts;
    HIP_TRY(prepare_spec(ts));
    if (ts.enabled) {
      HIP_TRY(launch_tasks((const int32_t*)p->row_ptr.ptr, ts.H, ts.nqt_head, ts.ntr, ts.refine_q, 0, 0, ts.order, 0,
                           ts.parts, ts.slot_base, ts.tasks, dst, s, ts.dev_split, ts.slots, ts.split_tiles));
      spec_launched = true;
    }
    // When a column array sized for every block is modest, the compaction is
    // queued before the statistics synchronization, so it overlaps the host's
    // wait and plan selection (not with the static scratch, whose space is
    // sized by the exact count instead).
    early_compact = !arena && cols_bound <= kEarlyCompactBytes;
    if (early_compact) {
      HIP_TRY(p->alloc(cols_bound, &p->cols));
      HIP_TRY(launch_compact(r.mask, nrows, p->nkb, (int32_t*)p->row_ptr.ptr, (int32_t*)p->cols.ptr,
                             (int32_t*)p->rsig.ptr, s));
    }
  }
  // Wait for the statistics alone (the compaction may still run): spin on the
  // sequence number the scan kernel stores last.  With the static scratch:
  // one stream-ordered copy of the device record and a stream synchronization.
  if (host) {
    const bsa_status ws = wait_host_seq(&host->seq, seq, s, "mask statistics");
    if (ws != BSA_OK) return ws;
    std::memcpy(&p->stats, host, sizeof(MaskStats));
  } else {
    HIP_TRY(hipMemcpyAsync(&p->stats, dst, sizeof(MaskStats), hipMemcpyDeviceToHost, s));
    HIP_TRY(hipStreamSynchronize(s));
  }
  const double total_blocks = (double)r.H * p->nqb * p->nkb;
  const double density = p->stats.nnz / total_blocks;
  const double runcov = p->stats.nnz ? (double)p->stats.long_run / (double)p->stats.nnz : 0.0;
  const double skew = p->stats.nnz ? (double)p->stats.max_row_nnz * nrows / (double)p->stats.nnz : 0.0;

  // ---- regime lookup and ranked fallback ------------------------------------
  const auto t0 = std::chrono::steady_clock::now();
  Selection sel;
  if (r.force_plan >= 0) {
    sel.regime = -2;
    sel.candidates = {r.force_plan};
  } else {
    sel = lookup(r, density, runcov, skew);
  }
  const CatalogEntry* chosen = nullptr;
  PlanShape shape;
  std::string why = "no candidate";
  // with the static scratch: the bytes left once the block-CSR columns
  // (compacted after the statistics) are carved
  const size_t nnz_cols =
      early_compact ? 0 : arena_size(sizeof(int32_t) * std::max<size_t>((size_t)p->stats.nnz, 1));
  const size_t arena_left = arena ? (arena->left() > nnz_cols ? arena->left() - nnz_cols : 0) : 0;
  if (arena && arena->left() < nnz_cols)
    return fail(BSA_ERR_UNSUPPORTED, "request needs %zu bytes of block-CSR columns, %zu of the %zu-byte static "
                "scratch are left", nnz_cols, arena->left(), arena->cap);
  for (int c : sel.candidates) {
    const CatalogEntry& e = catalog()[c];
    if (!attn_launcher(e.tq, e.tkv, e.d)) continue;
    PlanShape sh = shape_plan(e, r, p->stats, p->dev);
    if (arena && plan_bytes(e, r, sh, p->stats, p->nqb, p->nkb) > arena_left) {
      why = "buffers exceed the static scratch";
      continue;
    }
    if (eligible(e, r, sh.ws_bytes, &why)) {
      chosen = &e;
      shape = sh;
      break;
    }
  }
  const auto t1 = std::chrono::steady_clock::now();
  if (!chosen)
    return fail(BSA_ERR_UNSUPPORTED, "no eligible plan for B=(%d,%d) d=%d (%s)", r.block_q, r.block_kv, r.d,
                why.c_str());
  p->entry = chosen;
  p->shape = shape;

  // ---- block-CSR columns (unless queued before the synchronization) ----------
  const size_t nnz = (size_t)p->stats.nnz;
  if (!early_compact) {
    HIP_TRY(p->alloc(sizeof(int32_t) * std::max<size_t>(nnz, 1), &p->cols));
    HIP_TRY(launch_compact(r.mask, nrows, p->nkb, (int32_t*)p->row_ptr.ptr, (int32_t*)p->cols.ptr,
                           (int32_t*)p->rsig.ptr, s));
  }

  // ---- launch preparation: tile list of the selected mapping -------------------
  const int cq = shape.mq.coarsen, ckv = shape.mk.coarsen;
  p->coarse = cq > 1 || ckv > 1;
  if (p->coarse) {
    p->ntr = (int)cdiv(p->nqb, cq);
    const int ntc = (int)cdiv(p->nkb, ckv);
    const int ntrows = r.H * p->ntr;
    HIP_TRY(p->alloc(sizeof(int32_t) * (size_t)ntrows, &p->trow_cnt));
    HIP_TRY(p->alloc(sizeof(int32_t) * ((size_t)ntrows + 1), &p->trow_ptr_buf));
    HIP_TRY(p->alloc(sizeof(int32_t) * std::max<size_t>(nnz, 1), &p->tcol_buf));
    HIP_TRY(p->alloc(sizeof(uint32_t) * std::max<size_t>(nnz, 1), &p->tbits_buf));
    HIP_TRY(p->alloc(sizeof(int32_t) * (size_t)ntrows, &p->tsig_buf));
    HIP_TRY(launch_coarsen((int32_t*)p->row_ptr.ptr, (int32_t*)p->cols.ptr, r.H, p->nqb, p->nkb, cq, ckv, p->ntr,
                           ntc, (int32_t*)p->trow_cnt.ptr, nullptr, nullptr, nullptr, nullptr, s));
    HIP_TRY(launch_scan((int32_t*)p->trow_cnt.ptr, (int32_t*)p->trow_ptr_buf.ptr, ntrows, nullptr, 0, nullptr,
                        nullptr, 0, s));
    HIP_TRY(launch_coarsen((int32_t*)p->row_ptr.ptr, (int32_t*)p->cols.ptr, r.H, p->nqb, p->nkb, cq, ckv, p->ntr,
                           ntc, nullptr, (int32_t*)p->trow_ptr_buf.ptr, (int32_t*)p->tcol_buf.ptr,
                           (uint32_t*)p->tbits_buf.ptr, (int32_t*)p->tsig_buf.ptr, s));
    p->trow_ptr = (const int32_t*)p->trow_ptr_buf.ptr;
    p->tcol = (const int32_t*)p->tcol_buf.ptr;
    p->tbits = (const uint32_t*)p->tbits_buf.ptr;
    p->tsig = (const int32_t*)p->tsig_buf.ptr;
  } else {
    p->ntr = p->nqb;
    p->trow_ptr = (const int32_t*)p->row_ptr.ptr;
    p->tcol = (const int32_t*)p->cols.ptr;
    p->tbits = nullptr;
    p->tsig = (const int32_t*)p->rsig.ptr;
  }

  // ---- tasks and split-K partitions -----------------------------------------
  const int64_t nqt = shape.nqt;
  const bool spec_hit = spec_launched && chosen->id == pred_id && shape.groups == 0;
  if (!spec_hit) {
    HIP_TRY(p->alloc(sizeof(int32_t) * (size_t)nqt, &p->parts));
    HIP_TRY(p->alloc(sizeof(int32_t) * (size_t)nqt, &p->slot_off));
    HIP_TRY(p->alloc(sizeof(Task) * (size_t)std::max<int64_t>(shape.tasks_upper, 1), &p->tasks));
  }
  const int64_t max_len = shape.split > 0 ? shape.split
                                          : std::min<int64_t>((int64_t)shape.mq.coarsen * p->stats.max_row_nnz,
                                                              1 << 30);
  if (shape.groups > 0) {
    HIP_TRY(p->alloc(sizeof(int32_t) * (size_t)(shape.groups + 1), &p->seg_ptr));
    HIP_TRY(launch_tasks_stream(p->trow_ptr, r.H, shape.nqt_head, p->ntr, shape.mq.refine, shape.groups,
                                (int32_t*)p->parts.ptr, (int32_t*)p->slot_off.ptr, (Task*)p->tasks.ptr,
                                (int32_t*)p->seg_ptr.ptr, dst, s));
  } else if (spec_hit) {
    // the speculative builder made this plan's task list (same entry, same
    // statistics, the same balance rule on the device): take its buffers
    std::swap(p->parts, p->spec_parts);
    std::swap(p->slot_off, p->spec_slot);
    std::swap(p->tasks, p->spec_tasks);
    std::swap(p->split_tiles, p->spec_split);
  } else {
    if (shape.split > 0) HIP_TRY(p->alloc(sizeof(int32_t) * (size_t)nqt, &p->split_tiles));
    HIP_TRY(launch_tasks(p->trow_ptr, r.H, shape.nqt_head, p->ntr, shape.mq.refine, shape.split, shape.split_min,
                         chosen->order,
                         (int32_t)max_len, (int32_t*)p->parts.ptr, (int32_t*)p->slot_off.ptr,
                         (Task*)p->tasks.ptr, dst, s, -1, 0, (int32_t*)p->split_tiles.ptr, p->tsig,
                         (int32_t)cdiv(p->nkb, ckv)));
  }
  if (!arena) pred_store(pkey, predictable(*chosen, r) && shape.groups == 0 ? chosen->id : -1);
  if (shape.slots_upper > 0) HIP_TRY(p->alloc((size_t)shape.ws_bytes, &p->ws));
  const bool queues = chosen->xcd_remap > 0 && shape.groups == 0;
  const int64_t gran = queues ? 8 * (int64_t)chosen->xcd_remap : 1;
  // per-XCD queues: spare workgroups for the fast XCDs to steal with
  const int64_t spare = queues ? cdiv(std::max<int64_t>(shape.tasks_upper, 1), kXcdSpareDiv) : 0;
  p->grid = shape.groups > 0 ? shape.groups
                             : cdiv(std::max<int64_t>(shape.tasks_upper, 1) + spare, gran) * gran;
  if (queues) HIP_TRY(p->alloc(8 * sizeof(unsigned long long), &p->xq));
  if (p->grid >= (int64_t(1) << 31)) return fail(BSA_ERR_UNSUPPORTED, "too many tasks");
  HIP_TRY(hipGetLastError());

  bsa_plan_info& in = p->info;
  in.plan_id = chosen->id;
  in.regime = sel.regime;
  in.tile_q = chosen->tq;
  in.tile_kv = chosen->tkv;
  in.coarsen_q = cq;
  in.coarsen_kv = ckv;
  in.refine_q = shape.mq.refine;
  in.refine_kv = shape.mk.refine;
  in.split_items = shape.split;
  in.split_threshold = shape.split_min;
  in.max_row_nnz = (int32_t)p->stats.max_row_nnz;
  in.nnz_blocks = (int64_t)p->stats.nnz;
  in.n_tile_rows = (int64_t)r.H * p->ntr;
  in.n_items = -1;  // counts live on the device (the exports return them)
  in.n_tasks = -1;
  in.grid = p->grid;
  in.workspace_bytes = shape.slots_upper > 0 ? shape.ws_bytes : 0;
  in.long_run_blocks = (int64_t)p->stats.long_run;
  in.density = density;
  in.run_coverage = runcov;
  in.row_skew = skew;
  in.host_select_us = std::chrono::duration<double, std::micro>(t1 - t0).count();
  in.tasks_predicted = spec_hit ? 1 : 0;
  if (!arena) {
    HIP_TRY(event_get(p->dev, false, &p->done));
    HIP_TRY(hipEventRecord(p->done, s));
    p->last = p->done;
  }
  drain.ok = true;
  return BSA_OK;
}

bsa_status bsa_plan_create(const bsa_request* req, void* stream, bsa_plan** out) {
  if (!out) return fail(BSA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  std::unique_ptr<bsa_plan> p;
  const bsa_status st = plan_create_impl(req, (hipStream_t)stream, p, nullptr);
  if (st != BSA_OK) return st;
  *out = p.release();
  return BSA_OK;
}

// Tensor arguments of a run for a request with its batch folded into H:
// non-null, 16-byte aligned, O disjoint from Q, K and V.
static bsa_status check_tensors(const bsa_request& r, const void* q, const void* k, const void* v, const void* o) {
  if (!q || !k || !v || !o) return fail(BSA_ERR_INVALID_ARG, "NULL tensor pointer");
  for (const void* ptr : {q, k, v, o})
    if (((uintptr_t)ptr) & 15) return fail(BSA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  const uintptr_t bytes = (uintptr_t)r.H * r.N * r.d * 2;
  for (const void* in : {q, k, v}) {
    const uintptr_t a = (uintptr_t)in, b = (uintptr_t)o;
    if (a < b + bytes && b < a + bytes) return fail(BSA_ERR_INVALID_ARG, "O overlaps Q, K or V");
  }
  return BSA_OK;
}

// guard: nullptr, or a device word that the kernels read as the task count
// (0: the run does nothing; the speculative run of the plan cache).
static bsa_status run_impl(const bsa_plan* p, const void* q, const void* k, const void* v, void* o,
                           hipStream_t s, bool timed, float* attn_ms, float* merge_ms,
                           const unsigned long long* guard) {
  if (!p) return fail(BSA_ERR_INVALID_ARG, "plan is NULL");
  const bsa_request& r = p->req;
  {
    const bsa_status cs = check_tensors(r, q, k, v, o);
    if (cs != BSA_OK) return cs;
  }
  const CatalogEntry& e = *p->entry;
  AttnLauncher fn = attn_launcher(e.tq, e.tkv, e.d);
  if (!fn) return fail(BSA_ERR_UNSUPPORTED, "no kernel for plan %s", e.name.c_str());
  AttnArgs a{};
  a.q = (const __bf16*)q;
  a.k = (const __bf16*)k;
  a.v = (const __bf16*)v;
  a.o = (__bf16*)o;
  a.tasks = (const Task*)p->tasks.ptr;
  a.n_tasks = guard ? guard : &((const MaskStats*)p->stats_dev.ptr)->n_tasks;
  a.tcol = p->tcol;
  a.tbits = p->tbits;
  float* ws = (float*)p->ws.ptr;
  const int64_t slots = p->shape.slots_upper;
  a.ws_m = ws;
  a.ws_l = ws ? ws + slots * e.tq : nullptr;
  a.ws_o = ws ? ws + 2 * slots * e.tq : nullptr;
  // layout: HND = [batch*H][N][d] (one run of heads), NHD = [batch][N][H][d]
  const bool nhd = r.layout == BSA_LAYOUT_NHD;
  a.heads = nhd ? p->heads : r.H;
  a.batch_stride = nhd ? (int64_t)r.N * p->heads * r.d : 0;
  a.head_stride = nhd ? r.d : (int64_t)r.N * r.d;
  a.row_stride = nhd ? p->heads * r.d : r.d;
  a.N = r.N;
  a.sub_log2 = ilog2(p->shape.mk.refine);
  a.bkv_log2 = ilog2(r.block_kv);
  a.coarsen_kv = p->shape.mk.coarsen;
  a.coarsen_q = p->shape.mq.coarsen;
  a.bq = r.block_q;
  a.xcd_remap = p->shape.groups > 0 ? 0 : e.xcd_remap;
  a.xq = a.xcd_remap > 0 ? (unsigned long long*)p->xq.ptr : nullptr;
  a.seg_ptr = p->shape.groups > 0 ? (const int32_t*)p->seg_ptr.ptr : nullptr;
  a.grid = (int32_t)p->grid;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)r.d));
  if (a.xq) HIP_TRY(launch_xq_init(a.xq, a.n_tasks, a.xcd_remap, s));
  if (timed) {
    for (auto& ev : p->ev)
      if (!ev) HIP_TRY(event_get(p->dev, true, &ev));
    HIP_TRY(hipEventRecord(p->ev[0], s));
  }
  HIP_TRY(fn(a, (int)p->grid, s));
  if (timed) HIP_TRY(hipEventRecord(p->ev[1], s));
  if (p->shape.split > 0 || p->shape.groups > 0) {
    MergeArgs m{};
    m.o = (__bf16*)o;
    m.guard = guard;
    m.heads = a.heads;
    m.batch_stride = a.batch_stride;
    m.head_stride = a.head_stride;
    m.row_stride = a.row_stride;
    m.parts = (const int32_t*)p->parts.ptr;
    m.slot_base = (const int32_t*)p->slot_off.ptr;
    m.ws_m = a.ws_m;
    m.ws_l = a.ws_l;
    m.ws_o = a.ws_o;
    m.N = r.N;
    m.n_qtiles_head = p->shape.nqt_head;
    m.tq = e.tq;
    m.d = e.d;
    // with the builder's list of split tiles, a fixed grid loops over their
    // items (most query tiles are not split)
    int32_t grid_items = 0;
    if (p->split_tiles.ptr && p->shape.groups == 0) {
      m.split_tiles = (const int32_t*)p->split_tiles.ptr;
      m.n_split = &((const MaskStats*)p->stats_dev.ptr)->n_split;
      grid_items = (int32_t)std::min<int64_t>(p->shape.nqt * (e.d / kMergeCols), 8LL * device_cus(p->dev));
    }
    HIP_TRY(launch_merge(m, (int32_t)p->shape.nqt, s, grid_items));
  }
  if (!timed && p->done) {
    HIP_TRY(hipEventRecord(p->done, s));
    p->last = p->done;
  }
  if (timed) {
    HIP_TRY(hipEventRecord(p->ev[2], s));
    p->last = p->ev[2];
    HIP_TRY(hipEventSynchronize(p->ev[2]));
    float t = 0;
    HIP_TRY(hipEventElapsedTime(&t, p->ev[0], p->ev[1]));
    if (attn_ms) *attn_ms = t;
    HIP_TRY(hipEventElapsedTime(&t, p->ev[1], p->ev[2]));
    if (merge_ms) *merge_ms = t;
  }
  return BSA_OK;
}

bsa_status bsa_run(const bsa_plan* p, const void* q, const void* k, const void* v, void* o, void* stream) {
  return run_impl(p, q, k, v, o, (hipStream_t)stream, false, nullptr, nullptr, nullptr);
}

bsa_status bsa_run_timed(const bsa_plan* p, const void* q, const void* k, const void* v, void* o, void* stream,
                         float* attn_ms, float* merge_ms) {
  return run_impl(p, q, k, v, o, (hipStream_t)stream, true, attn_ms, merge_ms, nullptr);
}

bsa_status bsa_attention_noalloc(const bsa_request* req, const void* q, const void* k, const void* v, void* o,
                                 void* stream) {
  {
    const bsa_status vs = validate_request(req);
    if (vs != BSA_OK) return vs;
    const bsa_status cs = check_tensors(folded(*req), q, k, v, o);
    if (cs != BSA_OK) return cs;
  }
  void* base = nullptr;
  size_t cap = 0;
  HIP_TRY(static_scratch(&base, &cap));
  // the last 64 KiB of the array are never carved: a guard band between
  // the final buffer and the end of the array
  Arena arena;
  arena.base = (char*)base;
  arena.cap = cap - (size_t(64) << 10);
  hipStream_t s = (hipStream_t)stream;
  std::unique_ptr<bsa_plan> p;
  const bsa_status st = plan_create_impl(req, s, p, &arena);
  if (st != BSA_OK) return st;
  // the plan's buffers stay in the scratch (nothing is returned to a cache),
  // so the kernels queued here may outlive the host-side plan record
  return run_impl(p.get(), q, k, v, o, s, false, nullptr, nullptr, nullptr);
}

bsa_status bsa_plan_destroy(bsa_plan* p) {
  if (!p) return BSA_OK;
  // wait for the plan's latest stream work (its creation or last run) before
  // its device memory returns to the cache
  hipError_t e = p->last ? hipEventSynchronize(p->last) : hipDeviceSynchronize();
  delete p;
  if (e != hipSuccess) return fail(BSA_ERR_HIP, "waiting for the plan's work: %s", hipGetErrorString(e));
  return BSA_OK;
}

bsa_status bsa_plan_get_info(const bsa_plan* p, bsa_plan_info* info) {
  if (!p || !info) return fail(BSA_ERR_INVALID_ARG, "NULL argument");
  *info = p->info;
  return BSA_OK;
}

bsa_status bsa_plan_export_csr(const bsa_plan* p, int32_t* row_ptr, int32_t* cols, int64_t cap_cols) {
  if (!p || !row_ptr || !cols) return fail(BSA_ERR_INVALID_ARG, "NULL argument");
  if (cap_cols < (int64_t)p->stats.nnz) return fail(BSA_ERR_INVALID_ARG, "cols capacity too small");
  const size_t nrows = (size_t)p->req.H * p->nqb;
  HIP_TRY(hipDeviceSynchronize());
  HIP_TRY(hipMemcpy(row_ptr, p->row_ptr.ptr, sizeof(int32_t) * (nrows + 1), hipMemcpyDeviceToHost));
  if (p->stats.nnz)
    HIP_TRY(hipMemcpy(cols, p->cols.ptr, sizeof(int32_t) * (size_t)p->stats.nnz, hipMemcpyDeviceToHost));
  return BSA_OK;
}

bsa_status bsa_plan_export_tiles(const bsa_plan* p, int32_t* head, int32_t* q_tile, int32_t* kv_tile,
                                 uint32_t* bits, int64_t cap, int64_t* count) {
  if (!p || !count) return fail(BSA_ERR_INVALID_ARG, "NULL argument");
  HIP_TRY(hipDeviceSynchronize());
  MaskStats st{};
  HIP_TRY(hipMemcpy(&st, p->stats_dev.ptr, sizeof st, hipMemcpyDeviceToHost));
  const size_t nt = (size_t)st.n_tasks;
  std::vector<Task> tasks(nt);
  if (nt) HIP_TRY(hipMemcpy(tasks.data(), p->tasks.ptr, sizeof(Task) * nt, hipMemcpyDeviceToHost));
  const size_t ntrows = (size_t)p->req.H * p->ntr;
  int32_t nitems = 0;
  HIP_TRY(hipMemcpy(&nitems, p->trow_ptr + ntrows, sizeof(int32_t), hipMemcpyDeviceToHost));
  std::vector<int32_t> tcol(nitems);
  std::vector<uint32_t> tbits;
  if (nitems) HIP_TRY(hipMemcpy(tcol.data(), p->tcol, sizeof(int32_t) * nitems, hipMemcpyDeviceToHost));
  if (p->tbits) {
    tbits.resize(nitems);
    if (nitems) HIP_TRY(hipMemcpy(tbits.data(), p->tbits, sizeof(uint32_t) * nitems, hipMemcpyDeviceToHost));
  }
  const int rkv = p->shape.mk.refine;
  const int tkv = p->entry->tkv;
  const int N = p->req.N;
  const uint32_t full = (p->shape.mq.coarsen * p->shape.mk.coarsen >= 32)
                            ? 0xffffffffu
                            : ((1u << (p->shape.mq.coarsen * p->shape.mk.coarsen)) - 1u);
  int64_t n = 0;
  for (const Task& t : tasks) {
    for (int it = t.begin; it < t.end; ++it) {
      for (int sub = 0; sub < rkv; ++sub) {
        const int kt = tcol[it] * rkv + sub;
        if ((int64_t)kt * tkv >= N) continue;
        if (n < cap && head && q_tile && kv_tile && bits) {
          head[n] = t.head;
          q_tile[n] = t.qtile;
          kv_tile[n] = kt;
          bits[n] = p->tbits ? tbits[it] : full;
        }
        ++n;
      }
    }
  }
  *count = n;
  if (n > cap) return fail(BSA_ERR_INVALID_ARG, "capacity %lld < %lld tiles", (long long)cap, (long long)n);
  return BSA_OK;
}

bsa_status bsa_plan_export_tasks(const bsa_plan* p, int32_t* head, int32_t* q_tile, int32_t* begin,
                                 int32_t* end, int32_t* slot, int64_t cap, int64_t* count) {
  if (!p || !count) return fail(BSA_ERR_INVALID_ARG, "NULL argument");
  HIP_TRY(hipDeviceSynchronize());
  MaskStats st{};
  HIP_TRY(hipMemcpy(&st, p->stats_dev.ptr, sizeof st, hipMemcpyDeviceToHost));
  const int64_t nt = (int64_t)st.n_tasks;
  *count = nt;
  if (nt > cap) return fail(BSA_ERR_INVALID_ARG, "capacity %lld < %lld tasks", (long long)cap, (long long)nt);
  if (nt == 0) return BSA_OK;
  if (!head || !q_tile || !begin || !end || !slot) return fail(BSA_ERR_INVALID_ARG, "NULL array");
  std::vector<Task> tasks((size_t)nt);
  HIP_TRY(hipMemcpy(tasks.data(), p->tasks.ptr, sizeof(Task) * (size_t)nt, hipMemcpyDeviceToHost));
  for (int64_t i = 0; i < nt; ++i) {
    head[i] = tasks[i].head;
    q_tile[i] = tasks[i].qtile;
    begin[i] = tasks[i].begin;
    end[i] = tasks[i].end;
    slot[i] = tasks[i].slot;
  }
  return BSA_OK;
}

bsa_status bsa_plan_cache_create(int32_t capacity, int64_t max_mask_bytes, bsa_plan_cache** out) {
  if (!out) return fail(BSA_ERR_INVALID_ARG, "NULL argument");
  if (capacity < 1 || capacity > 64) return fail(BSA_ERR_INVALID_ARG, "capacity %d not in [1, 64]", capacity);
  if (max_mask_bytes < 0) return fail(BSA_ERR_INVALID_ARG, "max_mask_bytes < 0");
  bsa_plan_cache* c = new (std::nothrow) bsa_plan_cache();
  if (!c) return fail(BSA_ERR_NO_MEMORY, "host allocation failed");
  c->capacity = capacity;
  c->max_bytes = max_mask_bytes;
  *out = c;
  return BSA_OK;
}

bsa_status bsa_plan_cache_get(bsa_plan_cache* c, const bsa_request* req, void* stream, bsa_plan** out,
                              int32_t* hit) {
  return cache_acquire(c, req, (hipStream_t)stream, nullptr, out, hit);
}

bsa_status bsa_plan_cache_run(bsa_plan_cache* c, const bsa_request* req, const void* q, const void* k,
                              const void* v, void* o, void* stream, int32_t* hit) {
  const RunIO io{q, k, v, o};
  bsa_plan* p = nullptr;
  return cache_acquire(c, req, (hipStream_t)stream, &io, &p, hit);
}

bsa_status bsa_plan_cache_destroy(bsa_plan_cache* c) {
  if (!c) return BSA_OK;
  {
    std::lock_guard<std::mutex> lk(c->mu);
    for (auto& e : c->entries) drop_entry(e);
    c->entries.clear();
    for (auto& kv : c->flags) pool_release(&kv.second);
  }
  delete c;
  return BSA_OK;
}

}  // extern "C"

namespace {
// Destroys a cache entry's plan (after its latest stream work) and returns
// its mask copy once the copy has completed.
void drop_entry(bsa_plan_cache::Entry& e) {
  if (e.plan) (void)bsa_plan_destroy(e.plan);
  e.plan = nullptr;
  if (e.copied) {
    (void)hipEventSynchronize(e.copied);
    event_put(e.dev, false, e.copied);
    e.copied = nullptr;
  }
  pool_release(&e.mask_copy);
  pool_release(&e.guard);
}
}  // namespace
