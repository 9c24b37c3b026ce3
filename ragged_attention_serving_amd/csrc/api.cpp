// libxattn C ABI: plan (host schedule, double-buffered staging) and run (launches).
//
// Double buffering follows page "mstar.engine.resources.attn.cross",
// FlashInferCrossManager.force_double_buffer: a plan is staged in a pinned host
// buffer and copied to the device with a non-blocking copy, so planning step N+1
// into the same buffer before step N's copy (and the runs that read it) retired would
// race. Each handle therefore owns two slots; plan N writes slot N % 2, and run reads
// the latest slot.
//
// Before a slot is rewritten:
//  * its previous host-to-device copy must have read the pinned buffer (the slot's
//    `uploaded` event);
//  * every run that read the slot's device copy or workspace must be done, or be
//    ordered before the new copy. Runs on the plan's own stream are: the new copy is
//    queued behind them. A run on another stream records the slot's fence, and a plan
//    on another stream than the one the slot last used drains that stream first.
// Runs of one slot whose schedule splits contexts share the slot's fp32 workspace, so a
// run on another stream than the latest such run first waits for that stream.
// So the common case, plan and runs on one stream, records nothing per run.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "xattn.h"
#include "kernels.h"
#include "partition.h"

using xattn::AttnParams;
using xattn::Schedule;

namespace {

thread_local std::string g_err;

int set_err(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_err(hipError_t e, const char* what) {
  return set_err(XATTN_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int env_int(const char* name, int dflt) {
  const char* s = std::getenv(name);
  return s && *s ? std::atoi(s) : dflt;
}

size_t align_words(size_t n) { return (n + 63) & ~static_cast<size_t>(63); }

constexpr size_t kMaxTimingRecs = 65536;

struct Slot {
  void* host = nullptr;  // pinned staging
  size_t host_cap = 0;
  void* dev = nullptr;
  size_t dev_cap = 0;
  float* ws = nullptr;  // [ws_rows][d] partial O, then [ws_rows] partial lse
  size_t ws_cap = 0;    // bytes
  hipEvent_t fence = nullptr;     // drains the slot's previous plan stream on a stream change
  hipEvent_t uploaded = nullptr;  // the slot's host-to-device copy
  void* plan_stream = nullptr;    // stream of that copy
  bool uploaded_rec = false;      // `uploaded` was recorded
  // runs on streams other than the plan's: one event per stream, after its latest run
  std::vector<std::pair<void*, hipEvent_t>> foreign;
  size_t foreign_live = 0;        // entries recorded since the slot was last planned
  // the split workspace is one buffer per slot: the stream of the latest run that used
  // it since the slot was planned, and an event a run on another stream waits on
  void* ws_stream = nullptr;
  bool ws_used = false;
  hipEvent_t ws_event = nullptr;
  bool ready = false;
  // schedule summary and device offsets (in int32 words from dev)
  Schedule sched;
  size_t off_reqs = 0, off_units[xattn::FAM_COUNT] = {0, 0, 0}, off_merges = 0, off_pages = 0;
  size_t off_kv_start = 0;
  // graph-stable layout: section capacities (elements) that only grow, what every run
  // launches (the union over plans), and the generation of the layout
  size_t cap_reqs = 0, cap_units[xattn::FAM_COUNT] = {0, 0, 0}, cap_merges = 0, cap_pages = 0,
         cap_kv_start = 0;
  int64_t cap_ws_rows = 0;
  int run_fams = 0;       // bit f: family f is launched
  bool run_merge = false;
  int run_dec_rows = 0;
  std::vector<int64_t> layout_key;
  int64_t layout_gen = 0;
  int32_t dtype = 0, hq = 0, hkv = 0, d = 0, page_size = 0, mask = 0, block = 0;
  int64_t pool_bytes = 0;  // bytes of each of the K and V pools
};

}  // namespace

struct TimingRec {
  int stage;
  hipEvent_t start, stop;
};

struct xattn_plan_s {
  Slot slot[2];
  int flags = 0;  // XATTN_PLAN_GRAPH_STABLE
  int cur = -1;
  int device = 0;
  int timing_every = 0;  // record kernel events on every n-th run (0: off)
  int64_t runs = 0;
  std::vector<hipEvent_t> event_pool;
  std::vector<TimingRec> timing_recs;
};

namespace {

// Grows a buffer geometrically. Freeing the old one is safe while runs may still read
// it: hipFree and hipHostFree synchronise the device before they release memory.
int ensure(void** ptr, size_t* cap, size_t need, bool pinned) {
  if (*cap >= need && *ptr) return XATTN_OK;
  size_t want = need < 4096 ? 4096 : need + need / 4;
  if (*ptr) {
    hipError_t e = pinned ? hipHostFree(*ptr) : hipFree(*ptr);
    *ptr = nullptr;
    *cap = 0;
    if (e != hipSuccess) return hip_err(e, "free");
  }
  hipError_t e = pinned ? hipHostMalloc(ptr, want, hipHostMallocDefault) : hipMalloc(ptr, want);
  if (e != hipSuccess) {
    *ptr = nullptr;
    (void)hipGetLastError();
    return set_err(XATTN_ERR_OOM, std::string(pinned ? "hipHostMalloc" : "hipMalloc") + " failed: " +
                                      hipGetErrorString(e));
  }
  *cap = want;
  return XATTN_OK;
}

void log_schedule(const Schedule& s) {
  std::fprintf(stderr,
               "[xattn] plan: units f32=%zu dec=%zu (rows %d) mma=%zu; chunks %d/%d/%d; "
               "merge rows %zu; workspace rows %lld; kv tokens %lld\n",
               s.units[0].size(), s.units[1].size(), s.dec_rows, s.units[2].size(), s.chunk[0],
               s.chunk[1], s.chunk[2], s.merges.size(), static_cast<long long>(s.ws_rows),
               static_cast<long long>(s.total_kv));
}

void fill_info(const Schedule& s, xattn_schedule_info* info) {
  for (int f = 0; f < xattn::FAM_COUNT; ++f) {
    info->num_units[f] = static_cast<int32_t>(s.units[f].size());
    info->chunk_tokens[f] = s.units[f].empty() ? 0 : s.chunk[f];
  }
  info->decode_rows = s.dec_rows;
  info->num_merge_rows = static_cast<int32_t>(s.merges.size());
  info->workspace_rows = s.ws_rows;
  info->total_kv_tokens = s.total_kv;
  info->visible_pairs = s.visible_pairs;
  info->layout_generation = 0;
  info->slot = -1;
  info->reserved = 0;
}

xattn::PlanArgs make_args(const int32_t* qo_indptr, const int32_t* kv_indptr,
                          const int32_t* kv_page_indices, const int32_t* kv_last_page_len,
                          int32_t batch_size, int32_t num_qo_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t page_size, int64_t num_pages, int32_t mask_mode,
                          int32_t block_size, float sm_scale, int32_t dtype, int32_t force_chunk) {
  xattn::PlanArgs a;
  a.qo_indptr = qo_indptr;
  a.kv_indptr = kv_indptr;
  a.kv_page_indices = kv_page_indices;
  a.kv_last_page_len = kv_last_page_len;
  a.batch = batch_size;
  a.hq = num_qo_heads;
  a.hkv = num_kv_heads;
  a.d = head_dim;
  a.page_size = page_size;
  a.num_pages = num_pages;
  a.mask = mask_mode;
  a.block = block_size;
  a.sm_scale = sm_scale;
  a.dtype = dtype;
  a.force_chunk = force_chunk;
  return a;
}

}  // namespace

extern "C" {

const char* xattn_last_error(void) { return g_err.c_str(); }

int xattn_schedule(const int32_t* qo_indptr, const int32_t* kv_indptr,
                   const int32_t* kv_page_indices, const int32_t* kv_last_page_len,
                   int32_t batch_size, int32_t num_qo_heads, int32_t num_kv_heads,
                   int32_t head_dim, int32_t page_size, int64_t num_pages, int32_t mask_mode,
                   int32_t block_size, int32_t dtype, int32_t force_chunk,
                   xattn_schedule_info* info, int32_t* units, int32_t* merges) {
  if (!info) return set_err(XATTN_ERR_INVALID_ARG, "info is NULL");
  Schedule s;
  std::string err;
  const xattn::PlanArgs a = make_args(qo_indptr, kv_indptr, kv_page_indices, kv_last_page_len,
                                      batch_size, num_qo_heads, num_kv_heads, head_dim, page_size,
                                      num_pages, mask_mode, block_size, 0.f, dtype, force_chunk);
  const int rc = xattn::build_schedule(a, s, err);
  if (rc != XATTN_OK) return set_err(rc, err);
  fill_info(s, info);
  if (units) {
    int32_t* dst = units;
    for (int f = 0; f < xattn::FAM_COUNT; ++f) {
      std::memcpy(dst, s.units[f].data(), s.units[f].size() * sizeof(xattn::Unit));
      dst += s.units[f].size() * 8;
    }
  }
  if (merges) std::memcpy(merges, s.merges.data(), s.merges.size() * sizeof(xattn::Merge));
  return XATTN_OK;
}

int xattn_plan(xattn_plan_t* plan, const int32_t* qo_indptr, const int32_t* kv_indptr,
               const int32_t* kv_page_indices, const int32_t* kv_last_page_len,
               int32_t batch_size, int32_t num_qo_heads, int32_t num_kv_heads,
               int32_t head_dim, int32_t page_size, int64_t num_pages, int32_t mask_mode,
               int32_t block_size, float sm_scale, int32_t dtype, void* stream) {
  if (!plan) return set_err(XATTN_ERR_INVALID_ARG, "plan is NULL");
  Schedule s;
  std::string err;
  xattn::PlanArgs a =
      make_args(qo_indptr, kv_indptr, kv_page_indices, kv_last_page_len, batch_size, num_qo_heads,
                num_kv_heads, head_dim, page_size, num_pages, mask_mode, block_size, sm_scale, dtype,
                env_int("XATTN_FORCE_CHUNK", 0));
  a.tile_rows = env_int("XATTN_TILE_ROWS", 0);
  const int rc = xattn::build_schedule(a, s, err);
  if (rc != XATTN_OK) return set_err(rc, err);
  if (env_int("XATTN_LOG", 0)) log_schedule(s);

  bool created = false;
  if (*plan == nullptr) {
    *plan = new xattn_plan_s();
    created = true;
    (void)hipGetDevice(&(*plan)->device);
  }
  xattn_plan_s* h = *plan;
  auto fail = [&](int code) {
    if (created) {
      xattn_plan_destroy(h);
      *plan = nullptr;
    }
    return code;
  };
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev != h->device) return fail(set_err(XATTN_ERR_INVALID_ARG, "plan used on another device"));

  const int si = h->cur < 0 ? 0 : (h->cur ^ 1);
  Slot& sl = h->slot[si];
  hipError_t e;
  if (!sl.fence) {
    if ((e = hipEventCreateWithFlags(&sl.fence, hipEventDisableTiming)) != hipSuccess)
      return fail(hip_err(e, "hipEventCreate"));
    if ((e = hipEventCreateWithFlags(&sl.uploaded, hipEventDisableTiming)) != hipSuccess)
      return fail(hip_err(e, "hipEventCreate"));
    if ((e = hipEventCreateWithFlags(&sl.ws_event, hipEventDisableTiming)) != hipSuccess)
      return fail(hip_err(e, "hipEventCreate"));
  }
  if (sl.uploaded_rec) {
    // the previous copy out of the pinned buffer must be done before it is rewritten
    if ((e = hipEventSynchronize(sl.uploaded)) != hipSuccess) return fail(hip_err(e, "hipEventSynchronize"));
    if (stream != sl.plan_stream) {
      // runs on the slot's old stream are not ordered before a copy on this one: drain it
      if ((e = hipEventRecord(sl.fence, static_cast<hipStream_t>(sl.plan_stream))) != hipSuccess)
        return fail(hip_err(e, "hipEventRecord"));
      if ((e = hipEventSynchronize(sl.fence)) != hipSuccess) return fail(hip_err(e, "hipEventSynchronize"));
    }
  }
  for (size_t i = 0; i < sl.foreign_live; ++i) {
    // runs that used another stream than the plan's
    if ((e = hipEventSynchronize(sl.foreign[i].second)) != hipSuccess) return fail(hip_err(e, "hipEventSynchronize"));
  }
  sl.foreign_live = 0;
  // every run that used the workspace is done or ordered before this plan's copy, which
  // every later run of the slot follows
  sl.ws_used = false;

  // device image (int32 words): header | reqs | units per family | merges | page indices |
  // kv starts. The header holds each family's unit count and the merge count, which the
  // kernels read in a graph-stable handle. There the sections are laid out by capacities
  // that only grow (a quarter of headroom when they do), so offsets and buffers stay put
  // from plan to plan while the schedule fits, and the workspace likewise.
  const bool stable = (h->flags & XATTN_PLAN_GRAPH_STABLE) != 0;
  auto fit = [&](size_t& cap, size_t need) {
    if (!stable) cap = need;
    else if (need > cap) cap = need + need / 4;
    return cap;
  };
  size_t words = 0;
  constexpr size_t kHeaderWords = 64;
  words += kHeaderWords;
  const size_t off_reqs = words;
  words = align_words(words + fit(sl.cap_reqs, s.reqs.size()));
  size_t off_units[xattn::FAM_COUNT];
  for (int f = 0; f < xattn::FAM_COUNT; ++f) {
    off_units[f] = words;
    words = align_words(words + fit(sl.cap_units[f], s.units[f].size()) * 8);
  }
  const size_t off_merges = words;
  words = align_words(words + fit(sl.cap_merges, s.merges.size()) * 4);
  const size_t off_pages = words;
  words = align_words(words + fit(sl.cap_pages, s.pages.size()));
  const size_t off_kv_start = words;
  words = align_words(words + fit(sl.cap_kv_start, s.kv_start.size()));
  const size_t bytes = words * sizeof(int32_t);
  if (!stable) sl.cap_ws_rows = s.ws_rows;
  else if (s.ws_rows > sl.cap_ws_rows) sl.cap_ws_rows = s.ws_rows + s.ws_rows / 4;

  int st;
  if ((st = ensure(&sl.host, &sl.host_cap, bytes, true)) != XATTN_OK) return fail(st);
  if ((st = ensure(&sl.dev, &sl.dev_cap, bytes, false)) != XATTN_OK) return fail(st);
  const size_t ws_bytes = static_cast<size_t>(sl.cap_ws_rows) * (head_dim + 1) * sizeof(float);
  if (ws_bytes > 0) {
    void* w = sl.ws;
    if ((st = ensure(&w, &sl.ws_cap, ws_bytes, false)) != XATTN_OK) {
      sl.ws = nullptr;
      return fail(st);
    }
    sl.ws = static_cast<float*>(w);
  }

  int32_t* img = static_cast<int32_t*>(sl.host);
  std::memset(img, 0, kHeaderWords * sizeof(int32_t));
  for (int f = 0; f < xattn::FAM_COUNT; ++f) img[f] = static_cast<int32_t>(s.units[f].size());
  img[3] = static_cast<int32_t>(s.merges.size());
  std::memcpy(img + off_reqs, s.reqs.data(), s.reqs.size() * sizeof(int32_t));
  for (int f = 0; f < xattn::FAM_COUNT; ++f)
    std::memcpy(img + off_units[f], s.units[f].data(), s.units[f].size() * sizeof(xattn::Unit));
  std::memcpy(img + off_merges, s.merges.data(), s.merges.size() * sizeof(xattn::Merge));
  std::memcpy(img + off_pages, s.pages.data(), s.pages.size() * sizeof(int32_t));
  std::memcpy(img + off_kv_start, s.kv_start.data(), s.kv_start.size() * sizeof(int32_t));

  hipStream_t strm = static_cast<hipStream_t>(stream);
  if ((e = hipMemcpyAsync(sl.dev, sl.host, bytes, hipMemcpyHostToDevice, strm)) != hipSuccess)
    return fail(hip_err(e, "hipMemcpyAsync"));
  if ((e = hipEventRecord(sl.uploaded, strm)) != hipSuccess) return fail(hip_err(e, "hipEventRecord"));
  sl.uploaded_rec = true;
  sl.plan_stream = stream;

  sl.off_reqs = off_reqs;
  for (int f = 0; f < xattn::FAM_COUNT; ++f) sl.off_units[f] = off_units[f];
  sl.off_merges = off_merges;
  sl.off_pages = off_pages;
  sl.off_kv_start = off_kv_start;
  sl.dtype = dtype;
  sl.hq = num_qo_heads;
  sl.hkv = num_kv_heads;
  sl.d = head_dim;
  sl.page_size = page_size;
  sl.mask = mask_mode;
  sl.block = block_size;
  sl.pool_bytes = num_pages * page_size * static_cast<int64_t>(num_kv_heads) * head_dim *
                  (dtype == XATTN_BF16 ? 2 : 4);
  // what a run launches: this schedule's kernels, or in a graph-stable handle the union
  // over the slot's plans (a launch whose count is 0 this time exits at once)
  int fams = 0;
  for (int f = 0; f < xattn::FAM_COUNT; ++f)
    if (!s.units[f].empty()) fams |= 1 << f;
  sl.run_fams = stable ? (sl.run_fams | fams) : fams;
  sl.run_merge = stable ? (sl.run_merge || !s.merges.empty()) : !s.merges.empty();
  sl.run_dec_rows = stable ? std::max(sl.run_dec_rows, s.dec_rows) : s.dec_rows;
  // everything a captured run holds as a launch argument or launch shape; any change
  // starts a new layout generation
  std::vector<int64_t> key = {
      reinterpret_cast<int64_t>(sl.dev), reinterpret_cast<int64_t>(sl.ws), sl.cap_ws_rows,
      static_cast<int64_t>(off_reqs), static_cast<int64_t>(off_merges), static_cast<int64_t>(off_pages),
      static_cast<int64_t>(off_kv_start), static_cast<int64_t>(sl.cap_merges), sl.run_fams,
      sl.run_merge, sl.run_dec_rows, s.identity, s.group, s.tile_rows, dtype, num_qo_heads,
      num_kv_heads, head_dim, page_size, mask_mode, block_size,
      sl.pool_bytes > 0 && sl.pool_bytes <= static_cast<int64_t>(UINT32_MAX)};  // the tile kernel's load form
  for (int f = 0; f < xattn::FAM_COUNT; ++f) {
    key.push_back(static_cast<int64_t>(off_units[f]));
    key.push_back(static_cast<int64_t>(sl.cap_units[f]));
  }
  int32_t scale_bits;
  std::memcpy(&scale_bits, &s.scale, sizeof(scale_bits));
  key.push_back(scale_bits);
  if (key != sl.layout_key) {
    sl.layout_key = std::move(key);
    ++sl.layout_gen;
  }
  sl.sched = std::move(s);
  sl.ready = true;
  h->cur = si;
  return XATTN_OK;
}

int xattn_plan_create(xattn_plan_t* plan, int32_t flags) {
  if (!plan) return set_err(XATTN_ERR_INVALID_ARG, "plan is NULL");
  if (*plan) return set_err(XATTN_ERR_INVALID_ARG, "*plan is not NULL");
  if (flags & ~XATTN_PLAN_GRAPH_STABLE) return set_err(XATTN_ERR_INVALID_ARG, "unknown flags");
  xattn_plan_s* h = new xattn_plan_s();
  h->flags = flags;
  (void)hipGetDevice(&h->device);
  *plan = h;
  return XATTN_OK;
}

namespace {

// A launch on another stream than the plan's waits for the schedule's copy; on the same
// stream the copy already precedes it.
hipError_t slot_wait(Slot& sl, void* stream) {
  if (stream == sl.plan_stream) return hipSuccess;
  return hipStreamWaitEvent(static_cast<hipStream_t>(stream), sl.uploaded, 0);
}

// A launch on another stream than the plan's is not ordered before the slot's next copy
// by the stream: fence that stream (one event per stream, after its latest launch).
hipError_t slot_mark(Slot& sl, void* stream) {
  if (stream == sl.plan_stream) return hipSuccess;
  size_t i = 0;
  while (i < sl.foreign_live && sl.foreign[i].first != stream) ++i;
  if (i == sl.foreign_live) {
    if (i == sl.foreign.size()) {
      hipEvent_t ev = nullptr;
      const hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
      if (e != hipSuccess) return e;
      sl.foreign.emplace_back(stream, ev);
    }
    sl.foreign[i].first = stream;
    ++sl.foreign_live;
  }
  return hipEventRecord(sl.foreign[i].second, static_cast<hipStream_t>(stream));
}

// Runs of a split schedule share the slot's workspace (partial rows, then the merge that
// reads them): a run on another stream than the latest run that used it waits for that
// stream, so such runs execute one after another. Runs on one stream are ordered anyway,
// and record nothing.
hipError_t ws_order(Slot& sl, void* stream) {
  if (sl.ws_used && sl.ws_stream != stream) {
    hipError_t e = hipEventRecord(sl.ws_event, static_cast<hipStream_t>(sl.ws_stream));
    if (e == hipSuccess) e = hipStreamWaitEvent(static_cast<hipStream_t>(stream), sl.ws_event, 0);
    if (e != hipSuccess) return e;
  }
  sl.ws_used = true;
  sl.ws_stream = stream;
  return hipSuccess;
}

}  // namespace

}  // extern "C"

namespace {

// Argument checks shared by the run entry points.
int check_run_args(xattn_plan_t plan, const void* q, const void* k_pages, const void* v_pages,
                   void* out, float* lse) {
  if (!plan || plan->cur < 0 || !plan->slot[plan->cur].ready)
    return set_err(XATTN_ERR_INVALID_ARG, "run without a successful plan");
  const Schedule& s = plan->slot[plan->cur].sched;
  size_t nunits = 0;
  for (int f = 0; f < xattn::FAM_COUNT; ++f) nunits += s.units[f].size();
  if (nunits > 0 && (!q || !out)) return set_err(XATTN_ERR_INVALID_ARG, "q and out are required");
  if (s.total_kv > 0 && (!k_pages || !v_pages))
    return set_err(XATTN_ERR_INVALID_ARG, "k_pages and v_pages are required");
  const uintptr_t mis = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_pages) |
                        reinterpret_cast<uintptr_t>(v_pages) | reinterpret_cast<uintptr_t>(out);
  if (mis & 15) return set_err(XATTN_ERR_INVALID_ARG, "q, k_pages, v_pages and out must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(lse) & 3) return set_err(XATTN_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  return XATTN_OK;
}

// Launches the current slot's attention kernels, and the merge when contexts were split,
// on `stream`, with the split workspace at ws_o ([rows][d]) and ws_lse ([rows]).
// `timing` allows the per-kernel events of xattn_plan_set_timing.
int launch_run(xattn_plan_t plan, const void* q, const void* k_pages, const void* v_pages, void* out,
               float* lse, void* stream, float* ws_o, float* ws_lse, bool timing) {
  Slot& sl = plan->slot[plan->cur];
  const Schedule& s = sl.sched;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  hipError_t e;
  const bool stable = (plan->flags & XATTN_PLAN_GRAPH_STABLE) != 0;

  const int32_t* dev = static_cast<const int32_t*>(sl.dev);
  AttnParams p{};
  p.q = q;
  p.k = k_pages;
  p.v = v_pages;
  p.out = out;
  p.lse = lse;
  p.ws_o = ws_o;
  p.ws_lse = ws_lse;
  p.reqs = dev + sl.off_reqs;
  p.pages = s.identity ? nullptr : dev + sl.off_pages;
  p.merges = dev + sl.off_merges;
  p.num_merges = static_cast<int32_t>(s.merges.size());
  p.hq = sl.hq;
  p.hkv = sl.hkv;
  p.d = sl.d;
  p.group = s.group;
  p.page_size = sl.page_size;
  p.page_shift = -1;
  if ((sl.page_size & (sl.page_size - 1)) == 0) {
    int sh = 0;
    while ((1 << sh) < sl.page_size) ++sh;
    p.page_shift = sh;
  }
  p.mask = sl.mask;
  p.block = sl.mask == 2 ? sl.block : 1;
  p.tile_rows = s.tile_rows;
  p.scale = s.scale;
  p.scale_log2 = s.scale * 1.4426950408889634f;
  p.pool_bytes = sl.pool_bytes;

  // optional per-kernel events (xattn_plan_set_timing)
  const bool timed = timing && plan->timing_every > 0 && plan->runs++ % plan->timing_every == 0 &&
                     plan->timing_recs.size() < kMaxTimingRecs;
  auto event = [&](hipEvent_t* ev) -> hipError_t {
    if (!plan->event_pool.empty()) {
      *ev = plan->event_pool.back();
      plan->event_pool.pop_back();
      return hipSuccess;
    }
    return hipEventCreate(ev);
  };
  // the runtime stamps the events with the kernel's own start and end (Launch)
  auto launch_for = [&](xattn::Launch& l) -> hipError_t {
    l.stream = strm;
    if (!timed) return hipSuccess;
    hipError_t r = event(&l.start);
    if (r == hipSuccess) r = event(&l.stop);
    return r;
  };
  auto launched = [&](int stage, const xattn::Launch& l) {
    if (timed) plan->timing_recs.push_back(TimingRec{stage, l.start, l.stop});
  };
  auto unused = [&](const xattn::Launch& l) {  // a failed launch hands its events back
    if (l.start) plan->event_pool.push_back(l.start);
    if (l.stop) plan->event_pool.push_back(l.stop);
  };

  // a graph-stable handle launches every family the slot has seen with grids of the
  // slot's capacity; the kernels read the real counts from the image header
  for (int f = 0; f < xattn::FAM_COUNT; ++f) {
    if (stable ? !(sl.run_fams & (1 << f)) : s.units[f].empty()) continue;
    p.units = dev + sl.off_units[f];
    p.num_units = static_cast<int32_t>(stable ? sl.cap_units[f] : s.units[f].size());
    p.unit_count = stable ? dev + f : nullptr;
    if (p.num_units == 0) continue;
    xattn::Launch l;
    if ((e = launch_for(l)) != hipSuccess) return unused(l), hip_err(e, "timing event");
    if (f == xattn::FAM_F32) e = xattn::launch_attn_f32(p, l);
    else if (f == xattn::FAM_DEC) e = xattn::launch_attn_decode(p, stable ? sl.run_dec_rows : s.dec_rows, l);
    else e = xattn::launch_attn_mma(p, l);
    if (e != hipSuccess) return unused(l), hip_err(e, "attention kernel launch");
    launched(f, l);
  }
  if (stable) {
    p.num_merges = sl.run_merge ? static_cast<int32_t>(sl.cap_merges) : 0;
    p.merge_count = dev + 3;
  }
  if (p.num_merges > 0) {
    xattn::Launch l;
    if ((e = launch_for(l)) != hipSuccess) return unused(l), hip_err(e, "timing event");
    if ((e = xattn::launch_merge(p, sl.dtype, l)) != hipSuccess) return unused(l), hip_err(e, "merge kernel launch");
    launched(3, l);
  }
  return XATTN_OK;
}

}  // namespace

extern "C" {

int xattn_run(xattn_plan_t plan, const void* q, const void* k_pages, const void* v_pages, void* out,
              float* lse, void* stream) {
  int rc = check_run_args(plan, q, k_pages, v_pages, out, lse);
  if (rc != XATTN_OK) return rc;
  Slot& sl = plan->slot[plan->cur];
  const Schedule& s = sl.sched;
  hipError_t e;
  if ((e = slot_wait(sl, stream)) != hipSuccess) return hip_err(e, "hipStreamWaitEvent");
  const bool stable = (plan->flags & XATTN_PLAN_GRAPH_STABLE) != 0;
  if ((stable ? sl.run_merge : !s.merges.empty()) && (e = ws_order(sl, stream)) != hipSuccess)
    return hip_err(e, "workspace order");
  float* ws_lse = sl.ws ? sl.ws + static_cast<size_t>(sl.cap_ws_rows) * sl.d : nullptr;
  if ((rc = launch_run(plan, q, k_pages, v_pages, out, lse, stream, sl.ws, ws_lse, true)) != XATTN_OK)
    return rc;
  if ((e = slot_mark(sl, stream)) != hipSuccess) return hip_err(e, "hipEventRecord");
  return XATTN_OK;
}

int xattn_run_noalloc(xattn_plan_t plan, const void* q, const void* k_pages, const void* v_pages,
                      void* out, float* lse, void* stream) {
  int rc = check_run_args(plan, q, k_pages, v_pages, out, lse);
  if (rc != XATTN_OK) return rc;
  Slot& sl = plan->slot[plan->cur];
  const Schedule& s = sl.sched;
  if (stream != sl.plan_stream)
    return set_err(XATTN_ERR_INVALID_ARG,
                   "xattn_run_noalloc runs on the stream of the latest xattn_plan only");
  const bool stable = (plan->flags & XATTN_PLAN_GRAPH_STABLE) != 0;
  float* ws_o = nullptr;
  float* ws_lse = nullptr;
  if (stable ? sl.run_merge : !s.merges.empty()) {
    // every split row is written by its chunk's unit before the merge of the same run
    // reads it, so the scratch needs no clearing
    const int64_t rows = stable ? sl.cap_ws_rows : s.ws_rows;
    const size_t need = static_cast<size_t>(rows) * (sl.d + 1) * sizeof(float);
    if (need > xattn::static_scratch_bytes())
      return set_err(XATTN_ERR_UNSUPPORTED,
                     "split workspace of " + std::to_string(need) + " bytes exceeds the static scratch of " +
                         std::to_string(xattn::static_scratch_bytes()) + " bytes; use xattn_run");
    hipError_t e = xattn::static_scratch(&ws_o);
    if (e != hipSuccess) return hip_err(e, "hipGetSymbolAddress");
    ws_lse = ws_o + static_cast<size_t>(rows) * sl.d;
  }
  return launch_run(plan, q, k_pages, v_pages, out, lse, stream, ws_o, ws_lse, false);
}

int xattn_write_kv(xattn_plan_t plan, const void* k_src, const void* v_src, void* k_pages,
                   void* v_pages, void* stream) {
  if (!plan || plan->cur < 0 || !plan->slot[plan->cur].ready)
    return set_err(XATTN_ERR_INVALID_ARG, "write_kv without a successful plan");
  Slot& sl = plan->slot[plan->cur];
  const Schedule& s = sl.sched;
  if (s.total_kv == 0) return XATTN_OK;
  if (s.total_kv > INT32_MAX)
    return set_err(XATTN_ERR_UNSUPPORTED, "contexts of more than 2^31-1 rows in total");
  if (!k_src || !v_src || !k_pages || !v_pages)
    return set_err(XATTN_ERR_INVALID_ARG, "k_src, v_src, k_pages and v_pages are required");
  const uintptr_t mis = reinterpret_cast<uintptr_t>(k_src) | reinterpret_cast<uintptr_t>(v_src) |
                        reinterpret_cast<uintptr_t>(k_pages) | reinterpret_cast<uintptr_t>(v_pages);
  if (mis & 15) return set_err(XATTN_ERR_INVALID_ARG, "k_src, v_src, k_pages and v_pages must be 16-byte aligned");
  const int batch = static_cast<int>(s.reqs.size() / 4);
  int max_kv = 0;
  for (int r = 0; r < batch; ++r) max_kv = std::max(max_kv, s.reqs[4 * r + 2]);
  const int groups = xattn::write_kv_groups(max_kv);
  if (static_cast<int64_t>(batch) * groups > INT32_MAX)
    return set_err(XATTN_ERR_UNSUPPORTED, "too many context blocks for one launch");

  hipStream_t strm = static_cast<hipStream_t>(stream);
  hipError_t e;
  if ((e = slot_wait(sl, stream)) != hipSuccess) return hip_err(e, "hipStreamWaitEvent");
  const int32_t* dev = static_cast<const int32_t*>(sl.dev);
  xattn::WriteParams w{};
  w.k_src = k_src;
  w.v_src = v_src;
  w.k_pages = k_pages;
  w.v_pages = v_pages;
  w.reqs = dev + sl.off_reqs;
  w.kv_start = dev + sl.off_kv_start;
  w.pages = s.identity ? nullptr : dev + sl.off_pages;
  w.batch = batch;
  w.groups = groups;
  w.page_size = sl.page_size;
  w.page_shift = -1;
  if ((sl.page_size & (sl.page_size - 1)) == 0) {
    int sh = 0;
    while ((1 << sh) < sl.page_size) ++sh;
    w.page_shift = sh;
  }
  w.row_bytes = sl.hkv * sl.d * (sl.dtype == XATTN_BF16 ? 2 : 4);
  xattn::Launch l;
  l.stream = strm;
  if ((e = xattn::launch_write_kv(w, l)) != hipSuccess) return hip_err(e, "context write launch");
  if ((e = slot_mark(sl, stream)) != hipSuccess) return hip_err(e, "hipEventRecord");
  return XATTN_OK;
}

int xattn_plan_ready(xattn_plan_t plan) {
  if (!plan) return set_err(XATTN_ERR_INVALID_ARG, "plan is NULL");
  const Slot& sl = plan->slot[plan->cur < 0 ? 0 : (plan->cur ^ 1)];
  if (sl.uploaded_rec) {
    const hipError_t e = hipEventQuery(sl.uploaded);
    if (e == hipErrorNotReady) return 0;
    if (e != hipSuccess) return hip_err(e, "hipEventQuery");
  }
  for (size_t i = 0; i < sl.foreign_live; ++i) {
    const hipError_t e = hipEventQuery(sl.foreign[i].second);
    if (e == hipErrorNotReady) return 0;
    if (e != hipSuccess) return hip_err(e, "hipEventQuery");
  }
  return 1;
}

int xattn_plan_info(xattn_plan_t plan, xattn_schedule_info* info) {
  if (!plan || !info) return set_err(XATTN_ERR_INVALID_ARG, "NULL argument");
  if (plan->cur < 0) return set_err(XATTN_ERR_INVALID_ARG, "no schedule yet");
  fill_info(plan->slot[plan->cur].sched, info);
  info->layout_generation = plan->slot[plan->cur].layout_gen;
  info->slot = plan->cur;
  return XATTN_OK;
}

int xattn_plan_set_timing(xattn_plan_t plan, int every) {
  if (!plan) return set_err(XATTN_ERR_INVALID_ARG, "plan is NULL");
  plan->timing_every = every > 0 ? every : 0;
  plan->runs = 0;
  return XATTN_OK;
}

int xattn_plan_timing(xattn_plan_t plan, double* ms, int32_t* launches) {
  if (!plan || !ms || !launches) return set_err(XATTN_ERR_INVALID_ARG, "NULL argument");
  for (int i = 0; i < 4; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  int rc = XATTN_OK;
  for (const TimingRec& r : plan->timing_recs) {
    float t = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.start, r.stop);
    if (e != hipSuccess && rc == XATTN_OK) rc = hip_err(e, "hipEventElapsedTime");
    ms[r.stage] += t;
    launches[r.stage] += 1;
    plan->event_pool.push_back(r.start);
    plan->event_pool.push_back(r.stop);
  }
  plan->timing_recs.clear();
  return rc;
}

void xattn_plan_destroy(xattn_plan_t plan) {
  if (!plan) return;
  for (const TimingRec& r : plan->timing_recs) {
    (void)hipEventSynchronize(r.stop);
    plan->event_pool.push_back(r.start);
    plan->event_pool.push_back(r.stop);
  }
  for (hipEvent_t ev : plan->event_pool) (void)hipEventDestroy(ev);
  for (Slot& sl : plan->slot) {
    // runs on the plan's stream and on other streams must be done before the buffers go
    if (sl.uploaded_rec && sl.fence && hipEventRecord(sl.fence, static_cast<hipStream_t>(sl.plan_stream)) == hipSuccess)
      (void)hipEventSynchronize(sl.fence);
    for (size_t i = 0; i < sl.foreign_live; ++i) (void)hipEventSynchronize(sl.foreign[i].second);
    for (auto& f : sl.foreign) (void)hipEventDestroy(f.second);
    if (sl.ws_used && sl.ws_event &&
        hipEventRecord(sl.ws_event, static_cast<hipStream_t>(sl.ws_stream)) == hipSuccess)
      (void)hipEventSynchronize(sl.ws_event);
    if (sl.fence) (void)hipEventDestroy(sl.fence);
    if (sl.uploaded) (void)hipEventDestroy(sl.uploaded);
    if (sl.ws_event) (void)hipEventDestroy(sl.ws_event);
    if (sl.host) (void)hipHostFree(sl.host);
    if (sl.dev) (void)hipFree(sl.dev);
    if (sl.ws) (void)hipFree(sl.ws);
  }
  delete plan;
}

}  // extern "C"
