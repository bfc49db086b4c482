// C ABI of the K-Means library: argument checks, workspace carving, the
// per-iteration launch sequence and the chunked host-streaming pipeline.
//
// Citations name the page "Flash-KMeans: Fast and Memory-Efficient Exact
// K-Means" (gist.science summary of paper 2603.09229); "tech §n" is a section
// of its technical summary.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <condition_variable>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <mutex>
#include <string>
#include <thread>
#include <unordered_map>
#include <utility>
#include <vector>

#include "../../include/kmeans.h"
#include "copy_pool.hpp"
#include "km_internal.hpp"

using namespace km;

// --------------------------------------------------------------- errors ----

static thread_local std::string g_last_error;

static km_status fail(km_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

#define KM_HIP(call)                                                                               \
  do {                                                                                             \
    hipError_t e_ = (call);                                                                        \
    if (e_ != hipSuccess) return fail(KM_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_)); \
  } while (0)

// --------------------------------------------------------------- timing ----

namespace {
struct TimingRegistry {
  std::mutex mu;
  int mode = 0;  // 0 off, 1 every phase, 2 the "assign" phase only
  std::unordered_map<std::string, std::vector<std::pair<hipEvent_t, hipEvent_t>>> rec;
};
TimingRegistry& timing() {
  static TimingRegistry r;
  return r;
}

// Timing events carry no system-scope fence: they only take timestamps, and the
// fence (a cache writeback and invalidate per record) would slow the work it
// brackets.  Readers synchronise the device before reading them.
#ifndef KM_TIMING_EVENT_FLAGS
#define KM_TIMING_EVENT_FLAGS hipEventDisableSystemFence
#endif

// Brackets the launches made by `fn` with events on `stream` when timing is on.
template <class F>
hipError_t timed(const char* phase, hipStream_t stream, F&& fn) {
  TimingRegistry& T = timing();
  bool on;
  {
    std::lock_guard<std::mutex> g(T.mu);
    on = T.mode == 1 || (T.mode == 2 && std::strcmp(phase, "assign") == 0);
  }
  if (!on) return fn();
  hipEvent_t a, b;
  hipError_t e = hipEventCreateWithFlags(&a, KM_TIMING_EVENT_FLAGS);
  if (e != hipSuccess) return e;
  e = hipEventCreateWithFlags(&b, KM_TIMING_EVENT_FLAGS);
  if (e != hipSuccess) return e;
  e = hipEventRecord(a, stream);
  if (e != hipSuccess) return e;
  e = fn();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, stream);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> g(T.mu);
  T.rec[phase].emplace_back(a, b);
  return hipSuccess;
}
}  // namespace

#define KM_TIMED(phase, stream, body)                                                     \
  do {                                                                                    \
    hipError_t e_ = timed(phase, stream, [&]() -> hipError_t { body; });                  \
    if (e_ != hipSuccess) return fail(KM_ERR_HIP, std::string(phase) + ": " + hipGetErrorString(e_)); \
  } while (0)

// ------------------------------------------------ device and planner ----

namespace {
// The last-level cache of the GPU at PCI location (domain, bus, device), from
// the KFD topology (the largest cache of the highest level listed for its
// node); 0 when not found.
int64_t kfd_llc_bytes(int domain, int bus, int dev) {
  int64_t best = 0;
  for (int node = 0; node < 256; ++node) {
    const std::string base = "/sys/class/kfd/kfd/topology/nodes/" + std::to_string(node);
    std::ifstream props(base + "/properties");
    if (!props) {
      if (node > 0) break;
      continue;
    }
    int64_t loc = -1, dom = -1, simds = 0;
    std::string key;
    int64_t val;
    while (props >> key >> val) {
      if (key == "location_id") loc = val;
      else if (key == "domain") dom = val;
      else if (key == "simd_count") simds = val;
    }
    // location_id = bus << 8 | device << 3 | function
    if (simds <= 0 || dom != domain || (loc >> 8) != bus || ((loc >> 3) & 31) != dev) continue;
    // A gfx950 node lists every compute unit's L1 caches (over 500 entries)
    // before its L2 and its Infinity Cache: walk them all.
    int best_level = 0;
    for (int c = 0; c < (1 << 16); ++c) {
      std::ifstream cp(base + "/caches/" + std::to_string(c) + "/properties");
      if (!cp) break;
      int64_t level = 0, size_kb = 0;
      while (cp >> key >> val) {
        if (key == "level") level = val;
        else if (key == "size") size_kb = val;
      }
      if (level > best_level || (level == best_level && size_kb * 1024 > best)) {
        best_level = (int)level;
        best = size_kb * 1024;
      }
    }
    break;
  }
  return best;
}

DeviceInfo query_device(int dev) {
  DeviceInfo d{256, 160 * 1024, 4 << 20, (int64_t)256 << 20, false, "defaults"};  // MI355X
  int cus = 0, lds = 0, l2 = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return d;
  d.cus = cus;
  if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) == hipSuccess && lds > 0)
    d.lds_bytes = lds;
  if (hipDeviceGetAttribute(&l2, hipDeviceAttributeL2CacheSize, dev) == hipSuccess && l2 > 0) d.l2_bytes = l2;
  int domain = 0, bus = 0, pdev = 0;
  (void)hipDeviceGetAttribute(&domain, hipDeviceAttributePciDomainID, dev);
  (void)hipDeviceGetAttribute(&bus, hipDeviceAttributePciBusId, dev);
  (void)hipDeviceGetAttribute(&pdev, hipDeviceAttributePciDeviceId, dev);
  const int64_t llc = kfd_llc_bytes(domain, bus, pdev);
  d.queried = true;
  if (llc > d.l2_bytes) {
    d.llc_bytes = llc;
    d.llc_from = "KFD topology";
    return d;
  }
  // No larger level listed (the topology hidden from this process): gfx950
  // parts carry a 256 MiB Infinity Cache; any other device keeps its L2.
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) == hipSuccess && std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) {
    d.llc_bytes = (int64_t)256 << 20;
    d.llc_from = "gfx950";
  } else {
    (void)hipGetLastError();
    d.llc_bytes = d.l2_bytes;
    d.llc_from = "L2";
  }
  return d;
}

constexpr int kOverrides = 9;
std::atomic<int> g_override[kOverrides];  // PlanOverride fields, in order
const char* const kOverrideKeys[kOverrides] = {"assign_kernel", "assign_fold", "assign_split", "reduce_tile",
                                               "radix_items", "small_update", "sort_scan", "sort_rank",
                                               "radix_bits"};
}  // namespace

namespace km {
const DeviceInfo& device_info() {
  static std::mutex mu;
  static std::vector<DeviceInfo*> cache;  // per device ordinal, kept for the life of the process
  static const DeviceInfo fallback{256, 160 * 1024, 4 << 20, (int64_t)256 << 20, false, "defaults"};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fallback;
  }
  std::lock_guard<std::mutex> g(mu);
  if ((int)cache.size() <= dev) cache.resize((size_t)dev + 1, nullptr);
  if (!cache[(size_t)dev]) cache[(size_t)dev] = new DeviceInfo(query_device(dev));
  return *cache[(size_t)dev];
}

PlanOverride plan_override() {
  PlanOverride p;
  p.assign_kernel = g_override[0].load(std::memory_order_relaxed);
  p.assign_fold = g_override[1].load(std::memory_order_relaxed);
  p.assign_split = g_override[2].load(std::memory_order_relaxed);
  p.reduce_tile = g_override[3].load(std::memory_order_relaxed);
  p.radix_items = g_override[4].load(std::memory_order_relaxed);
  p.small_update = g_override[5].load(std::memory_order_relaxed);
  p.sort_scan = g_override[6].load(std::memory_order_relaxed);
  p.sort_rank = g_override[7].load(std::memory_order_relaxed);
  p.radix_bits = g_override[8].load(std::memory_order_relaxed);
  return p;
}
}  // namespace km

// ---------------------------------------------------------- validation ----

static bool dtype_ok(km_dtype dt) { return dt == KM_F32 || dt == KM_BF16 || dt == KM_F16; }
static bool aligned(const void* p, size_t a) { return ((uintptr_t)p) % a == 0; }
static const int64_t kMaxN = (int64_t)1 << 31;

static km_status check_sizes(int64_t N, int64_t D, int64_t K, km_dtype dt, bool need_d) {
  if (!dtype_ok(dt)) return fail(KM_ERR_INVALID_VALUE, "dtype must be KM_F32, KM_BF16 or KM_F16");
  if (N < 0 || N >= kMaxN) return fail(KM_ERR_INVALID_VALUE, "N must satisfy 0 <= N < 2^31");
  if (K < 1 || K >= kMaxN) return fail(KM_ERR_INVALID_VALUE, "K must satisfy 1 <= K < 2^31");
  if (need_d) {
    if (D < 1) return fail(KM_ERR_INVALID_VALUE, "D must be >= 1");
    if (D > kMaxD)
      return fail(KM_ERR_UNSUPPORTED, "D=" + std::to_string(D) + " exceeds the supported maximum " +
                                          std::to_string(kMaxD));
    if (K * D >= kMaxN * 64) return fail(KM_ERR_UNSUPPORTED, "K*D too large");
  }
  return KM_OK;
}

// ----------------------------------------------------------- geometry -----

static AssignGeom assign_geom(int64_t N, int64_t D, int64_t K, km_dtype dt, int64_t B = 1) {
  return make_assign_geom(N, D, K, (int)dt, B);
}

static SortGeom sort_geom(int64_t N, int64_t K) {
  SortGeom g;
  g.N = N;
  g.K = K;
  int kb = 0;
  while (kb < 31 && ((int64_t)1 << kb) <= K - 1) ++kb;
  if (kb < 1) kb = 1;
  g.kbits = kb;
  const PlanOverride ov = plan_override();
  g.items = radix_items(N);
  // Digits of up to 8 bits (ranked by wavefront ballots) where they save one of at most three passes and blocks
  // hold at most 4,096 keys; otherwise up to 6 (per-thread counters, faster at an equal pass count).  (Measured on
  // gfx950, uniform ids: 2^20 keys of 16 bits sort in 53.7 us in two 8-bit passes against 60.7 in three 6-bit
  // ones, 2^22 in 83.5 against 90.7, 2^20 keys of 8 bits in 26.9 us in one pass against 36.4 in two; 19-bit ids
  // in three 8-bit passes 78.2 against 75.4 in four 6-bit ones; at an equal pass count the ballot ranking is
  // 14-20% slower, and 77% slower in 8,192-key blocks.)
  const int p6 = (kb + kMaxDigitBits - 1) / kMaxDigitBits, p8 = (kb + kMaxWaveDigitBits - 1) / kMaxWaveDigitBits;
  const bool wide = p8 < p6 && p6 <= 3 && g.items <= 16;
  const int maxb = ov.radix_bits ? ov.radix_bits : (wide ? kMaxWaveDigitBits : kMaxDigitBits);
  g.npass = (kb + maxb - 1) / maxb;
  const int base = kb / g.npass, rem = kb % g.npass;
  for (int p = 0; p < 6; ++p) g.bits[p] = p < g.npass ? base + (p < rem ? 1 : 0) : 0;
  const int64_t blk = (int64_t)kRadixThreads * g.items;
  g.nblk = (N + blk - 1) / blk;
  int64_t m = 1;
  for (int p = 0; p < g.npass; ++p) {
    const int64_t len = ((int64_t)1 << g.bits[p]) * g.nblk;
    if (len > m) m = len;
  }
  g.count_len = m;
  g.scan_mode = ov.sort_scan;
  g.wave_rank = ov.sort_rank == 2 || maxb > kMaxDigitBits;
  return g;
}

// Bump allocator over the caller's workspace (256-byte aligned pieces).
struct Carve {
  uint8_t* base;
  size_t used = 0;
  explicit Carve(void* b) : base((uint8_t*)b) {}
  template <class T>
  T* take(size_t count) {
    used = (used + 255) / 256 * 256;
    T* p = base ? (T*)(base + used) : nullptr;
    used += count * sizeof(T);
    return p;
  }
};

struct SortBufs {
  int32_t *key_a, *val_a, *key_b, *val_b;
  uint32_t *counts, *scan_part;
  int32_t* off;
};

static SortBufs carve_sort(Carve& c, const SortGeom& g) {
  SortBufs b;
  const size_t n = (size_t)(g.N > 0 ? g.N : 1);
  b.key_a = c.take<int32_t>(n);
  b.val_a = c.take<int32_t>(n);
  b.key_b = c.take<int32_t>(n);
  b.val_b = c.take<int32_t>(n);
  b.counts = c.take<uint32_t>((size_t)g.count_len);
  b.scan_part = c.take<uint32_t>((size_t)scan_part_len(g.count_len));
  b.off = c.take<int32_t>((size_t)g.K + 1);
  return b;
}

struct UpdateBufs {
  SortBufs s;
  float* carry_sum;
  int32_t* carry_cnt;
  float* group_sum;
  int32_t* group_cnt;
  float* small_sum;  // chunk sums of the small-codebook update
  int32_t* small_cnt;
};

// g: the whole update (all B problems); B problems of g.N / B points and g.K / B clusters each.
static UpdateBufs carve_update(Carve& c, const SortGeom& g, int64_t D, km_dtype dt, int64_t B = 1) {
  UpdateBufs u;
  u.s = carve_sort(c, g);
  const int64_t kper = g.K / B;
  const int64_t nsmall = kper <= kSmallMaxK ? B * small_chunks(g.N / B) * kper : 1;
  u.small_sum = c.take<float>((size_t)(nsmall > 0 ? nsmall : 1) * (size_t)reduce_dc((int)dt, D));
  u.small_cnt = c.take<int32_t>((size_t)(nsmall > 0 ? nsmall : 1));
  const int64_t ntiles = reduce_carry_tiles((int)dt, D, g.N);  // (a streamed chunk may hold fewer points)
  u.carry_sum = c.take<float>((size_t)(ntiles > 0 ? ntiles : 1) * 2 * (size_t)reduce_dc((int)dt, D));
  u.carry_cnt = c.take<int32_t>((size_t)(ntiles > 0 ? ntiles : 1) * 2);
  const int64_t tpb = reduce_tpb((int)dt, D);
  const int64_t ngroups = (ntiles + tpb - 1) / tpb;
  u.group_sum = c.take<float>((size_t)(ngroups > 0 ? ngroups : 1) * (size_t)reduce_dc((int)dt, D));
  u.group_cnt = c.take<int32_t>((size_t)(ngroups > 0 ? ngroups : 1));
  return u;
}

struct FitBufs {
  void* frag;
  void* split;  // scratch of a split FlashAssign sweep (NULL: none)
  UpdateBufs u;
  int32_t* assign;
  float* min_dist;
  double* obj_part;
};

// split: room for a split FlashAssign sweep (the streamed fit sizes its buffers for its largest chunk and
// does not split)
static FitBufs carve_fit(Carve& c, int64_t N, int64_t D, int64_t K, km_dtype dt, bool split = true) {
  FitBufs f;
  const AssignGeom g = assign_geom(N, D, K, dt);
  f.frag = c.take<uint8_t>(g.frag_bytes());
  const size_t sb = split ? assign_split_bytes(g, N, 1) : 0;
  f.split = sb ? c.take<uint8_t>(sb) : nullptr;
  f.u = carve_update(c, sort_geom(N, K), D, dt);
  const size_t n = (size_t)(N > 0 ? N : 1);
  f.assign = c.take<int32_t>(n);
  f.min_dist = c.take<float>(n);
  f.obj_part = c.take<double>((size_t)objective_partials(N));
  return f;
}

struct StreamBufs {
  FitBufs f;  // sized for one chunk
  void* xbuf[2];
  float* acc_sum;
  int64_t* acc_cnt;
};

// The streamed fit's warm-start order: every chunk's sorted ids and point order from the last iteration,
// kept for the next (two int32 per row of X).
struct WarmOrder {
  int32_t* keys;
  int32_t* vals;
};
static WarmOrder carve_warm_order(Carve& c, int64_t N) {
  const size_t n = (size_t)(N > 0 ? N : 1);
  WarmOrder w;
  w.keys = c.take<int32_t>(n);
  w.vals = c.take<int32_t>(n);
  return w;
}

static StreamBufs carve_streamed(Carve& c, int64_t rows, int64_t D, int64_t K, km_dtype dt) {
  StreamBufs s;
  s.f = carve_fit(c, rows, D, K, dt, /*split=*/false);
  const size_t xb = (size_t)rows * (size_t)D * (size_t)dtype_size((int)dt);
  s.xbuf[0] = c.take<uint8_t>(xb);
  s.xbuf[1] = c.take<uint8_t>(xb);
  s.acc_sum = c.take<float>((size_t)K * (size_t)D);
  s.acc_cnt = c.take<int64_t>((size_t)K);
  return s;
}

// Batched fit: B problems of one shape.  The update treats the batch as one
// problem of B*N points and B*K clusters (composite id b*K + k), so one sort
// and one segmented reduction serve every problem.
struct BatchBufs {
  void* frag;  // B x frag_bytes
  void* split;  // scratch of a split FlashAssign sweep (NULL: none)
  UpdateBufs u;
  int32_t* ids;  // B*N composite ids
  float* min_dist;
};

static BatchBufs carve_batched(Carve& c, int64_t B, int64_t N, int64_t D, int64_t K, km_dtype dt) {
  BatchBufs b;
  const AssignGeom g = assign_geom(N, D, K, dt, B);
  b.frag = c.take<uint8_t>((size_t)B * g.frag_bytes());
  const size_t sb = assign_split_bytes(g, N, B);
  b.split = sb ? c.take<uint8_t>(sb) : nullptr;
  b.u = carve_update(c, sort_geom(B * N, B * K), D, dt, B);
  const size_t n = (size_t)(B * N > 0 ? B * N : 1);
  b.ids = c.take<int32_t>(n);
  b.min_dist = c.take<float>(n);
  return b;
}

static km_status check_batch(int64_t B, int64_t N, int64_t D, int64_t K, km_dtype dt) {
  km_status st = check_sizes(N, D, K, dt, true);
  if (st != KM_OK) return st;
  if (B < 1 || B >= kMaxN) return fail(KM_ERR_INVALID_VALUE, "B must satisfy 1 <= B < 2^31");
  if (B * N >= kMaxN) return fail(KM_ERR_UNSUPPORTED, "B*N must be < 2^31");
  if (B * K >= kMaxN) return fail(KM_ERR_UNSUPPORTED, "B*K must be < 2^31");
  if (B * K * D >= kMaxN * 64) return fail(KM_ERR_UNSUPPORTED, "B*K*D too large");
  return KM_OK;
}

static size_t workspace_bytes_batched_impl(int64_t B, int64_t N, int64_t D, int64_t K, km_dtype dt) {
  Carve c(nullptr);
  carve_batched(c, B, N, D, K, dt);
  return (c.used + 255) / 256 * 256;
}

static size_t workspace_bytes_impl(km_op op, int64_t N, int64_t D, int64_t K, km_dtype dt, int64_t chunk_rows) {
  Carve c(nullptr);
  switch (op) {
    case KM_OP_ASSIGN: {
      const AssignGeom g = assign_geom(N, D, K, dt);
      c.take<uint8_t>(g.frag_bytes());
      c.take<uint8_t>(assign_split_bytes(g, N, 1));
      break;
    }
    case KM_OP_SORT: carve_sort(c, sort_geom(N, K)); break;
    case KM_OP_UPDATE: carve_update(c, sort_geom(N, K), D, dt); break;
    case KM_OP_FIT: carve_fit(c, N, D, K, dt); break;
    case KM_OP_FIT_STREAMED:
    case KM_OP_FIT_STREAMED_WARM:
    case KM_OP_FIT_STREAMED_RESIDENT: {
      const int64_t rows = chunk_rows < N ? chunk_rows : (N > 0 ? N : 1);
      carve_streamed(c, rows, D, K, dt);
      if (op != KM_OP_FIT_STREAMED) carve_warm_order(c, N);
      if (op == KM_OP_FIT_STREAMED_RESIDENT) {
        c.used = (c.used + 255) / 256 * 256;  // the resident copy starts where the warm layout's size ends
        c.used += (size_t)N * (size_t)D * (size_t)dtype_size((int)dt);
      }
      break;
    }
    default: return 0;
  }
  return (c.used + 255) / 256 * 256;
}

static km_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return KM_OK;
  if (!ws) return fail(KM_ERR_WORKSPACE, "workspace pointer is NULL");
  if (!aligned(ws, 256)) return fail(KM_ERR_INVALID_VALUE, "workspace must be 256-byte aligned");
  if (ws_bytes < need)
    return fail(KM_ERR_WORKSPACE, "workspace too small: " + std::to_string(ws_bytes) + " < " + std::to_string(need));
  return KM_OK;
}

// ------------------------------------------------ host staging copies ----
//
// X in pageable host memory cannot be read by the DMA engine directly: each
// piece is first copied into a pinned staging slot by a small pool of host
// threads (the copy is bound by host memory bandwidth, one thread is not
// enough to keep up with the host link), then uploaded from the slot.

namespace {
CopyPool& copy_pool() {
  static CopyPool pool([] {
    if (const char* e = std::getenv("KM_STAGE_THREADS")) {
      const int v = std::atoi(e);
      if (v >= 1 && v <= 256) return v - 1;
    }
    const int hc = (int)std::thread::hardware_concurrency();
    return std::max(0, std::min(8, hc - 1));
  }());
  return pool;
}
}  // namespace

constexpr int kStageSlots = 4;

// ---------------------------------------------------- launch sequences ----

// perm/prev (optional): the previous iteration's sorted order and sorted keys (warm start).
// prepped: the fragments of C are already in `frag` (written by the last update).
// split: scratch for a split sweep (assign_split_bytes; NULL: never split).
static km_status run_assign(const void* X, km_dtype dt, int64_t N, int64_t D, const float* C, int64_t K,
                            int32_t* assign, float* min_dist, void* frag, hipStream_t s,
                            const int32_t* perm = nullptr, const int32_t* prev = nullptr, bool prepped = false,
                            void* split = nullptr) {
  const AssignGeom g = assign_geom(N, D, K, dt);
  if (!prepped) KM_TIMED("prep", s, return launch_prep(g, C, frag, s));
  if (N > 0)
    KM_TIMED("assign", s, return launch_flash_assign(g, X, N, frag, assign, min_dist, s, perm, prev, 1, 0, split));
  return KM_OK;
}

// Argsort (+ cluster offsets when `offsets`); returns the sorted keys and values (the inverse map).
static km_status run_sort(const int32_t* assign, int64_t N, int64_t K, const SortBufs& b, int32_t* perm_out,
                          int32_t** keys, int32_t** vals, hipStream_t s, bool offsets = true,
                          int32_t* keys_out = nullptr) {
  const SortGeom g = sort_geom(N, K);
  // ping-pong through set a / set b; the last pass may write the caller's perm (and sorted ids)
  int32_t* kf = keys_out ? keys_out : ((g.npass % 2) ? b.key_a : b.key_b);
  int32_t* vf = perm_out ? perm_out : ((g.npass % 2) ? b.val_a : b.val_b);
  KM_TIMED("sort", s, return launch_argsort(g, assign, b.key_a, b.val_a, b.key_b, b.val_b, kf, vf, b.counts,
                                            b.scan_part, s));
  *keys = kf;
  *vals = vf;
  if (offsets) KM_TIMED("segments", s, return launch_boundaries(kf, N, K, b.off, s));
  return KM_OK;
}

constexpr int64_t kFuseFragMaxK = 8192;  // largest codebook whose fix-up also writes the operand fragments

// sorted_keys/sorted_vals (optional out): where the argsort left the sorted
// assignment and the point order, valid until the workspace is used again;
// NULL when the small-codebook path ran (it sorts on chip only).
// B > 1: N points of B problems (N / B each) with K / B clusters each and ids b*(K/B) + k.
// keep_keys/keep_vals (optional, sorted path): where the argsort writes the sorted ids and point order, so
// they outlive the call (the streamed fit's per-chunk warm-start order).
// frag/geom/prepped (optional): FlashAssign's fragment buffer and geometry for
// the next assignment; *prepped tells whether this update already wrote the
// fragments of C_new (then the next assignment skips its centroid preparation).
static km_status run_update(const void* X, km_dtype dt, int64_t N, int64_t D, const int32_t* assign, int64_t K,
                            const float* C_prev, float* C_new, int32_t* counts, const UpdateBufs& u, int mode,
                            float* acc_sum, int64_t* acc_cnt, hipStream_t s, const int32_t** sorted_keys = nullptr,
                            const int32_t** sorted_vals = nullptr, int64_t B = 1, void* frag = nullptr,
                            const AssignGeom* geom = nullptr, bool* prepped = nullptr, int32_t* keep_keys = nullptr,
                            int32_t* keep_vals = nullptr) {
  if (sorted_keys) *sorted_keys = nullptr;
  if (sorted_vals) *sorted_vals = nullptr;
  if (prepped) *prepped = false;
  const bool deep = deep_rows((int)dt, D);  // rows beyond one lane group: no small-codebook path, column strips
  if (mode == MODE_MEAN && !deep && plan_override().small_update != 1 &&
      (K / B <= kSmallMaxK || small_owner_fits(B, N / B, K / B))) {
    SmallArgs a;
    a.X = X;
    a.dt = (int)dt;
    a.B = B;
    a.N = N / B;
    a.D = D;
    a.K = K / B;
    a.ids = assign;
    a.id_mul = K / B;
    a.C_prev = C_prev;
    a.C_new = C_new;
    a.counts = counts;
    a.part_sum = u.small_sum;
    a.part_cnt = u.small_cnt;
    a.frag = (frag && geom && prepped) ? frag : nullptr;
    a.f_stride = geom ? (int64_t)(geom->frag_bytes() / 16) : 0;
    if (geom) a.cfg = geom->cfg;
    a.emitted = prepped;
    KM_TIMED("reduce", s, return launch_small_update(a, s));
    return KM_OK;
  }
  int32_t *keys = nullptr, *vals = nullptr;
  // the segmented reduction writes the cluster offsets itself (it sees every id change)
  km_status st = run_sort(assign, N, K, u.s, keep_vals, &keys, &vals, s, /*offsets=*/N == 0, keep_keys);
  if (st != KM_OK) return st;
  if (sorted_keys) *sorted_keys = keys;
  if (sorted_vals) *sorted_vals = vals;
  ReduceArgs a;
  a.X = X;
  a.dt = (int)dt;
  a.N = N;
  a.D = D;
  a.K = K;
  a.keys = keys;
  a.vals = vals;
  a.off = u.s.off;
  a.carry_sum = u.carry_sum;
  a.carry_cnt = u.carry_cnt;
  a.group_sum = u.group_sum;
  a.group_cnt = u.group_cnt;
  a.mode = mode;
  a.C_prev = C_prev;
  a.C_new = C_new;
  a.counts = counts;
  a.acc_sum = acc_sum;
  a.acc_cnt = acc_cnt;
  // The fix-up writes the next assignment's operands when it is cheaper than a separate preparation: one
  // wavefront per cluster against one workgroup per 32 centroids (measured on gfx950: a gain up to K = 4096,
  // a loss at K = 65536, where most clusters would keep a wavefront only for this).
  if (mode == MODE_MEAN && frag && geom && prepped && K / B <= kFuseFragMaxK && !deep) {
    a.frag = frag;
    a.f_stride = (int64_t)(geom->frag_bytes() / 16);
    a.kper = K / B;
    a.cfg = geom->cfg;
  }
  const int64_t nstrips = reduce_strips((int)dt, D);  // 1 unless the rows are deep
  for (int64_t strip = 0; strip < nstrips; ++strip) {
    a.strip = strip;
    KM_TIMED("reduce", s, return launch_segment_reduce(a, s));
    KM_TIMED("finalize", s, return launch_fixup(a, s));
  }
  if (a.frag) *prepped = true;
  return KM_OK;
}

// ------------------------------------------------------------ entry points --

namespace km {
// The argument checks of kmeans_fit other than the workspace (shared with kmeans_fit_noalloc).
km_status fit_args_check(const void* X, km_dtype dt, int64_t N, int64_t D, int64_t K, const float* C, int32_t iters,
                         const int32_t* assign, const int32_t* counts, const double* objective) {
  km_status st = check_sizes(N, D, K, dt, true);
  if (st != KM_OK) return st;
  if (iters < 0) return fail(KM_ERR_INVALID_VALUE, "iters must be >= 0");
  if (!C || (N > 0 && !X)) return fail(KM_ERR_INVALID_VALUE, "X and C must be non-NULL");
  if (!aligned(X, dt == KM_F32 ? 4 : 2) || !aligned(C, 4) || !aligned(assign, 4) || !aligned(counts, 4) ||
      !aligned(objective, 8))
    return fail(KM_ERR_INVALID_VALUE, "misaligned pointer");
  return KM_OK;
}

km_status fail_with(km_status s, const char* msg) { return fail(s, msg); }
}  // namespace km

extern "C" {

size_t kmeans_workspace_bytes(km_op op, int64_t N, int64_t D, int64_t K, km_dtype dt, int64_t chunk_rows) {
  const bool need_d = op != KM_OP_SORT;
  if (check_sizes(N, need_d ? D : 1, K, op == KM_OP_SORT ? KM_F32 : dt, need_d) != KM_OK) return 0;
  if ((op == KM_OP_FIT_STREAMED || op == KM_OP_FIT_STREAMED_WARM || op == KM_OP_FIT_STREAMED_RESIDENT) &&
      chunk_rows < 1)
    return 0;
  return workspace_bytes_impl(op, N, D, K, dt, chunk_rows);
}

km_status kmeans_assign(const void* X, km_dtype dt, int64_t N, int64_t D, const float* C, int64_t K, int32_t* assign,
                        float* min_dist, void* ws, size_t ws_bytes, void* stream) {
  km_status st = check_sizes(N, D, K, dt, true);
  if (st != KM_OK) return st;
  if (!C || (N > 0 && (!X || !assign))) return fail(KM_ERR_INVALID_VALUE, "X, C and assign must be non-NULL");
  if (!aligned(X, dt == KM_F32 ? 4 : 2) || !aligned(C, 4) || !aligned(assign, 4) || !aligned(min_dist, 4))
    return fail(KM_ERR_INVALID_VALUE, "misaligned pointer");
  st = check_ws(ws, ws_bytes, workspace_bytes_impl(KM_OP_ASSIGN, N, D, K, dt, 0));
  if (st != KM_OK) return st;
  Carve c(ws);
  const AssignGeom g = assign_geom(N, D, K, dt);
  void* frag = c.take<uint8_t>(g.frag_bytes());
  const size_t sb = assign_split_bytes(g, N, 1);
  void* split = sb ? c.take<uint8_t>(sb) : nullptr;
  return run_assign(X, dt, N, D, C, K, assign, min_dist, frag, (hipStream_t)stream, nullptr, nullptr, false, split);
}

km_status kmeans_sort_by_cluster(const int32_t* assign, int64_t N, int64_t K, int32_t* perm, int32_t* offsets,
                                 void* ws, size_t ws_bytes, void* stream) {
  km_status st = check_sizes(N, 1, K, KM_F32, false);
  if (st != KM_OK) return st;
  if (N > 0 && (!assign || !perm)) return fail(KM_ERR_INVALID_VALUE, "assign and perm must be non-NULL");
  if (!aligned(assign, 4) || !aligned(perm, 4) || !aligned(offsets, 4))
    return fail(KM_ERR_INVALID_VALUE, "misaligned pointer");
  st = check_ws(ws, ws_bytes, workspace_bytes_impl(KM_OP_SORT, N, 1, K, KM_F32, 0));
  if (st != KM_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  Carve c(ws);
  const SortBufs b = carve_sort(c, sort_geom(N, K));
  int32_t *keys = nullptr, *vals = nullptr;
  if (N > 0) {
    st = run_sort(assign, N, K, b, perm, &keys, &vals, s);
    if (st != KM_OK) return st;
  } else {
    KM_TIMED("segments", s, return launch_boundaries(b.key_a, 0, K, b.off, s));
  }
  if (offsets) KM_HIP(hipMemcpyAsync(offsets, b.off, sizeof(int32_t) * (size_t)(K + 1), hipMemcpyDeviceToDevice, s));
  return KM_OK;
}

km_status kmeans_update(const void* X, km_dtype dt, int64_t N, int64_t D, const int32_t* assign, int64_t K,
                        const float* C_prev, float* C_new, int32_t* counts, void* ws, size_t ws_bytes, void* stream) {
  km_status st = check_sizes(N, D, K, dt, true);
  if (st != KM_OK) return st;
  if (!C_prev || !C_new || (N > 0 && (!X || !assign)))
    return fail(KM_ERR_INVALID_VALUE, "X, assign, C_prev and C_new must be non-NULL");
  if (!aligned(X, dt == KM_F32 ? 4 : 2) || !aligned(assign, 4) || !aligned(C_prev, 4) || !aligned(C_new, 4) ||
      !aligned(counts, 4))
    return fail(KM_ERR_INVALID_VALUE, "misaligned pointer");
  st = check_ws(ws, ws_bytes, workspace_bytes_impl(KM_OP_UPDATE, N, D, K, dt, 0));
  if (st != KM_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  Carve c(ws);
  const UpdateBufs u = carve_update(c, sort_geom(N, K), D, dt);
  if (N == 0) {  // every cluster is empty: keep C_prev
    if (counts) KM_HIP(launch_zero(counts, sizeof(int32_t) * (size_t)K, s));
    if (C_new != C_prev)
      KM_HIP(hipMemcpyAsync(C_new, C_prev, sizeof(float) * (size_t)(K * D), hipMemcpyDeviceToDevice, s));
    return KM_OK;
  }
  return run_update(X, dt, N, D, assign, K, C_prev, C_new, counts, u, MODE_MEAN, nullptr, nullptr, s);
}

km_status kmeans_fit(const void* X, km_dtype dt, int64_t N, int64_t D, int64_t K, float* C, int32_t iters,
                     int32_t* assign, int32_t* counts, double* objective, void* ws, size_t ws_bytes, void* stream) {
  km_status st = km::fit_args_check(X, dt, N, D, K, C, iters, assign, counts, objective);
  if (st != KM_OK) return st;
  st = check_ws(ws, ws_bytes, workspace_bytes_impl(KM_OP_FIT, N, D, K, dt, 0));
  if (st != KM_OK) return st;
  if (iters == 0) return KM_OK;
  hipStream_t s = (hipStream_t)stream;
  Carve c(ws);
  const FitBufs f = carve_fit(c, N, D, K, dt);
  int32_t* a = assign ? assign : f.assign;
  // From the second iteration on, the assign visits points in the order of the
  // previous argsort and starts each from its previous centroid's group.
  const int32_t *order = nullptr, *prev = nullptr;
  const AssignGeom geom = assign_geom(N, D, K, dt);
  bool prepped = false;  // the last update already wrote the centroid fragments
  for (int32_t t = 0; t < iters; ++t) {
    st = run_assign(X, dt, N, D, C, K, a, objective ? f.min_dist : nullptr, f.frag, s, order, prev, prepped,
                    f.split);
    if (st != KM_OK) return st;
    if (objective) KM_TIMED("objective", s, return launch_objective(f.min_dist, N, f.obj_part, objective + t, 0, s));
    if (N == 0) {
      if (counts) KM_HIP(launch_zero(counts, sizeof(int32_t) * (size_t)K, s));
      continue;
    }
    st = run_update(X, dt, N, D, a, K, C, C, counts, f.u, MODE_MEAN, nullptr, nullptr, s, &prev, &order, 1, f.frag,
                    &geom, &prepped);
    if (st != KM_OK) return st;
  }
  return KM_OK;
}

size_t kmeans_workspace_bytes_batched(int64_t B, int64_t N, int64_t D, int64_t K, km_dtype dt) {
  if (check_batch(B, N, D, K, dt) != KM_OK) return 0;
  return workspace_bytes_batched_impl(B, N, D, K, dt);
}

km_status kmeans_fit_batched(const void* X, km_dtype dt, int64_t B, int64_t N, int64_t D, int64_t K, float* C,
                             int32_t iters, int32_t* assign, int32_t* counts, double* objective, void* ws,
                             size_t ws_bytes, void* stream) {
  km_status st = check_batch(B, N, D, K, dt);
  if (st != KM_OK) return st;
  if (iters < 0) return fail(KM_ERR_INVALID_VALUE, "iters must be >= 0");
  if (!C || (N > 0 && !X)) return fail(KM_ERR_INVALID_VALUE, "X and C must be non-NULL");
  if (!aligned(X, dt == KM_F32 ? 4 : 2) || !aligned(C, 4) || !aligned(assign, 4) || !aligned(counts, 4) ||
      !aligned(objective, 8))
    return fail(KM_ERR_INVALID_VALUE, "misaligned pointer");
  st = check_ws(ws, ws_bytes, workspace_bytes_batched_impl(B, N, D, K, dt));
  if (st != KM_OK) return st;
  if (iters == 0) return KM_OK;
  hipStream_t s = (hipStream_t)stream;
  Carve c(ws);
  const BatchBufs b = carve_batched(c, B, N, D, K, dt);
  const AssignGeom g = assign_geom(N, D, K, dt, B);
  bool prepped = false;  // the last update already wrote the centroid fragments
  for (int32_t t = 0; t < iters; ++t) {
    if (!prepped) KM_TIMED("prep", s, return launch_prep(g, C, b.frag, s, B));
    if (N > 0)
      KM_TIMED("assign", s,
               return launch_flash_assign(g, X, N, b.frag, b.ids, objective ? b.min_dist : nullptr, s, nullptr,
                                          nullptr, B, (int32_t)K, b.split));
    if (objective)
      KM_TIMED("objective", s, return launch_objective_batched(b.min_dist, B, N, objective + (int64_t)t * B, s));
    if (N == 0) {
      if (counts) KM_HIP(launch_zero(counts, sizeof(int32_t) * (size_t)(B * K), s));
      continue;
    }
    st = run_update(X, dt, B * N, D, b.ids, B * K, C, C, counts, b.u, MODE_MEAN, nullptr, nullptr, s, nullptr,
                    nullptr, B, b.frag, &g, &prepped);
    if (st != KM_OK) return st;
  }
  if (assign && N > 0) KM_TIMED("finalize", s, return launch_local_ids(b.ids, B, N, K, assign, s));
  return KM_OK;
}

km_status kmeans_fit_streamed(const void* X_host, km_dtype dt, int64_t N, int64_t D, int64_t K, float* C,
                              int32_t iters, int64_t chunk_rows, int32_t* assign_host, int32_t* counts,
                              double* objective, void* ws, size_t ws_bytes, void* compute_stream,
                              void* copy_stream, void* stage_host, size_t stage_bytes) {
  km_status st = check_sizes(N, D, K, dt, true);
  if (st != KM_OK) return st;
  if (iters < 0) return fail(KM_ERR_INVALID_VALUE, "iters must be >= 0");
  if (chunk_rows < 1) return fail(KM_ERR_INVALID_VALUE, "chunk_rows must be >= 1");
  if (!C || (N > 0 && !X_host)) return fail(KM_ERR_INVALID_VALUE, "X_host and C must be non-NULL");
  if (!copy_stream || copy_stream == compute_stream)
    return fail(KM_ERR_INVALID_VALUE, "copy_stream must be a non-NULL stream distinct from compute_stream");
  if (!aligned(X_host, dt == KM_F32 ? 4 : 2) || !aligned(C, 4) || !aligned(assign_host, 4) ||
      !aligned(counts, 4) || !aligned(objective, 8))
    return fail(KM_ERR_INVALID_VALUE, "misaligned pointer");
  const size_t es = (size_t)dtype_size((int)dt);
  const size_t row_bytes = (size_t)D * es;
  size_t slot_bytes = 0;
  if (stage_host) {
    slot_bytes = stage_bytes / kStageSlots / row_bytes * row_bytes;
    if (slot_bytes == 0)
      return fail(KM_ERR_INVALID_VALUE, "stage_bytes must hold at least " + std::to_string(kStageSlots) + " rows");
  }
  st = check_ws(ws, ws_bytes, workspace_bytes_impl(KM_OP_FIT_STREAMED, N, D, K, dt, chunk_rows));
  if (st != KM_OK) return st;
  if (iters == 0) return KM_OK;
  hipStream_t cs = (hipStream_t)compute_stream, xs = (hipStream_t)copy_stream;
  const int64_t rows = chunk_rows < N ? chunk_rows : (N > 0 ? N : 1);
  // With room for every chunk's order (KM_OP_FIT_STREAMED_WARM), iterations after the first assign each chunk
  // warm, in the order of its last argsort (the same results, bit for bit; only the order of work changes).
  const size_t warm_bytes = workspace_bytes_impl(KM_OP_FIT_STREAMED_WARM, N, D, K, dt, chunk_rows);
  const bool warm = ws_bytes >= warm_bytes;
  // Workspace beyond the warm layout: a device copy of the leading chunks that fit whole (uploaded in the first
  // iteration, read from device memory afterwards).  Chunk ch is resident iff its last row is below res_rows.
  uint8_t* const xres = warm && ws_bytes > warm_bytes ? (uint8_t*)ws + warm_bytes : nullptr;
  const int64_t res_rows = xres ? (int64_t)((ws_bytes - warm_bytes) / row_bytes) : 0;
  Carve c(ws);
  const StreamBufs b = carve_streamed(c, rows, D, K, dt);
  const WarmOrder wo = warm ? carve_warm_order(c, N) : WarmOrder{nullptr, nullptr};
  const int64_t nchunks = N > 0 ? (N + rows - 1) / rows : 0;
  const AssignGeom g = assign_geom(rows, D, K, dt);

  // ready[b]: chunk buffer b is filled; freed[b]: its compute is done; slot_done[s]: staging slot s uploaded
  std::vector<hipEvent_t> events;
  struct EventGuard {
    std::vector<hipEvent_t>& ev;
    ~EventGuard() {
      for (hipEvent_t e : ev) (void)hipEventDestroy(e);
    }
  } guard{events};
  hipEvent_t ready[2], freed[2], slot_done[kStageSlots], start, res_ready;
  for (hipEvent_t* e : {&ready[0], &ready[1], &freed[0], &freed[1], &start, &res_ready}) {
    KM_HIP(hipEventCreateWithFlags(e, hipEventDisableTiming));
    events.push_back(*e);
  }
  // The chunk buffers live in the workspace, which earlier work on the compute
  // stream may still be using (a previous call, or memory the caller's
  // allocator recycled in compute-stream order): uploads start after it.
  KM_HIP(hipEventRecord(start, cs));
  KM_HIP(hipStreamWaitEvent(xs, start, 0));
  if (stage_host)
    for (int i = 0; i < kStageSlots; ++i) {
      KM_HIP(hipEventCreateWithFlags(&slot_done[i], hipEventDisableTiming));
      events.push_back(slot_done[i]);
    }
  uint64_t slot_seq = 0;
  // On every return, error or not, with staging: wait until the uploads already issued from the slots are
  // done, so the caller may free or reuse the staging buffer (and pageable X) as soon as the call returns.
  struct StagingDrain {
    const bool on;
    const uint64_t& seq;
    hipEvent_t* done;
    ~StagingDrain() {
      if (on)
        for (uint64_t i = 0; i < seq && i < (uint64_t)kStageSlots; ++i) (void)hipEventSynchronize(done[i]);
    }
  } drain{stage_host != nullptr, slot_seq, slot_done};
  // Fault injection for tests of the error path: KM_FAULT_INJECT_UPLOAD=n makes the n-th chunk upload of
  // this call fail before it is issued, as a failed copy would (the call returns KM_ERR_HIP).
  int64_t fail_upload = 0, uploads = 0;
  if (const char* e = std::getenv("KM_FAULT_INJECT_UPLOAD")) fail_upload = std::atoll(e);
  // Upload `bytes` of host X to `dst`: one copy from pinned X, or slot by slot through the staging ring.
  auto upload = [&](uint8_t* dst, const uint8_t* src, size_t bytes) -> hipError_t {
    if (++uploads == fail_upload) return hipErrorUnknown;
    if (!stage_host) return hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, xs);
    for (size_t off = 0; off < bytes; off += slot_bytes, ++slot_seq) {
      const size_t n = std::min(slot_bytes, bytes - off);
      const int sl = (int)(slot_seq % kStageSlots);
      hipError_t e;
      if (slot_seq >= (uint64_t)kStageSlots && (e = hipEventSynchronize(slot_done[sl])) != hipSuccess) return e;
      uint8_t* slot = (uint8_t*)stage_host + (size_t)sl * slot_bytes;
      copy_pool().copy(slot, src + off, n);
      if ((e = hipMemcpyAsync(dst + off, slot, n, hipMemcpyHostToDevice, xs)) != hipSuccess) return e;
      if ((e = hipEventRecord(slot_done[sl], xs)) != hipSuccess) return e;
    }
    return hipSuccess;
  };

  int64_t seq = 0;  // counter of the chunks that go through the two chunk buffers: buffer = seq % 2
  for (int32_t t = 0; t < iters; ++t) {
    KM_TIMED("prep", cs, return launch_prep(g, C, b.f.frag, cs));
    KM_HIP(launch_zero(b.acc_sum, sizeof(float) * (size_t)(K * D), cs));
    KM_HIP(launch_zero(b.acc_cnt, sizeof(int64_t) * (size_t)K, cs));
    if (objective && nchunks == 0) KM_HIP(launch_zero(objective + t, sizeof(double), cs));
    for (int64_t ch = 0; ch < nchunks; ++ch) {
      const int64_t r0 = ch * rows;
      const int64_t nr = (N - r0) < rows ? (N - r0) : rows;
      const bool resident = xres && r0 + nr <= res_rows;
      const int buf = resident ? -1 : (int)(seq % 2);
      void* xdev;
      if (resident) {  // uploaded once, into its own place in the resident copy
        xdev = xres + (size_t)r0 * row_bytes;
        if (t == 0) {
          KM_TIMED("h2d", xs,
                   return upload((uint8_t*)xdev, (const uint8_t*)X_host + (size_t)r0 * row_bytes,
                                 (size_t)nr * row_bytes));
          KM_HIP(hipEventRecord(res_ready, xs));
          KM_HIP(hipStreamWaitEvent(cs, res_ready, 0));
        }
      } else {
        xdev = b.xbuf[buf];
        // copy stream: wait until the compute of the chunk that last used this buffer is done
        if (seq >= 2) KM_HIP(hipStreamWaitEvent(xs, freed[buf], 0));
        KM_TIMED("h2d", xs,
                 return upload((uint8_t*)xdev, (const uint8_t*)X_host + (size_t)r0 * row_bytes,
                               (size_t)nr * row_bytes));
        KM_HIP(hipEventRecord(ready[buf], xs));
        KM_HIP(hipStreamWaitEvent(cs, ready[buf], 0));
      }
      // compute stream: assign the chunk, then fold its per-cluster sums into the totals
      int32_t* ck = warm ? wo.keys + r0 : nullptr;  // this chunk's order from the last iteration
      int32_t* cv = warm ? wo.vals + r0 : nullptr;
      KM_TIMED("assign", cs,
               return launch_flash_assign(g, xdev, nr, b.f.frag, b.f.assign, objective ? b.f.min_dist : nullptr,
                                          cs, t > 0 ? cv : nullptr, t > 0 ? ck : nullptr));
      if (objective)
        KM_TIMED("objective", cs,
                 return launch_objective(b.f.min_dist, nr, b.f.obj_part, objective + t, ch > 0 ? 1 : 0, cs));
      const UpdateBufs u = b.f.u;
      st = run_update(xdev, dt, nr, D, b.f.assign, K, nullptr, nullptr, nullptr, u, MODE_ACCUM, b.acc_sum,
                      b.acc_cnt, cs, nullptr, nullptr, 1, nullptr, nullptr, nullptr, ck, cv);
      if (st != KM_OK) return st;
      if (assign_host && t == iters - 1)
        KM_TIMED("d2h", cs,
                 return hipMemcpyAsync(assign_host + r0, b.f.assign, sizeof(int32_t) * (size_t)nr,
                                       hipMemcpyDeviceToHost, cs));
      if (!resident) {
        KM_HIP(hipEventRecord(freed[buf], cs));
        ++seq;
      }
    }
    KM_TIMED("finalize", cs, return launch_finalize_accum(b.acc_sum, b.acc_cnt, K, D, C, counts, cs));
  }
  // With staging, return only once the last uploads have left the slots, so
  // the staging buffer (and pageable X) can be reused as soon as this returns.
  if (stage_host)
    for (uint64_t i = 0; i < slot_seq && i < (uint64_t)kStageSlots; ++i) KM_HIP(hipEventSynchronize(slot_done[i]));
  return KM_OK;  // (the drain guard then finds every slot done)
}

km_status kmeans_plan_override(const char* key, int64_t value) {
  if (!key) return fail(KM_ERR_INVALID_VALUE, "key must be non-NULL");
  for (int i = 0; i < kOverrides; ++i)
    if (std::strcmp(key, kOverrideKeys[i]) == 0) {
      const bool ok = value == 0 ||
                      (i == 0 && (value == 1 || value == 2)) || (i == 1 && (value == 1 || value == 2)) ||
                      (i == 2 && value >= 1 && value <= 64) || (i == 3 && (value == 1 || value == 2)) ||
                      (i == 4 && (value == 8 || value == 16 || value == 32)) || (i == 5 && value == 1) ||
                      (i == 6 && (value == 1 || value == 2)) || (i == 7 && (value == 1 || value == 2)) ||
                      (i == 8 && value >= 5 && value <= kMaxWaveDigitBits);
      if (!ok) return fail(KM_ERR_INVALID_VALUE, std::string("value out of range for ") + key);
      g_override[i].store((int)value, std::memory_order_relaxed);
      return KM_OK;
    }
  return fail(KM_ERR_INVALID_VALUE, std::string("unknown planner key ") + key);
}

km_status kmeans_plan_describe(int64_t N, int64_t D, int64_t K, km_dtype dt, char* buf, size_t len) {
  km_status st = check_sizes(N, D, K, dt, true);
  if (st != KM_OK) return st;
  if (!buf || len == 0) return fail(KM_ERR_INVALID_VALUE, "buf must be non-NULL with len > 0");
  const DeviceInfo& dv = device_info();
  const AssignGeom g = assign_geom(N, D, K, dt);
  auto same = [](const AssignCfg& a, const AssignCfg& b) {
    return a.rows == b.rows && a.KB == b.KB && a.NB == b.NB && a.CT == b.CT && a.W == b.W;
  };
  const char* kernel = is_deep_cfg((int)dt, g.cfg)                                       ? "depth-tiled"
                       : dt == KM_F32                                                    ? "fp32"
                       : g.cfg.KB <= kWide8MaxKB && same(g.cfg, wide8_cfg(g.cfg.KB)) ? "single-accumulator"
                                                                                         : "pipelined";
  const int64_t splits = assign_splits(g, N, 1);
  const SortGeom sg = sort_geom(N, K);
  const bool small = !deep_rows((int)dt, D) && plan_override().small_update != 1 &&
                     (K <= kSmallMaxK || small_owner_fits(1, N, K));
  char upd[256];
  if (small)
    std::snprintf(upd, sizeof upd, "on-chip small-codebook");
  else
    std::snprintf(upd, sizeof upd,
                  "sorted, %d radix pass(es) of %d keys/thread, %s count scans, %s ranks, segment tile %lld, "
                  "%lld column strip(s)",
                  sg.npass, sg.items, sg.scan_mode == 1 ? "whole-table" : (sg.scan_mode == 2 ? "per-digit" : "in-scatter or per-digit"),
                  sg.wave_rank ? "wavefront" : "thread-counter", (long long)reduce_tile((int)dt, D, N),
                  (long long)reduce_strips((int)dt, D));
  char out[640];
  std::snprintf(out, sizeof out,
                "assign: %s kernel, %d depth blocks, %d point groups/wave, %d groups/tile, %d waves, cold argmax %s, "
                "%lld centroid range(s); update: %s; workspace %zu bytes; device: %d CUs, LLC %lld MiB (%s)",
                kernel, g.cfg.KB, g.cfg.NB, g.cfg.CT, g.cfg.W, g.lazy ? "folded" : "exact", (long long)splits, upd,
                workspace_bytes_impl(KM_OP_FIT, N, D, K, dt, 0), dv.cus, (long long)(dv.llc_bytes >> 20),
                dv.llc_from);
  std::snprintf(buf, len, "%s", out);
  return KM_OK;
}

const char* kmeans_status_string(km_status s) {
  switch (s) {
    case KM_OK: return "success";
    case KM_ERR_INVALID_VALUE: return "invalid argument";
    case KM_ERR_UNSUPPORTED: return "unsupported shape";
    case KM_ERR_WORKSPACE: return "workspace missing or too small";
    case KM_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* kmeans_last_error(void) { return g_last_error.c_str(); }

km_status kmeans_timing_enable(int enable) {
  TimingRegistry& T = timing();
  std::lock_guard<std::mutex> g(T.mu);
  if (enable < 0 || enable > 2) return fail(KM_ERR_INVALID_VALUE, "timing mode must be 0, 1 or 2");
  T.mode = enable;
  return KM_OK;
}

km_status kmeans_timing_read(const char* phase, double* total_ms, int64_t* launches) {
  if (!phase || !total_ms || !launches) return fail(KM_ERR_INVALID_VALUE, "NULL argument");
  TimingRegistry& T = timing();
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
  {
    std::lock_guard<std::mutex> g(T.mu);
    auto it = T.rec.find(phase);
    if (it != T.rec.end()) ev = it->second;
  }
  double sum = 0.0;
  for (auto& p : ev) {
    KM_HIP(hipEventSynchronize(p.second));
    float ms = 0.0f;
    KM_HIP(hipEventElapsedTime(&ms, p.first, p.second));
    sum += ms;
  }
  *total_ms = sum;
  *launches = (int64_t)ev.size();
  return KM_OK;
}

km_status kmeans_timing_reset(void) {
  TimingRegistry& T = timing();
  std::lock_guard<std::mutex> g(T.mu);
  for (auto& kv : T.rec)
    for (auto& p : kv.second) {
      (void)hipEventDestroy(p.first);
      (void)hipEventDestroy(p.second);
    }
  T.rec.clear();
  return KM_OK;
}

}  // extern "C"
