// mita_api.hip — the C ABI (include/mita.h): host-side validation, work-space
// planning and the launch sequence of the MiTA forward pass.  No device code
// here; every step of the computation runs in the kernels of the other
// translation units.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "mita.h"
#include "mita_internal.hpp"

namespace mita {
namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& why) {
  g_last_error = why;
  return status;
}

int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// stage profiler
// ---------------------------------------------------------------------------

// in launch order; step 4 (bucketing) runs inside the scan and merge stages
enum Stage {
  kStagePool = 0,
  kStageThreshold,
  kStageRoute,
  kStageScan,
  kStageMerge,
  kStageAttend,
  kStageSmall,  // the one-launch path for short sequences (all five steps)
  kStageBw0,    // the backward pass's steps (BwStep order) follow
  kStageCount = kStageBw0 + kBwStepCount
};
const char* kStageNames[kStageCount] = {
    "pool",         "landmark_threshold", "route",           "landmark_scan",
    "landmark_merge", "expert_attend",    "single_launch",   "bw_zero",
    "bw_pool",      "bw_landmark_fwd",    "bw_bucket",       "bw_attend",
    "bw_cross",     "bw_pool_grad"};

struct Profiler {
  bool enabled = false;
  std::vector<hipEvent_t> free_events;
  struct Pending {
    int stage;
    hipEvent_t a, b;
  };
  std::vector<Pending> pending;
  double ms[kStageCount] = {};
  int64_t calls = 0;

  hipEvent_t get() {
    if (!free_events.empty()) {
      hipEvent_t e = free_events.back();
      free_events.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  void drain() {
    for (auto& p : pending) {
      float t = 0.f;
      if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&t, p.a, p.b) == hipSuccess)
        ms[p.stage] += t;
      free_events.push_back(p.a);
      free_events.push_back(p.b);
    }
    pending.clear();
  }
};
Profiler g_prof;

struct StageTimer {
  int stage;
  hipStream_t st;
  hipEvent_t a = nullptr, b = nullptr;
  // on: false for the no-allocation entry point (the profiler creates events)
  StageTimer(int s, hipStream_t stream, bool on) : stage(s), st(stream) {
    if (on && g_prof.enabled) {
      a = g_prof.get();
      b = g_prof.get();
      if (a && b) hipEventRecord(a, st);
    }
  }
  ~StageTimer() {
    if (a && b) {
      hipEventRecord(b, st);
      g_prof.pending.push_back({stage, a, b});
    }
  }
};

// ---------------------------------------------------------------------------
// device attributes (cached per device)
// ---------------------------------------------------------------------------

int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------------------
// per-device state: the cached work spaces
//
// One block per calling stream (up to kWsStreams per device), kept between
// calls and reused while it is large enough.  Calls on one stream are
// ordered by that stream, so a call's kernels never overlap the previous
// call's use of the block.  A block that is too small is released with
// hipFreeAsync on its stream and replaced by a larger hipMallocAsync block.
// Each call records the entry's event on its stream after its last kernel;
// when a new stream takes over the least recently used entry, it waits for
// that event on the GPU (hipStreamWaitEvent) and frees the old block in its
// own order.  The old stream's handle is never used again (it may have been
// destroyed), and the host never waits.  The device mutex is held for the
// whole enqueue sequence of a call, so calls from several host threads on
// one stream do not interleave their kernels.
// ---------------------------------------------------------------------------

constexpr int kWsStreams = 8;

// The no-allocation entry point's work space: one array per device, sized
// for every workload of this build's limits up to kScratchBytes (64 MiB: the
// 2^20-token, 4-head workload needs about 60 MB).  In host code `scratch`
// names a host-side stand-in, never a device address: host code only ever
// uses the address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = size_t{64} << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

struct DeviceState {
  std::mutex mu;
  void* scratch_ptr = nullptr;  // this device's copy of `scratch` (device address)
  struct Ws {
    hipStream_t st = nullptr;
    void* p = nullptr;
    size_t bytes = 0;
    uint64_t used = 0;
    hipEvent_t done = nullptr;  // recorded on st after each call that used p
  } ws[kWsStreams];
  uint64_t clock = 0;
};
DeviceState g_dev[64];

// the current device's state; the caller holds its mutex while using it
DeviceState* device_state() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  return &g_dev[dev];
}

// A work-space block of at least `bytes` for calls on stream st, and its
// entry (the caller records entry->done on st after enqueueing the call).
// Returns MITA_OK, MITA_ERR_OOM (allocation failed) or MITA_ERR_HIP (a wait
// or free failed; the old block is then kept, not leaked).
int workspace_for(DeviceState& ds, hipStream_t st, size_t bytes, void** out,
                  DeviceState::Ws** entry) {
  ++ds.clock;
  DeviceState::Ws* e = nullptr;
  for (auto& w : ds.ws)
    if (w.p != nullptr && w.st == st) e = &w;
  if (e == nullptr) {  // a free entry, else the least recently used one
    for (auto& w : ds.ws)
      if (w.p == nullptr) {
        e = &w;
        break;
      }
    if (e == nullptr) {
      e = &ds.ws[0];
      for (auto& w : ds.ws)
        if (w.used < e->used) e = &w;
    }
  }
  if (e->done == nullptr) {
    const hipError_t ec = hipEventCreateWithFlags(&e->done, hipEventDisableTiming);
    if (ec != hipSuccess) {
      e->done = nullptr;
      return fail(MITA_ERR_HIP, std::string("hipEventCreateWithFlags: ") + hipGetErrorString(ec));
    }
  }
  if (e->p != nullptr && (e->st != st || e->bytes < bytes)) {
    // Another stream's block (taken over), or this stream's block grown too
    // small.  The calls that used it end with e->done; st waits for that on
    // the GPU and frees the block in its own order.
    hipError_t ef = hipStreamWaitEvent(st, e->done, 0);
    if (ef == hipSuccess) ef = hipFreeAsync(e->p, st);
    if (ef != hipSuccess)
      return fail(MITA_ERR_HIP, std::string("releasing a cached work space: ") +
                                    hipGetErrorString(ef));
    e->p = nullptr;
    e->bytes = 0;
  }
  if (e->p == nullptr) {
    const size_t want = bytes + bytes / 4;  // room for somewhat larger calls
    void* p = nullptr;
    const hipError_t ea = hipMallocAsync(&p, want, st);
    if (ea != hipSuccess || p == nullptr)
      return fail(MITA_ERR_OOM, std::string("work-space allocation failed: ") +
                                    hipGetErrorString(ea != hipSuccess ? ea
                                                                       : hipErrorOutOfMemory));
    e->p = p;
    e->bytes = want;
  }
  e->st = st;
  e->used = ds.clock;
  *out = e->p;
  *entry = e;
  return MITA_OK;
}

// This device's address of the static scratch array, looked up once per
// device (the caller holds the device mutex, with that device current).
int scratch_for(DeviceState& ds, void** out) {
  if (ds.scratch_ptr == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return fail(MITA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                    hipGetErrorString(e != hipSuccess ? e : hipErrorInvalidSymbol));
    }
    ds.scratch_ptr = p;
  }
  *out = ds.scratch_ptr;
  return MITA_OK;
}

// ---------------------------------------------------------------------------
// validation (host only, before any HIP call)
// ---------------------------------------------------------------------------

int validate(const void* Q, const void* K, const void* V, int dtype, int64_t B, int64_t H,
             int64_t N, int64_t d, const mita_grid* grid, int64_t m, int64_t k, float scale,
             const float* out, const int32_t* idx_out, const int32_t* route_out,
             const mita_intermediates* dbg, Shape* s) {
  if (!Q || !K || !V) return fail(MITA_ERR_INVALID_ARG, "Q, K and V must be non-null");
  if (!out || !idx_out || !route_out)
    return fail(MITA_ERR_INVALID_ARG, "out, idx_out and route_out must be non-null");
  if (dtype != MITA_F32 && dtype != MITA_BF16)
    return fail(MITA_ERR_INVALID_ARG, "dtype must be MITA_F32 or MITA_BF16");
  if (B < 1 || H < 1 || N < 1) return fail(MITA_ERR_INVALID_ARG, "B, H and N must be >= 1");
  if (d < 1) return fail(MITA_ERR_INVALID_ARG, "d must be >= 1");
  if (N >= (int64_t(1) << 31)) return fail(MITA_ERR_INVALID_ARG, "N must be < 2^31");
  if (B > (int64_t(1) << 30) || H > (int64_t(1) << 30) || B * H > 65535)
    return fail(MITA_ERR_UNSUPPORTED, "B*H must be <= 65535 in this build");
  if (d != kD) return fail(MITA_ERR_UNSUPPORTED, "only d == 64 is supported in this build");
  if ((B * H) > (int64_t(1) << 40) / (N * d))
    return fail(MITA_ERR_INVALID_ARG, "B*H*N*d must be < 2^40");
  if (m < 1 || m > N) return fail(MITA_ERR_INVALID_ARG, "m must satisfy 1 <= m <= N");
  if (k < 1 || k > N) return fail(MITA_ERR_INVALID_ARG, "k must satisfy 1 <= k <= N");
  if (m > kMaxM) return fail(MITA_ERR_UNSUPPORTED, "m must be <= 64 in this build");
  if (k > kMaxK) return fail(MITA_ERR_UNSUPPORTED, "k must be <= 64 in this build");
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(MITA_ERR_INVALID_ARG, "scale must be finite and > 0");
  mita_grid gr = grid ? *grid : mita_grid{1, static_cast<int32_t>(N), 1, static_cast<int32_t>(m)};
  if (gr.gh < 1 || gr.gw < 1 || gr.mh < 1 || gr.mw < 1)
    return fail(MITA_ERR_INVALID_ARG, "grid sizes must be >= 1");
  if (int64_t(gr.gh) * gr.gw != N) return fail(MITA_ERR_INVALID_ARG, "grid gh*gw must equal N");
  if (int64_t(gr.mh) * gr.mw != m) return fail(MITA_ERR_INVALID_ARG, "grid mh*mw must equal m");
  if (gr.mh > gr.gh || gr.mw > gr.gw)
    return fail(MITA_ERR_INVALID_ARG, "landmark grid must not exceed the token grid");
  const void* ptrs[] = {Q, K, V, out, idx_out, route_out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(MITA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (dbg) {
    const void* dp[] = {dbg->ql, dbg->vl, dbg->perm, dbg->offsets};
    for (const void* p : dp)
      if (p && !aligned16(p))
        return fail(MITA_ERR_INVALID_ARG, "intermediate pointers must be 16-byte aligned");
  }
  s->B = B;
  s->H = H;
  s->BH = B * H;
  s->N = N;
  s->m = static_cast<int>(m);
  s->k = static_cast<int>(k);
  s->gh = gr.gh;
  s->gw = gr.gw;
  s->mh = gr.mh;
  s->mw = gr.mw;
  s->scale = scale;
  s->dtype = dtype;
  return MITA_OK;
}

// largest pooling window of the grid (same bin rule as the kernels)
int64_t max_window(const Shape& s) {
  int64_t best = 0;
  for (int i = 0; i < s.m; ++i) {
    const int64_t a = i / s.mw, c = i % s.mw;
    const int64_t r0 = (a * s.gh) / s.mh, r1 = ((a + 1) * s.gh + s.mh - 1) / s.mh;
    const int64_t c0 = (c * s.gw) / s.mw, c1 = ((c + 1) * s.gw + s.mw - 1) / s.mw;
    const int64_t w = (r1 - r0) * (c1 - c0);
    if (w > best) best = w;
  }
  return best;
}

void derive(Shape& s, int cus) {
  s.cus = cus;
  s.mpad = static_cast<int>(round_up(s.m, 32));
  s.kpad = static_cast<int>(round_up(s.k, 32));
  s.scan_waves = s.m <= 16 ? 1 : (s.m <= 32 ? 2 : 4);
  s.mrows = s.scan_waves * 16;
  // landmark scan.  bf16: three blocks per CU (the kernel's register and LDS
  // budget), each taking every splits-th 64-key tile of its head, at least 8
  // tiles per block.  fp32: one block per CU, contiguous chunks of at least
  // 512 keys.
  const int64_t ktiles = cdiv(s.N, kTileKeys);
  if (s.dtype == MITA_BF16) {
    int64_t splits = cdiv(3 * static_cast<int64_t>(cus), s.BH);
    if (splits > ktiles / 8) splits = ktiles / 8;
    if (splits < 1) splits = 1;
    s.scan_splits = static_cast<int>(splits);
    s.scan_chunk = 0;
  } else {
    int64_t chunk = round_up(cdiv(s.N * s.BH, static_cast<int64_t>(cus)), kTileKeys);
    if (chunk < 512) chunk = 512;
    if (chunk > round_up(s.N, kTileKeys)) chunk = round_up(s.N, kTileKeys);
    s.scan_chunk = static_cast<int>(chunk);
    s.scan_splits = static_cast<int>(cdiv(s.N, chunk));
  }
  // merge of the scan partials in two levels when there are many splits
  s.merge_parts = s.scan_splits > 32 ? 8 : 1;
  s.pool_splits = static_cast<int>(cdiv(max_window(s), kPoolChunk));
  s.pool_direct = max_window(s) <= kPoolDirectMax;
  // top-k pre-threshold from group maxima (a group = gs consecutive keys;
  // the threshold is the k-th largest maximum).  Large N: a sample of the
  // 64-key tiles, a quarter of them (at most 1024 per head) when that gives
  // at least 256 samples, else half of them when that does (32K-64K keys: a
  // pass over every key cost more than the extra candidates a half sample
  // lets through).  Below that, every key: singly up to kThetaMaxGroups keys
  // (exact k-th largest score), else in 16-key groups.  Off when there are
  // fewer than k keys.
  s.theta_groups = 0;
  s.theta_gs = 64;
  s.theta_sampled = false;
  if (s.N >= s.k) {
    if (ktiles / 2 >= 256) {
      int64_t groups = ktiles / 4 >= 256 ? ktiles / 4 : ktiles / 2;
      if (groups > 1024) groups = 1024;
      groups = groups / kThetaTilesPerBlock * kThetaTilesPerBlock;
      s.theta_sampled = true;
      s.theta_groups = static_cast<int>(groups);
    } else if (s.N <= kThetaMaxGroups) {
      s.theta_gs = 1;
      s.theta_groups = static_cast<int>(s.N);
    } else if (cdiv(s.N, 16) <= kThetaMaxGroups) {
      s.theta_gs = 16;
      s.theta_groups = static_cast<int>(cdiv(s.N, 16));
    } else {
      s.theta_gs = 64;
      s.theta_groups = static_cast<int>(ktiles);
    }
  }
  s.NA = s.N * s.s;
  // routing and bucketing segments: 1024 queries, or 256 when 1024-query
  // segments would give fewer than four routing blocks per CU (a routing
  // block is latency-bound: at 2^16 tokens x 4 heads, one 1024-query block
  // per CU took 15 us)
  s.rseg = (s.s == 1 && cdiv(s.NA, kRouteSeg) * s.BH < 4 * static_cast<int64_t>(cus))
               ? kRouteSegSmall
               : kRouteSeg;
  s.nseg = static_cast<int>(cdiv(s.NA, s.rseg));
  // expert attention: work items of up to 16 tiles, keeping >= 2 items per CU
  // (fewer, larger items stage each expert less often: -4% to -7% per step
  // at long1d_16k and seg_32x32 against >= 4 items per CU; 8 was slower)
  const int64_t tiles = cdiv(s.NA, kAttendTile);
  int64_t tpb = (tiles * s.BH) / (2 * static_cast<int64_t>(cus));
  tpb = tpb < 1 ? 1 : (tpb > kAttendMaxTpb ? kAttendMaxTpb : tpb);
  s.attend_tpb = static_cast<int>(tpb);
  // items: sum over experts of ceil(t_e / tpb) with t_e = ceil(c_e / 64);
  // the t_e add up to at most tiles + m - 1, and each ceil adds at most
  // (tpb - 1) / tpb, so tiles / tpb + m bounds them
  s.attend_items = static_cast<int>(cdiv(tiles, tpb) + s.m);
  // short items (bf16, s = 1, under 256 queries per expert on average):
  // 2-wave blocks of ipb consecutive work items, ipb chosen so that every
  // block of the launch is resident at once (about three per CU); with at
  // most 64 items per head they are assigned to the blocks by size instead
  s.attend_short = s.dtype == MITA_BF16 && s.s == 1 && s.N < kAttendShortItems * static_cast<int64_t>(s.m);
  {
    const int64_t per_head = std::max<int64_t>(1, 3 * static_cast<int64_t>(cus) / s.BH);
    s.attend_ipb = static_cast<int>(std::min<int64_t>(
        kAttendIpbMax, std::max<int64_t>(1, cdiv(s.attend_items, per_head))));
    s.attend_nbx = static_cast<int>(cdiv(s.attend_items, s.attend_ipb));
  }
  s.attend_balanced = s.attend_short && s.attend_items <= 64;
  s.small = small_path_fits(s);
  s.medium = !s.small && medium_path_fits(s);
  if (s.medium) {  // exact selection inside the one launch: no pre-threshold
    s.theta_groups = 0;
    s.theta_sampled = false;
  }
}

}  // namespace

size_t plan_workspace(const Shape& s, Workspace* ws, char* base) {
  size_t off = 0;
  if (s.small) {  // the one-launch path keeps everything in LDS
    *ws = Workspace{};
    return 0;
  }
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off += (bytes + 255) / 256 * 256;
    return p;
  };
  const size_t BH = static_cast<size_t>(s.BH), es = s.dtype == MITA_BF16 ? 2 : 4;
  ws->pool_part = reinterpret_cast<double*>(take(BH * s.m * s.pool_splits * kD * sizeof(double)));
  ws->ql = take(BH * s.m * kD * es);
  if (s.theta_groups > 0) {
    ws->gmax = reinterpret_cast<uint32_t*>(take(BH * s.m * s.theta_groups * sizeof(uint32_t)));
    ws->theta = reinterpret_cast<float*>(take(BH * s.mrows * sizeof(float)));
  } else {
    ws->gmax = nullptr;
    ws->theta = nullptr;
  }
  if (s.medium) {  // no split partials
    ws->vl = reinterpret_cast<float*>(take(BH * s.m * kD * sizeof(float)));
    ws->offsets = reinterpret_cast<int32_t*>(take(BH * (s.m + 1) * 4));
    ws->item_start = reinterpret_cast<int32_t*>(take(BH * (s.m + 1) * 4));
    ws->perm = reinterpret_cast<int32_t*>(take(BH * s.NA * 4));
    if (s.attend_balanced)
      ws->item_blocks =
          reinterpret_cast<int32_t*>(take(BH * s.attend_nbx * s.attend_ipb * 4));
    return off;
  }
  const size_t parts = BH * s.scan_splits * s.mrows;
  ws->part_keys = reinterpret_cast<uint64_t*>(take(parts * kTopCap * sizeof(uint64_t)));
  ws->part_cnt = reinterpret_cast<int32_t*>(take(parts * sizeof(int32_t)));
  ws->part_stats = reinterpret_cast<float*>(take(parts * 2 * sizeof(float)));
  ws->part_acc = reinterpret_cast<float*>(take(parts * kD * sizeof(float)));
  if (s.merge_parts > 1) {
    const size_t parts2 = BH * s.merge_parts * s.mrows;
    ws->part2_keys = reinterpret_cast<uint64_t*>(take(parts2 * kTopCap * sizeof(uint64_t)));
    ws->part2_cnt = reinterpret_cast<int32_t*>(take(parts2 * sizeof(int32_t)));
    ws->part2_stats = reinterpret_cast<float*>(take(parts2 * 2 * sizeof(float)));
    ws->part2_acc = reinterpret_cast<float*>(take(parts2 * kD * sizeof(float)));
  }
  ws->vl = reinterpret_cast<float*>(take(BH * s.m * kD * sizeof(float)));
  ws->counts = reinterpret_cast<int32_t*>(take(BH * s.nseg * s.m * 4));
  ws->colpre = reinterpret_cast<int32_t*>(take(BH * s.nseg * s.m * 4));
  ws->totals = reinterpret_cast<int32_t*>(take(BH * s.m * 4));
  ws->offsets = reinterpret_cast<int32_t*>(take(BH * (s.m + 1) * 4));
  ws->item_start = reinterpret_cast<int32_t*>(take(BH * (s.m + 1) * 4));
  ws->item_order = reinterpret_cast<int32_t*>(take(BH * (2 * s.m + 1) * 4));
  if (s.attend_balanced)
    ws->item_blocks = reinterpret_cast<int32_t*>(take(BH * s.attend_nbx * s.attend_ipb * 4));
  ws->perm = reinterpret_cast<int32_t*>(take(BH * s.NA * 4));
  if (s.s > 1) {
    ws->pacc = reinterpret_cast<float*>(take(BH * s.NA * kD * sizeof(float)));
    ws->pstat = reinterpret_cast<float*>(take(BH * s.NA * 2 * sizeof(float)));
  }
  return off;
}

}  // namespace mita

using namespace mita;

extern "C" {

int mita_version(void) { return MITA_VERSION; }

const char* mita_status_string(int status) {
  switch (status) {
    case MITA_OK: return "success";
    case MITA_ERR_INVALID_ARG: return "invalid argument";
    case MITA_ERR_UNSUPPORTED: return "unsupported by this build";
    case MITA_ERR_OOM: return "work-space allocation failed";
    case MITA_ERR_HIP: return "HIP runtime or launch error";
    case MITA_ERR_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

const char* mita_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

namespace {

// The forward pass: validation, work space, then every launch on `stream`.
// use_scratch: take the device's static scratch array instead of a cached
// stream-ordered block (no allocation of any kind).
int forward_impl(const void* Q, const void* K, const void* V, int dtype, int64_t B, int64_t H,
                 int64_t N, int64_t d, const mita_grid* grid, int64_t m, int64_t k, int64_t sx,
                 float scale, float* out, int32_t* idx_out, int32_t* route_out, void* stream,
                 const mita_intermediates* dbg, bool use_scratch) {
  try {
    g_last_error.clear();
    Shape s;
    int rc = validate(Q, K, V, dtype, B, H, N, d, grid, m, k, scale, out, idx_out, route_out, dbg,
                      &s);
    if (rc != MITA_OK) return rc;
    if (sx < 1 || sx > m) return fail(MITA_ERR_INVALID_ARG, "s must satisfy 1 <= s <= m");
    if (sx > kMaxS) return fail(MITA_ERR_UNSUPPORTED, "s must be <= 8 in this build");
    if (sx > 1 && dtype != MITA_BF16)
      return fail(MITA_ERR_UNSUPPORTED, "s > 1 needs bfloat16 inputs in this build");
    if (sx > 1 && N * sx >= (int64_t(1) << 31))
      return fail(MITA_ERR_UNSUPPORTED, "N * s must be < 2^31");
    s.s = static_cast<int>(sx);
    const char* inject = std::getenv("MITA_FAULT_INJECT");
    if (inject && std::strcmp(inject, "alloc") == 0)
      return fail(MITA_ERR_OOM, "work-space allocation failed (injected by MITA_FAULT_INJECT)");

    hipStream_t st = static_cast<hipStream_t>(stream);
    derive(s, device_cus());
    Workspace ws;
    const size_t bytes = plan_workspace(s, &ws, nullptr);
    if (use_scratch && bytes > kScratchBytes)
      return fail(MITA_ERR_UNSUPPORTED,
                  "mita_forward_noalloc: this call needs " + std::to_string(bytes) +
                      " bytes of work space, more than the static scratch array's " +
                      std::to_string(kScratchBytes) + " bytes (use mita_forward)");
    DeviceState* ds = device_state();
    if (ds == nullptr) return fail(MITA_ERR_HIP, "no current HIP device");
    std::lock_guard<std::mutex> lk(ds->mu);  // the whole enqueue sequence
    void* ql_copy = dbg ? dbg->ql : nullptr;
    float* vl_copy = dbg ? dbg->vl : nullptr;
    int32_t* perm_copy = dbg ? dbg->perm : nullptr;
    int32_t* off_copy = dbg ? dbg->offsets : nullptr;
    const bool inject_launch = inject && std::strcmp(inject, "launch") == 0;
    void* base = nullptr;
    DeviceState::Ws* entry = nullptr;
    if (use_scratch) {
      // looked up on the entry point's first call on this device, whichever
      // path the call takes
      rc = scratch_for(*ds, &base);
      if (rc != MITA_OK) return rc;
    }
    if (s.small) {
      // one launch, no work space (nothing to allocate, no event to record)
      hipError_t e = inject_launch ? hipErrorLaunchFailure : hipSuccess;
      if (e == hipSuccess) {
        StageTimer t(kStageSmall, st, !use_scratch);
        e = launch_small(s, Q, K, V, out, idx_out, route_out, ql_copy, vl_copy, perm_copy,
                         off_copy, st);
      }
      if (!use_scratch && g_prof.enabled && e == hipSuccess) g_prof.calls += 1;
      if (e != hipSuccess)
        return fail(MITA_ERR_HIP, std::string("launch of stage single_launch failed: ") +
                                      hipGetErrorString(e));
      return MITA_OK;
    }
    if (!use_scratch) {
      rc = workspace_for(*ds, st, bytes, &base, &entry);
      if (rc != MITA_OK) {
        (void)hipGetLastError();
        return rc;
      }
    }
    plan_workspace(s, &ws, static_cast<char*>(base));
    hipError_t e = hipSuccess;

    const char* where = "pool";
    if (inject_launch) e = hipErrorLaunchFailure;
    if (e == hipSuccess) {
      StageTimer t(kStagePool, st, !use_scratch);
      e = launch_pool(s, Q, ws, ql_copy, 0, s.BH, st);
    }
    // All on the caller's stream, in this order.  Mid-length bf16 heads:
    // pool; the landmark scan and exact selection, routing and bucketing in
    // one launch; the expert attention.  Otherwise: pool; the top-k
    // pre-threshold's group maxima; routing (the pre-threshold's selection as
    // its leading blocks); the landmark scan (step 4's prefix over the
    // routing counts as its trailing blocks); the merge (step 4's scatter as
    // leading blocks of its first pass); the expert attention.  Bucketing
    // rides in launches that follow routing anyway, so the call needs no
    // second stream and no events.
    if (s.medium) {
      if (e == hipSuccess) {
        where = "landmark_scan";
        StageTimer t(kStageScan, st, !use_scratch);
        e = launch_medium(s, Q, K, V, ws, idx_out, route_out, vl_copy, off_copy, perm_copy, st);
      }
    } else {
      if (e == hipSuccess && s.theta_groups > 0) {
        where = "landmark_threshold";
        StageTimer t(kStageThreshold, st, !use_scratch);
        e = launch_threshold(s, K, ws, st);
      }
      if (e == hipSuccess) {
        where = "route";
        StageTimer t(kStageRoute, st, !use_scratch);
        e = s.s > 1 ? launch_route_s(s, Q, ws, route_out, st)
                    : launch_route(s, Q, ws, route_out, st);
      }
      if (e == hipSuccess) {
        where = "landmark_scan";
        StageTimer t(kStageScan, st, !use_scratch);
        e = launch_scan(s, K, V, ws, route_out, st);
      }
      if (e == hipSuccess) {
        where = "landmark_merge";
        StageTimer t(kStageMerge, st, !use_scratch);
        e = launch_merge(s, ws, idx_out, vl_copy, route_out, off_copy, perm_copy, st);
      }
    }
    if (e == hipSuccess) {
      where = "expert_attend";
      StageTimer t(kStageAttend, st, !use_scratch);
      e = s.s > 1 ? launch_attend_multi(s, Q, K, V, idx_out, ws, out, st)
                  : launch_attend(s, Q, K, V, idx_out, ws, out, st);
    }
    if (!use_scratch && g_prof.enabled && e == hipSuccess) g_prof.calls += 1;
    if (entry != nullptr) {
      // the block is in use until here on st (see workspace_for)
      const hipError_t er = hipEventRecord(entry->done, st);
      if (e == hipSuccess && er != hipSuccess) {
        where = "work-space event";
        e = er;
      }
    }
    if (e != hipSuccess)
      return fail(MITA_ERR_HIP, std::string("launch of stage ") + where +
                                    " failed: " + hipGetErrorString(e));
    return MITA_OK;
  } catch (...) {
    return fail(MITA_ERR_INTERNAL, "unexpected exception inside mita_forward");
  }
}

// The backward pass: validation, work space, then its steps on `stream`.
int backward_impl(const void* Q, const void* K, const void* V, int dtype, int64_t B, int64_t H,
                  int64_t N, int64_t d, const mita_grid* grid, int64_t m, int64_t k, float scale,
                  const int32_t* idx, const int32_t* routes, const float* dout, float* dQ,
                  float* dK, float* dV, void* stream) {
  try {
    g_last_error.clear();
    if (!idx || !routes || !dout || !dQ || !dK || !dV)
      return fail(MITA_ERR_INVALID_ARG, "idx, routes, dout, dQ, dK and dV must be non-null");
    Shape s;
    int rc = validate(Q, K, V, dtype, B, H, N, d, grid, m, k, scale, dQ, idx, routes, nullptr, &s);
    if (rc != MITA_OK) return rc;
    for (const void* p : {static_cast<const void*>(dout), static_cast<const void*>(dK),
                          static_cast<const void*>(dV)})
      if (!aligned16(p)) return fail(MITA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    if (dQ == dK || dQ == dV || dK == dV)
      return fail(MITA_ERR_INVALID_ARG, "dQ, dK and dV must be distinct buffers");
    const char* inject = std::getenv("MITA_FAULT_INJECT");
    if (inject && std::strcmp(inject, "alloc") == 0)
      return fail(MITA_ERR_OOM, "work-space allocation failed (injected by MITA_FAULT_INJECT)");
    hipStream_t st = static_cast<hipStream_t>(stream);
    derive(s, device_cus());  // the pooling geometry (pool_splits, pool_direct)
    const BwPlan bp = plan_backward(s, device_cus());
    BwWorkspace ws;
    const size_t bytes = plan_bw_workspace(s, bp, &ws, nullptr);
    DeviceState* ds = device_state();
    if (ds == nullptr) return fail(MITA_ERR_HIP, "no current HIP device");
    std::lock_guard<std::mutex> lk(ds->mu);
    void* base = nullptr;
    DeviceState::Ws* entry = nullptr;
    rc = workspace_for(*ds, st, bytes, &base, &entry);
    if (rc != MITA_OK) {
      (void)hipGetLastError();
      return rc;
    }
    plan_bw_workspace(s, bp, &ws, static_cast<char*>(base));
    hipError_t e = (inject && std::strcmp(inject, "launch") == 0) ? hipErrorLaunchFailure
                                                                  : hipSuccess;
    int where = 0;
    for (int i = 0; i < kBwStepCount && e == hipSuccess; ++i) {
      where = i;
      StageTimer t(kStageBw0 + i, st, true);
      e = launch_backward(s, bp, ws, Q, K, V, idx, routes, dout, dQ, dK, dV, st, i, i);
    }
    if (g_prof.enabled && e == hipSuccess) g_prof.calls += 1;
    const hipError_t er = hipEventRecord(entry->done, st);  // the block is in use until here
    if (e != hipSuccess)
      return fail(MITA_ERR_HIP, std::string("launch of backward stage ") +
                                    kStageNames[kStageBw0 + where] + " failed: " +
                                    hipGetErrorString(e));
    if (er != hipSuccess)
      return fail(MITA_ERR_HIP, std::string("work-space event: ") + hipGetErrorString(er));
    return MITA_OK;
  } catch (...) {
    return fail(MITA_ERR_INTERNAL, "unexpected exception inside mita_backward");
  }
}

}  // namespace

extern "C" {

int mita_backward(const void* Q, const void* K, const void* V, int dtype, int64_t B, int64_t H,
                  int64_t N, int64_t d, const mita_grid* grid, int64_t m, int64_t k,
                  float scale, const int32_t* idx, const int32_t* routes, const float* dout,
                  float* dQ, float* dK, float* dV, void* stream) {
  return backward_impl(Q, K, V, dtype, B, H, N, d, grid, m, k, scale, idx, routes, dout, dQ, dK,
                       dV, stream);
}

int mita_forward_ex(const void* Q, const void* K, const void* V, int dtype, int64_t B, int64_t H,
                    int64_t N, int64_t d, const mita_grid* grid, int64_t m, int64_t k,
                    float scale, float* out, int32_t* idx_out, int32_t* route_out, void* stream,
                    const mita_intermediates* dbg) {
  return forward_impl(Q, K, V, dtype, B, H, N, d, grid, m, k, 1, scale, out, idx_out, route_out,
                      stream, dbg, false);
}

int mita_forward_s(const void* Q, const void* K, const void* V, int dtype, int64_t B, int64_t H,
                   int64_t N, int64_t d, const mita_grid* grid, int64_t m, int64_t k, int64_t s,
                   float scale, float* out, int32_t* idx_out, int32_t* routes_out,
                   void* stream) {
  return forward_impl(Q, K, V, dtype, B, H, N, d, grid, m, k, s, scale, out, idx_out, routes_out,
                      stream, nullptr, false);
}

int mita_forward_noalloc(const void* Q, const void* K, const void* V, int dtype, int64_t B,
                         int64_t H, int64_t N, int64_t d, const mita_grid* grid, int64_t m,
                         int64_t k, float scale, float* out, int32_t* idx_out,
                         int32_t* route_out, void* stream) {
  return forward_impl(Q, K, V, dtype, B, H, N, d, grid, m, k, 1, scale, out, idx_out, route_out,
                      stream, nullptr, true);
}

int mita_forward(const void* Q, const void* K, const void* V, int dtype, int64_t B, int64_t H,
                 int64_t N, int64_t d, const mita_grid* grid, int64_t m, int64_t k, float scale,
                 float* out, int32_t* idx_out, int32_t* route_out, void* stream) {
  return mita_forward_ex(Q, K, V, dtype, B, H, N, d, grid, m, k, scale, out, idx_out, route_out,
                         stream, nullptr);
}

int mita_dense_attention(const void* Q, const void* K, const void* V, int dtype, int64_t B,
                         int64_t H, int64_t N, int64_t d, float scale, float* out, void* stream) {
  try {
    if (!Q || !K || !V || !out) return fail(MITA_ERR_INVALID_ARG, "Q, K, V and out must be non-null");
    if (dtype != MITA_F32 && dtype != MITA_BF16)
      return fail(MITA_ERR_INVALID_ARG, "dtype must be MITA_F32 or MITA_BF16");
    if (B < 1 || H < 1 || N < 1) return fail(MITA_ERR_INVALID_ARG, "B, H and N must be >= 1");
    if (d < 1) return fail(MITA_ERR_INVALID_ARG, "d must be >= 1");
    if (N >= (int64_t(1) << 31)) return fail(MITA_ERR_INVALID_ARG, "N must be < 2^31");
    if (B * H > 65535) return fail(MITA_ERR_UNSUPPORTED, "B*H must be <= 65535 in this build");
    if (dtype != MITA_BF16)
      return fail(MITA_ERR_UNSUPPORTED, "the dense baseline supports bf16 inputs only");
    if (d != kD && d != 2 * kD)
      return fail(MITA_ERR_UNSUPPORTED, "the dense baseline supports d == 64 and d == 128");
    if (B * H * N > (int64_t(1) << 40) / d)
      return fail(MITA_ERR_INVALID_ARG, "B*H*N*d must be < 2^40");
    if (!(scale > 0.0f) || !std::isfinite(scale))
      return fail(MITA_ERR_INVALID_ARG, "scale must be finite and > 0");
    for (const void* p : {Q, K, V, static_cast<const void*>(out)})
      if (!aligned16(p)) return fail(MITA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
    const hipError_t e = launch_dense(dtype, Q, K, V, B * H, N, d, scale, out,
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
      return fail(MITA_ERR_HIP, std::string("launch of the dense kernel failed: ") +
                                    hipGetErrorString(e));
    return MITA_OK;
  } catch (...) {
    return fail(MITA_ERR_INTERNAL, "unexpected exception inside mita_dense_attention");
  }
}

int mita_release_workspace(void* stream) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  DeviceState* ds = device_state();
  if (ds == nullptr) return fail(MITA_ERR_HIP, "no current HIP device");
  std::lock_guard<std::mutex> lk(ds->mu);
  for (auto& w : ds->ws) {
    if (w.p == nullptr || w.st != st) continue;
    const hipError_t e = hipFreeAsync(w.p, st);  // after the calls already on st
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(MITA_ERR_HIP, std::string("hipFreeAsync: ") + hipGetErrorString(e));
    }
    w.p = nullptr;
    w.bytes = 0;
    w.st = nullptr;
  }
  return MITA_OK;
}

int mita_profile_enable(int enabled) {
  try {
    if (enabled) {
      g_prof.drain();
      for (double& v : g_prof.ms) v = 0.0;
      g_prof.calls = 0;
      g_prof.enabled = true;
    } else {
      g_prof.enabled = false;
    }
    return MITA_OK;
  } catch (...) {
    return fail(MITA_ERR_INTERNAL, "profiler failure");
  }
}

int mita_profile_stage_count(void) { return kStageCount; }

const char* mita_profile_stage_name(int stage) {
  return (stage >= 0 && stage < kStageCount) ? kStageNames[stage] : "";
}

int mita_profile_read(double* ms_per_stage, int64_t* calls, int n_stages) {
  try {
    if (!ms_per_stage || !calls || n_stages < 1)
      return fail(MITA_ERR_INVALID_ARG, "profile_read needs output arrays");
    g_prof.drain();
    for (int i = 0; i < n_stages && i < kStageCount; ++i) ms_per_stage[i] = g_prof.ms[i];
    *calls = g_prof.calls;
    return MITA_OK;
  } catch (...) {
    return fail(MITA_ERR_INTERNAL, "profiler failure");
  }
}

}  // extern "C"
