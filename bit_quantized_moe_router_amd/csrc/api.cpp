// C ABI of the MoE layer: argument validation, workspace carving, the chunk
// loop and the GEMV/GEMM dispatch.  Host code only; it enqueues kernels on the
// caller's stream and never allocates device memory, synchronises or reads
// device data (the optional kernel-timing mode aside, which only records
// events and synchronises inside moe_profile_read).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "launch.h"

using namespace moe;

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

constexpr int kDefaultTileRows = 128;
constexpr int kDefaultGemvMaxRows = 8;  // measured: the GEMV path is faster at every T <= 8 (the decode maximum)
// With batch_invariant = 1 both paths give the same bits, so the threshold only
// picks the faster: measured, the GEMV path with the grouped GEMM's arithmetic
// is faster up to 4 rows (26 us at T = 1 against 47 us) and slower from 5.
constexpr int kDefaultGemvMaxRowsBi = 4;
constexpr int kMaxRowsDecode = 8;

moe_status validate_desc(const moe_layer_desc* d) {
  if (!d) return fail(MOE_ERR_INVALID_ARGUMENT, "desc is null");
  if (d->group_size != 64) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "group_size must be 64 (got %d)", d->group_size);
  if (d->hidden <= 0 || d->hidden % 64 || d->hidden > 8192)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "hidden must be a positive multiple of 64 <= 8192 (got %d)", d->hidden);
  if (d->inter <= 0 || d->inter % 64 || d->inter > 4096)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "inter must be a positive multiple of 64 <= 4096 (got %d)", d->inter);
  if (d->shared_inter < 0 || d->shared_inter % 64 || d->shared_inter > 4096)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "shared_inter must be 0 or a multiple of 64 <= 4096 (got %d)", d->shared_inter);
  if (d->n_experts < 1 || d->n_experts > 512)
    return fail(MOE_ERR_UNSUPPORTED_SHAPE, "n_experts must be in 1..512 (got %d)", d->n_experts);
  if (d->top_k < 1 || d->top_k > 16) return fail(MOE_ERR_INVALID_ARGUMENT, "top_k must be in 1..16 (got %d)", d->top_k);
  if (d->top_k > d->n_experts)
    return fail(MOE_ERR_INVALID_ARGUMENT, "top_k (%d) exceeds n_experts (%d)", d->top_k, d->n_experts);
  if (d->gemv_max_rows < -1 || d->gemv_max_rows > kMaxRowsDecode)
    return fail(MOE_ERR_INVALID_ARGUMENT, "gemv_max_rows must be in -1..8 (got %d)", d->gemv_max_rows);
  if (d->max_chunk < 1 || d->max_chunk > 8192)
    return fail(MOE_ERR_INVALID_ARGUMENT, "max_chunk must be in 1..8192 (got %d)", d->max_chunk);
  const int bm = d->tile_rows;
  if (!(bm == 0 || bm == 16 || bm == 32 || bm == 64 || bm == 128))
    return fail(MOE_ERR_INVALID_ARGUMENT, "tile_rows must be 0, 16, 32, 64 or 128 (got %d)", bm);
  if (d->host_sync_routing != 0 && d->host_sync_routing != 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "host_sync_routing must be 0 or 1 (got %d)", d->host_sync_routing);
  if (d->dequant_pass != 0 && d->dequant_pass != 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "dequant_pass must be 0 or 1 (got %d)", d->dequant_pass);
  if (d->batch_invariant != 0 && d->batch_invariant != 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "batch_invariant must be 0 or 1 (got %d)", d->batch_invariant);
  return MOE_OK;
}

int tile_rows(const moe_layer_desc* d) { return d->tile_rows ? d->tile_rows : kDefaultTileRows; }
int imax(const moe_layer_desc* d) { return d->inter > d->shared_inter ? d->inter : d->shared_inter; }

int64_t max_tiles_for(const moe_layer_desc* d, int64_t T) {
  if (T <= 0) return 1;
  const int64_t BM = tile_rows(d), k = d->top_k, E = d->n_experts;
  const int64_t tk = T * k;
  return (tk + BM - 1) / BM + (E < tk ? E : tk) + (d->shared_inter > 0 ? (T + BM - 1) / BM : 0);
}

// Schedule entries: the tiles, plus one more for each tile of more than
// BM/2 rows that the schedule may cut in two.
int64_t max_sched_for(const moe_layer_desc* d, int64_t T) {
  const int64_t mt = max_tiles_for(d, T), BM = tile_rows(d);
  if (T <= 0 || BM < 64) return mt;
  return mt + (T * d->top_k + (d->shared_inter > 0 ? T : 0)) / (BM / 2 + 1);
}

struct Blob {
  int64_t expert_bytes, gateup_bytes, shared_base, shared_gateup_bytes, trailer, total;
};

Blob blob_geom(const moe_layer_desc* d) {
  const int64_t H = d->hidden, I = d->inter, Is = d->shared_inter, E = d->n_experts;
  Blob b;
  b.gateup_bytes = (I / 32) * (H / 64) * 2 * kBlockBytes;
  b.expert_bytes = b.gateup_bytes + (H / 32) * (I / 64) * kBlockBytes;
  b.shared_base = E * b.expert_bytes;
  b.shared_gateup_bytes = (Is / 32) * (H / 64) * 2 * kBlockBytes;
  b.trailer = b.shared_base + (Is ? b.shared_gateup_bytes + (H / 32) * (Is / 64) * kBlockBytes : 0);
  b.total = b.trailer + kTrailerBytes;
  return b;
}

struct Ws {
  size_t logits, wnorm, xsum, x16, ids, tw, counts, offsets, sorted, inv, tiles, sched, n_tiles, active, n_active, segs,
      hbuf, obuf, dpart, wdq;
  size_t span;     // bytes of one chunk's area (logits .. obuf)
  int areas;       // 1, or 2: a second chunk area follows the first
  size_t total;
};

size_t al(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace of one chunk: routing outputs, gathered activations and the
// GEMMs' intermediates.  With areas = 2 it is there twice, so two chunks can
// be in flight at once (one per stream).  Offsets are relative to an area's
// base, except wdq's, which is relative to the workspace.
Ws ws_layout(const moe_layer_desc* d, int64_t Tc, int areas = 1) {
  const int64_t E = d->n_experts, k = d->top_k, H = d->hidden, Im = imax(d);
  const int64_t rows = Tc * k + Tc;
  Ws w;
  size_t o = 0;
  w.logits = o; o += al(4 * Tc * E * 4);  // 4 partial slices of the screened logits
  w.wnorm = o; o += al(4 * E * 8);
  w.xsum = o; o += al(Tc * (H / 64) * 4);
  w.x16 = o; o += al(Tc * H * 2);
  w.ids = o; o += al(Tc * k * 4);
  w.tw = o; o += al(Tc * k * 4);
  w.counts = o; o += al(E * 4);
  w.offsets = o; o += al((E + 1) * 4);
  w.sorted = o; o += al(Tc * k * 4);
  w.inv = o; o += al(Tc * k * 4);
  w.tiles = o; o += al(max_tiles_for(d, Tc) * 3 * 4);
  w.sched = o; o += al((1 + max_sched_for(d, Tc)) * 16);  // count, then an int4 descriptor per entry
  w.n_tiles = o; o += al(4);
  w.active = o; o += al(E * 4);
  w.n_active = o; o += al(4);
  w.segs = o; o += al(((Tc * k + kSegAssign - 1) / kSegAssign) * E * 4);  // per-segment expert counts
  w.hbuf = o; o += al(rows * Im * 2);
  // obuf (grouped-GEMM path) and dpart (decode GEMV path: partial outputs
  // [T*k + T][Imax/32][H] fp32, T <= 8) are never live together: one region.
  const int64_t Td = Tc < kMaxRowsDecode ? Tc : kMaxRowsDecode;
  const int64_t dpart_bytes = (Td * k + Td) * (Im / 32) * H * 4;
  w.obuf = o;
  w.dpart = o;
  o += al((Tc * k + Tc) * H * 2 > dpart_bytes ? (Tc * k + Tc) * H * 2 : dpart_bytes);
  w.span = o;
  w.areas = areas;
  o *= areas;
  // Separate-dequant measurement only: an fp16 copy of the blob's blocks.
  w.wdq = o;
  if (d->dequant_pass) o += al(blob_geom(d).total / kBlockBytes * kDqBlockBytes);
  w.total = o;
  return w;
}

template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

// ---- device check -------------------------------------------------------
std::mutex g_dev_mu;
int g_dev_ok[64];   // 0 = unknown, 1 = gfx950, -1 = other
int g_dev_cus[64];  // compute units

moe_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_DEVICE_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    g_dev_ok[dev] = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_dev_cus[dev] = p.multiProcessorCount;
  }
  if (g_dev_ok[dev] != 1) return fail(MOE_ERR_DEVICE_UNSUPPORTED, "device %d is not gfx950", dev);
  return MOE_OK;
}

// Long tiles the schedule keeps whole: one round of gate/up workgroups over
// the device (after check_device on the current device).
int max_long_tiles(const moe_layer_desc* d) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  return g_dev_cus[dev] * gemm_wgs_per_cu() / gateup_col_tiles(d->inter, d->shared_inter);
}

// ---- kernel timing (measurement mode) ----------------------------------------
constexpr int kNumKernels = 11;
struct Pending {
  int kid;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
uint32_t g_prof_mask = 0;  // bit i: time kernel id i
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_event_pool;
double g_prof_ms[kNumKernels];
int g_prof_n[kNumKernels];

hipEvent_t get_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  // No system-scope fence on record: the profiling events must not flush the
  // caches between the kernels they time (device-scope ordering suffices
  // for timestamps read back with hipEventSynchronize).
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// Launch `fn(KTime)` (returning hipError_t).  When timing is on, the events
// go to the launcher, which has its first kernel stamp the start and its last
// kernel the end; both are also recorded just before, so a call that
// enqueues nothing reads 0.
template <class F>
moe_status timed(int kid, hipStream_t s, const char* what, F fn) {
  Pending p{kid, nullptr, nullptr};
  const bool on = kid >= 0 && ((g_prof_mask >> kid) & 1u);
  if (on) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    p.a = get_event();
    p.b = get_event();
    if (p.a && p.b) {
      (void)hipEventRecord(p.a, s);
      (void)hipEventRecord(p.b, s);
    }
  }
  KTime kt;
  if (on && p.a && p.b) {
    kt.start = p.a;
    kt.stop = p.b;
  }
  hipError_t e = fn(kt);
  if (on && p.a && p.b) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_pending.push_back(p);
  }
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

#define TRY(x)                     \
  do {                             \
    moe_status _s = (x);           \
    if (_s != MOE_OK) return _s;   \
  } while (0)

LayerArgs layer_args(const moe_layer_desc* d, const void* packed) {
  const Blob b = blob_geom(d);
  LayerArgs L;
  L.blob = static_cast<const uint8_t*>(packed);
  L.H = d->hidden;
  L.E = d->n_experts;
  L.k = d->top_k;
  L.I = d->inter;
  L.Is = d->shared_inter;
  L.expert_bytes = b.expert_bytes;
  L.gateup_bytes = b.gateup_bytes;
  L.shared_base = b.shared_base;
  L.shared_gateup_bytes = b.shared_gateup_bytes;
  L.small_scales = reinterpret_cast<const int32_t*>(L.blob + b.trailer);
  L.wdq = nullptr;
  return L;
}

struct RouteOut {
  int32_t *ids, *counts, *offsets, *sorted, *inv, *tiles, *sched, *n_tiles, *active, *n_active, *segs;
  float *tw, *logits, *xsum;
  double* wsq;
  uint16_t* x16;
};

moe_status run_route(const moe_layer_desc* d, const uint16_t* x, int T, const float* wr,
                     const float* bias, const RouteOut& o, hipStream_t s) {
  const int E = d->n_experts, k = d->top_k, H = d->hidden;
  bool two = false;
  TRY(timed(0, s, "router logits", [&](const KTime& kt) {
    return launch_route_logits(x, T, H, wr, bias, E, k, o.logits, o.wsq, o.ids, o.tw, o.xsum, o.x16, o.segs, s,
                               &two, kt);
  }));
  if (!two) {
    // Few tokens: exact logits are already there; top-k + metadata in one launch.
    return timed(2, s, "top-k + routing metadata", [&](const KTime& kt) {
      return launch_topk_meta(o.logits, T, E, k, o.ids, o.tw, tile_rows(d), d->shared_inter > 0 ? 1 : 0,
                              o.counts, o.offsets, o.sorted, o.tiles, o.n_tiles, o.active, o.n_active, o.inv,
                              o.sched, s, kt);
    });
  }
  TRY(timed(1, s, "top-k", [&](const KTime& kt) {
    return launch_route_select(x, T, H, wr, bias, E, k, o.logits, o.wsq, o.ids, o.tw, o.x16, o.segs, s, kt);
  }));
  TRY(timed(2, s, "routing metadata", [&](const KTime& kt) {
    return launch_meta(o.ids, T, k, E, tile_rows(d), d->shared_inter > 0 ? 1 : 0, max_long_tiles(d), o.counts,
                       o.offsets, o.sorted, o.tiles, o.n_tiles, o.active, o.n_active, o.inv, o.sched, o.segs,
                       s, kt);  // segment counts taken by the exact top-k
  }));
  return MOE_OK;
}

void* area_base(void* ws, const Ws& w, int area) { return static_cast<char*>(ws) + (area ? w.span : 0); }

RouteOut ws_route(void* ws, const Ws& w) {
  RouteOut o;
  o.logits = at<float>(ws, w.logits);
  o.wsq = at<double>(ws, w.wnorm);
  o.xsum = at<float>(ws, w.xsum);
  o.x16 = at<uint16_t>(ws, w.x16);
  o.ids = at<int32_t>(ws, w.ids);
  o.tw = at<float>(ws, w.tw);
  o.counts = at<int32_t>(ws, w.counts);
  o.offsets = at<int32_t>(ws, w.offsets);
  o.sorted = at<int32_t>(ws, w.sorted);
  o.inv = at<int32_t>(ws, w.inv);
  o.tiles = at<int32_t>(ws, w.tiles);
  o.sched = at<int32_t>(ws, w.sched);
  o.n_tiles = at<int32_t>(ws, w.n_tiles);
  o.active = at<int32_t>(ws, w.active);
  o.n_active = at<int32_t>(ws, w.n_active);
  o.segs = at<int32_t>(ws, w.segs);
  return o;
}

ChunkArgs chunk_args(const moe_layer_desc* d, const uint16_t* x, int Tc, const RouteOut& o, void* ws,
                     const Ws& w, float* y) {
  ChunkArgs C;
  C.x = x;
  C.x16 = o.x16;
  C.T = Tc;
  C.Tk = Tc * d->top_k;
  C.xsum = o.xsum;
  C.ids = o.ids;
  C.tw = o.tw;
  C.counts = o.counts;
  C.offsets = o.offsets;
  C.sorted = o.sorted;
  C.inv = o.inv;
  C.tiles = o.tiles;
  C.sched = o.sched;
  C.n_tiles = o.n_tiles;
  C.active = o.active;
  C.n_active = o.n_active;
  C.hbuf = at<uint16_t>(ws, w.hbuf);
  C.obuf = at<uint16_t>(ws, w.obuf);
  C.y = y;
  C.Imax = imax(d);
  return C;
}

moe_status forward_checks(const moe_layer_desc* d, const void* packed, const float* wr,
                          const uint16_t* x, int32_t T, const float* y, const void* ws,
                          size_t ws_bytes) {
  TRY(validate_desc(d));
  if (T < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "T must be >= 0 (got %d)", T);
  if (T == 0) return MOE_OK;
  if (!packed || !wr || !x || !y || !ws) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer argument");
  const int64_t Tc = T < d->max_chunk ? T : d->max_chunk;
  const size_t need = ws_layout(d, Tc).total;
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < required %zu", ws_bytes, need);
  return MOE_OK;
}

// The GEMMs of one routed chunk, on stream s (chunk_combine follows them).
moe_status chunk_gemms(const moe_layer_desc* d, const LayerArgs& L, const uint16_t* x, int Tc, const RouteOut& o,
                       float* y, void* area, void* ws, const Ws& w, hipStream_t s) {
  const ChunkArgs C = chunk_args(d, x, Tc, o, area, w, y);
  LayerArgs Lc = L;
  if (d->dequant_pass) {
    Lc.wdq = at<uint8_t>(ws, w.wdq);
    TRY(timed(8, s, "separate dequant", [&](const KTime& kt) { return launch_dequant_active(Lc, C, s, kt); }));
  }
  int mt = (int)max_sched_for(d, Tc);
  if (d->host_sync_routing) {
    // Measurement of the host round trip: read the schedule's entry count
    // back, wait for it, and size the GEMM grids from it.
    int32_t hdr[4] = {0, 0, 0, 0};
    hipError_t e = hipMemcpyAsync(hdr, o.sched, sizeof(hdr), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "routing read-back: %s", hipGetErrorString(e));
    if (hdr[0] < 0 || hdr[0] > mt) return fail(MOE_ERR_HIP, "routing read-back: bad entry count %d", hdr[0]);
    mt = hdr[0];
  }
  TRY(timed(3, s, "gate/up GEMM", [&](const KTime& kt) { return launch_gateup_gemm(Lc, C, mt, s, kt); }));
  TRY(timed(4, s, "down GEMM", [&](const KTime& kt) { return launch_down_gemm(Lc, C, mt, s, kt); }));
  return MOE_OK;
}

// The per-token combine of one chunk whose down GEMM is ordered before it on stream s.
moe_status chunk_combine(const moe_layer_desc* d, const LayerArgs& L, const uint16_t* x, int Tc, const RouteOut& o,
                         float* y, void* area, const Ws& w, hipStream_t s) {
  const ChunkArgs C = chunk_args(d, x, Tc, o, area, w, y);
  TRY(timed(7, s, "combine", [&](const KTime& kt) { return launch_combine(L, C, s, kt); }));
  return MOE_OK;
}

// ---- the second stream ----------------------------------------------------------
// Per device, a second stream (non-blocking, default priority) that runs every
// other chunk beside the caller's stream.  Events without timing order the two
// streams; they come from a per-device pool and go back to it once every wait
// on them is enqueued (a wait takes the event's state at the time it is
// enqueued).
std::mutex g_side_mu;
hipStream_t g_side[64];
std::vector<hipEvent_t> g_sync_pool[64];

struct SyncEvents {
  int dev = 0;
  std::vector<hipEvent_t> used;
  ~SyncEvents() {
    std::lock_guard<std::mutex> lk(g_side_mu);
    for (hipEvent_t e : used) g_sync_pool[dev].push_back(e);
  }
  moe_status get(hipEvent_t* out) {
    {
      std::lock_guard<std::mutex> lk(g_side_mu);
      if (!g_sync_pool[dev].empty()) {
        *out = g_sync_pool[dev].back();
        g_sync_pool[dev].pop_back();
        used.push_back(*out);
        return MOE_OK;
      }
    }
    hipError_t e = hipEventCreateWithFlags(out, hipEventDisableTiming);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipEventCreateWithFlags: %s", hipGetErrorString(e));
    used.push_back(*out);
    return MOE_OK;
  }
  // Stream `waiter` waits for what is enqueued on `src` so far.
  moe_status order(hipStream_t src, hipStream_t waiter) {
    hipEvent_t ev = nullptr;
    TRY(get(&ev));
    hipError_t e = hipEventRecord(ev, src);
    if (e == hipSuccess) e = hipStreamWaitEvent(waiter, ev, 0);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "stream ordering: %s", hipGetErrorString(e));
    return MOE_OK;
  }
};

moe_status side_stream(int* dev_out, hipStream_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_DEVICE_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_side_mu);
  if (!g_side[dev]) {
    hipStream_t st = nullptr;
    e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipStreamCreateWithFlags: %s", hipGetErrorString(e));
    g_side[dev] = st;
  }
  *dev_out = dev;
  *out = g_side[dev];
  return MOE_OK;
}

// ---- decode without allocation (moe_forward_decode_static) -------------------
// The workspace of moe_forward_decode_static: a fixed device array that each
// GPU the library runs on holds until the process ends.  Host code never uses
// the array's name as an address (it is the host-side stand-in); the device
// address is taken once per device with hipGetSymbolAddress, with that device
// current, and kept in g_scratch_ptr.  Every call on one GPU shares the array,
// so calls that overlap on one GPU race.  No decode kernel reads a workspace
// byte it has not written in the same call, so nothing needs clearing.
constexpr size_t kStaticScratchBytes = MOE_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

moe_status static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_DEVICE_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// The grouped GEMM path over T tokens, max_chunk tokens at a time.  With one
// chunk area in the workspace every chunk is routed and run on the caller's
// stream, one after the other.  With two (and more than one chunk), chunks
// alternate between the caller's stream (even chunks, area 0) and the second
// stream (odd chunks, area 1), so two chunks are in flight at once: the
// routing of one runs beside the other's GEMMs, and the GEMMs of both share
// the device.  The tokens of different chunks are independent, so the only
// orderings are the call's inputs before the second stream's work, each
// stream's own order for the reuse of its area, and the second stream's work
// joined to the caller's stream before the call returns.
moe_status prefill_loop(const moe_layer_desc* d, const void* packed, const float* wr, const float* bias,
                        const uint16_t* x, int T, float* y, void* ws, size_t ws_bytes, bool may_overlap,
                        hipStream_t s) {
  const LayerArgs L = layer_args(d, packed);
  const int chunk = d->max_chunk, H = d->hidden;
  const int nch = (T + chunk - 1) / chunk;
  const int64_t Tc0 = T < chunk ? T : chunk;
  auto rows = [&](int c) { return T - c * chunk < chunk ? T - c * chunk : chunk; };
  const Ws w2 = ws_layout(d, Tc0, 2);
  const bool two = nch > 1 && may_overlap && !d->host_sync_routing && !d->dequant_pass && ws_bytes >= w2.total;
  if (!two) {
    const Ws w = ws_layout(d, Tc0);
    const RouteOut o = ws_route(ws, w);
    for (int c = 0; c < nch; c++) {
      const int64_t off = (int64_t)c * chunk * H;
      TRY(run_route(d, x + off, rows(c), wr, bias, o, s));
      TRY(chunk_gemms(d, L, x + off, rows(c), o, y + off, ws, ws, w, s));
      TRY(chunk_combine(d, L, x + off, rows(c), o, y + off, ws, w, s));
    }
    return MOE_OK;
  }
  int dev = 0;
  hipStream_t side = nullptr;
  TRY(side_stream(&dev, &side));
  SyncEvents ev;
  ev.dev = dev;
  TRY(ev.order(s, side));  // the inputs and the workspace's previous users come first
  // When the last chunk runs on the second stream, its combine runs on the
  // caller's stream after an event that follows that chunk's down GEMM: the
  // wait then overlaps the other chunk's combine, and it orders all of the
  // second stream's work before the call's end on the caller's stream, so no
  // separate join is needed.
  const bool last_on_side = (nch - 1) & 1;
  auto body = [&]() -> moe_status {
    for (int c = 0; c < nch; c++) {
      hipStream_t st = c & 1 ? side : s;
      void* area = area_base(ws, w2, c & 1);
      const RouteOut o = ws_route(area, w2);
      const int64_t off = (int64_t)c * chunk * H;
      TRY(run_route(d, x + off, rows(c), wr, bias, o, st));
      TRY(chunk_gemms(d, L, x + off, rows(c), o, y + off, area, ws, w2, st));
      hipStream_t cs = st;
      if (c == nch - 1 && last_on_side) {
        TRY(ev.order(side, s));
        cs = s;
      }
      TRY(chunk_combine(d, L, x + off, rows(c), o, y + off, area, w2, cs));
    }
    return MOE_OK;
  };
  const moe_status st = body();
  if (st != MOE_OK) {
    // Best effort, keeping the first error: leave nothing of the call unjoined.
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) == hipSuccess) {
      if (hipEventRecord(e, side) == hipSuccess) (void)hipStreamWaitEvent(s, e, 0);
      (void)hipEventDestroy(e);
    }
    return st;
  }
  return last_on_side ? MOE_OK : ev.order(side, s);
}

// Decode after the argument checks; may_overlap is false for the
// static-scratch entry point, which must not create the routing stream.
moe_status decode_impl(const moe_layer_desc* desc, const void* packed, const float* router_w,
                       const float* logit_bias, const uint16_t* x, int32_t T, float* y, void* ws, size_t ws_bytes,
                       bool may_overlap, void* stream) {
  // T > R* (and always T > 8, the GEMV's largest row count) takes the grouped-GEMM path.
  const int R = desc->gemv_max_rows >= 0 ? desc->gemv_max_rows
                : desc->batch_invariant ? kDefaultGemvMaxRowsBi : kDefaultGemvMaxRows;
  const bool gemv = T <= R && T <= desc->max_chunk && (int64_t)T * desc->hidden <= 32768;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!gemv) return prefill_loop(desc, packed, router_w, logit_bias, x, T, y, ws, ws_bytes, may_overlap, s);
  const LayerArgs L = layer_args(desc, packed);
  const Ws w = ws_layout(desc, T);
  const RouteOut o = ws_route(ws, w);
  // Exact logits; then the top-k, gate/up and split down projection; then the
  // fixed-order sum of the partial outputs.
  bool two = false;
  float* part = at<float>(ws, w.dpart);
  TRY(timed(0, s, "router logits", [&](const KTime& kt) {
    return launch_route_logits(x, T, desc->hidden, router_w, logit_bias, desc->n_experts, desc->top_k, o.logits,
                               o.wsq, o.ids, o.tw, nullptr, nullptr, nullptr, s, &two, kt);
  }));
  const ChunkArgs C = chunk_args(desc, x, T, o, ws, w, y);
  if (desc->batch_invariant) {
    // The grouped-GEMM path's arithmetic: gate/up into fp16 h rows, then down + combine.
    TRY(timed(5, s, "top-k + gate/up GEMV (grouped-GEMM arithmetic)", [&](const KTime& kt) {
      return launch_gemv_gateup_bi(L, C, o.logits, C.hbuf, o.ids, o.tw, s, kt);
    }));
    TRY(timed(6, s, "down GEMV + combine (grouped-GEMM arithmetic)", [&](const KTime& kt) {
      return launch_gemv_down_bi(L, C, C.hbuf, o.ids, o.tw, s, kt);
    }));
    return MOE_OK;
  }
  TRY(timed(5, s, "top-k + gate/up + split down GEMV", [&](const KTime& kt) {
    return launch_gemv_experts(L, C, o.logits, part, s, kt);
  }));
  TRY(timed(6, s, "partial-output sum", [&](const KTime& kt) { return launch_gemv_reduce(L, C, part, s, kt); }));
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_packed_bytes(const moe_layer_desc* desc, size_t* bytes) {
  TRY(validate_desc(desc));
  if (!bytes) return fail(MOE_ERR_INVALID_ARGUMENT, "bytes is null");
  *bytes = (size_t)blob_geom(desc).total;
  return MOE_OK;
}

moe_status moe_workspace_bytes(const moe_layer_desc* desc, int32_t max_tokens, size_t* bytes) {
  TRY(validate_desc(desc));
  if (!bytes) return fail(MOE_ERR_INVALID_ARGUMENT, "bytes is null");
  if (max_tokens < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "max_tokens must be >= 0");
  const int64_t Tc = max_tokens < desc->max_chunk ? max_tokens : desc->max_chunk;
  // Beyond one chunk, room for a second chunk area (two chunks in flight).
  *bytes = ws_layout(desc, Tc > 0 ? Tc : 1, max_tokens > desc->max_chunk ? 2 : 1).total;
  return MOE_OK;
}

moe_status moe_max_tiles(const moe_layer_desc* desc, int32_t T, int32_t* n) {
  TRY(validate_desc(desc));
  if (!n) return fail(MOE_ERR_INVALID_ARGUMENT, "n is null");
  if (T < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "T must be >= 0");
  *n = (int32_t)max_tiles_for(desc, T);
  return MOE_OK;
}

int32_t moe_default_gemv_max_rows(void) { return kDefaultGemvMaxRows; }

moe_status moe_pack_weights(const moe_layer_desc* desc, moe_qmatrix gate, moe_qmatrix up,
                            moe_qmatrix down, moe_qmatrix sh_gate, moe_qmatrix sh_up,
                            moe_qmatrix sh_down, void* packed, size_t packed_bytes, void* stream) {
  TRY(validate_desc(desc));
  const Blob b = blob_geom(desc);
  auto bad = [](const moe_qmatrix& m) { return !m.codes || !m.scales || !m.biases; };
  if (!packed || bad(gate) || bad(up) || bad(down))
    return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (desc->shared_inter > 0 && (bad(sh_gate) || bad(sh_up) || bad(sh_down)))
    return fail(MOE_ERR_INVALID_ARGUMENT, "null shared-expert pointer");
  if (packed_bytes < (size_t)b.total)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "packed buffer %zu bytes < required %lld", packed_bytes,
                (long long)b.total);
  TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = desc->hidden, I = desc->inter, Is = desc->shared_inter, E = desc->n_experts;
  uint8_t* dst = static_cast<uint8_t*>(packed);
  auto pack = [&](const moe_qmatrix& m, int M, int N, int K, int64_t base, int64_t stride_m,
                  int64_t stride_nb, int64_t stride_g) -> moe_status {
    PackArgs P{m.codes, m.scales, m.biases, dst, M, N, K, base, stride_m, stride_nb, stride_g,
               reinterpret_cast<int32_t*>(dst + b.trailer)};
    hipError_t e = launch_pack(P, s);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "pack launch failed: %s", hipGetErrorString(e));
    return MOE_OK;
  };
  {
    hipError_t e = launch_pack_trailer(dst + b.trailer, s);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "pack launch failed: %s", hipGetErrorString(e));
  }
  const int64_t gu_nb = (int64_t)(H / 64) * 2 * kBlockBytes, gu_g = 2 * kBlockBytes;
  TRY(pack(gate, E, I, H, 0, b.expert_bytes, gu_nb, gu_g));
  TRY(pack(up, E, I, H, kBlockBytes, b.expert_bytes, gu_nb, gu_g));
  TRY(pack(down, E, H, I, b.gateup_bytes, b.expert_bytes, (int64_t)(I / 64) * kBlockBytes, kBlockBytes));
  if (Is > 0) {
    TRY(pack(sh_gate, 1, Is, H, b.shared_base, 0, gu_nb, gu_g));
    TRY(pack(sh_up, 1, Is, H, b.shared_base + kBlockBytes, 0, gu_nb, gu_g));
    TRY(pack(sh_down, 1, H, Is, b.shared_base + b.shared_gateup_bytes, 0,
             (int64_t)(Is / 64) * kBlockBytes, kBlockBytes));
  }
  return MOE_OK;
}

moe_status moe_route(const moe_layer_desc* desc, const uint16_t* x, int32_t T, const float* router_w,
                     const float* logit_bias, const moe_routing* out, void* ws, size_t ws_bytes,
                     void* stream) {
  TRY(validate_desc(desc));
  if (T < 0 || T > desc->max_chunk)
    return fail(MOE_ERR_INVALID_ARGUMENT, "T must be in 0..max_chunk (got %d)", T);
  if (T == 0) return MOE_OK;
  if (!x || !router_w || !out || !ws) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer argument");
  if (!out->topk_ids || !out->topk_weights || !out->expert_counts || !out->expert_offsets ||
      !out->sorted_assign || !out->tile_map || !out->n_tiles)
    return fail(MOE_ERR_INVALID_ARGUMENT, "null routing output pointer");
  const Ws w = ws_layout(desc, T);
  if (ws_bytes < w.total)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < required %zu", ws_bytes, w.total);
  TRY(check_device());
  RouteOut o = ws_route(ws, w);
  o.ids = out->topk_ids;
  o.tw = out->topk_weights;
  o.counts = out->expert_counts;
  o.offsets = out->expert_offsets;
  o.sorted = out->sorted_assign;
  o.tiles = out->tile_map;
  o.n_tiles = out->n_tiles;
  return run_route(desc, x, T, router_w, logit_bias, o, static_cast<hipStream_t>(stream));
}

moe_status moe_forward_prefill(const moe_layer_desc* desc, const void* packed, const float* router_w,
                               const float* logit_bias, const uint16_t* x, int32_t T, float* y, void* ws,
                               size_t ws_bytes, void* stream) {
  TRY(forward_checks(desc, packed, router_w, x, T, y, ws, ws_bytes));
  if (T == 0) return MOE_OK;
  TRY(check_device());
  return prefill_loop(desc, packed, router_w, logit_bias, x, T, y, ws, ws_bytes, true,
                      static_cast<hipStream_t>(stream));
}

moe_status moe_forward_decode(const moe_layer_desc* desc, const void* packed, const float* router_w,
                              const float* logit_bias, const uint16_t* x, int32_t T, float* y, void* ws,
                              size_t ws_bytes, void* stream) {
  TRY(forward_checks(desc, packed, router_w, x, T, y, ws, ws_bytes));
  if (T == 0) return MOE_OK;
  TRY(check_device());
  return decode_impl(desc, packed, router_w, logit_bias, x, T, y, ws, ws_bytes, true, stream);
}

moe_status moe_forward_decode_static(const moe_layer_desc* desc, const void* packed, const float* router_w,
                                     const float* logit_bias, const uint16_t* x, int32_t T, float* y,
                                     void* stream) {
  TRY(validate_desc(desc));
  if (T < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "T must be >= 0 (got %d)", T);
  if (T == 0) return MOE_OK;
  if (desc->host_sync_routing || desc->dequant_pass)
    return fail(MOE_ERR_INVALID_ARGUMENT, "the static-scratch decode takes neither host_sync_routing nor dequant_pass");
  if (!packed || !router_w || !x || !y) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer argument");
  const size_t need = ws_layout(desc, T < desc->max_chunk ? T : desc->max_chunk).total;
  if (need > kStaticScratchBytes)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "this layer needs %zu bytes of scratch at T=%d; the static scratch holds %zu",
                need, T, kStaticScratchBytes);
  TRY(check_device());
  void* ws = nullptr;
  TRY(static_scratch(&ws));
  TRY(forward_checks(desc, packed, router_w, x, T, y, ws, kStaticScratchBytes));
  return decode_impl(desc, packed, router_w, logit_bias, x, T, y, ws, kStaticScratchBytes, false, stream);
}

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "MOE_ERR_UNSUPPORTED_SHAPE";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_DEVICE_UNSUPPORTED: return "MOE_ERR_DEVICE_UNSUPPORTED";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t max_workgroups,
                                 void* stream) {
  if (!src || !sink || max_workgroups < 1 || (reinterpret_cast<uintptr_t>(src) & 15) || (bytes & 15))
    return fail(MOE_ERR_INVALID_ARGUMENT, "probe: null pointer, max_workgroups < 1, or src/bytes not 16-byte aligned");
  TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  return timed(9, s, "stream-read probe",
               [&](const KTime& kt) { return launch_stream_read(src, bytes, sink, max_workgroups, s, kt); });
}

moe_status moe_probe_mfma_rate(int32_t iters, int32_t workgroups, uint64_t* clocks, uint32_t* sink, void* stream) {
  if (iters < 1 || workgroups < 1 || !sink) return fail(MOE_ERR_INVALID_ARGUMENT, "probe: iters, workgroups or sink");
  TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  return timed(10, s, "MFMA-rate probe",
               [&](const KTime& kt) { return launch_mfma_rate(iters, workgroups, clocks, sink, s, kt); });
}

moe_status moe_profile_enable(int32_t mask) {
  g_prof_mask = (uint32_t)mask;
  return MOE_OK;
}

moe_status moe_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& p : g_pending) {
    (void)hipEventSynchronize(p.b);
    g_event_pool.push_back(p.a);
    g_event_pool.push_back(p.b);
  }
  g_pending.clear();
  for (int i = 0; i < kNumKernels; i++) {
    g_prof_ms[i] = 0.0;
    g_prof_n[i] = 0;
  }
  return MOE_OK;
}

moe_status moe_profile_read(int32_t kernel_id, double* total_ms, int32_t* launches) {
  if (kernel_id < 0 || kernel_id >= kNumKernels || !total_ms || !launches)
    return fail(MOE_ERR_INVALID_ARGUMENT, "bad profile query");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& p : g_pending) {
    hipError_t e = hipEventSynchronize(p.b);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(e));
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, p.a, p.b);
    g_prof_ms[p.kid] += ms;
    g_prof_n[p.kid] += 1;
    g_event_pool.push_back(p.a);
    g_event_pool.push_back(p.b);
  }
  g_pending.clear();
  *total_ms = g_prof_ms[kernel_id];
  *launches = g_prof_n[kernel_id];
  return MOE_OK;
}

}  // extern "C"
