// C ABI of libfkmeans: argument validation, workspace layout, path dispatch,
// the Lloyd loop and the optional timing trace. Every numeric step runs in
// the kernels of norms.hip, assign.hip and update.hip.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "fk_internal.hpp"

namespace fk {
LaunchEvents& launch_events() {
  static thread_local LaunchEvents ev;
  return ev;
}
}  // namespace fk

namespace {

using fk::UpdateWs;

constexpr int64_t kI32Max = 0x7FFFFFFF;
constexpr int64_t kElemLimit = (int64_t)1 << 62;

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int elem_bytes(int dt) { return dt == FK_F32 ? 4 : 2; }

bool valid_dt(int dt) { return dt == FK_F32 || dt == FK_F16 || dt == FK_BF16; }

bool mul_ok(int64_t a, int64_t b, int64_t c) {
  if (a == 0 || b == 0 || c == 0) return true;
  if (a > kElemLimit / b) return false;
  const int64_t ab = a * b;
  return ab <= kElemLimit / c;
}

bool valid_sizes(int64_t B, int64_t N, int64_t d, int64_t K) {
  if (B < 0 || N < 0 || d < 1 || K < 1) return false;
  if (N >= kI32Max || K >= kI32Max || d >= kI32Max || B >= kI32Max) return false;
  return mul_ok(B, N, d) && mul_ok(B, K, d);
}

fk_status_t hip_status(hipError_t e) { return e == hipSuccess ? FK_OK : FK_ERR_HIP; }

bool force_splitd() {
  const char* v = getenv("FK_FORCE_SPLITD");
  return v && v[0] == '1';
}

hipError_t run_assign(const void* x, const void* c_lp, const float* cn, int dt, int64_t B,
                      int64_t N, int64_t d, int64_t K, int32_t* ids, hipStream_t s) {
  if (!force_splitd() && fk::smalld_supported(dt, d))
    return fk::launch_assign_smalld(x, c_lp, cn, dt, B, N, d, K, ids, s);
  return fk::launch_assign_splitd(x, c_lp, cn, dt, B, N, d, K, ids, s);
}

// Workspace beyond the update's: rounded centroids, norms, counts, shift,
// and (for the tol test) copies of the ids and centres of the last iteration
// whose stop decision is still pending.
struct LloydWs {
  UpdateWs upd;
  void* c_lp;
  float* cnorm;
  int32_t* counts;
  float* shift;
  int32_t* ids_bak;
  float* centers_bak;
};

size_t lloyd_extra_bytes(int dt, int64_t B, int64_t N, int64_t d, int64_t K) {
  return align256((size_t)B * K * d * elem_bytes(dt)) + align256((size_t)B * K * 4) * 2 +
         align256((size_t)B * 4) + align256((size_t)B * N * 4) + align256((size_t)B * K * d * 4);
}

LloydWs carve_lloyd(void* base, int dt, int64_t B, int64_t N, int64_t d, int64_t K) {
  LloydWs w;
  w.upd = fk::carve_update_ws(base, B, N, d, K);
  char* p = static_cast<char*>(base) + fk::update_ws_bytes(B, N, d, K);
  w.c_lp = p;
  p += align256((size_t)B * K * d * elem_bytes(dt));
  w.cnorm = reinterpret_cast<float*>(p);
  p += align256((size_t)B * K * 4);
  w.counts = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)B * K * 4);
  w.shift = reinterpret_cast<float*>(p);
  p += align256((size_t)B * 4);
  w.ids_bak = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)B * N * 4);
  w.centers_bak = reinterpret_cast<float*>(p);
  return w;
}

// Page-locked host copies of the shift of the two most recent iterations and
// the events that say they have arrived; released on every return path.
struct ShiftReadback {
  float* host = nullptr;
  hipEvent_t ev[2] = {nullptr, nullptr};
  bool ok = false;
  explicit ShiftReadback(int64_t B) {
    ok = hipHostMalloc((void**)&host, (size_t)2 * B * sizeof(float), hipHostMallocDefault) ==
             hipSuccess &&
         hipEventCreateWithFlags(&ev[0], hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&ev[1], hipEventDisableTiming) == hipSuccess;
  }
  ~ShiftReadback() {   // teardown errors have no one to report to
    for (int i = 0; i < 2; ++i)
      if (ev[i]) (void)hipEventSynchronize(ev[i]), (void)hipEventDestroy(ev[i]);
    if (host) (void)hipHostFree(host);
  }
};

// Workspace of the host-streamed loop: two chunk buffers, the chunk's ids,
// the update scratch for one chunk, the running sums and counts, the
// chunk's counts, rounded centroids, norms, shift and shift partials.
struct HostWs {
  void* xbuf[2];
  int32_t* ids_chunk;
  UpdateWs upd;
  float* sums;
  int32_t* counts;
  int32_t* counts_chunk;
  void* c_lp;
  float* cnorm;
  float* shift;
  float* part;
};

size_t host_ws_bytes(int dt, int64_t B, int64_t chunk, int64_t d, int64_t K) {
  return 2 * align256((size_t)B * chunk * d * elem_bytes(dt)) + align256((size_t)B * chunk * 4) +
         fk::update_ws_bytes(B, chunk, d, K) + align256((size_t)B * K * d * 4) +
         2 * align256((size_t)B * K * 4) + align256((size_t)B * K * d * elem_bytes(dt)) +
         align256((size_t)B * K * 4) + align256((size_t)B * 4) +
         align256((size_t)B * fk::sums_fin_blocks(K, d) * 4);
}

HostWs carve_host(void* base, int dt, int64_t B, int64_t chunk, int64_t d, int64_t K) {
  HostWs w;
  char* p = static_cast<char*>(base);
  for (int i = 0; i < 2; ++i) {
    w.xbuf[i] = p;
    p += align256((size_t)B * chunk * d * elem_bytes(dt));
  }
  w.ids_chunk = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)B * chunk * 4);
  w.upd = fk::carve_update_ws(p, B, chunk, d, K);
  p += fk::update_ws_bytes(B, chunk, d, K);
  w.sums = reinterpret_cast<float*>(p);
  p += align256((size_t)B * K * d * 4);
  w.counts = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)B * K * 4);
  w.counts_chunk = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)B * K * 4);
  w.c_lp = p;
  p += align256((size_t)B * K * d * elem_bytes(dt));
  w.cnorm = reinterpret_cast<float*>(p);
  p += align256((size_t)B * K * 4);
  w.shift = reinterpret_cast<float*>(p);
  p += align256((size_t)B * 4);
  w.part = reinterpret_cast<float*>(p);
  return w;
}

// The copy stream and events of one host-streamed call, released on every
// return path.
struct StreamSet {
  hipStream_t copy = nullptr;
  hipEvent_t ready[2] = {nullptr, nullptr};
  hipEvent_t free_[2] = {nullptr, nullptr};
  bool ok = false;
  StreamSet() {
    ok = hipStreamCreateWithFlags(&copy, hipStreamNonBlocking) == hipSuccess;
    for (int i = 0; i < 2 && ok; ++i)
      ok = hipEventCreateWithFlags(&ready[i], hipEventDisableTiming) == hipSuccess &&
           hipEventCreateWithFlags(&free_[i], hipEventDisableTiming) == hipSuccess;
  }
  ~StreamSet() {   // teardown errors have no one to report to
    if (copy) (void)hipStreamSynchronize(copy);
    for (int i = 0; i < 2; ++i) {
      if (ready[i]) (void)hipEventDestroy(ready[i]);
      if (free_[i]) (void)hipEventDestroy(free_[i]);
    }
    if (copy) (void)hipStreamDestroy(copy);
  }
};

// ---------------------------------------------------------------------------
// trace
// Per iteration: the norms kernel's start and end, the assign kernel's start
// and end (stamped by the kernels' own launches, so the trace adds nothing to
// the stream between them), and, for the last iteration a call traces, a
// marker after its update. An iteration's update runs from its assign's end
// to the next iteration's norms start, or to that marker.
enum TraceEv { kNormsStart, kNormsEnd, kAssignStart, kAssignEnd, kUpdateEnd, kTraceEvs };
struct Trace {
  bool on = false;
  int32_t capacity = 0;
  int32_t used = 0;
  std::vector<hipEvent_t> ev;       // kTraceEvs per iteration
  std::vector<char> has_end;        // kUpdateEnd recorded
};
Trace g_trace;

void trace_release() {
  for (hipEvent_t e : g_trace.ev) (void)hipEventDestroy(e);
  g_trace.ev.clear();
  g_trace.has_end.clear();
  g_trace.on = false;
  g_trace.capacity = g_trace.used = 0;
}

hipEvent_t trace_event(int32_t it, int which) {
  return g_trace.ev[(size_t)it * kTraceEvs + which];
}

// Hands the next timed launch a start and end event; if no kernel took them
// (nothing to launch), they become plain stream markers at that point.
struct TimedPhase {
  bool on;
  TimedPhase(bool tr, hipEvent_t a, hipEvent_t b) : on(tr) {
    if (on) fk::launch_events() = fk::LaunchEvents{a, b};
  }
  hipError_t finish(hipStream_t s) {
    if (!on) return hipSuccess;
    on = false;
    fk::LaunchEvents& le = fk::launch_events();
    if (!le.start && !le.stop) return hipSuccess;
    const fk::LaunchEvents ev = le;
    le = fk::LaunchEvents();
    hipError_t e = hipEventRecord(ev.start, s);
    return e != hipSuccess ? e : hipEventRecord(ev.stop, s);
  }
  ~TimedPhase() {
    if (on) fk::launch_events() = fk::LaunchEvents();
  }
};

}  // namespace

// ---------------------------------------------------------------------------
// Workspace of fk_update_noalloc: one array per GPU, part of the library's
// code object (each device that loads the library holds its own copy until
// the process ends). In host code `scratch` names a host-side stand-in, not
// device memory: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is ever handed to a kernel.
static_assert(FK_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte units");
static __device__ __align__(256) unsigned char scratch[FK_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

struct ScratchPtrs {
  std::once_flag once[kMaxDevices];
  void* ptr[kMaxDevices] = {};
  hipError_t err[kMaxDevices] = {};
};
ScratchPtrs g_scratch;

// The current device's scratch address (null with *e set on failure).
void* scratch_ptr(hipError_t* e) {
  int dev = -1;
  *e = hipGetDevice(&dev);
  if (*e != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *e = hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(g_scratch.once[dev], [dev]() {
    void* p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch.err[dev] = r;
    g_scratch.ptr[dev] = r == hipSuccess ? p : nullptr;
  });
  *e = g_scratch.err[dev];
  return g_scratch.ptr[dev];
}

}  // namespace

extern "C" {

const char* fk_status_string(fk_status_t st) {
  switch (st) {
    case FK_OK: return "FK_OK";
    case FK_ERR_INVALID: return "FK_ERR_INVALID: invalid argument";
    case FK_ERR_UNSUPPORTED: return "FK_ERR_UNSUPPORTED: shape not supported";
    case FK_ERR_WORKSPACE: return "FK_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case FK_ERR_HIP: return "FK_ERR_HIP: HIP launch or runtime error";
  }
  return "unknown status";
}

int32_t fk_version(void) { return 100; }

size_t fk_workspace_size(fk_dtype_t dt, int64_t B, int64_t N, int64_t d, int64_t K) {
  if (!valid_dt(dt) || !valid_sizes(B, N, d, K)) return 0;
  const size_t n = fk::update_ws_bytes(B, N, d, K) + lloyd_extra_bytes(dt, B, N, d, K);
  return n < 256 ? 256 : n;   // never 0 for a valid problem (0 flags bad arguments)
}

fk_status_t fk_norms(const float* c, void* c_lp, float* cnorm, fk_dtype_t dt, int64_t B,
                     int64_t K, int64_t d, hipStream_t stream) {
  if (!valid_dt(dt) || !valid_sizes(B, 0, d, K)) return FK_ERR_INVALID;
  if (B > 0 && (!c || !c_lp || !cnorm)) return FK_ERR_INVALID;
  return hip_status(fk::launch_norms(c, c_lp, cnorm, dt, B * K, d, stream));
}

fk_status_t fk_assign(const void* x, const void* c_lp, const float* cnorm, fk_dtype_t dt,
                      int64_t B, int64_t N, int64_t d, int64_t K, int32_t* ids,
                      hipStream_t stream) {
  if (!valid_dt(dt) || !valid_sizes(B, N, d, K)) return FK_ERR_INVALID;
  if (B * N > 0 && (!x || !c_lp || !cnorm || !ids)) return FK_ERR_INVALID;
  const hipError_t e = run_assign(x, c_lp, cnorm, dt, B, N, d, K, ids, stream);
  if (e == hipErrorNotSupported || e == hipErrorInvalidConfiguration) return FK_ERR_UNSUPPORTED;
  return hip_status(e);
}

fk_status_t fk_update(const void* x, const int32_t* ids, fk_dtype_t dt, int64_t B, int64_t N,
                      int64_t d, int64_t K, float* c, int32_t* counts, float* shift, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
  if (!valid_dt(dt) || !valid_sizes(B, N, d, K)) return FK_ERR_INVALID;
  if (B > 0 && (!c || !counts || !shift)) return FK_ERR_INVALID;
  if (B * N > 0 && (!x || !ids)) return FK_ERR_INVALID;
  if (B == 0) return FK_OK;
  if (!ws || ((uintptr_t)ws & 255) || ws_bytes < fk::update_ws_bytes(B, N, d, K))
    return FK_ERR_WORKSPACE;
  const UpdateWs w = fk::carve_update_ws(ws, B, N, d, K);
  const hipError_t e = fk::launch_update(x, ids, dt, B, N, d, K, c, counts, shift, w, stream);
  if (e == hipErrorInvalidConfiguration) return FK_ERR_UNSUPPORTED;
  return hip_status(e);
}

fk_status_t fk_update_noalloc(const void* x, const int32_t* ids, fk_dtype_t dt, int64_t B,
                              int64_t N, int64_t d, int64_t K, float* c, int32_t* counts,
                              float* shift, hipStream_t stream) {
  if (!valid_dt(dt) || !valid_sizes(B, N, d, K)) return FK_ERR_INVALID;
  if (B > 0 && (!c || !counts || !shift)) return FK_ERR_INVALID;
  if (B * N > 0 && (!x || !ids)) return FK_ERR_INVALID;
  if (B == 0) return FK_OK;
  if (fk::update_ws_bytes(B, N, d, K) > (size_t)FK_NOALLOC_SCRATCH_BYTES) return FK_ERR_WORKSPACE;
  hipError_t e = hipSuccess;
  void* ws = scratch_ptr(&e);
  if (!ws) return FK_ERR_HIP;
  const UpdateWs w = fk::carve_update_ws(ws, B, N, d, K);
  e = fk::launch_update(x, ids, dt, B, N, d, K, c, counts, shift, w, stream);
  if (e == hipErrorInvalidConfiguration) return FK_ERR_UNSUPPORTED;
  return hip_status(e);
}

fk_status_t fk_update_partial(const void* x, const int32_t* ids, fk_dtype_t dt, int64_t B,
                              int64_t N, int64_t d, int64_t K, float* sums, int32_t* counts,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!valid_dt(dt) || !valid_sizes(B, N, d, K)) return FK_ERR_INVALID;
  if (B > 0 && (!sums || !counts)) return FK_ERR_INVALID;
  if (B * N > 0 && (!x || !ids)) return FK_ERR_INVALID;
  if (B == 0 || N == 0) return FK_OK;
  if (!ws || ((uintptr_t)ws & 255) || ws_bytes < fk_workspace_size(dt, B, N, d, K))
    return FK_ERR_WORKSPACE;
  const LloydWs w = carve_lloyd(ws, dt, B, N, d, K);
  const hipError_t e = fk::launch_update_accumulate(x, ids, dt, B, N, d, K, sums, counts,
                                                    w.counts, w.upd, stream);
  if (e == hipErrorInvalidConfiguration) return FK_ERR_UNSUPPORTED;
  return hip_status(e);
}

fk_status_t fk_lloyd(const void* x, fk_dtype_t dt, int64_t B, int64_t N, int64_t d, int64_t K,
                     const void* init, int32_t max_iter, float tol, int32_t* ids, float* centers,
                     int32_t* n_iter, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!valid_dt(dt) || !valid_sizes(B, N, d, K)) return FK_ERR_INVALID;
  if (max_iter < 0 || !(tol >= 0.f) || !n_iter) return FK_ERR_INVALID;
  if (B > 0 && !centers) return FK_ERR_INVALID;
  if (B * N > 0 && (!x || !ids)) return FK_ERR_INVALID;
  *n_iter = 0;
  if (B == 0) return FK_OK;
  if (!ws || ((uintptr_t)ws & 255) || ws_bytes < fk_workspace_size(dt, B, N, d, K))
    return FK_ERR_WORKSPACE;
  const LloydWs w = carve_lloyd(ws, dt, B, N, d, K);
  // no init: resume from the fp32 centres already in `centers`
  hipError_t e = init ? fk::launch_widen(init, centers, dt, B * K * d, stream) : hipSuccess;
  if (e != hipSuccess) return FK_ERR_HIP;
  if (max_iter == 0) return hip_status(fk::launch_fill_i32(ids, 0, B * N, stream));

  // With tol > 0 the stop decision for iteration t is taken while iteration
  // t + 1 already runs: t's shift comes back to page-locked host memory
  // asynchronously, and its ids and centres are copied aside. If t turns out
  // to have converged, those copies replace what t + 1 wrote, so the result
  // is exactly that of stopping after t; the GPU never waits for the host.
  const bool test = tol > 0.f;
  const bool defer = !test && N > 0;
  ShiftReadback rb(test ? B : 1);
  if (test && !rb.ok) return FK_ERR_HIP;
  int32_t done = 0, pending = -1;
  const size_t ids_bytes = (size_t)B * N * 4, c_bytes = (size_t)B * K * d * 4;
  const int32_t first_slot = g_trace.used;
  for (int32_t t = 0; t < max_iter; ++t) {
    const bool tr = g_trace.on && g_trace.used < g_trace.capacity;
    const int32_t slot = g_trace.used;
    // without the tol test, the previous update's long clusters are divided
    // by this norms pass (it reads the centres anyway): one launch less
    {
      TimedPhase ph(tr, tr ? trace_event(slot, kNormsStart) : nullptr,
                    tr ? trace_event(slot, kNormsEnd) : nullptr);
      e = fk::launch_norms(centers, w.c_lp, w.cnorm, dt, B * K, d, stream,
                           defer && t > 0 ? fk::pending_finish(w.upd, K) : fk::PendingFinish());
      if (e != hipSuccess || ph.finish(stream) != hipSuccess) return FK_ERR_HIP;
    }
    {
      TimedPhase ph(tr, tr ? trace_event(slot, kAssignStart) : nullptr,
                    tr ? trace_event(slot, kAssignEnd) : nullptr);
      e = run_assign(x, w.c_lp, w.cnorm, dt, B, N, d, K, ids, stream);
      if (e == hipErrorNotSupported || e == hipErrorInvalidConfiguration) return FK_ERR_UNSUPPORTED;
      if (e != hipSuccess || ph.finish(stream) != hipSuccess) return FK_ERR_HIP;
    }
    // the shift is only read for the tol test
    e = fk::launch_update(x, ids, dt, B, N, d, K, centers, w.counts, test ? w.shift : nullptr,
                          w.upd, stream, defer);
    if (e == hipErrorInvalidConfiguration) return FK_ERR_UNSUPPORTED;
    if (e != hipSuccess) return FK_ERR_HIP;
    if (tr) {
      // the last iteration this call can trace ends with a marker of its own
      if (slot == g_trace.capacity - 1 || t == max_iter - 1) {
        if (hipEventRecord(trace_event(slot, kUpdateEnd), stream) != hipSuccess) return FK_ERR_HIP;
        g_trace.has_end[slot] = 1;
      }
      ++g_trace.used;
    }
    done = t + 1;
    if (!test) continue;
    float* hs = rb.host + (size_t)(t & 1) * B;
    if (hipMemcpyAsync(hs, w.shift, (size_t)B * sizeof(float), hipMemcpyDeviceToHost,
                       stream) != hipSuccess ||
        hipEventRecord(rb.ev[t & 1], stream) != hipSuccess)
      return FK_ERR_HIP;
    if (pending >= 0) {                          // decide on the previous iteration
      if (hipEventSynchronize(rb.ev[pending & 1]) != hipSuccess) return FK_ERR_HIP;
      const float* ps = rb.host + (size_t)(pending & 1) * B;
      float mx = ps[0];
      for (int64_t b = 1; b < B; ++b) mx = ps[b] > mx ? ps[b] : mx;
      if (mx < tol) {                            // it converged: undo iteration t
        if (hipMemcpyAsync(ids, w.ids_bak, ids_bytes, hipMemcpyDeviceToDevice, stream) !=
                hipSuccess ||
            hipMemcpyAsync(centers, w.centers_bak, c_bytes, hipMemcpyDeviceToDevice, stream) !=
                hipSuccess)
          return FK_ERR_HIP;
        done = pending + 1;
        break;
      }
    }
    if (t + 1 < max_iter) {                      // keep t's results until t is decided
      if (hipMemcpyAsync(w.ids_bak, ids, ids_bytes, hipMemcpyDeviceToDevice, stream) !=
              hipSuccess ||
          hipMemcpyAsync(w.centers_bak, centers, c_bytes, hipMemcpyDeviceToDevice, stream) !=
              hipSuccess)
        return FK_ERR_HIP;
      pending = t;
    }
  }
  if (defer && done > 0 && fk::launch_finish(centers, w.upd, B, d, K, stream) != hipSuccess)
    return FK_ERR_HIP;
  // a tol stop ends the loop early: its last traced iteration gets the marker
  if (g_trace.on && g_trace.used > first_slot && !g_trace.has_end[g_trace.used - 1]) {
    if (hipEventRecord(trace_event(g_trace.used - 1, kUpdateEnd), stream) != hipSuccess)
      return FK_ERR_HIP;
    g_trace.has_end[g_trace.used - 1] = 1;
  }
  if (test && hipStreamSynchronize(stream) != hipSuccess) return FK_ERR_HIP;
  *n_iter = done;
  return FK_OK;
}

size_t fk_workspace_size_host(fk_dtype_t dt, int64_t B, int64_t chunk, int64_t d, int64_t K) {
  if (!valid_dt(dt) || chunk < 1 || !valid_sizes(B, chunk, d, K)) return 0;
  const size_t n = host_ws_bytes(dt, B, chunk, d, K);
  return n < 256 ? 256 : n;
}

fk_status_t fk_lloyd_host(const void* x_host, fk_dtype_t dt, int64_t B, int64_t N, int64_t d,
                          int64_t K, const void* init, int32_t max_iter, float tol,
                          int64_t chunk, int32_t* ids, float* centers, int32_t* n_iter,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!valid_dt(dt) || !valid_sizes(B, N, d, K) || chunk < 1) return FK_ERR_INVALID;
  if (max_iter < 0 || !(tol >= 0.f) || !n_iter) return FK_ERR_INVALID;
  if (B > 0 && !centers) return FK_ERR_INVALID;
  if (B * N > 0 && (!x_host || !ids)) return FK_ERR_INVALID;
  *n_iter = 0;
  if (B == 0) return FK_OK;
  if (!ws || ((uintptr_t)ws & 255) || ws_bytes < fk_workspace_size_host(dt, B, chunk, d, K))
    return FK_ERR_WORKSPACE;
  const HostWs w = carve_host(ws, dt, B, chunk, d, K);
  if (init && fk::launch_widen(init, centers, dt, B * K * d, stream) != hipSuccess)
    return FK_ERR_HIP;
  if (max_iter == 0) {
    if (fk::launch_fill_i32(ids, 0, B * N, stream) != hipSuccess) return FK_ERR_HIP;
    return hip_status(hipStreamSynchronize(stream));
  }
  StreamSet ss;
  if (!ss.ok) return FK_ERR_HIP;
  const size_t es = (size_t)elem_bytes(dt);
  const int64_t cmax = chunk < N ? chunk : N;
  const int64_t nchunks = N > 0 ? (N + cmax - 1) / cmax : 0;
  for (int i = 0; i < 2; ++i)
    if (hipEventRecord(ss.free_[i], stream) != hipSuccess) return FK_ERR_HIP;
  std::vector<float> host_shift(tol > 0.f ? (size_t)B : 0);
  int32_t done = 0;
  for (int32_t t = 0; t < max_iter; ++t) {
    if (fk::launch_norms(centers, w.c_lp, w.cnorm, dt, B * K, d, stream) != hipSuccess ||
        fk::launch_zero_sums(w.sums, w.counts, B, K, d, stream) != hipSuccess)
      return FK_ERR_HIP;
    for (int64_t i = 0; i < nchunks; ++i) {
      const int slot = (int)(i & 1);
      const int64_t n0 = i * cmax, cn = (N - n0) < cmax ? (N - n0) : cmax;
      // copy stream: the slot's previous chunk is done, then x[:, n0:n0+cn]
      if (hipStreamWaitEvent(ss.copy, ss.free_[slot], 0) != hipSuccess ||
          hipMemcpy2DAsync(w.xbuf[slot], (size_t)cn * d * es,
                           static_cast<const char*>(x_host) + (size_t)n0 * d * es,
                           (size_t)N * d * es, (size_t)cn * d * es, (size_t)B,
                           hipMemcpyHostToDevice, ss.copy) != hipSuccess ||
          hipEventRecord(ss.ready[slot], ss.copy) != hipSuccess ||
          hipStreamWaitEvent(stream, ss.ready[slot], 0) != hipSuccess)
        return FK_ERR_HIP;
      hipError_t e = run_assign(w.xbuf[slot], w.c_lp, w.cnorm, dt, B, cn, d, K, w.ids_chunk,
                                stream);
      if (e == hipErrorNotSupported || e == hipErrorInvalidConfiguration) return FK_ERR_UNSUPPORTED;
      if (e != hipSuccess) return FK_ERR_HIP;
      if (hipMemcpy2DAsync(ids + n0, (size_t)N * 4, w.ids_chunk, (size_t)cn * 4, (size_t)cn * 4,
                           (size_t)B, hipMemcpyDeviceToDevice, stream) != hipSuccess)
        return FK_ERR_HIP;
      e = fk::launch_update_accumulate(w.xbuf[slot], w.ids_chunk, dt, B, cn, d, K, w.sums,
                                       w.counts, w.counts_chunk, w.upd, stream);
      if (e == hipErrorInvalidConfiguration) return FK_ERR_UNSUPPORTED;
      if (e != hipSuccess || hipEventRecord(ss.free_[slot], stream) != hipSuccess)
        return FK_ERR_HIP;
    }
    if (fk::launch_finalize_sums(w.sums, w.counts, centers, tol > 0.f ? w.shift : nullptr,
                                 w.part, B, K, d, stream) != hipSuccess)
      return FK_ERR_HIP;
    done = t + 1;
    if (tol > 0.f) {
      if (hipMemcpyAsync(host_shift.data(), w.shift, (size_t)B * sizeof(float),
                         hipMemcpyDeviceToHost, stream) != hipSuccess ||
          hipStreamSynchronize(stream) != hipSuccess)
        return FK_ERR_HIP;
      float mx = host_shift[0];
      for (int64_t b = 1; b < B; ++b) mx = host_shift[b] > mx ? host_shift[b] : mx;
      if (mx < tol) break;
    }
  }
  *n_iter = done;
  return hip_status(hipStreamSynchronize(stream));
}

fk_status_t fk_trace_begin(int32_t capacity) {
  if (capacity < 1) return FK_ERR_INVALID;
  trace_release();
  g_trace.ev.resize((size_t)capacity * kTraceEvs);
  g_trace.has_end.assign((size_t)capacity, 0);
  for (auto& e : g_trace.ev) {
    if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
      trace_release();
      return FK_ERR_HIP;
    }
  }
  g_trace.capacity = capacity;
  g_trace.used = 0;
  g_trace.on = true;
  return FK_OK;
}

fk_status_t fk_trace_end(fk_trace_t* out) {
  if (!out) return FK_ERR_INVALID;
  memset(out, 0, sizeof(*out));
  if (!g_trace.on) return FK_ERR_INVALID;
  fk_status_t st = FK_OK;
  for (int32_t i = 0; i < g_trace.used && st == FK_OK; ++i) {
    float a = 0.f, b = 0.f, c = 0.f;
    // the update ends at the next iteration's norms start, or at the marker
    const bool own_end = g_trace.has_end[i] || i + 1 == g_trace.used;
    const hipEvent_t uend =
        own_end ? trace_event(i, kUpdateEnd) : trace_event(i + 1, kNormsStart);
    if (!g_trace.has_end[i] && own_end) {        // no marker was recorded: nothing to end on
      st = FK_ERR_INVALID;
      break;
    }
    if (hipEventSynchronize(uend) != hipSuccess ||
        hipEventElapsedTime(&a, trace_event(i, kNormsStart), trace_event(i, kNormsEnd)) !=
            hipSuccess ||
        hipEventElapsedTime(&b, trace_event(i, kAssignStart), trace_event(i, kAssignEnd)) !=
            hipSuccess ||
        hipEventElapsedTime(&c, trace_event(i, kAssignEnd), uend) != hipSuccess) {
      st = FK_ERR_HIP;
      break;
    }
    out->norms_ms += a;
    out->assign_ms += b;
    out->update_ms += c;
    out->iterations += 1;
  }
  trace_release();
  return st;
}

}  // extern "C"
