// C ABI of the frame-wise GDN forward: argument validation, workspace layout
// and dispatch to the HIP kernels.  Declarations and the contract are in
// include/gdn.h.
//
// Layout of this file: argument checks; per-device state (timing events,
// the side streams of the segmented schedule, fused-kernel launch sizes);
// the two schedules of the MFMA path; the extern "C" entry points.
#include "gdn.h"
#include "gdn_attn.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdlib>
#include <limits>
#include <mutex>
#include <utility>
#include <vector>

#include "gdn_backward.h"
#include "gdn_launch.h"

namespace {

constexpr int64_t kMaxFrames = (int64_t{1} << 24) - 1;  // B*H*T: one workgroup per frame
constexpr int64_t kSegmentFrames = 64;                   // frames per segment, overlapped schedule
// The backward cuts a sequence into at most 3 segments of at least
// kSegmentFrames frames.  Its reverse chain waits on a cross-stream hand-off
// per segment, and fewer, longer segments pay fewer of them while still
// overlapping the chains with the streaming kernels.  Measured on the 60 s
// workload (two boxes, segments of F frames, each box against itself):
// F = 32, 64, 96, 128, 192: 12.69, 12.55, 12.54, 12.38, 12.21 ms; then
// F = 192, 256, 321, 481, 961 (3 segments at 321, one at 961): 11.99,
// 11.91, 11.81, 12.01, 14.13 ms.
constexpr int64_t kBwdMaxSegments = 3;
constexpr int64_t kFusedMinT = 32;                       // shorter sequences take the three-kernel path
constexpr int64_t kMapSlots = 3;                         // segments whose maps the MFMA path holds at once
constexpr size_t kMapFrameBytes = 128 * 128 * 4;         // one packed G, U or M of one frame (D = 128)

struct Dims {
  int64_t B, H, T, S, D;
  int64_t heads, frames;
  size_t in_elems, state_elems, map_elems;  // per tensor
};

// a * b for a, b >= 0, false on overflow
bool mul_ok(int64_t a, int64_t b, int64_t* r) {
  if (a < 0 || b < 0) return false;
  if (b != 0 && a > std::numeric_limits<int64_t>::max() / b) return false;
  *r = a * b;
  return true;
}

bool valid_dtype(int d) { return d == GDN_F32 || d == GDN_BF16; }
size_t dsize(int d) { return d == GDN_BF16 ? 2 : 4; }

// Validates the shape; use_s selects whether S takes part.  allow_empty
// admits B, H, T or S of 0 (the whole calls: nothing to do, or only the
// state to set); the stage entry points need every size >= 1.
int check_shape(const gdn_shape* s, bool use_s, Dims* out, bool allow_empty = false) {
  if (!s) return GDN_E_NULLPTR;
  Dims d{};
  d.B = s->B;
  d.H = s->H;
  d.T = s->T;
  d.S = use_s ? s->S : 1;
  d.D = s->D;
  const int64_t lo = allow_empty ? 0 : 1;
  if (d.B < lo || d.H < lo || d.T < lo || d.S < lo || d.D < 1) return GDN_E_SHAPE;
  if (!gdn_supports_d(d.D)) return GDN_E_UNSUPPORTED_D;
  if (d.S > std::numeric_limits<int>::max() / 256) return GDN_E_SHAPE;
  int64_t heads, frames, tmp;
  if (!mul_ok(d.B, d.H, &heads) || heads > kMaxFrames || !mul_ok(heads, d.T, &frames)) return GDN_E_SHAPE;
  if (frames > kMaxFrames) return GDN_E_SHAPE;
  int64_t in_elems, map_elems;
  if (!mul_ok(frames, d.S, &tmp) || !mul_ok(tmp, d.D, &in_elems)) return GDN_E_SHAPE;
  if (!mul_ok(frames, d.D * d.D, &map_elems)) return GDN_E_SHAPE;
  // keep every byte count well inside 64 bits
  if (in_elems > (int64_t{1} << 56) || map_elems > (int64_t{1} << 56)) return GDN_E_SHAPE;
  d.heads = heads;
  d.frames = frames;
  d.in_elems = (size_t)in_elems;
  d.state_elems = (size_t)(heads * d.D * d.D);
  d.map_elems = (size_t)map_elems;
  *out = d;
  return GDN_OK;
}

struct Range {
  const void* p;
  size_t bytes;
};

bool overlap(const Range& a, const Range& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Every output must be disjoint from every other buffer.  The one exception
// is the output `same_out` coinciding exactly (same address, same size) with
// the input `same_in` (state_out == state_in for in-place streaming).
bool aliasing_ok(const Range* outs, int nout, const Range* ins, int nin,
                 const void* same_out = nullptr, const void* same_in = nullptr) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j) {
      if (!overlap(outs[i], ins[j])) continue;
      const bool exact = outs[i].p == ins[j].p && outs[i].bytes == ins[j].bytes;
      if (exact && same_out && outs[i].p == same_out && ins[j].p == same_in) continue;
      return false;
    }
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return false;
  }
  return true;
}

bool fast_path(int in_dtype, int64_t D) { return in_dtype == GDN_BF16 && D == 128; }

// The fused kernel takes bf16, D == 128 sequences longer than one segment
// of the three-kernel schedule while it is enabled: gdn_set_fused switches
// it; GDN_FUSED=0 in the environment makes the default "disabled".
std::atomic<int>& fused_enabled() {
  static std::atomic<int> on{[] {
    const char* e = std::getenv("GDN_FUSED");
    return e && std::atoi(e) == 0 ? 0 : 1;
  }()};
  return on;
}

// Polls before a bounded wait of the fused kernel or of the split single-frame
// kernel gives up (0: each kernel's default);
// gdn_set_spin_limit sets it.
std::atomic<uint32_t>& spin_limit() {
  static std::atomic<uint32_t> polls{0};
  return polls;
}

bool fused_path(int in_dtype, const Dims& d) {
  return fused_enabled().load() && fast_path(in_dtype, d.D) && d.T > kFusedMinT;
}

// The single-frame kernels take bf16, D == 128 calls of one frame while
// they are enabled: gdn_set_single_frame switches them; GDN_SINGLE_FRAME=0
// in the environment makes the default "disabled".
std::atomic<int>& single_frame_enabled() {
  static std::atomic<int> on{[] {
    const char* e = std::getenv("GDN_SINGLE_FRAME");
    return e && std::atoi(e) == 0 ? 0 : 1;
  }()};
  return on;
}

bool frame1_path(int in_dtype, const Dims& d) {
  return single_frame_enabled().load() && fast_path(in_dtype, d.D) && d.T == 1;
}

int hip_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_E_HIP; }

size_t round256(size_t x) { return (x + 255) & ~size_t{255}; }

// ---------------------------------------------------------------------------
// per-device state, created on first use and kept for the life of the process
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;

void teardown();

// The library's own HIP objects (the timing events and the side streams
// and events below) are destroyed by an exit handler registered right
// after the first of them is created.  The HIP runtime registers its own
// exit-time clean-up when it starts, which is before that, and exit
// handlers run in reverse order of registration: this one runs first, while
// the runtime is still whole, and the objects never outlive it.
void register_teardown() {
  static std::once_flag once;
  std::call_once(once, [] { std::atexit(teardown); });
}

// Per-launch HIP events of gdn_frame_fwd_timed: a pair around every kernel,
// on the stream that kernel is launched on.  One pool per device, grown on
// demand and kept for the life of the process.
struct Recorder {
  std::vector<hipEvent_t>* pool;
  std::vector<int> kind;  // kernel kind of pair i
  hipError_t begin(hipStream_t st) {
    const size_t i = 2 * kind.size();
    while (pool->size() < i + 2) {
      hipEvent_t e;
      hipError_t err = hipEventCreate(&e);
      if (err != hipSuccess) return err;
      pool->push_back(e);
      register_teardown();
    }
    return hipEventRecord((*pool)[i], st);
  }
  hipError_t end(hipStream_t st, int k) {
    hipError_t err = hipEventRecord((*pool)[2 * kind.size() + 1], st);
    if (err == hipSuccess) kind.push_back(k);
    return err;
  }
};
std::vector<hipEvent_t> g_timing_pool[kMaxDevices];
std::mutex g_timing_mu;

// Side streams of the overlapped schedule, one pair per device, created on
// first use (non-blocking, default priority) and kept for the life of the
// process, with the events that chain them.  g_side_mu serialises the
// enqueue of a whole call, so calls from several host threads never
// interleave their records and waits on these events.
struct Side {
  hipStream_t state_st, out_st;
  hipEvent_t fork, built, state_done, out_done;
  hipEvent_t stated[kMapSlots], output[kMapSlots];  // per map slot: its state pass, its output done
  bool ready;
};
Side g_side[kMaxDevices];
std::mutex g_side_mu;

hipError_t side_init(Side& sd) {
  if (sd.ready) return hipSuccess;
  hipError_t e;
  if ((e = hipStreamCreateWithFlags(&sd.state_st, hipStreamNonBlocking)) != hipSuccess) return e;
  if ((e = hipStreamCreateWithFlags(&sd.out_st, hipStreamNonBlocking)) != hipSuccess) return e;
  for (hipEvent_t* ev : {&sd.fork, &sd.built, &sd.state_done, &sd.out_done, &sd.stated[0], &sd.stated[1],
                         &sd.stated[2], &sd.output[0], &sd.output[1], &sd.output[2]})
    if ((e = hipEventCreateWithFlags(ev, hipEventDisableTiming)) != hipSuccess) return e;
  sd.ready = true;
  register_teardown();
  return hipSuccess;
}

// Fused launches on one device run one after another.  The fused kernel
// needs no co-residency guarantee, but each launch holds up to 16
// state-pass workgroups of every XCD while they wait for workers, so enough
// of them at once on several streams could fill an XCD's 64 slots with
// state-pass workgroups and leave none for workers (their bounded waits
// would then end them with an error).  Per device: the event recorded after
// the last fused launch and its stream; a launch on another stream waits
// for it on the GPU.  Not under stream capture, whose graph must not depend
// on work outside it.  A stream handle reused after its stream was
// destroyed counts as the same stream.
struct FusedOrder {
  hipEvent_t done;
  hipStream_t last;
  bool have, ready;
};
FusedOrder g_fused_order[kMaxDevices];
std::mutex g_fused_mu;

// Frames per segment of the overlapped schedule (GDN_SEGMENT_FRAMES
// overrides the default; read once).
int64_t segment_frames() {
  static const int64_t f = [] {
    const char* e = std::getenv("GDN_SEGMENT_FRAMES");
    const long v = e ? std::strtol(e, nullptr, 10) : 0;
    return v >= 1 && v <= (1L << 24) ? (int64_t)v : int64_t{kSegmentFrames};
  }();
  return f;
}

// Segments of the MFMA path: ceil(T / F) of (nearly) equal length, at most
// `cap` frames each; the maps of segment i live in slot i % slots of each
// of the three map buffers.
struct Segments {
  int64_t n, cap, slots;
};
Segments segments_of(int64_t T) {
  const int64_t F = segment_frames();
  const int64_t n = (T + F - 1) / F;
  return {n, (T + n - 1) / n, n < kMapSlots ? n : kMapSlots};
}
size_t slot_bytes(const Dims& d, const Segments& g) { return round256((size_t)(d.heads * g.cap) * kMapFrameBytes); }

void teardown() {
  {
    std::lock_guard<std::mutex> lock(g_side_mu);
    for (Side& sd : g_side) {
      if (!sd.ready) continue;
      for (hipEvent_t ev : {sd.fork, sd.built, sd.state_done, sd.out_done, sd.stated[0], sd.stated[1],
                            sd.stated[2], sd.output[0], sd.output[1], sd.output[2]})
        (void)hipEventDestroy(ev);
      (void)hipStreamDestroy(sd.state_st);
      (void)hipStreamDestroy(sd.out_st);
      sd.ready = false;
    }
  }
  {
    std::lock_guard<std::mutex> lock(g_fused_mu);
    for (FusedOrder& fo : g_fused_order) {
      if (!fo.ready) continue;
      (void)hipEventDestroy(fo.done);
      fo.ready = fo.have = false;
    }
  }
  std::lock_guard<std::mutex> lock(g_timing_mu);
  for (auto& pool : g_timing_pool) {
    for (hipEvent_t ev : pool) (void)hipEventDestroy(ev);
    pool.clear();
  }
}

// Per-device facts queried once: the launch size of the fused kernel (0
// when the device cannot host it: too few compute units, or workgroups not
// dealt evenly over eight XCDs with ids 0-7, which the one-time probe in
// gdn::fused_topology_ok checks), and whether workgroups b and b + 8 share
// an XCD, as the split single-frame form needs (gdn::frame1_pairs_share_xcd).
struct DevInfo {
  int fused_grid[2];  // [out_bf16]
  bool frame_pairs;   // the split single-frame form can run (gdn::frame1_pairs_share_xcd)
  bool ready;
};
DevInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

hipError_t dev_info(DevInfo** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  DevInfo& di = g_dev[dev];
  if (!di.ready) {
    int cus = 0;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    for (int b = 0; b < 2; ++b) {
      int grid = gdn::fused_grid(b != 0, cus);
      bool even = false;
      if (grid > 0 && (e = gdn::fused_topology_ok(grid, &even)) != hipSuccess) return e;
      di.fused_grid[b] = even ? grid : 0;
    }
    if ((e = gdn::frame1_pairs_share_xcd(&di.frame_pairs)) != hipSuccess) return e;
    di.ready = true;
  }
  *out = &di;
  return hipSuccess;
}

// Whether the current device's facts are known already (no probe needed):
// then *pairs says if the split single-frame form can run on it.
bool known_frame_pairs(bool* pairs) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return false;
  }
  std::lock_guard<std::mutex> lock(g_dev_mu);
  if (!g_dev[dev].ready) return false;
  *pairs = g_dev[dev].frame_pairs;
  return true;
}

// A new nonzero value for every eager split single-frame call: the
// kernel's pair words carry it, so a word left by an earlier call never
// matches.
uint32_t next_epoch() {
  static std::atomic<uint32_t> epoch{0};
  uint32_t e = epoch.fetch_add(1) + 1;
  while (e == 0) e = epoch.fetch_add(1) + 1;
  return e;
}

// The fused kernel's launch size for a call on the current device, 0 when
// the call does not take it.  *queried is false when the device could not
// be queried (no device): callers then assume a device that hosts it.
int fused_launch(int in_dtype, const Dims& d, bool out_bf16, bool* queried) {
  *queried = true;
  if (!fused_path(in_dtype, d)) return 0;
  DevInfo* di = nullptr;
  if (dev_info(&di) != hipSuccess) {
    (void)hipGetLastError();
    *queried = false;
    return 0;
  }
  return di->fused_grid[out_bf16 ? 1 : 0];
}

// Workspace bytes of each path (D x D maps of the frames the path holds at
// once); SIZE_MAX when the path cannot take the shape.
size_t path_workspace(const Dims& d, int in_dtype, int path) {
  if (d.in_elems == 0) return 0;
  switch (path) {
    case GDN_PATH_FUSED:
      return fast_path(in_dtype, d.D) && d.T > kFusedMinT ? (size_t)gdn::fused_workspace_bytes(d.heads)
                                                          : SIZE_MAX;
    case GDN_PATH_FRAME:
      return fast_path(in_dtype, d.D) && d.T == 1 ? (size_t)gdn::frame1_workspace_bytes(d.heads) : SIZE_MAX;
    case GDN_PATH_MFMA: {
      if (!fast_path(in_dtype, d.D)) return SIZE_MAX;
      const Segments g = segments_of(d.T);
      return (size_t)(3 * g.slots) * slot_bytes(d, g);
    }
    case GDN_PATH_PLAIN:
      return 3 * round256(d.map_elems * sizeof(float));
    default:
      return SIZE_MAX;
  }
}

// ---------------------------------------------------------------------------
// schedules
// ---------------------------------------------------------------------------
// One kernel launch, bracketed by timing events when rec is set.
template <typename F>
hipError_t timed(Recorder* rec, hipStream_t st, int kind, F&& launch) {
  hipError_t e;
  if (rec && (e = rec->begin(st)) != hipSuccess) return e;
  if ((e = launch()) != hipSuccess) return e;
  return rec ? rec->end(st, kind) : hipSuccess;
}

// The MFMA path: build, state pass and output over the segments.  Segment
// i's state pass needs its own build and segment i-1's state pass; its
// output needs its own state pass.  Builds run on the caller's stream,
// state passes and outputs on the two side streams, so build(i+1),
// state(i) and output(i-1) overlap: the state pass is a chain of short
// latency-bound steps on a few CUs, while build and output stream from HBM
// on the rest.  The maps of segment i use slot i % 3 of each map buffer, so
// build(i) also waits for state(i-3) (the last reader of its G, U slot) and
// state(i) for output(i-3) (the last reader of its M slot); the workspace
// then holds three segments instead of the whole sequence.  With one
// segment everything runs on the caller's stream.
hipError_t run_mfma(const Dims& d, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const float* gamma, const float* beta, const float* state_in, float ks, void* out,
                    bool out_bf16, float* state_out, char* ws, hipStream_t s, Recorder* rec) {
  const Segments g = segments_of(d.T);
  const size_t sb = slot_bytes(d, g);
  const int S = (int)d.S;
  // map buffers of segment i: G, U and M slots, each `sb` bytes
  auto G = [&](int64_t i) { return ws + (size_t)(i % g.slots) * sb; };
  auto U = [&](int64_t i) { return reinterpret_cast<float*>(ws + (size_t)(g.slots + i % g.slots) * sb); };
  auto M = [&](int64_t i) { return ws + (size_t)(2 * g.slots + i % g.slots) * sb; };
  auto build = [&](hipStream_t st, int64_t i, int64_t t0, int64_t t1) {
    return timed(rec, st, 0, [&] {
      return gdn::launch_build_bf16_d128(k, v, G(i), true, U(i), d.heads, d.T, t0, t1, S, ks, {g.cap, t0}, st);
    });
  };
  auto state = [&](hipStream_t st, int64_t i, int64_t t0, int64_t t1) {
    return timed(rec, st, 1, [&] {
      return gdn::launch_state_d128(G(i), true, U(i), gamma, beta, t0 ? state_out : state_in, M(i), false,
                                    state_out, d.heads, d.T, t0, t1, {g.cap, t0}, st);
    });
  };
  auto output = [&](hipStream_t st, int64_t i, int64_t t0, int64_t t1) {
    return timed(rec, st, 2, [&] {
      return gdn::launch_output_bf16_d128(q, M(i), true, out, out_bf16, d.heads, d.T, t0, t1, S, {g.cap, t0}, st);
    });
  };
  hipError_t e;
  if (g.n == 1) {
    if ((e = build(s, 0, 0, d.T)) != hipSuccess) return e;
    if ((e = state(s, 0, 0, d.T)) != hipSuccess) return e;
    return output(s, 0, 0, d.T);
  }
  int dev = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_side_mu);
  Side& sd = g_side[dev];
  if ((e = side_init(sd)) != hipSuccess) return e;
  // fork: the side streams start after everything already on the caller's stream
  if ((e = hipEventRecord(sd.fork, s)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(sd.state_st, sd.fork, 0)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(sd.out_st, sd.fork, 0)) != hipSuccess) return e;
  // Each wait is enqueued after the record it refers to and before that
  // event is recorded again (three segments later), so the events are reused.
  hipError_t err = hipSuccess;
  for (int64_t i = 0; i < g.n && err == hipSuccess; ++i) {
    const int64_t t0 = i * d.T / g.n, t1 = (i + 1) * d.T / g.n;  // balanced, at most g.cap frames
    const int slot = (int)(i % kMapSlots);
    if (i >= kMapSlots && (err = hipStreamWaitEvent(s, sd.stated[slot], 0)) != hipSuccess) break;
    if ((err = build(s, i, t0, t1)) != hipSuccess) break;
    if ((err = hipEventRecord(sd.built, s)) != hipSuccess) break;
    if ((err = hipStreamWaitEvent(sd.state_st, sd.built, 0)) != hipSuccess) break;
    if (i >= kMapSlots && (err = hipStreamWaitEvent(sd.state_st, sd.output[slot], 0)) != hipSuccess) break;
    if ((err = state(sd.state_st, i, t0, t1)) != hipSuccess) break;
    if ((err = hipEventRecord(sd.stated[slot], sd.state_st)) != hipSuccess) break;
    if ((err = hipStreamWaitEvent(sd.out_st, sd.stated[slot], 0)) != hipSuccess) break;
    if ((err = output(sd.out_st, i, t0, t1)) != hipSuccess) break;
    err = hipEventRecord(sd.output[slot], sd.out_st);
  }
  // join, also after a failed launch, so the caller's stream stays ordered
  // after whatever was enqueued
  if ((e = hipEventRecord(sd.state_done, sd.state_st)) != hipSuccess) return e;
  if ((e = hipEventRecord(sd.out_done, sd.out_st)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(s, sd.state_done, 0)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(s, sd.out_done, 0)) != hipSuccess) return e;
  return err;
}

// ---------------------------------------------------------------------------
// the backward schedule
// ---------------------------------------------------------------------------
struct BwdArgs {
  const uint16_t *q, *k, *v, *d_out;
  const float *gamma, *beta, *state_in, *d_state_out;
  float *dq, *dk, *dv, *dgamma, *dbeta, *d_state_in;
  float ks;  // key scale of the forward
};
struct BwdBuffers {
  float *G, *U, *M_all, *P, *LB, *partials, *fstate;
};

// gdn_frame_bwd over min(ceil(T / F), kBwdMaxSegments) segments, on the side streams of the
// overlapped forward schedule.  First the forward is recomputed (G_t, U_t in
// the packed forms of the forward, every M_t in float32): (K, V) builds on
// the caller's stream, the state pass (a chain)
// segment by segment on the state stream, and dq = dO M per segment on the
// output stream as its states appear.  Then the reverse-time state pass
// walks the segments from the last to the first on the state stream, the
// state gradient carried through d_state_in; each segment waits for its
// P_t = dO_t^T Q_t, built on the caller's stream right after the (K, V)
// builds in the same reverse order (so the pass can start as soon as the
// forward chain ends), and its dk, dv (one kernel) follow on the output
// stream, behind the last dq.  (A third stream for them, measured,
// lets them take bandwidth from the P builds the chain waits for.)  The chains run on a few CUs while the
// builds and token contractions stream from HBM on the rest.  No kernel's
// arithmetic depends on the segmentation.  With one segment everything runs
// on the caller's stream.
hipError_t run_bwd(const Dims& d, const BwdArgs& a, const BwdBuffers& b, hipStream_t s) {
  const int64_t F = segment_frames();
  const int64_t nseg = std::min((d.T + F - 1) / F, kBwdMaxSegments);
  const int S = (int)d.S;
  const int64_t H = d.heads, T = d.T;
  auto seg = [&](int64_t i) { return std::make_pair(i * T / nseg, (i + 1) * T / nseg); };
  auto build_kv = [&](hipStream_t st, int64_t t0, int64_t t1) {
    return gdn::launch_build_bf16_d128(a.k, a.v, b.G, true, b.U, H, T, t0, t1, S, a.ks, {T, 0}, st);
  };
  // P_t = dO_t^T Q_t: the build's second map with (K, V) = (Q, dO); its first (Q^T Q) is not stored
  auto build_p = [&](hipStream_t st, int64_t t0, int64_t t1) {
    return gdn::launch_build_bf16_d128(a.q, a.d_out, nullptr, false, b.P, H, T, t0, t1, S, 1.f, {T, 0}, st);
  };
  auto state_fwd = [&](hipStream_t st, int64_t t0, int64_t t1) {
    return gdn::launch_state_d128(b.G, true, b.U, a.gamma, a.beta, t0 ? b.fstate : a.state_in, b.M_all, true,
                                  b.fstate, H, T, t0, t1, {T, 0}, st);
  };
  auto dq = [&](hipStream_t st, int64_t t0, int64_t t1) {
    return gdn::launch_output_bwd_d128(a.d_out, b.M_all, a.dq, true, H, T, t0, t1, S, st);  // dq = dO M
  };
  auto state_bwd = [&](hipStream_t st, int64_t t0, int64_t t1) {
    const float* carry = t1 == T ? a.d_state_out : a.d_state_in;
    return gdn::launch_state_bwd_d128(b.G, b.U, b.P, b.M_all, a.state_in, a.gamma, a.beta, carry, b.LB,
                                      b.partials, a.d_state_in, H, T, t0, t1, st);
  };
  auto grads = [&](hipStream_t st, int64_t t0, int64_t t1) {  // dk = V LB + K S, dv = K LB^T
    return gdn::launch_dkv_bwd_d128(a.v, a.k, b.LB, b.M_all, a.state_in, a.gamma, a.ks, a.dk, a.dv, H, T, t0, t1, S,
                                    st);
  };
  auto reduce = [&]() { return gdn::launch_bwd_reduce(b.partials, a.dgamma, a.dbeta, d.frames, s); };
  hipError_t e;
  if (nseg == 1) {
    if ((e = build_kv(s, 0, T)) != hipSuccess || (e = state_fwd(s, 0, T)) != hipSuccess ||
        (e = dq(s, 0, T)) != hipSuccess || (e = build_p(s, 0, T)) != hipSuccess || (e = state_bwd(s, 0, T)) != hipSuccess ||
        (e = grads(s, 0, T)) != hipSuccess)
      return e;
    return reduce();
  }
  int dev = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_side_mu);
  Side& sd = g_side[dev];
  if ((e = side_init(sd)) != hipSuccess) return e;
  if ((e = hipEventRecord(sd.fork, s)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(sd.state_st, sd.fork, 0)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(sd.out_st, sd.fork, 0)) != hipSuccess) return e;
  // each wait is enqueued right after the record it refers to, so the events are reused
  auto hand_off = [&](hipStream_t from, hipEvent_t ev, hipStream_t to) {
    hipError_t err = hipEventRecord(ev, from);
    return err == hipSuccess ? hipStreamWaitEvent(to, ev, 0) : err;
  };
  hipError_t err = hipSuccess;
  for (int64_t i = 0; i < nseg && err == hipSuccess; ++i) {
    const auto [t0, t1] = seg(i);
    if ((err = build_kv(s, t0, t1)) != hipSuccess) break;
    if ((err = hand_off(s, sd.built, sd.state_st)) != hipSuccess) break;
    if ((err = state_fwd(sd.state_st, t0, t1)) != hipSuccess) break;
    if ((err = hand_off(sd.state_st, sd.stated[0], sd.out_st)) != hipSuccess) break;
    err = dq(sd.out_st, t0, t1);
  }
  for (int64_t i = nseg - 1; i >= 0 && err == hipSuccess; --i) {
    const auto [t0, t1] = seg(i);
    if ((err = build_p(s, t0, t1)) != hipSuccess) break;
    if ((err = hand_off(s, sd.built, sd.state_st)) != hipSuccess) break;
    if ((err = state_bwd(sd.state_st, t0, t1)) != hipSuccess) break;
    if ((err = hand_off(sd.state_st, sd.stated[0], sd.out_st)) != hipSuccess) break;
    err = grads(sd.out_st, t0, t1);
  }
  // join, also after a failed launch, so the caller's stream stays ordered
  if ((e = hipEventRecord(sd.state_done, sd.state_st)) != hipSuccess) return e;
  if ((e = hipEventRecord(sd.out_done, sd.out_st)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(s, sd.state_done, 0)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(s, sd.out_done, 0)) != hipSuccess) return e;
  return err == hipSuccess ? reduce() : err;
}

// Gates computed from activations (gdn_frame_fwd_gated): per-token
// pre-activations a, b [B, H, T, S], per-head A_log, dt_bias [H]; the gates
// are written to gamma, beta [B, H, T].
struct GateIn {
  const float *a, *b, *A_log, *dt_bias;
  float *gamma, *beta;
};

int frame_fwd_impl(const gdn_shape* shape, int in_dtype, int out_dtype, const void* q, const void* k,
                   const void* v, const float* gamma, const float* beta, const float* state_in, float ks,
                   void* out, float* state_out, void* workspace, size_t workspace_bytes,
                   void* stream, Recorder* rec, const GateIn* gate = nullptr) {
  Dims d;
  int st = check_shape(shape, true, &d, true);
  if (st != GDN_OK) return st;
  if (!std::isfinite(ks)) return GDN_E_VALUE;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return GDN_E_DTYPE;
  // a pointer may be null exactly when its tensor has no elements
  const bool has_in = d.in_elems > 0, has_fr = d.frames > 0, has_st = d.heads > 0;
  if (gate) {
    // a frame's gates average its tokens: frames need tokens
    if (has_fr && d.S == 0) return GDN_E_SHAPE;
    if (has_fr && (!gate->a || !gate->b || !gate->A_log || !gate->dt_bias || !gate->gamma || !gate->beta))
      return GDN_E_NULLPTR;
    gamma = gate->gamma;
    beta = gate->beta;
  }
  if ((has_in && (!q || !k || !v || !out)) || (has_fr && (!gamma || !beta)) || (has_st && !state_out))
    return GDN_E_NULLPTR;
  const size_t inb = d.in_elems * dsize(in_dtype), outb = d.in_elems * dsize(out_dtype);
  const size_t stb = d.state_elems * 4, gb = (size_t)d.frames * 4;
  const size_t gab = (size_t)d.frames * (size_t)d.S * 4, parb = (size_t)d.H * 4;
  // inputs (gamma, beta only when given) and, with gates, their inputs
  const Range ins[] = {{q, inb}, {k, inb}, {v, inb}, {gate ? nullptr : gamma, gb}, {gate ? nullptr : beta, gb},
                       {state_in, state_in ? stb : 0}, {gate ? gate->a : nullptr, gab},
                       {gate ? gate->b : nullptr, gab}, {gate ? gate->A_log : nullptr, parb},
                       {gate ? gate->dt_bias : nullptr, parb}};
  // The workspace a path needs, checked on the host before anything is
  // enqueued: null, too small, misaligned or overlapping another buffer.
  auto workspace_ok = [&](size_t need, int* status) {
    if (need > 0 && (!workspace || workspace_bytes < need || (uintptr_t)workspace % 256 != 0)) {
      *status = GDN_E_WORKSPACE;
      return false;
    }
    const Range outs[] = {{out, outb}, {state_out, stb}, {workspace, need}, {gate ? gamma : nullptr, gb},
                          {gate ? beta : nullptr, gb}};
    if (!aliasing_ok(outs, 5, ins, 10, state_out, state_in)) {
      *status = GDN_E_ALIAS;
      return false;
    }
    return true;
  };
  const bool ob = out_dtype == GDN_BF16;
  const int planned = !has_in ? GDN_PATH_PLAIN
                      : fused_path(in_dtype, d) ? GDN_PATH_FUSED
                      : frame1_path(in_dtype, d) ? GDN_PATH_FRAME
                      : fast_path(in_dtype, d.D) ? GDN_PATH_MFMA
                                                 : GDN_PATH_PLAIN;
  // the planned path's workspace first, with no device query (the
  // single-frame kernel runs without one, and uses one that is big enough)
  if (!workspace_ok(has_in && planned != GDN_PATH_FRAME ? path_workspace(d, in_dtype, planned) : 0, &st)) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!has_in) {
    // no heads: nothing to do; no frames: state_out = state_in; frames
    // without tokens: G_t = U_t = 0, each step only decays the state (not
    // with computed gates, refused above)
    if (!has_st) return GDN_OK;
    if (!has_fr)
      return hip_status(timed(rec, s, 1, [&] { return gdn::launch_state_fill(state_in, state_out, d.state_elems, s); }));
    return hip_status(timed(rec, s, 1, [&] {
      return gdn::launch_decay(gamma, state_in, state_out, d.heads, d.T, (int)d.D, s);
    }));
  }
  char* ws = static_cast<char*>(workspace);
  if (planned == GDN_PATH_FUSED) {
    bool queried = true;
    const int grid = fused_launch(in_dtype, d, ob, &queried);
    if (!queried) return GDN_E_HIP;
    if (grid > 0) {
      int dev = 0;
      if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_E_HIP;
      hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
      if (hipStreamIsCapturing(s, &cap) != hipSuccess) return GDN_E_HIP;
      const bool ordered = cap == hipStreamCaptureStatusNone;
      std::lock_guard<std::mutex> lock(g_fused_mu);
      FusedOrder& fo = g_fused_order[dev];
      if (ordered && !fo.ready) {
        if (hipEventCreateWithFlags(&fo.done, hipEventDisableTiming) != hipSuccess) return GDN_E_HIP;
        fo.ready = true;
        register_teardown();
      }
      if (ordered && fo.have && fo.last != s && hipStreamWaitEvent(s, fo.done, 0) != hipSuccess) return GDN_E_HIP;
      // the gates first, into gamma, beta, which the fused kernel then reads
      // as inputs (one pass over the activations, which the state pass has
      // no slack to take on, nor the build items, the kernel's throughput)
      if (gate && timed(rec, s, 0, [&] {
            return gdn::launch_frame_gates(gate->a, gate->b, gate->A_log, gate->dt_bias, gate->gamma, gate->beta,
                                           d.frames, (int)d.H, (int)d.T, (int)d.S, s);
          }) != hipSuccess)
        return GDN_E_HIP;
      const hipError_t e = timed(rec, s, 1, [&] {
        return gdn::launch_fused(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                 static_cast<const uint16_t*>(v), gamma, beta, state_in, out, ob, state_out,
                                 workspace, d.heads, d.T, (int)d.S, ks, spin_limit().load(), grid, s);
      });
      if (e != hipSuccess) return GDN_E_HIP;
      if (ordered) {
        if (hipEventRecord(fo.done, s) != hipSuccess) return GDN_E_HIP;
        fo.last = s;
        fo.have = true;
      }
      return GDN_OK;
    }
    // this device cannot host the fused kernel: the three-kernel schedule,
    // whose workspace is larger
    if (!workspace_ok(path_workspace(d, in_dtype, GDN_PATH_MFMA), &st)) return st;
  }
  if (planned == GDN_PATH_FRAME) {
    // the token halves of a row block on two workgroups when the workspace
    // holds their hand-off (checked for overlap like any workspace) and the
    // device deals each pair of workgroups to one XCD (its one-time probe
    // runs on the null stream: not while this stream is being captured, so
    // a capture before any eager call on the device takes one workgroup per
    // block)
    void* pair_ws = nullptr;
    uint32_t epoch = 0;  // 0: the captured form of the swap
    const size_t pneed = path_workspace(d, in_dtype, GDN_PATH_FRAME);
    if (pneed > 0 && workspace && workspace_bytes >= pneed && (uintptr_t)workspace % 256 == 0) {
      if (!workspace_ok(pneed, &st)) return st;
      hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
      if (hipStreamIsCapturing(s, &cap) != hipSuccess) return GDN_E_HIP;
      const bool eager = cap == hipStreamCaptureStatusNone;
      bool pairs = false;
      if (!known_frame_pairs(&pairs) && eager) {
        DevInfo* di = nullptr;
        if (dev_info(&di) != hipSuccess) {
          (void)hipGetLastError();
          return GDN_E_HIP;
        }
        pairs = di->frame_pairs;
      }
      if (pairs) {
        pair_ws = workspace;
        if (eager) epoch = next_epoch();
      }
    }
    if (gate && timed(rec, s, 0, [&] {
          return gdn::launch_frame_gates(gate->a, gate->b, gate->A_log, gate->dt_bias, gate->gamma, gate->beta,
                                         d.frames, (int)d.H, (int)d.T, (int)d.S, s);
        }) != hipSuccess)
      return GDN_E_HIP;
    return hip_status(timed(rec, s, 1, [&] {
      return gdn::launch_frame1(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                static_cast<const uint16_t*>(v), gamma, beta, state_in, out, ob, state_out,
                                d.heads, (int)d.S, ks, pair_ws, epoch, spin_limit().load(), s);
    }));
  }
  // separate kernels: the gates first, into gamma, beta
  if (gate && timed(rec, s, 0, [&] {
        return gdn::launch_frame_gates(gate->a, gate->b, gate->A_log, gate->dt_bias, gate->gamma, gate->beta,
                                       d.frames, (int)d.H, (int)d.T, (int)d.S, s);
      }) != hipSuccess)
    return GDN_E_HIP;
  if (fast_path(in_dtype, d.D))
    return hip_status(run_mfma(d, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                               static_cast<const uint16_t*>(v), gamma, beta, state_in, ks, out, ob, state_out,
                               ws, s, rec));
  // plain path: G_t, U_t, M_t of every frame in float32
  const size_t slot = round256(d.map_elems * sizeof(float));
  float* G = reinterpret_cast<float*>(ws);
  float* U = reinterpret_cast<float*>(ws + slot);
  float* M_all = reinterpret_cast<float*>(ws + 2 * slot);
  hipError_t e;
  if ((e = timed(rec, s, 0, [&] {
         return gdn::launch_build_generic(k, v, in_dtype == GDN_BF16, G, U, d.frames, (int)d.S, (int)d.D, ks, s);
       })) != hipSuccess)
    return GDN_E_HIP;
  if ((e = timed(rec, s, 1, [&] {
         return gdn::launch_state_generic(G, U, gamma, beta, state_in, M_all, state_out, d.heads, d.T, (int)d.D, s);
       })) != hipSuccess)
    return GDN_E_HIP;
  if ((e = timed(rec, s, 2, [&] {
         return gdn::launch_output_generic(q, in_dtype == GDN_BF16, M_all, out, ob, d.frames, (int)d.S, (int)d.D,
                                           s);
       })) != hipSuccess)
    return GDN_E_HIP;
  return GDN_OK;
}

int frame_bwd_impl(const gdn_shape* shape, int in_dtype, const void* q, const void* k, const void* v,
                   const float* gamma, const float* beta, const float* state_in, float ks, const void* d_out,
                   const float* d_state_out, float* dq, float* dk, float* dv, float* dgamma, float* dbeta,
                   float* d_state_in, void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  int st = check_shape(shape, true, &d, true);
  if (st != GDN_OK) return st;
  if (!valid_dtype(in_dtype)) return GDN_E_DTYPE;
  if (in_dtype != GDN_BF16) return GDN_E_DTYPE;
  if (d.D != 128) return GDN_E_UNSUPPORTED_D;
  if (!std::isfinite(ks)) return GDN_E_VALUE;
  // a pointer may be null exactly when its tensor has no elements
  const bool has_in = d.in_elems > 0, has_fr = d.frames > 0, has_st = d.heads > 0;
  if ((has_in && (!q || !k || !v || !d_out || !dq || !dk || !dv)) ||
      (has_fr && (!gamma || !beta || !dgamma || !dbeta)) || (has_st && !d_state_in))
    return GDN_E_NULLPTR;
  const size_t need = gdn_bwd_workspace_bytes(shape, in_dtype);
  if (need > 0 && (!workspace || workspace_bytes < need || (uintptr_t)workspace % 256 != 0))
    return GDN_E_WORKSPACE;
  const size_t inb = d.in_elems * 2, gradb = d.in_elems * 4;
  const size_t stb = d.state_elems * 4, gb = (size_t)d.frames * 4;
  const Range outs[] = {{dq, gradb}, {dk, gradb}, {dv, gradb}, {dgamma, gb}, {dbeta, gb},
                        {d_state_in, stb}, {workspace, need}};
  const Range ins[] = {{q, inb}, {k, inb}, {v, inb}, {gamma, gb}, {beta, gb}, {state_in, state_in ? stb : 0},
                       {d_out, inb}, {d_state_out, d_state_out ? stb : 0}};
  if (!aliasing_ok(outs, 7, ins, 8, d_state_in, d_state_out)) return GDN_E_ALIAS;
  if (!has_in) {
    // no heads: nothing to do; no frames: d_state_in = d_state_out; frames
    // without tokens: the backward of the pure decay
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!has_st) return GDN_OK;
    if (!has_fr) return hip_status(gdn::launch_state_fill(d_state_out, d_state_in, d.state_elems, s));
    return hip_status(gdn::launch_decay_bwd(gamma, state_in, d_state_out, dgamma, dbeta, d_state_in, d.heads, d.T,
                                            (int)d.D, s));
  }

  const size_t slot = round256(d.map_elems * sizeof(float));
  char* ws = static_cast<char*>(workspace);
  BwdBuffers b;
  b.G = reinterpret_cast<float*>(ws);
  b.U = reinterpret_cast<float*>(ws + slot);
  b.M_all = reinterpret_cast<float*>(ws + 2 * slot);
  b.P = reinterpret_cast<float*>(ws + 3 * slot);
  b.LB = reinterpret_cast<float*>(ws + 4 * slot);
  b.partials = reinterpret_cast<float*>(ws + 5 * slot);
  b.fstate = reinterpret_cast<float*>(ws + 5 * slot +
                                      round256((size_t)d.frames * gdn::kBwdParts * 2 * sizeof(float)));
  const BwdArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                  static_cast<const uint16_t*>(d_out), gamma, beta, state_in, d_state_out,
                  dq, dk, dv, dgamma, dbeta, d_state_in, ks};
  return hip_status(run_bwd(d, a, b, static_cast<hipStream_t>(stream)));
}

}  // namespace

namespace gdn {
// gdn_frame_fwd on a workspace the caller provides by other means (the
// no-allocation entry point's scratch array).
int frame_fwd_in(const gdn_shape* shape, int in_dtype, int out_dtype, const void* q, const void* k, const void* v,
                 const float* gamma, const float* beta, const float* state_in, void* out, float* state_out,
                 void* workspace, size_t workspace_bytes, void* stream) {
  return frame_fwd_impl(shape, in_dtype, out_dtype, q, k, v, gamma, beta, state_in, 1.f, out, state_out, workspace,
                        workspace_bytes, stream, nullptr);
}
}  // namespace gdn

// ---------------------------------------------------------------------------
// entry points
// ---------------------------------------------------------------------------
extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_str(int s) {
  switch (s) {
    case GDN_OK: return "ok";
    case GDN_E_NULLPTR: return "a required pointer is NULL";
    case GDN_E_SHAPE: return "invalid shape (negative size, a stage call with a size of 0, too large, or overflow)";
    case GDN_E_DTYPE: return "unsupported dtype";
    case GDN_E_UNSUPPORTED_D: return "unsupported head dim (multiples of 16 up to 128)";
    case GDN_E_WORKSPACE: return "workspace missing or too small";
    case GDN_E_ALIAS: return "an output overlaps another buffer";
    case GDN_E_HIP: return "HIP runtime or launch error";
    case GDN_E_VALUE: return "an argument value is outside its domain (a non-finite key scale)";
    case GDN_E_TIMEOUT: return "an internal wait of the fused kernel ran out; frames not produced are NaN";
    case GDN_E_TOO_LARGE:
      return "the call needs more scratch memory than gdn_frame_fwd_noalloc holds (GDN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int gdn_set_fused(int enabled) { return fused_enabled().exchange(enabled ? 1 : 0); }

int gdn_set_single_frame(int enabled) { return single_frame_enabled().exchange(enabled ? 1 : 0); }

unsigned gdn_set_spin_limit(unsigned polls) { return spin_limit().exchange(polls); }

int gdn_supports_d(int64_t D) { return D >= 16 && D <= 128 && D % 16 == 0; }

int gdn_path(const gdn_shape* shape, int in_dtype) {
  Dims d;
  if (!valid_dtype(in_dtype) || check_shape(shape, true, &d, true) != GDN_OK) return -1;
  if (d.in_elems == 0) return GDN_PATH_PLAIN;
  if (fused_path(in_dtype, d)) {
    bool queried = true;
    // float32 and bf16 outputs have the same launch size
    if (fused_launch(in_dtype, d, false, &queried) > 0 || !queried) return GDN_PATH_FUSED;
  }
  if (frame1_path(in_dtype, d)) return GDN_PATH_FRAME;
  return fast_path(in_dtype, d.D) ? GDN_PATH_MFMA : GDN_PATH_PLAIN;
}

size_t gdn_path_workspace_bytes(const gdn_shape* shape, int in_dtype, int path) {
  Dims d;
  if (!valid_dtype(in_dtype) || check_shape(shape, true, &d, true) != GDN_OK) return SIZE_MAX;
  return path_workspace(d, in_dtype, path);
}

size_t gdn_workspace_bytes(const gdn_shape* shape, int in_dtype) {
  Dims d;
  if (!valid_dtype(in_dtype) || check_shape(shape, true, &d, true) != GDN_OK || d.in_elems == 0) return 0;
  if (fused_path(in_dtype, d)) {
    bool queried = true;
    const int grid = fused_launch(in_dtype, d, false, &queried);
    // no device to ask: what the three-kernel schedule needs, the larger
    return path_workspace(d, in_dtype, grid > 0 ? GDN_PATH_FUSED : GDN_PATH_MFMA);
  }
  if (frame1_path(in_dtype, d)) return path_workspace(d, in_dtype, GDN_PATH_FRAME);
  return path_workspace(d, in_dtype, fast_path(in_dtype, d.D) ? GDN_PATH_MFMA : GDN_PATH_PLAIN);
}

int gdn_attn_fwd(const gdn_shape* shape, int in_dtype, const gdn_attn_layout* layout, const void* q, const void* k,
                 const void* v, float* out, float* lse, void* stream) {
  if (!shape || !layout) return GDN_E_NULLPTR;
  const int64_t B = shape->B, H = shape->H, T = shape->T, S = shape->S, D = shape->D;
  if (B < 0 || H < 0 || T < 0 || S < 0) return GDN_E_SHAPE;
  if (!valid_dtype(in_dtype)) return GDN_E_DTYPE;
  if (D != 128) return GDN_E_UNSUPPORTED_D;
  if (in_dtype != GDN_BF16) return GDN_E_DTYPE;
  const gdn_attn_layout& L = *layout;
  if (L.sink < 0 || L.first_chunk < 1 || L.chunk < 1 || L.window < 1) return GDN_E_VALUE;
  int64_t heads, tokens, elems;
  if (!mul_ok(B, H, &heads) || !mul_ok(T, S, &tokens) || tokens >= (int64_t{1} << 30)) return GDN_E_SHAPE;
  if (!mul_ok(heads, tokens, &elems) || elems > (int64_t{1} << 40)) return GDN_E_SHAPE;
  if (elems == 0) return GDN_OK;
  if (!q || !k || !v || !out) return GDN_E_NULLPTR;
  const size_t inb = (size_t)elems * D * 2, outb = (size_t)elems * D * 4, lseb = (size_t)elems * 4;
  const Range outs[] = {{out, outb}, {lse, lse ? lseb : 0}};
  const Range ins[] = {{q, inb}, {k, inb}, {v, inb}};
  if (!aliasing_ok(outs, 2, ins, 3)) return GDN_E_ALIAS;
  // layout fields beyond T frames change nothing; clamp them into int range
  auto clampT = [&](int64_t x) { return (int)(x < T + 1 ? x : T + 1); };
  return hip_status(gdn::launch_attn_d128(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                          static_cast<const uint16_t*>(v), out, lse, heads, (int)T, (int)S,
                                          clampT(L.sink), clampT(L.first_chunk), clampT(L.chunk), clampT(L.window),
                                          static_cast<hipStream_t>(stream)));
}

int gdn_fused_status(const void* workspace, void* stream) {
  if (!workspace) return GDN_E_NULLPTR;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t word = 0;
  if (hipMemcpyAsync(&word, gdn::fused_error_word(workspace), sizeof word, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return GDN_E_HIP;
  return word == 0 ? GDN_OK : GDN_E_TIMEOUT;
}

int gdn_build_maps(const gdn_shape* shape, int in_dtype, const void* k, const void* v, float* G,
                   float* U, void* stream) {
  Dims d;
  int st = check_shape(shape, true, &d);
  if (st != GDN_OK) return st;
  if (!valid_dtype(in_dtype)) return GDN_E_DTYPE;
  if (!k || !v || !G || !U) return GDN_E_NULLPTR;
  const size_t inb = d.in_elems * dsize(in_dtype), mapb = d.map_elems * 4;
  const Range outs[] = {{G, mapb}, {U, mapb}};
  const Range ins[] = {{k, inb}, {v, inb}};
  if (!aliasing_ok(outs, 2, ins, 2)) return GDN_E_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fast_path(in_dtype, d.D))
    return hip_status(gdn::launch_build_bf16_d128(static_cast<const uint16_t*>(k),
                                                  static_cast<const uint16_t*>(v), G, false, U,
                                                  d.heads, d.T, 0, d.T, (int)d.S, 1.f, {d.T, 0}, s));
  return hip_status(gdn::launch_build_generic(k, v, in_dtype == GDN_BF16, G, U, d.frames, (int)d.S,
                                              (int)d.D, 1.f, s));
}

int gdn_state_pass(const gdn_shape* shape, const float* G, const float* U, const float* gamma,
                   const float* beta, const float* state_in, float* M_all, float* state_out,
                   void* stream) {
  Dims d;
  int st = check_shape(shape, false, &d);
  if (st != GDN_OK) return st;
  if (!G || !U || !gamma || !beta || !state_out) return GDN_E_NULLPTR;
  const size_t mapb = d.map_elems * 4, stb = d.state_elems * 4, gb = (size_t)d.frames * 4;
  const Range outs[] = {{M_all, M_all ? mapb : 0}, {state_out, stb}};
  const Range ins[] = {{G, mapb}, {U, mapb}, {gamma, gb}, {beta, gb}, {state_in, state_in ? stb : 0}};
  if (!aliasing_ok(outs, 2, ins, 5, state_out, state_in)) return GDN_E_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d.D == 128)
    return hip_status(gdn::launch_state_d128(G, false, U, gamma, beta, state_in, M_all, true, state_out,
                                             d.heads, d.T, 0, d.T, {d.T, 0}, s));
  return hip_status(gdn::launch_state_generic(G, U, gamma, beta, state_in, M_all, state_out,
                                              d.heads, d.T, (int)d.D, s));
}

int gdn_output(const gdn_shape* shape, int in_dtype, int out_dtype, const void* q,
               const float* M_all, void* out, void* stream) {
  Dims d;
  int st = check_shape(shape, true, &d);
  if (st != GDN_OK) return st;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return GDN_E_DTYPE;
  if (!q || !M_all || !out) return GDN_E_NULLPTR;
  const size_t inb = d.in_elems * dsize(in_dtype), outb = d.in_elems * dsize(out_dtype);
  const Range outs[] = {{out, outb}};
  const Range ins[] = {{q, inb}, {M_all, d.map_elems * 4}};
  if (!aliasing_ok(outs, 1, ins, 2)) return GDN_E_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool ob = out_dtype == GDN_BF16;
  if (fast_path(in_dtype, d.D))
    return hip_status(gdn::launch_output_bf16_d128(static_cast<const uint16_t*>(q), M_all, false, out,
                                                   ob, d.heads, d.T, 0, d.T, (int)d.S, {d.T, 0}, s));
  return hip_status(gdn::launch_output_generic(q, in_dtype == GDN_BF16, M_all, out, ob, d.frames,
                                               (int)d.S, (int)d.D, s));
}

int gdn_frame_fwd(const gdn_shape* shape, int in_dtype, int out_dtype, const void* q, const void* k,
                  const void* v, const float* gamma, const float* beta, const float* state_in,
                  void* out, float* state_out, void* workspace, size_t workspace_bytes,
                  void* stream) {
  return frame_fwd_impl(shape, in_dtype, out_dtype, q, k, v, gamma, beta, state_in, 1.f, out, state_out,
                        workspace, workspace_bytes, stream, nullptr);
}

int gdn_frame_fwd_ks(const gdn_shape* shape, int in_dtype, int out_dtype, const void* q, const void* k,
                     const void* v, const float* gamma, const float* beta, const float* state_in, float key_scale,
                     void* out, float* state_out, void* workspace, size_t workspace_bytes, void* stream) {
  return frame_fwd_impl(shape, in_dtype, out_dtype, q, k, v, gamma, beta, state_in, key_scale, out, state_out,
                        workspace, workspace_bytes, stream, nullptr);
}

int gdn_frame_fwd_gated(const gdn_shape* shape, int in_dtype, int out_dtype, const void* q, const void* k,
                        const void* v, const float* gate_a, const float* gate_b, const float* A_log,
                        const float* dt_bias, const float* state_in, float key_scale, void* out, float* state_out,
                        float* gamma, float* beta, void* workspace, size_t workspace_bytes, void* stream) {
  const GateIn g{gate_a, gate_b, A_log, dt_bias, gamma, beta};
  return frame_fwd_impl(shape, in_dtype, out_dtype, q, k, v, nullptr, nullptr, state_in, key_scale, out, state_out,
                        workspace, workspace_bytes, stream, nullptr, &g);
}

int gdn_frame_fwd_timed(const gdn_shape* shape, int in_dtype, int out_dtype, const void* q,
                        const void* k, const void* v, const float* gamma, const float* beta,
                        const float* state_in, void* out, float* state_out, void* workspace,
                        size_t workspace_bytes, void* stream, float* kernel_ms, int* launches) {
  if (!kernel_ms || !launches) return GDN_E_NULLPTR;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_E_HIP;
  std::lock_guard<std::mutex> lock(g_timing_mu);
  Recorder rec{&g_timing_pool[dev], {}};
  const int st = frame_fwd_impl(shape, in_dtype, out_dtype, q, k, v, gamma, beta, state_in, 1.f, out,
                                state_out, workspace, workspace_bytes, stream, &rec);
  if (st != GDN_OK) return st;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return GDN_E_HIP;
  for (int i = 0; i < 3; ++i) {
    kernel_ms[i] = 0.f;
    launches[i] = 0;
  }
  for (size_t i = 0; i < rec.kind.size(); ++i) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, (*rec.pool)[2 * i], (*rec.pool)[2 * i + 1]) != hipSuccess) return GDN_E_HIP;
    kernel_ms[rec.kind[i]] += ms;
    launches[rec.kind[i]] += 1;
  }
  return GDN_OK;
}

size_t gdn_bwd_workspace_bytes(const gdn_shape* shape, int in_dtype) {
  Dims d;
  if (!valid_dtype(in_dtype) || check_shape(shape, true, &d, true) != GDN_OK || d.in_elems == 0) return 0;
  // G, U (packed forms), M_all, P and LB (float32), then the dgamma/dbeta
  // partial sums and the recomputed final state
  return 5 * round256(d.map_elems * sizeof(float)) +
         round256((size_t)d.frames * gdn::kBwdParts * 2 * sizeof(float)) +
         round256(d.state_elems * sizeof(float));
}


int gdn_frame_bwd(const gdn_shape* shape, int in_dtype, const void* q, const void* k, const void* v,
                  const float* gamma, const float* beta, const float* state_in, const void* d_out,
                  const float* d_state_out, float* dq, float* dk, float* dv, float* dgamma, float* dbeta,
                  float* d_state_in, void* workspace, size_t workspace_bytes, void* stream) {
  return frame_bwd_impl(shape, in_dtype, q, k, v, gamma, beta, state_in, 1.f, d_out, d_state_out, dq, dk, dv,
                        dgamma, dbeta, d_state_in, workspace, workspace_bytes, stream);
}

int gdn_frame_bwd_ks(const gdn_shape* shape, int in_dtype, const void* q, const void* k, const void* v,
                     const float* gamma, const float* beta, const float* state_in, float key_scale,
                     const void* d_out, const float* d_state_out, float* dq, float* dk, float* dv, float* dgamma,
                     float* dbeta, float* d_state_in, void* workspace, size_t workspace_bytes, void* stream) {
  return frame_bwd_impl(shape, in_dtype, q, k, v, gamma, beta, state_in, key_scale, d_out, d_state_out, dq, dk,
                        dv, dgamma, dbeta, d_state_in, workspace, workspace_bytes, stream);
}

}  // extern "C"
