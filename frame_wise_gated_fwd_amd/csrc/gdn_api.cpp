// C ABI of the frame-wise GDN forward: argument validation, workspace layout
// and dispatch to the HIP kernels.  Declarations and the contract are in
// include/gdn.h.
#include "gdn.h"

#include <hip/hip_runtime.h>

#include <limits>
#include <mutex>

#include "gdn_launch.h"

namespace {

constexpr int64_t kMaxFrames = (int64_t{1} << 24) - 1;  // B*H*T: one workgroup per frame

struct Dims {
  int64_t B, H, T, S, D;
  int64_t heads, frames;
  size_t in_elems, state_elems, map_elems;  // per tensor
};

bool mul_ok(int64_t a, int64_t b, int64_t* r) {
  if (a <= 0 || b <= 0) return false;
  if (a > std::numeric_limits<int64_t>::max() / b) return false;
  *r = a * b;
  return true;
}

bool valid_dtype(int d) { return d == GDN_F32 || d == GDN_BF16; }
size_t dsize(int d) { return d == GDN_BF16 ? 2 : 4; }

// Validates the shape; use_s selects whether S takes part.
int check_shape(const gdn_shape* s, bool use_s, Dims* out) {
  if (!s) return GDN_E_NULLPTR;
  Dims d{};
  d.B = s->B;
  d.H = s->H;
  d.T = s->T;
  d.S = use_s ? s->S : 1;
  d.D = s->D;
  if (d.B < 1 || d.H < 1 || d.T < 1 || d.S < 1 || d.D < 1) return GDN_E_SHAPE;
  if (!gdn_supports_d(d.D)) return GDN_E_UNSUPPORTED_D;
  if (d.S > std::numeric_limits<int>::max() / 256) return GDN_E_SHAPE;
  int64_t heads, frames, tmp;
  if (!mul_ok(d.B, d.H, &heads) || !mul_ok(heads, d.T, &frames)) return GDN_E_SHAPE;
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

bool pipelined(int in_dtype, const Dims& d) {
  return fast_path(in_dtype, d.D) && gdn::pipeline_supported(d.heads, d.S);
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

int hip_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_E_HIP; }

size_t round256(size_t x) { return (x + 255) & ~size_t{255}; }

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_str(int s) {
  switch (s) {
    case GDN_OK: return "ok";
    case GDN_E_NULLPTR: return "a required pointer is NULL";
    case GDN_E_SHAPE: return "invalid shape (size < 1, too large, or overflow)";
    case GDN_E_DTYPE: return "unsupported dtype";
    case GDN_E_UNSUPPORTED_D: return "unsupported head dim (multiples of 16 up to 128)";
    case GDN_E_WORKSPACE: return "workspace missing or too small";
    case GDN_E_ALIAS: return "an output overlaps another buffer";
    case GDN_E_HIP: return "HIP runtime or launch error";
    default: return "unknown status";
  }
}

int gdn_supports_d(int64_t D) { return D >= 16 && D <= 128 && D % 16 == 0; }

int gdn_path(const gdn_shape* shape, int in_dtype) {
  Dims d;
  if (!valid_dtype(in_dtype) || check_shape(shape, true, &d) != GDN_OK) return -1;
  if (pipelined(in_dtype, d)) return GDN_PATH_PIPELINED;
  return fast_path(in_dtype, d.D) ? GDN_PATH_MFMA : GDN_PATH_PLAIN;
}

size_t gdn_workspace_bytes(const gdn_shape* shape, int in_dtype) {
  Dims d;
  if (!valid_dtype(in_dtype) || check_shape(shape, true, &d) != GDN_OK) return 0;
  if (pipelined(in_dtype, d)) return round256((size_t)gdn::pipeline_workspace_bytes(d.heads));
  return 3 * round256(d.map_elems * sizeof(float));
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
                                                  d.frames, (int)d.S, s));
  return hip_status(gdn::launch_build_generic(k, v, in_dtype == GDN_BF16, G, U, d.frames, (int)d.S,
                                              (int)d.D, s));
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
    return hip_status(gdn::launch_state_d128(G, false, U, gamma, beta, state_in, M_all, state_out,
                                             d.heads, d.T, s));
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
                                                   ob, d.frames, (int)d.S, s));
  return hip_status(gdn::launch_output_generic(q, in_dtype == GDN_BF16, M_all, out, ob, d.frames,
                                               (int)d.S, (int)d.D, s));
}

namespace {

// Events for gdn_frame_fwd_timed, one set per device, created on first use.
constexpr int kMaxDevices = 64;
hipEvent_t g_events[kMaxDevices][4];
bool g_events_ready[kMaxDevices];
std::mutex g_events_mu;

int frame_fwd_impl(const gdn_shape* shape, int in_dtype, int out_dtype, const void* q, const void* k,
                   const void* v, const float* gamma, const float* beta, const float* state_in,
                   void* out, float* state_out, void* workspace, size_t workspace_bytes,
                   void* stream, hipEvent_t* ev);

}  // namespace

int gdn_frame_fwd(const gdn_shape* shape, int in_dtype, int out_dtype, const void* q, const void* k,
                  const void* v, const float* gamma, const float* beta, const float* state_in,
                  void* out, float* state_out, void* workspace, size_t workspace_bytes,
                  void* stream) {
  return frame_fwd_impl(shape, in_dtype, out_dtype, q, k, v, gamma, beta, state_in, out, state_out,
                        workspace, workspace_bytes, stream, nullptr);
}

int gdn_frame_fwd_timed(const gdn_shape* shape, int in_dtype, int out_dtype, const void* q,
                        const void* k, const void* v, const float* gamma, const float* beta,
                        const float* state_in, void* out, float* state_out, void* workspace,
                        size_t workspace_bytes, void* stream, float* kernel_ms) {
  if (!kernel_ms) return GDN_E_NULLPTR;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_E_HIP;
  {
    std::lock_guard<std::mutex> lock(g_events_mu);
    if (!g_events_ready[dev]) {
      for (int i = 0; i < 4; ++i)
        if (hipEventCreate(&g_events[dev][i]) != hipSuccess) return GDN_E_HIP;
      g_events_ready[dev] = true;
    }
  }
  hipEvent_t* ev = g_events[dev];
  const int st = frame_fwd_impl(shape, in_dtype, out_dtype, q, k, v, gamma, beta, state_in, out,
                                state_out, workspace, workspace_bytes, stream, ev);
  if (st != GDN_OK) return st;
  if (hipEventSynchronize(ev[3]) != hipSuccess) return GDN_E_HIP;
  for (int i = 0; i < 3; ++i)
    if (hipEventElapsedTime(&kernel_ms[i], ev[i], ev[i + 1]) != hipSuccess) return GDN_E_HIP;
  return GDN_OK;
}

namespace {

int frame_fwd_impl(const gdn_shape* shape, int in_dtype, int out_dtype, const void* q, const void* k,
                   const void* v, const float* gamma, const float* beta, const float* state_in,
                   void* out, float* state_out, void* workspace, size_t workspace_bytes,
                   void* stream, hipEvent_t* ev) {
  Dims d;
  int st = check_shape(shape, true, &d);
  if (st != GDN_OK) return st;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return GDN_E_DTYPE;
  if (!q || !k || !v || !gamma || !beta || !out || !state_out) return GDN_E_NULLPTR;
  const size_t need = gdn_workspace_bytes(shape, in_dtype);
  if (!workspace || workspace_bytes < need) return GDN_E_WORKSPACE;
  if ((uintptr_t)workspace % 256 != 0) return GDN_E_WORKSPACE;
  const size_t inb = d.in_elems * dsize(in_dtype), outb = d.in_elems * dsize(out_dtype);
  const size_t stb = d.state_elems * 4, gb = (size_t)d.frames * 4;
  const Range outs[] = {{out, outb}, {state_out, stb}, {workspace, need}};
  const Range ins[] = {{q, inb}, {k, inb}, {v, inb}, {gamma, gb}, {beta, gb},
                       {state_in, state_in ? stb : 0}};
  if (!aliasing_ok(outs, 3, ins, 6, state_out, state_in)) return GDN_E_ALIAS;

  if (pipelined(in_dtype, d)) {
    const int cus = device_cus();
    if (cus <= 0) return GDN_E_HIP;
    return hip_status(gdn::launch_pipeline(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
        gamma, beta, state_in, out, out_dtype == GDN_BF16, state_out, workspace, d.heads, d.T, (int)d.S, cus,
        static_cast<hipStream_t>(stream), ev));
  }
  // Workspace: G_t, U_t, M_t of every frame (packed forms on the MFMA path).
  const size_t slot = round256(d.map_elems * sizeof(float));
  char* ws = static_cast<char*>(workspace);
  void* G = ws;
  float* U = reinterpret_cast<float*>(ws + slot);
  void* M_all = ws + 2 * slot;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fast = fast_path(in_dtype, d.D);
  const bool ob = out_dtype == GDN_BF16;
  hipError_t e;
  if (ev && hipEventRecord(ev[0], s) != hipSuccess) return GDN_E_HIP;
  if (fast)
    e = gdn::launch_build_bf16_d128(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                                    G, true, U, d.frames, (int)d.S, s);
  else
    e = gdn::launch_build_generic(k, v, in_dtype == GDN_BF16, static_cast<float*>(G), U, d.frames,
                                  (int)d.S, (int)d.D, s);
  if (e != hipSuccess) return GDN_E_HIP;
  if (ev && hipEventRecord(ev[1], s) != hipSuccess) return GDN_E_HIP;
  if (fast)
    e = gdn::launch_state_d128(G, true, U, gamma, beta, state_in, M_all, state_out, d.heads, d.T, s);
  else
    e = gdn::launch_state_generic(static_cast<float*>(G), U, gamma, beta, state_in,
                                  static_cast<float*>(M_all), state_out, d.heads, d.T, (int)d.D, s);
  if (e != hipSuccess) return GDN_E_HIP;
  if (ev && hipEventRecord(ev[2], s) != hipSuccess) return GDN_E_HIP;
  if (fast)
    e = gdn::launch_output_bf16_d128(static_cast<const uint16_t*>(q), M_all, true, out, ob, d.frames,
                                     (int)d.S, s);
  else
    e = gdn::launch_output_generic(q, in_dtype == GDN_BF16, static_cast<float*>(M_all), out, ob,
                                   d.frames, (int)d.S, (int)d.D, s);
  if (e != hipSuccess) return GDN_E_HIP;
  if (ev && hipEventRecord(ev[3], s) != hipSuccess) return GDN_E_HIP;
  return GDN_OK;
}

}  // namespace

}  // extern "C"
