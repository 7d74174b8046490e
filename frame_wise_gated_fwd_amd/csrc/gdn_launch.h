// Internal launchers (host side).  Arguments are validated by gdn_api.cpp
// before any of these is called; each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

// ---- MFMA path: bf16 inputs, D == 128 --------------------------------------
// The per-frame matrices G_t, U_t, M_t pass between the three kernels either
// as float32 row-major (the stage entry points) or "packed" (gdn_packed.h:
// G_t and M_t as bf16 hi/lo pairs, all three in the order the consumer's
// waves read them), which is what gdn_frame_fwd uses.  Every per-frame array
// is laid out [head][T]; each launcher covers frames [t0, t1) of every head.
//
// Where a launch's per-frame maps live: frame t of head h is map slot
// h * T + (t - t0) of the map buffers (T: frames per head in the buffers).
// The whole-sequence layout is {T, 0}; the segmented schedule keeps one
// segment per buffer, {frames per segment, first frame of the segment}.
struct MapLayout {
  int64_t T, t0;
};

// Launches of at most this many frames (heads x frames in the range) take the
// small-launch variants: a build that splits each frame's output rows over
// four workgroups and an output that splits each frame's tokens over several
// workgroups.  Both give bit-identical results to the full-size variants.
constexpr int64_t kFewFrames = 128;

// ks^2 K_t^T K_t and ks V_t^T K_t for frames [t0, t1) (ks: the key scale,
// 1 for none); packed_out selects the packed forms, else float32 row-major,
// where G may be null.
hipError_t launch_build_bf16_d128(const uint16_t* k, const uint16_t* v, void* G, bool packed_out,
                                  float* U, int64_t heads, int64_t T, int64_t t0, int64_t t1, int S, float ks,
                                  MapLayout ml, hipStream_t st);
// State pass over frames [t0, t1) for `heads` heads, starting from state_in
// (M_{t0-1}; null = zero) and leaving M_{t1-1} in state_out (which may equal
// state_in).  G and U are both packed or both float32; M_out (may be null)
// is float32 when m_f32, else packed (only with packed G and U).
hipError_t launch_state_d128(const void* G, bool packed, const float* U, const float* gamma,
                             const float* beta, const float* state_in, void* M_out, bool m_f32,
                             float* state_out, int64_t heads, int64_t T, int64_t t0, int64_t t1,
                             MapLayout ml, hipStream_t st);
// O_t = Q_t M_t^T for frames [t0, t1); out_bf16 selects the output dtype.
hipError_t launch_output_bf16_d128(const uint16_t* q, const void* M_all, bool packed_m, void* out,
                                   bool out_bf16, int64_t heads, int64_t T, int64_t t0, int64_t t1, int S,
                                   MapLayout ml, hipStream_t st);

// Token parts per frame for a launch of `frames` frames (1 unless the launch
// is small); the parts only split the tokens, not any reduction.
int token_split(int64_t frames, int S);

// ---- gates from activations (k_gate.hip, frame_gate.h) --------------------
// gamma, beta [frames] of every frame of [B, H, T] from the per-token gate
// pre-activations a, b [frames, S] and the per-head A_log, dt_bias [H].
hipError_t launch_frame_gates(const float* a, const float* b, const float* A_log, const float* dt_bias, float* gamma,
                              float* beta, int64_t frames, int H, int T, int S, hipStream_t st);

// ---- fused MFMA path: the three stages in one persistent kernel -------------
// bf16, D == 128.  Heads go in groups of at most 16, one launch (plus a
// tiny flag reset) per group.  fused_grid returns the launch size
// (workgroups resident at once on num_cus CUs) or 0 when the device cannot
// host the kernel's roles.  The workspace holds a control block, per-head
// flags and per-head rings (fused_workspace_bytes).  spin_limit: polls
// before an internal wait gives up (0: the default, a few seconds).
int64_t fused_workspace_bytes(int64_t heads);
int fused_grid(bool out_bf16, int num_cus);
// One-time check that a launch of `grid` workgroups is dealt evenly over
// eight XCDs with XCC_IDs 0-7 (a probe kernel on the null stream; waits).
hipError_t fused_topology_ok(int grid, bool* ok);
// Device address of the error word of the last fused launch that used this
// workspace (0: every wait completed).
const void* fused_error_word(const void* workspace);
hipError_t launch_fused(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* gamma,
                        const float* beta, const float* state_in, void* out, bool out_bf16,
                        float* state_out, void* workspace, int64_t heads, int64_t T, int S, float ks,
                        uint32_t spin_limit, int grid, hipStream_t st);

// ---- single frame (k_frame1.hip): T == 1, bf16, D == 128 -----------------
// One launch on `st`: every 16-row block of a head's M' (written to
// state_out) and the same 16 columns of O = Q M'^T.  With pair_ws (at least
// frame1_workspace_bytes(heads) bytes, 256-byte aligned; nonzero only for
// at most 16 heads) on a device where frame1_pairs_share_xcd holds, each
// row block's tokens split over two workgroups that swap partial sums
// through pair_ws (epoch: nonzero and new for every eager call, 0 for a
// call under stream capture);
// otherwise one workgroup per row block.  The two forms agree to float32
// rounding.  spin_limit: polls of the swap's bounded wait (0: the default,
// about a second); a workgroup whose wait runs out writes NaN to its output
// columns.
int64_t frame1_workspace_bytes(int64_t heads);
// Whether this device deals workgroups b and b + 8 to one XCD, which the
// split form needs (a one-time probe; null stream, synchronous).
hipError_t frame1_pairs_share_xcd(bool* ok);
hipError_t launch_frame1(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* gamma,
                         const float* beta, const float* state_in, void* out, bool out_bf16, float* state_out,
                         int64_t heads, int S, float ks, void* pair_ws, uint32_t epoch, uint32_t spin_limit,
                         hipStream_t st);

// ---- plain float32 path: any supported D, f32 or bf16 inputs ---------------
hipError_t launch_build_generic(const void* k, const void* v, bool in_bf16, float* G, float* U,
                                int64_t frames, int S, int D, float ks, hipStream_t st);
hipError_t launch_state_generic(const float* G, const float* U, const float* gamma,
                                const float* beta, const float* state_in, float* M_all,
                                float* state_out, int64_t heads, int64_t T, int D,
                                hipStream_t st);
hipError_t launch_output_generic(const void* q, bool in_bf16, const float* M_all, void* out,
                                 bool out_bf16, int64_t frames, int S, int D, hipStream_t st);

// ---- degenerate shapes (k_empty.hip), float32, any supported D ------------
// dst = src (n floats), or zeros when src is null; nothing when src == dst.
hipError_t launch_state_fill(const float* src, float* dst, int64_t n, hipStream_t st);
// Frames without tokens (S = 0): M_t = gamma_t M_{t-1} over T frames per
// head; state_out may equal state_in (null = zero).
hipError_t launch_decay(const float* gamma, const float* state_in, float* state_out, int64_t heads, int64_t T,
                        int D, hipStream_t st);
// Its backward for the loss <d_state_out, state_out>: dgamma, dbeta [heads, T]
// and d_state_in (may equal d_state_out; either state may be null = zero).
hipError_t launch_decay_bwd(const float* gamma, const float* state_in, const float* d_state_out, float* dgamma,
                            float* dbeta, float* d_state_in, int64_t heads, int64_t T, int D, hipStream_t st);

// ---- softmax attention with sinks and a local window (k_attn.hip) ---------
// bf16, D == 128; heads * (T * S) tokens; out float32, lse float32 or null.
hipError_t launch_attn_d128(const uint16_t* q, const uint16_t* k, const uint16_t* v, float* out, float* lse,
                            int64_t heads, int T, int S, int sink, int first_chunk, int chunk, int window,
                            hipStream_t st);

// ---- gdn_api.cpp ------------------------------------------------------------
// gdn_frame_fwd's whole call on a caller-provided workspace (see gdn.h).
int frame_fwd_in(const gdn_shape* shape, int in_dtype, int out_dtype, const void* q, const void* k,
                 const void* v, const float* gamma, const float* beta, const float* state_in, void* out,
                 float* state_out, void* workspace, size_t workspace_bytes, void* stream);

}  // namespace gdn
