/*
 * gdn.h -- C ABI of the frame-wise Gated DeltaNet forward (and its backward
 * pass) on AMD Instinct MI355X (gfx950).
 *
 * What is computed.  The SANA-WM pages ("SANA-WM: NVIDIA puts a one-minute
 * world model on a single GPU", zhichai.net, section "1. Hybrid Linear
 * Attention -- Gated DeltaNet + Softmax") describe a recurrent state of
 * constant D x D size per head, a learned decay scalar gamma that multiplies
 * the previous state, a delta-rule strength beta that corrects only the
 * residual between prediction and target, and keys scaled by 1/sqrt(D*S).
 * bilibili cv49203711 (fourth key point) makes the recurrence frame-wise: one
 * step consumes a whole latent frame of S tokens.  This library implements,
 * per batch b, head h and frame t (K_t, V_t, Q_t are S x D):
 *
 *     G_t = K_t^T K_t                  (key x key)
 *     U_t = V_t^T K_t                  (value x key)
 *     M_t = M_{t-1} gamma_t (I - beta_t G_t) + beta_t U_t
 *     O_t = Q_t M_t^T
 *
 * with M_0 = state_in (zeros when NULL) and state_out = M_T.  gdn_frame_fwd
 * applies no key scaling: the caller passes keys already multiplied by
 * 1/sqrt(D*S).  gdn_frame_fwd_ks takes the scale as an argument instead and
 * applies it inside the build of G_t and U_t (keys as given, unscaled).
 *
 * Layout.  All tensors are dense, row-major, innermost index last:
 *     q, k, v, out   [B, H, T, S, D]
 *     gamma, beta    [B, H, T]          float32
 *     state_in/out   [B, H, D, D]       float32, state[b,h,i,j]: i value, j key
 *     G, U, M_all    [B, H, T, D, D]    float32 (stage entry points)
 *
 * Pointers.  Every tensor pointer is a device pointer owned by the caller.
 * The library allocates no device memory and keeps no per-call state; the
 * workspace is caller-provided.  `stream` is a hipStream_t (NULL: the null
 * stream).  Calls are asynchronous on that stream.
 *
 * Errors.  Argument errors are detected on the host before anything is
 * enqueued and returned synchronously; nothing is written then.  A failed
 * launch returns GDN_E_HIP.  Faults during execution surface at the caller's
 * next synchronisation.  Non-finite inputs are not checked: they propagate.
 *
 * Aliasing.  state_out may equal state_in exactly (in-place streaming), and
 * in gdn_frame_bwd d_state_in may equal d_state_out.  Any other overlap
 * between an output and any other buffer is GDN_E_ALIAS.
 *
 * Empty shapes.  gdn_frame_fwd, gdn_frame_bwd (and their _ks and _timed
 * forms) accept B, H, T or S of 0; a pointer may then be NULL exactly when
 * its tensor has no elements, and no workspace is needed (the workspace
 * queries return 0).  With B*H = 0 nothing is done.  With T = 0 no step is
 * taken: state_out = state_in (zeros when NULL), and in the backward
 * d_state_in = d_state_out.  With S = 0 every frame has G_t = U_t = 0, so
 * M_t = gamma_t M_{t-1} (one float32 product per frame); the backward then
 * gives dbeta = 0, dgamma_t = (prod_{u != t} gamma_u) <d_state_out,
 * state_in> and d_state_in = (prod_u gamma_u) d_state_out.  The stage entry
 * points (gdn_build_maps, gdn_state_pass, gdn_output) need every size >= 1.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 3

typedef enum {
  GDN_OK = 0,
  GDN_E_NULLPTR = 1,        /* a required pointer is NULL                     */
  GDN_E_SHAPE = 2,          /* a size is negative (or 0 in a stage call), too
                               large, or overflows 64 bits                    */
  GDN_E_DTYPE = 3,          /* unknown or unsupported dtype                   */
  GDN_E_UNSUPPORTED_D = 4,  /* head dim not one of the supported sizes        */
  GDN_E_WORKSPACE = 5,      /* workspace NULL or smaller than required        */
  GDN_E_ALIAS = 6,          /* an output overlaps another buffer              */
  GDN_E_HIP = 7,            /* a HIP runtime call or launch failed            */
  GDN_E_VALUE = 8,          /* an argument value is outside its domain        */
  GDN_E_TIMEOUT = 9,        /* gdn_fused_status: an internal wait of the fused
                               kernel ran out (see gdn_set_spin_limit)        */
  GDN_E_TOO_LARGE = 10      /* gdn_frame_fwd_noalloc: the call needs more
                               scratch than GDN_NOALLOC_SCRATCH_BYTES         */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef struct {
  int64_t B, H, T, S, D;
} gdn_shape;

/* ABI version (GDN_ABI_VERSION of the built library). */
int gdn_abi_version(void);

/* Static, human-readable name of a status code; never NULL. */
const char* gdn_status_str(int status);

/* Supported head dims: D in {16, 32, 48, ..., 128} (multiples of 16 up to
 * 128).  bf16 inputs with D == 128 take the MFMA path; every other
 * combination takes a plain float32 path. */
int gdn_supports_d(int64_t D);

/*
 * Enables (nonzero) or disables (0) the fused kernel (GDN_PATH_FUSED below)
 * for calls made after it returns, process-wide; returns the previous
 * setting.  The default is enabled unless the environment variable
 * GDN_FUSED is 0 when the library first needs the setting.  Both paths give
 * bit-identical results; the switch exists for comparison and testing.
 */
int gdn_set_fused(int enabled);

/*
 * Enables (nonzero) or disables (0) the single-frame kernels
 * (GDN_PATH_FRAME below) for calls made after it returns, process-wide;
 * returns the previous setting.  The default is enabled unless the
 * environment variable GDN_SINGLE_FRAME is 0 when the library first needs
 * the setting.  They sum a frame's tokens in another order than the other
 * paths, so a single-frame call agrees with the first frame of a longer call
 * to float32 rounding; disabled, single-frame calls take GDN_PATH_MFMA and
 * reproduce a longer call over the same frames bit for bit.
 */
int gdn_set_single_frame(int enabled);

/*
 * Testing aid for the failure paths of the kernels that wait on other
 * workgroups: the number of polls after which one of their waits gives up,
 * for launches made after it returns, process-wide; 0 restores each
 * kernel's default.  Returns the previous setting.
 *
 * Single frame, two-workgroup form (GDN_PATH_FRAME): the first of a pair to
 * finish its partial sums waits for the other's (default 2^20 polls, about
 * a second).  If the wait runs out, that workgroup writes NaN to its output
 * columns; the other, the second of the pair, still writes the pair's rows
 * of state_out correctly, and values that are not NaN are exact.
 *
 * Fused kernel (default 2^22 polls: seconds for a wait of the state pass,
 * about 20 s for one of the other workgroups, which poll less often).
 * Every wait is bounded so
 * that a failure ends the kernel instead of hanging it: the first wait that
 * runs out sets an error word in the workspace's control block, every other
 * wait then gives up at once, the state pass writes NaN to the rows of
 * state_out it had not finished, and every frame of `out` that was not
 * produced is written as NaN (each frame is then either exact or NaN).
 * gdn_fused_status reports the error word.  A tiny limit makes the waits run
 * out on purpose, with every workgroup still exiting normally.  The next
 * launch starts from a fresh control block.
 */
unsigned gdn_set_spin_limit(unsigned polls);

/*
 * Outcome of the last fused-path gdn_frame_fwd call (GDN_PATH_FUSED) that
 * used `workspace`: waits for `stream` (the call's stream), then reads the
 * error word of the workspace's control block.  GDN_OK: every internal wait
 * completed and the results are valid; GDN_E_TIMEOUT: a wait ran out (which
 * cannot happen while every workgroup of the launch is resident), and the
 * frames of `out` and rows of state_out not produced are NaN.  GDN_E_NULLPTR
 * for a NULL workspace; GDN_E_HIP if the copy or the wait fails.  Call it
 * before the workspace is reused; after a call on another path the result
 * is meaningless.
 */
int gdn_fused_status(const void* workspace, void* stream);

/*
 * Which implementation gdn_frame_fwd uses for this shape and input dtype on
 * the current device, with the current gdn_set_fused setting:
 *   GDN_PATH_MFMA   bf16, D == 128, T <= 32 (and longer sequences when the
 *                   fused kernel below is unavailable): three bf16-MFMA
 *                   kernels (build, state pass, output) with the per-frame
 *                   intermediates in the workspace.  When T > 64 the
 *                   frames are cut into
 *                   ceil(T / 64) segments of nearly equal length and the
 *                   build of segment i+1, the state pass of segment i and
 *                   the output of segment i-1 overlap: builds run on
 *                   `stream`, state passes and outputs on two
 *                   library-owned streams (created on first use per device,
 *                   non-blocking, default priority) that fork from and join
 *                   back to `stream` through events, so the call is ordered
 *                   on `stream` like a single kernel.  The environment
 *                   variable GDN_SEGMENT_FRAMES (read once per process)
 *                   replaces the 64.  Otherwise all three run on `stream`;
 *   GDN_PATH_FUSED  bf16, D == 128, T > 32: build, state pass and output in
 *                   one persistent kernel per group of at most 16 heads,
 *                   launched on `stream` at the size that fills the device
 *                   after a tiny flag-reset kernel.  Each head runs on one
 *                   XCD and its per-frame G_t, U_t, M_t pass between compute
 *                   units through that XCD's L2 instead of HBM.  Roles go
 *                   by the order in which workgroups start, so the kernel
 *                   makes progress with any number of them resident; fused
 *                   calls issued on different streams of one device run one
 *                   after another (ordered on the GPU by an event, except
 *                   while the stream is being captured).  Every
 *                   internal wait is bounded: if one runs out (only when
 *                   other work holds the device's compute units for longer
 *                   than the limit), the frames and state rows not produced
 *                   are NaN and gdn_fused_status reports it.  On a device
 *                   that cannot host its roles at full size or does not deal
 *                   workgroups evenly over eight XCDs with ids 0-7 (checked
 *                   once per device by a probe kernel on the null stream
 *                   that waits for it, at the first call or query that
 *                   needs the fact), or while the fused kernel is disabled
 *                   (gdn_set_fused), these shapes take GDN_PATH_MFMA.  When
 *                   no device can be queried (no GPU), gdn_path reports the
 *                   path of a device that hosts the fused kernel;
 *   GDN_PATH_FRAME  bf16, D == 128, T == 1 (one frame per call, as in
 *                   frame-by-frame generation): one launch on `stream`.
 *                   The step written per token, M' = gamma M + beta sum_s
 *                   (v_s - gamma M k_s) k_s^T, splits M' into blocks of 16
 *                   rows (8 per head) with no reduction between them; a
 *                   block's workgroup then computes the same 16 columns of
 *                   O = Q M'^T.  With at most 16 heads, a workspace of
 *                   gdn_workspace_bytes (the call runs without one) and a
 *                   device that deals workgroups b and b + 8 to one XCD
 *                   (a one-time probe on the null stream at the first
 *                   call; a capture made before any eager call on the
 *                   device takes the other form), each block's even and
 *                   odd 64-token tiles go to two workgroups that swap
 *                   partial sums through the workspace (bounded waits, see
 *                   gdn_set_spin_limit); otherwise one workgroup takes all
 *                   of a block's tiles.  The two forms agree to float32
 *                   rounding; each is deterministic, captured or not.
 *                   Equal to
 *                   GDN_PATH_MFMA's result to float32 rounding, not bit for
 *                   bit (gdn_set_single_frame).  While disabled,
 *                   GDN_PATH_MFMA;
 *   GDN_PATH_PLAIN  every other supported case: three float32 kernels on
 *                   `stream`; also empty shapes (one small float32 kernel
 *                   or none, see "Empty shapes" above);
 *   -1              invalid arguments.
 * Results do not depend on the segmentation: the state pass carries the
 * float32 state exactly from one segment to the next.
 */
enum { GDN_PATH_PLAIN = 0, GDN_PATH_MFMA = 1, GDN_PATH_FUSED = 2, GDN_PATH_FRAME = 3 };
int gdn_path(const gdn_shape* shape, int in_dtype);

/*
 * Workspace bytes a gdn_frame_fwd call with this shape and input dtype needs
 * on the current device: those of gdn_path's path (gdn_path_workspace_bytes),
 * or, when no device can be queried, of GDN_PATH_MFMA, which is at least as
 * large as GDN_PATH_FUSED's.  0 when the shape is invalid or empty.
 */
size_t gdn_workspace_bytes(const gdn_shape* shape, int in_dtype);

/*
 * Workspace bytes of one path for this shape and input dtype, a pure
 * function of its arguments (per frame map, D*D*4 bytes = 64 KiB at D = 128):
 *   GDN_PATH_FUSED  a control block and per-head flags, then rings of G_t,
 *                   U_t and M_t slots for at most 16 heads at a time: a few
 *                   MiB per head whatever T is (76 MiB for 16 heads);
 *   GDN_PATH_FRAME  up to 16 heads (B*H), what the two-workgroup form
 *                   uses: per 16-row block (8 per head) a 128-byte pair
 *                   word and two 8 KiB halves of partial sums, the words
 *                   rounded up to 256 bytes (2.0 MiB for 16 heads); 0 for
 *                   more heads; T == 1 only.  A single-frame call needs no
 *                   workspace: with a smaller one (or NULL) it runs one
 *                   workgroup per block;
 *   GDN_PATH_MFMA   the maps of at most three segments at once: with n =
 *                   ceil(T / 64) segments of at most c = ceil(T / n) frames,
 *                   3 * min(n, 3) buffers of B*H*c maps, each rounded up to
 *                   256 bytes (549 MiB for B*H = 16, T = 961);
 *   GDN_PATH_PLAIN  G_t, U_t and M_t of every frame in float32:
 *                   3 * B*H*T*D*D*4 bytes, each third rounded up to 256.
 * 0 for an empty shape; SIZE_MAX for an invalid shape or dtype, an unknown
 * path, or a path that cannot take the shape (fused: bf16, D == 128 and
 * T > 32 only; single frame: bf16, D == 128 and T == 1 only; MFMA: bf16 and
 * D == 128 only).
 */
size_t gdn_path_workspace_bytes(const gdn_shape* shape, int in_dtype, int path);

/*
 * The whole forward: O and M_T from q, k, v, gamma, beta and M_0.
 *   in_dtype   GDN_BF16 or GDN_F32: dtype of q, k, v.
 *   out_dtype  GDN_F32 (recommended) or GDN_BF16: dtype of out.
 *   state_in   M_0 or NULL for zeros.   state_out: M_T (may equal state_in).
 *   workspace  at least gdn_workspace_bytes(shape, in_dtype) bytes of device
 *              memory, 256-byte aligned; its contents on return are
 *              unspecified.  A call checks it against the need of the path
 *              it takes: GDN_E_WORKSPACE when NULL, misaligned or smaller.
 */
int gdn_frame_fwd(const gdn_shape* shape, int in_dtype, int out_dtype,
                  const void* q, const void* k, const void* v,
                  const float* gamma, const float* beta,
                  const float* state_in, void* out, float* state_out,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_frame_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It takes no workspace: its kernels use a scratch array of
 * GDN_NOALLOC_SCRATCH_BYTES compiled into the library, one copy per GPU,
 * resident from the first call on that GPU until the process ends.  The
 * call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); the caller still provides every input and output.  Shapes whose
 * workspace (gdn_workspace_bytes) exceeds the array return GDN_E_TOO_LARGE
 * before anything is enqueued: this covers every shape on the fused path
 * (bf16, D == 128, T > 32, any B*H) and three-kernel calls of up to about
 * 500 head-frames (16 heads x 32 frames).  Every call on a GPU shares that
 * GPU's array and leaves its contents behind: calls that overlap on one GPU
 * (concurrent streams, threads or processes sharing the library instance)
 * race and give wrong results; serialise them.  The state the kernels need
 * zeroed is cleared by a kernel at the start of each call.  Everything else
 * as gdn_frame_fwd (no key scale; same results bit for bit).
 */
#define GDN_NOALLOC_SCRATCH_BYTES (96u << 20)
int gdn_frame_fwd_noalloc(const gdn_shape* shape, int in_dtype, int out_dtype,
                          const void* q, const void* k, const void* v,
                          const float* gamma, const float* beta,
                          const float* state_in, void* out, float* state_out, void* stream);

/*
 * gdn_frame_fwd with the key scaling fused into the build: the keys K_t are
 * used as given and the recurrence runs on key_scale * K_t, i.e.
 *     G_t = key_scale^2 K_t^T K_t,    U_t = key_scale V_t^T K_t
 * (the pages scale keys by 1/sqrt(D*S): pass that value with unscaled keys).
 * Each map is its float32 sum times key_scale^2 or key_scale, one rounding,
 * so key_scale = 1 gives gdn_frame_fwd's result bit for bit.  key_scale must
 * be finite (else GDN_E_VALUE).  Everything else as gdn_frame_fwd.  The fused
 * prologue saves the caller a separate pass over K (read and write).
 */
int gdn_frame_fwd_ks(const gdn_shape* shape, int in_dtype, int out_dtype,
                     const void* q, const void* k, const void* v,
                     const float* gamma, const float* beta,
                     const float* state_in, float key_scale, void* out, float* state_out,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_frame_fwd with the gates computed from activations and the key scale
 * applied inside the build: the gate prologue fused into the scan (the pages
 * fuse "the GDN scan and gate operations" into custom kernels: "SANA-WM:
 * NVIDIA puts a one-minute world model on a single GPU", zhichai.net,
 * training pipeline).  The pages call gamma a learned decay scalar and beta
 * the delta-rule strength (section 1) but do not give their
 * parameterisation; the one taken here, per frame t of head h:
 *     gamma_t = exp(-exp(A_log[h]) * softplus(mean_s gate_a[t, s] + dt_bias[h]))
 *     beta_t  = sigmoid(mean_s gate_b[t, s])
 * with gate_a, gate_b the per-token pre-activations of the layer's gate
 * projections (one scalar per token and head) averaged over the frame's S
 * tokens, because one recurrent step consumes a whole latent frame.  Then the
 * recurrence of gdn_frame_fwd runs on key_scale * K with these gates.
 *   gate_a, gate_b  [B, H, T, S] float32 (device)
 *   A_log, dt_bias  [H] float32 (device): head h of every batch element
 *   gamma, beta     [B, H, T] float32 (device) outputs: the gates used
 *   key_scale       finite (else GDN_E_VALUE); 1 for keys already scaled
 * Everything else, the workspace included, as gdn_frame_fwd.  S must be at
 * least 1 when there are frames (a frame's gates average its tokens; else
 * GDN_E_SHAPE).  One small kernel computes the gates (one pass over the
 * pre-activations, token sums in one fixed order), then the call proceeds as
 * gdn_frame_fwd_ks on its path with them; results do not depend on the path
 * beyond what gdn_frame_fwd's do.
 */
int gdn_frame_fwd_gated(const gdn_shape* shape, int in_dtype, int out_dtype,
                        const void* q, const void* k, const void* v,
                        const float* gate_a, const float* gate_b,
                        const float* A_log, const float* dt_bias,
                        const float* state_in, float key_scale, void* out, float* state_out,
                        float* gamma, float* beta,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_frame_fwd, plus per-kernel durations: a pair of HIP events is recorded
 * around every kernel launch of the call, on the stream that launch uses;
 * the call waits for `stream` (which the call joins back to) and writes,
 * for kernel kinds 0 = build, 1 = state pass (the whole fused kernel on
 * the fused path, flag reset included; the single-frame kernel on
 * GDN_PATH_FRAME), 2 = output, the summed elapsed milliseconds to
 * kernel_ms[kind] and the number of launches to
 * launches[kind] (both host arrays of 3).  Launches of different kinds may overlap in time, so the
 * three sums can add up to more than the call.  Results are identical to
 * gdn_frame_fwd.  The events are created as needed and kept for the life of
 * the process; this entry point is for profiling and is not meant for graph
 * capture.
 */
int gdn_frame_fwd_timed(const gdn_shape* shape, int in_dtype, int out_dtype,
                        const void* q, const void* k, const void* v,
                        const float* gamma, const float* beta,
                        const float* state_in, void* out, float* state_out,
                        void* workspace, size_t workspace_bytes, void* stream,
                        float* kernel_ms, int* launches);

/*
 * Stage 1, the per-frame maps: G_t = K_t^T K_t and U_t = V_t^T K_t for every
 * (b, h, t), reducing over the S tokens of the frame.  G, U: [B,H,T,D,D] f32.
 */
int gdn_build_maps(const gdn_shape* shape, int in_dtype, const void* k, const void* v,
                   float* G, float* U, void* stream);

/*
 * Stage 2, the state pass: M_t = M_{t-1} gamma_t (I - beta_t G_t) + beta_t U_t
 * for t = 1..T in float32.  Writes every M_t to M_all ([B,H,T,D,D], may be
 * NULL when only the final state is wanted) and M_T to state_out.  The S
 * field of the shape is ignored.
 */
int gdn_state_pass(const gdn_shape* shape, const float* G, const float* U,
                   const float* gamma, const float* beta, const float* state_in,
                   float* M_all, float* state_out, void* stream);

/*
 * Stage 3, the output: O_t = Q_t M_t^T for every (b, h, t), M_t from M_all.
 */
int gdn_output(const gdn_shape* shape, int in_dtype, int out_dtype, const void* q,
               const float* M_all, void* out, void* stream);

/*
 * Backward pass (vector-Jacobian product) of gdn_frame_fwd.  The pages train
 * the model ("SANA-WM: NVIDIA puts a one-minute world model on a single
 * GPU", zhichai.net, training pipeline) without stating the gradients; these
 * are the exact derivative of the forward above.  With Lambda_t the total
 * gradient reaching M_t (d_out_t^T Q_t plus what flows back from M_{t+1}):
 *   dq_t = d_out_t M_t,   dv_t = beta_t K_t Lambda_t^T,
 *   dk_t = beta_t V_t Lambda_t + K_t (dG_t + dG_t^T),
 *          dG_t = -gamma_t beta_t M_{t-1}^T Lambda_t,
 *   dgamma_t = < Lambda_t, M_{t-1} (I - beta_t G_t) >,
 *   dbeta_t  = < Lambda_t, U_t - gamma_t M_{t-1} G_t >,
 *   d_state_in = gradient of M_0 (written even when state_in is NULL).
 * Supported: in_dtype GDN_BF16 with D == 128 (otherwise GDN_E_DTYPE or
 * GDN_E_UNSUPPORTED_D).  d_out has in_dtype; d_state_out is [B,H,D,D] f32 or
 * NULL (zero).  dq, dk, dv: [B,H,T,S,D] f32; dgamma, dbeta: [B,H,T] f32;
 * d_state_in: [B,H,D,D] f32 (may equal d_state_out, for chunked backward
 * passes that carry the state gradient: cutting a sequence into calls made
 * last chunk first, each given the next chunk's d_state_in as d_state_out
 * and its own forward state_in, gives the one-call result bit for bit).
 * The forward states are recomputed from q, k, v, gamma, beta and state_in.
 * Asynchronous on `stream`; for T > 64 the work runs in min(ceil(T / 64), 3)
 * segments of nearly equal length on the same library-owned side streams
 * as gdn_frame_fwd, forked from and joined back to `stream`, and results do
 * not depend on the segmentation.
 * Argument errors return before any launch.  workspace: at least
 * gdn_bwd_workspace_bytes(shape, in_dtype) bytes of device memory
 * (5 * B*H*T*D*D*4 bytes for the per-frame maps, plus 64 bytes per frame of
 * partial sums and one state, each rounded up to 256), 256-byte aligned; its
 * contents on return are unspecified.  gdn_bwd_workspace_bytes returns 0
 * for an invalid or empty shape.
 */
size_t gdn_bwd_workspace_bytes(const gdn_shape* shape, int in_dtype);
int gdn_frame_bwd(const gdn_shape* shape, int in_dtype,
                  const void* q, const void* k, const void* v,
                  const float* gamma, const float* beta, const float* state_in,
                  const void* d_out, const float* d_state_out,
                  float* dq, float* dk, float* dv, float* dgamma, float* dbeta,
                  float* d_state_in, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The backward of gdn_frame_fwd_ks: gradients with respect to the unscaled
 * keys given to it, dk = key_scale * (gradient with respect to
 * key_scale * K); the other gradients as gdn_frame_bwd's.  key_scale = 1
 * gives gdn_frame_bwd's result bit for bit; it must be finite (else
 * GDN_E_VALUE).  Same workspace as gdn_frame_bwd.
 */
int gdn_frame_bwd_ks(const gdn_shape* shape, int in_dtype,
                     const void* q, const void* k, const void* v,
                     const float* gamma, const float* beta, const float* state_in, float key_scale,
                     const void* d_out, const float* d_state_out,
                     float* dq, float* dk, float* dv, float* dgamma, float* dbeta,
                     float* d_state_in, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
