// The whole frame-wise GDN forward (bf16 inputs, head dim 128) as one
// persistent kernel that overlaps the three stages:
//   build   G_t = K_t^T K_t, U_t = V_t^T K_t      (parallel over frames)
//   state   M_t = M_{t-1} gamma_t (I - beta_t G_t) + beta_t U_t   (sequential)
//   output  O_t = Q_t M_t^T                        (parallel over frames)
// (the recurrence of "SANA-WM: NVIDIA puts a one-minute world model on a
// single GPU", zhichai.net, section 1; one step per latent frame, bilibili
// cv49203711, fourth key point).
//
// Why one kernel.  As separate kernels the per-frame maps G_t, U_t and the
// states M_t make a round trip through HBM (384 KB per head-frame against
// the 1,126 KB of q, k, v and O).  Here they pass between compute units
// through the L2 of one XCD and the memory-side cache behind it instead of
// making a round trip to HBM between kernels.
//
// Layout of the work.  MI355X has 8 XCDs, each with its own 4 MB L2.  Head h
// is handled entirely by XCD h % 8.  A workgroup learns its XCD from the
// XCC_ID hardware register and takes a ticket from that XCD's counter: the
// first tickets become state-pass workgroups (kParts per head, each owning
// kRows rows of M; rows of M evolve independently), the rest become
// workers that pull build and output items from the XCD's queue.  Two
// workgroups fit on a CU (every role stays within 256 registers per lane
// and 80 KB of LDS) and the launch fills the device; state-pass waves raise
// their issue priority so that a worker sharing their CU does not stretch
// the sequential chain.
//
// Progress without a co-residency guarantee.  The launch is an ordinary one
// (a cooperative launch costs about 20 us more per call and guarantees
// nothing the design needs).  Roles follow the order in which workgroups
// start on an XCD, not their ids: the first nh * kParts to take a ticket
// run the state pass, so a worker runs only once every state-pass
// workgroup of its XCD is running.  State-pass workgroups wait only for
// items, and every item waits only for earlier items or for state-pass
// progress that needs only earlier items (see the ring notes below), so any
// running worker can finish the lowest unfinished item.  The state pass
// holds at most 16 of an XCD's 64 workgroup slots, so as long as other work
// on the device drains, workers start (the library runs its fused launches
// of one device one at a time, so they never hold those slots together).
// Should none start within the bounded waits, the call ends with the error
// word set (see below), never hangs.
//
// Hand-off between CUs of one XCD.  The L2 is shared by the XCD's CUs and
// the vector L1 is write-through, so a producer makes data visible by
// waiting for its stores to be acknowledged (s_waitcnt vmcnt(0)) and then
// setting a flag; a consumer reads the flag from L2 (device-scope relaxed
// atomic load), invalidates its own L1 (buffer_inv sc0) and reads the data.
// Device-scope acquire/release would write back or invalidate whole L2s and
// is not needed within one XCD.
//
// Rings.  Per head: kRing.wg slots for G_t/U_t and kRing.wm slots for M_t,
// with monotonic per-slot flags (frame index + 1).  G_t is symmetric, so a
// build writes only its upper triangle (36 of 64 16 x 16 blocks per plane,
// 36 KB instead of 64) and the state pass reads the lower blocks as
// transposes of the upper ones, out of LDS.  The queue of an XCD
// lists, per head, the builds of frames 0 .. lag-1, then output(f) and
// build(f + lag) alternately, then the last outputs; those of the last
// wm frames are split over token parts (nothing waits for them, and after
// the state pass's last step they are the only work left).  Every wait of an item
// depends only on items earlier in the queue, or on state-pass progress that
// needs only such items (lag > kPrefetch + 1, lag <= wg + wm), and all
// workgroups are resident, so the lowest unfinished item can always proceed.
// Every wait is still bounded: one that runs out sets an error word, every
// other wait then gives up, the state pass writes NaN to state_out, and the
// kernel ends.
#include "frame_build.h"
#include "frame_output.h"
#include "gdn_common.h"
#include "gdn_launch.h"
#include "gdn_packed.h"

#include <cstddef>
#include <type_traits>
#include <utility>

namespace gdn {
namespace {

constexpr int D = 128;
constexpr int kXcd = 8;
constexpr int kPrefetch = 1;          // frames the state pass loads ahead
static_assert(kPrefetch == 1, "the state pass holds exactly one frame ahead in registers");
constexpr int kMaxHeadsPerXcd = 2;
constexpr int kMaxParts = 8;          // kRows >= 16
constexpr int kLdsW = D + 8;
constexpr int kChainWaves = 4;
static_assert(kMaxParts * kChainWaves <= 64, "a worker polls a head's per-wave flags from one wave");
constexpr uint32_t kSpinLimit = 1u << 22;  // default polls before a wait gives up (seconds)

// Ring shape: G/U slots, M slots and the queue distance from build(t) to
// output(t).  The queue distance must cover a build's duration in state-pass
// steps (a build takes ~40 us, a step ~4 us); every wait then depends only
// on earlier items as long as lag > kPrefetch + 1 and lag <= wg + wm (see
// the ring notes above).  Measured on the 60 s workload (same box, same
// inputs): with the wave-wide polls above and a cooperative launch, 4-8 M
// slots were 1-2 % faster than 12-28 (which are within 1 % of each other)
// on two boxes, 3 were 3 % slower; 24, 20 or 16 G/U slots starve the state
// pass (+30-40 %), and queue lags of 20-28 are within 1 %.  With the
// ordinary launch, 12 M slots against 6: the 961-frame call the same, an
// 81-frame call 1.5 % and 40-frame calls 1 % faster (20 slots: between).
// (Before those polls, with one lane loading each flag, 20 M slots were
// 2-3.5 % faster than 12, 36-40 G/U slots lost 2-5 %, and 96 overflowed the
// memory-side cache, +20 %.)
struct RingShape {
  int wg, wm, lag;
};
constexpr RingShape kRing{32, 12, 24};
static_assert(kRing.wg >= kPrefetch + 2 && kRing.wm >= 2 &&
                  kRing.lag > kPrefetch + 1 && kRing.lag <= kRing.wg + kRing.wm,
              "ring shape could stall the queue");

// Control block (zeroed before every launch) followed by per-head flags.
struct Ctrl {
  uint32_t error;
  uint32_t pad0[31];
  uint32_t ticket[kXcd];
  uint32_t pad1[24];
  uint32_t queue[kXcd];
  uint32_t pad2[24];
};
// Per-head flag block.  The state pass publishes per wave, so no extra
// workgroup barrier is needed to publish.
constexpr int kFlagGReady = 0;                                         // [wg]  frame + 1 of the G/U in the slot
constexpr int kFlagConsumed = kRing.wg;                                 // [parts][waves] frames loaded by the wave
constexpr int kFlagMReady = kFlagConsumed + kMaxParts * kChainWaves;   // [wm][parts][waves] frame + 1 of M rows
constexpr int kFlagOutDone = kFlagMReady + kRing.wm * kMaxParts * kChainWaves;  // [wm] frame + 1 staged by the output
constexpr int kFlagWords = (kFlagOutDone + kRing.wm + 63) / 64 * 64;  // whole cache lines per head

__device__ __forceinline__ uint32_t xcc_id() {
  // HW_REG_XCC_ID, bits [3:0]
  return __builtin_amdgcn_s_getreg((15 << 11) | (0 << 6) | 20) & 0xfu;
}
__device__ __forceinline__ uint32_t flag_load(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void flag_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void invalidate_l1() { asm volatile("buffer_inv sc0" ::: "memory"); }

// Spin until pred() holds, at most `limit` polls kSleep x 64 clocks apart;
// false if it never did or another wait already failed.  A state-pass wave
// polls one flag from one lane; a worker polls the 32 per-wave flags of a
// head from the 32 lanes of its first wave, one load instruction that reads
// the flags' one cache line once (pred must then give the same value in
// every lane of the wave).  Polls from many workgroups land on those few
// flag lines, and that traffic slows the whole XCD: with one lane loading
// the 32 flags one by one every 64 clocks, a call took 5-17 % longer than
// with a wave-wide load every ~0.4 us (more with a bf16 output, where it
// could double the call's time); the poll interval matters little once each
// poll is a single load.
constexpr int kStateSleep = 16;
constexpr int kWorkerSleep = 32;
template <int kSleep, typename Pred>
__device__ bool spin_until(Ctrl* ctrl, uint32_t limit, Pred pred) {
  for (uint32_t i = 0; i < limit; ++i) {
    if (pred()) return true;
    if ((i & 63) == 0 && flag_load(&ctrl->error)) return false;
    __builtin_amdgcn_s_sleep(kSleep);
  }
  if ((threadIdx.x & 63) == 0) __hip_atomic_store(&ctrl->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return false;
}

// True in every lane when the condition holds in every lane of the wave.
__device__ __forceinline__ bool wave_all(bool c) { return __builtin_amdgcn_ballot_w64(!c) == 0; }

struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* gamma;
  const float* beta;
  const float* state_in;
  void* out;
  float* state_out;
  char* ring;       // per head: kRing.wg x (Gp, Up) then kRing.wm x Mp, 64 KB each
  Ctrl* ctrl;
  uint32_t* flags;  // per head kFlagWords
  int heads, T, S;
  float ks;             // key scale: the build items write ks^2 G_t and ks U_t
  uint32_t spin_limit;  // polls before a wait gives up
};

__host__ __device__ constexpr int64_t ring_head_bytes(int wg, int wm) {
  return int64_t{2 * wg + wm} * packed::kFrameBytes;
}

struct Item {
  int kind;  // 0 build, 1 output
  int hl;    // head index within the XCD
  int t;     // frame
  int part;  // token part of a split output, -1 for the whole frame
};

// The outputs of the last tail_frames(T) frames are split over kTailParts
// token parts each.  No state-pass step waits for them (a step waits only
// for the output kRing.wm frames back), so their flag stores are never
// read; split, the output of the last frame no longer stretches the
// kernel's end by a whole frame's output on one workgroup (T = 40: 186
// against 192 us; 2 and 8 parts measure the same as 4).  Each token's
// arithmetic is unchanged.
constexpr int kTailParts = 4;
__device__ int tail_frames(int T) {
  const int L = T < kRing.lag ? T : kRing.lag;
  return L < kRing.wm ? L : kRing.wm;
}
__device__ int queue_items(int nh, int T) { return nh * (2 * T + tail_frames(T) * (kTailParts - 1)); }

// Item i of an XCD with nh heads.  Slot k = i / nh holds one item per head:
// builds of frames 0..L-1 (L = min(T, lag)), then alternately output(f) and
// build(f + L), then the outputs of frames T-L .. T-1, the last tail_frames
// of them as kTailParts slots each.
__device__ Item decode_item(int i, int nh, int T) {
  const int L = T < kRing.lag ? T : kRing.lag;
  const int k = i / nh, hl = i % nh;
  const int tail = tail_frames(T), kt = 2 * T - tail;  // slots before the split outputs
  if (k >= kt) return {1, hl, T - tail + (k - kt) / kTailParts, (k - kt) % kTailParts};
  if (k < L) return {0, hl, k, -1};
  const int j = k - L;
  if (j < 2 * (T - L)) return (j & 1) ? Item{0, hl, L + (j >> 1), -1} : Item{1, hl, j >> 1, -1};
  return {1, hl, T - L + (j - 2 * (T - L)), -1};
}

// G_t as the state pass holds it in LDS: the 36 upper-triangle 16 x 16
// blocks (row block rb <= column block cb) of each bf16 plane, 72 blocks of
// 512 B in the order of sym_block(); inside a block, lane slot n + 16 h holds
// the 8 bf16 of row n, columns 8h .. 8h+7 (one half of a packed Gp unit).
constexpr int kSymBlocks = 36;
constexpr int kSymChunks = kSymBlocks * 2 * 32;  // 16-byte chunks, both planes
__host__ __device__ constexpr int sym_block(int rb, int cb) { return rb * 8 - rb * (rb - 1) / 2 + (cb - rb); }

template <int kRows>
union __attribute__((aligned(16))) Lds {
  u32x4 build[build_lds_bytes<true>() / 16];
  uint16_t out[2][D][kOutLdsW];
  struct {
    uint16_t m[2][2][kRows][kLdsW];
    u32x4 g[kSymChunks];
  } chain;
};

// ---------------------------------------------------------------------------
// state pass: one workgroup owns rows [r0, r0 + kRows) of one head's M
// ---------------------------------------------------------------------------
// X = M G on bf16 MFMA in three passes (Ghi*Mhi + Glo*Mhi + Ghi*Mlo), as the
// stand-alone state pass: computed transposed, X^T = G M^T (G is symmetric),
// wave w owning G rows 32w .. 32w+31; each lane ends with 4 consecutive
// columns of kRows/16 rows of M.  The workgroup loads G_t's upper triangle
// a step ahead (9 chunks of 16 bytes per thread), puts it in LDS at the
// start of the step and reads its MFMA operands from there, lower blocks
// through transposed reads.  Each wave keeps its own flags: at the top of
// step t it waits only for memory operations it issued during step t-1
// (M_{t-1} stores, the loads of frame t, the flag loads for this step),
// publishes M_{t-1} and its progress, and checks the flags it loaded a step
// ahead.  Two barriers per step: after G_t is in LDS, and for the LDS
// hand-off of M between the waves.  A wave whose wait fails sets `abort` in
// LDS; after the barrier every wave sees it and all leave together.
template <int kRows>
__device__ void state_role(const Args& a, Lds<kRows>& lds, uint32_t* bcast, int head, int part) {
  constexpr int kParts = D / kRows;
  constexpr int kRB = kRows / 16;
  uint16_t (*Ml)[2][kRows][kLdsW] = lds.chain.m;
  u32x4* Gs = lds.chain.g;
  const int T = a.T;
  const int r0 = part * kRows;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int n = l & 15, g = l >> 4;
  uint32_t* fl = a.flags + (int64_t)head * kFlagWords;
  constexpr int kWG = kRing.wg, kWM = kRing.wm;
  char* ring = a.ring + head * ring_head_bytes(kWG, kWM);
  auto gp_slot = [&](int t) { return ring + (int64_t)(2 * (t % kWG)) * packed::kFrameBytes; };
  auto up_slot = [&](int t) { return ring + (int64_t)(2 * (t % kWG) + 1) * packed::kFrameBytes; };
  auto mp_slot = [&](int t) { return ring + (int64_t)(2 * kWG + t % kWM) * packed::kFrameBytes; };
  uint32_t* my_consumed = fl + kFlagConsumed + part * kChainWaves + w;
  auto my_mready = [&](int t) { return fl + kFlagMReady + ((t % kWM) * kParts + part) * kChainWaves + w; };

  auto row_of = [&](int rb) { return r0 + 16 * rb + n; };
  auto col_of = [&](int cb) { return 32 * w + 16 * cb + 4 * g; };
  const int64_t hoff = (int64_t)head * D * D;

  f32x4 Mreg[2][kRB];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
      Mreg[cb][rb] = a.state_in ? *reinterpret_cast<const f32x4*>(a.state_in + hoff + row_of(rb) * D + col_of(cb))
                                : (f32x4){0.f, 0.f, 0.f, 0.f};
  u32x2 mh[2][kRB], ml[2][kRB];
  auto split_m = [&]() {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        const u32x2 p0 = split2(Mreg[cb][rb][0], Mreg[cb][rb][1]);
        const u32x2 p1 = split2(Mreg[cb][rb][2], Mreg[cb][rb][3]);
        mh[cb][rb] = (u32x2){p0.x, p1.x};
        ml[cb][rb] = (u32x2){p0.y, p1.y};
      }
  };
  auto put_lds = [&](int buf) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        *reinterpret_cast<u32x2*>(&Ml[buf][0][16 * rb + n][col_of(cb)]) = mh[cb][rb];
        *reinterpret_cast<u32x2*>(&Ml[buf][1][16 * rb + n][col_of(cb)]) = ml[cb][rb];
      }
  };
  split_m();
  put_lds(0);
  // bcast[0] is the abort word: zeroed by the kernel entry before its
  // barrier, set to 1 by any wave whose wait fails, and read by every wave
  // only after the next barrier, so all waves leave the loop together.

  // gamma/beta: 64-frame windows per lane, read with readlane (scalar loads
  // would share the LDS wait counter)
  const float* gh = a.gamma + (int64_t)head * T;
  const float* bh = a.beta + (int64_t)head * T;
  auto win_load = [&](int t0, float& gv, float& bv) {
    const int tt = t0 + l;
    gv = tt < T ? gh[tt] : 0.f;
    bv = tt < T ? bh[tt] : 0.f;
  };
  float gwin, bwin, gnxt, bnxt;
  win_load(0, gwin, bwin);
  win_load(64, gnxt, bnxt);

  // one-frame register ring: 9 of the 2304 16-byte chunks of G_t's upper
  // triangle (the builders write only those halves of the packed units) and
  // this wave's U_t elements.  Chunk c = tid + 256 i is LDS chunk c; its
  // source in the packed slot is fixed per thread, computed once here.
  constexpr int kChunks = kSymChunks / 256;
  static_assert(kSymChunks % 256 == 0, "whole chunks per thread");
  int goff[kChunks];
#pragma unroll
  for (int i = 0; i < kChunks; ++i) {
    const int c = tid + 256 * i;
    const int blk = c >> 5, plane = blk & 1, slot = c & 31;
    int rb = 0, first = 0;
#pragma unroll
    for (int r = 1; r < 8; ++r)
      if ((blk >> 1) >= sym_block(r, r)) rb = r, first = sym_block(r, r);
    const int cbk = rb + ((blk >> 1) - first);  // column block of the 16 x 16 block
    goff[i] = ((((rb * 4 + (cbk >> 1)) * 2 + plane) << 10) + ((cbk & 1) << 9) + (slot << 4));
  }
  u32x4 rg[kChunks];
  f32x4 ru[2][kRB];
  auto load_frame = [&](int t) {
    if (t >= T) return;
    const char* Gp = gp_slot(t);
    const char* Up = up_slot(t);
#pragma unroll
    for (int i = 0; i < kChunks; ++i) rg[i] = *reinterpret_cast<const u32x4*>(Gp + goff[i]);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
        ru[cb][rb] = *reinterpret_cast<const f32x4*>(Up + ((((r0 >> 4) + rb) * 8 + 2 * w + cb) << 10) + 16 * l);
  };

  // Prologue: wait for build(0) (every wave for itself) and load frame 0.
  bool ok = true;
  if (l == 0) ok = spin_until<kStateSleep>(a.ctrl, a.spin_limit, [&] { return flag_load(fl + kFlagGReady) >= 1u; });
  ok = __builtin_amdgcn_readfirstlane((int)ok) != 0;
  if (!ok && l == 0) bcast[0] = 1;
  invalidate_l1();
  if (ok) load_frame(0);
  uint32_t gflag = 0, oflag = 0;  // flags for the next step, loaded a step ahead (lane 0)
  if (l == 0 && kPrefetch < T) gflag = flag_load(fl + kFlagGReady + kPrefetch % kWG);
  lds_barrier();
  ok = bcast[0] == 0;  // the same on every wave

  for (int t = 0; t < T && ok; ++t) {
    // Everything this wave issued in step t-1 is complete after this wait.
    wait_stores();
    // gamma_t and beta_t now, with nothing in flight: a readlane after the
    // flag loads below would wait for those loads too (the compiler cannot
    // count the loads in flight there, so it waits for all of them)
    const int tw = t & 63;
    const float gm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gwin), tw));
    const float bt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bwin), tw));
    if (tw == 63) {
      gwin = gnxt;
      bwin = bnxt;
      win_load(t + 65, gnxt, bnxt);
    }
    bool good = true;
    if (l == 0) {
      if (t > 0) flag_store(my_mready(t - 1), (uint32_t)t);
      flag_store(my_consumed, (uint32_t)(t + kPrefetch < T ? t + kPrefetch : T));
      const int tn = t + kPrefetch;
      if (tn < T && gflag < (uint32_t)(tn + 1))
        good = spin_until<kStateSleep>(a.ctrl, a.spin_limit, [&] {
          return flag_load(fl + kFlagGReady + tn % kWG) >= (uint32_t)(tn + 1);
        });
      if (good && t >= kWM && oflag < (uint32_t)(t - kWM + 1))
        good = spin_until<kStateSleep>(a.ctrl, a.spin_limit, [&] {
          return flag_load(fl + kFlagOutDone + t % kWM) >= (uint32_t)(t - kWM + 1);
        });
      // flags for step t + 1, in flight during this step
      if (t + 1 + kPrefetch < T) gflag = flag_load(fl + kFlagGReady + (t + 1 + kPrefetch) % kWG);
      if (t + 1 >= kWM) oflag = flag_load(fl + kFlagOutDone + (t + 1) % kWM);
    }
    good = __builtin_amdgcn_readfirstlane((int)good) != 0;
    // G_t into LDS (every wave's reads of G_{t-1} ended at the last barrier)
    if (good) {
#pragma unroll
      for (int i = 0; i < kChunks; ++i) Gs[tid + 256 * i] = rg[i];
    }
    lds_barrier();
    if (good) {
      const int buf = t & 1;
      f32x4 ureg[2][kRB];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) ureg[cb][rb] = ru[cb][rb];
      // refill the ring with frame t + 1 (its build is done)
      invalidate_l1();
      load_frame(t + kPrefetch);

      f32x4 acc[2][kRB];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) acc[cb][rb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        // A operand (cb, kb): lane (n, g) needs G[16(2w + cb) + n][32kb + 8g .. +7], in
        // 16 x 16 block (2w + cb, 2kb + g/2).  An upper block is read as stored; a lower
        // one is the transpose of block (2kb + g/2, 2w + cb): rows 8(g%2) + e, column n,
        // e = 0..7, two transposed reads in which lane (n, g) names row 8(g%2) + 4h + n/4
        // at columns 4(n%4) .. +3.
        u32x4 ahi[2], alo[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const int rbk = 2 * w + cb, cbk = 2 * kb + (g >> 1);
          if (rbk <= cbk) {
            const int c = sym_block(rbk, cbk) * 64 + n + 16 * (g & 1);
            ahi[cb] = Gs[c];
            alo[cb] = Gs[c + 32];
          } else {
            const uint16_t* hb = reinterpret_cast<const uint16_t*>(Gs + sym_block(cbk, rbk) * 64);
            const int r = 8 * (g & 1) + (n >> 2);
            const int e0 = (r + 16 * ((n & 3) >> 1)) * 8 + 4 * (n & 1);      // bf16 index, rows r
            const int e1 = (r + 4 + 16 * ((n & 3) >> 1)) * 8 + 4 * (n & 1);  // and r + 4
            const u32x2 h0 = lds_read_tr16(hb + e0), h1 = lds_read_tr16(hb + e1);
            const u32x2 l0 = lds_read_tr16(hb + 256 + e0), l1 = lds_read_tr16(hb + 256 + e1);
            ahi[cb] = (u32x4){h0.x, h0.y, h1.x, h1.y};
            alo[cb] = (u32x4){l0.x, l0.y, l1.x, l1.y};
          }
        }
        u32x4 bhi[kRB], blo[kRB];
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          bhi[rb] = *reinterpret_cast<const u32x4*>(&Ml[buf][0][16 * rb + n][32 * kb + 8 * g]);
          blo[rb] = *reinterpret_cast<const u32x4*>(&Ml[buf][1][16 * rb + n][32 * kb + 8 * g]);
        }
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) acc[cb][rb] = mfma16x16x32(ahi[cb], bhi[rb], acc[cb][rb]);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) acc[cb][rb] = mfma16x16x32(alo[cb], bhi[rb], acc[cb][rb]);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) acc[cb][rb] = mfma16x16x32(ahi[cb], blo[rb], acc[cb][rb]);
      }
      const float gb = gm * bt;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            Mreg[cb][rb][i] = fmaf(gm, Mreg[cb][rb][i], fmaf(-gb, acc[cb][rb][i], bt * ureg[cb][rb][i]));
      split_m();
      put_lds(buf ^ 1);
      // this wave's rows of M_t into the ring (the slot's previous frame is staged)
      char* Mp = mp_slot(t);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          *reinterpret_cast<u32x2*>(Mp + packed::m_chunk(row_of(rb), col_of(cb), 0)) = mh[cb][rb];
          *reinterpret_cast<u32x2*>(Mp + packed::m_chunk(row_of(rb), col_of(cb), 1)) = ml[cb][rb];
        }
    } else if (l == 0) {
      bcast[0] = 1;
    }
    lds_barrier();
    ok = bcast[0] == 0;
  }
  wait_stores();
  if (ok && l == 0) {
    flag_store(my_mready(T - 1), (uint32_t)T);
    flag_store(my_consumed, (uint32_t)T);
  }
  const float nan = __builtin_nanf("");
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
      *reinterpret_cast<f32x4*>(a.state_out + hoff + row_of(rb) * D + col_of(cb)) =
          ok ? Mreg[cb][rb] : (f32x4){nan, nan, nan, nan};
}

// ---------------------------------------------------------------------------
// workers
// ---------------------------------------------------------------------------
// NaN into rows [0, n) of an output frame (float32 or bf16 elements): what
// an output item writes when its wait gave up, so that every frame of `out`
// is either exact or NaN after a failed launch.  Kept out of line: inlined,
// its registers made the worker loop spill (and the kernel 4 % slower).
template <bool kOutBf16>
__device__ __attribute__((noinline)) void nan_fill(void* of, int n) {
  constexpr uint32_t w = kOutBf16 ? 0x7fc07fc0u : 0x7fc00000u;
  constexpr int kRowChunks = D * (kOutBf16 ? 2 : 4) / 16;
  u32x4* dst = static_cast<u32x4*>(of);
  for (int c = threadIdx.x; c < n * kRowChunks; c += blockDim.x) dst[c] = (u32x4){w, w, w, w};
}

template <bool kOutBf16, int kRows>
__device__ void worker_role(const Args& a, Lds<kRows>& lds, uint32_t* bcast, int xcd, int nh) {
  constexpr int kParts = D / kRows;
  const int T = a.T, S = a.S;
  constexpr int kWG = kRing.wg, kWM = kRing.wm;
  const int total = queue_items(nh, T);
  const int tid = threadIdx.x;
  for (;;) {
    if (tid == 0) bcast[2] = atomicAdd(&a.ctrl->queue[xcd], 1u);
    __syncthreads();
    const int i = (int)bcast[2];
    __syncthreads();  // everyone has read the item before thread 0 overwrites it
    if (i >= total) return;
    const Item it = decode_item(i, nh, T);
    const int head = it.hl * kXcd + xcd;
    uint32_t* fl = a.flags + (int64_t)head * kFlagWords;
    char* ring = a.ring + head * ring_head_bytes(kWG, kWM);
    const int64_t fr = (int64_t)head * T + it.t;
    if (it.kind == 0) {
      // build(t): every state-pass wave must have loaded the slot's previous frame
      if (tid < 64) {
        const uint32_t need = it.t >= kWG ? (uint32_t)(it.t - kWG + 1) : 0u;
        const bool ready = spin_until<kWorkerSleep>(a.ctrl, a.spin_limit, [&] {
          int ln = threadIdx.x;  // opaque: the lane's flag address is formed here, not kept live
          asm volatile("" : "+v"(ln));
          const uint32_t c = ln < kParts * kChainWaves ? flag_load(fl + kFlagConsumed + ln) : 0xffffffffu;
          return wave_all(c >= need);
        });
        if (tid == 0) bcast[3] = ready;
      }
      __syncthreads();
      if (!bcast[3]) continue;  // a wait gave up: drain the queue, building nothing
      char* gp = ring + (int64_t)(2 * (it.t % kWG)) * packed::kFrameBytes;
      float* up = reinterpret_cast<float*>(ring + (int64_t)(2 * (it.t % kWG) + 1) * packed::kFrameBytes);
      // two token iterations loaded ahead (one measured no faster); the
      // kernel fits its 256 registers per lane without spilling either way
      build_frame<true, 2, true>(a.k + fr * S * D, a.v + fr * S * D, S, lds.build, gp, up, a.ks);
      wait_stores();
      __syncthreads();
      if (tid == 0) flag_store(fl + kFlagGReady + it.t % kWG, (uint32_t)(it.t + 1));
    } else {
      // output(t): every state-pass wave's rows of M_t must be in the ring
      if (tid < 64) {
        const bool ready = spin_until<kWorkerSleep>(a.ctrl, a.spin_limit, [&] {
          int ln = threadIdx.x;  // opaque, as above
          asm volatile("" : "+v"(ln));
          const uint32_t c = ln < kParts * kChainWaves
                                 ? flag_load(fl + kFlagMReady + (it.t % kWM) * kParts * kChainWaves + ln)
                                 : 0xffffffffu;
          return wave_all(c >= (uint32_t)(it.t + 1));
        });
        if (tid == 0) bcast[3] = ready;
      }
      __syncthreads();
      const int s0 = it.part < 0 ? 0 : it.part * S / kTailParts;
      const int s1 = it.part < 0 ? S : (it.part + 1) * S / kTailParts;
      if (!bcast[3]) {  // a wait gave up: this frame's M_t never came
        nan_fill<kOutBf16>(static_cast<char*>(a.out) + (fr * S + s0) * D * (kOutBf16 ? 2 : 4), s1 - s0);
        continue;
      }
      invalidate_l1();
      const char* mp = ring + (int64_t)(2 * kWG + it.t % kWM) * packed::kFrameBytes;
      const int64_t tok = fr * S + s0;
      void* of = static_cast<char*>(a.out) + tok * D * (kOutBf16 ? 2 : 4);
      if (s1 > s0)
        output_frame<true, kOutBf16>(a.q + tok * D, mp, of, s1 - s0, lds.out, [&] {
          if (tid == 0) flag_store(fl + kFlagOutDone + it.t % kWM, (uint32_t)(it.t + 1));
        });
    }
  }
}

template <bool kOutBf16, int kRows>
__global__ __launch_bounds__(256, 2) void k_fused(Args a) {
  constexpr int kParts = D / kRows;
  __shared__ Lds<kRows> lds;
  __shared__ uint32_t bcast[4];
  const uint32_t xcd = xcc_id();
  if (xcd >= (uint32_t)kXcd) return;  // not an MI355X XCD id: take no part
  const int nh = (int)xcd < a.heads ? (a.heads - (int)xcd + kXcd - 1) / kXcd : 0;
  if (threadIdx.x == 0) {
    bcast[0] = 0;
    bcast[1] = atomicAdd(&a.ctrl->ticket[xcd], 1u);
  }
  __syncthreads();
  const int ticket = (int)bcast[1];
  __syncthreads();
  if (nh == 0) return;
  if (ticket < nh * kParts) {
    __builtin_amdgcn_s_setprio(3);
    state_role<kRows>(a, lds, bcast, (ticket / kParts) * kXcd + (int)xcd, ticket % kParts);
  } else {
    worker_role<kOutBf16, kRows>(a, lds, bcast, (int)xcd, nh);
  }
}

// Workgroups per XCC_ID value seen by one launch (the topology probe).
__device__ uint32_t g_xcc_seen[16];
__global__ void k_xcc_probe() {
  if (threadIdx.x == 0) atomicAdd(&g_xcc_seen[xcc_id()], 1u);
}

__global__ void k_fused_init(uint32_t* words, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) words[i] = 0;
}

// State-pass rows per workgroup: 16 (8 workgroups per head) keeps each
// sequential step short enough; 32 halves the state-pass workgroups but the
// longer step then limits the kernel (5.4 ms against 4.2 ms for the 60 s
// workload).
constexpr int kFusedRows = 16;

template <bool kOutBf16>
const void* fused_kernel() {
  return reinterpret_cast<const void*>(&k_fused<kOutBf16, kFusedRows>);
}


}  // namespace

int64_t fused_workspace_bytes(int64_t heads) {
  const int64_t h = heads < kXcd * kMaxHeadsPerXcd ? heads : kXcd * kMaxHeadsPerXcd;
  const int64_t ctrl = ((int64_t)sizeof(Ctrl) + kXcd * kMaxHeadsPerXcd * kFlagWords * 4 + 255) & ~int64_t{255};
  return ctrl + h * ring_head_bytes(kRing.wg, kRing.wm);
}

int fused_grid(bool out_bf16, int num_cus) {
  int pc = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&pc, out_bf16 ? fused_kernel<true>() : fused_kernel<false>(), 256,
                                                   0) != hipSuccess)
    return 0;
  // every XCD needs its state-pass workgroups and at least as many workers
  const int grid = pc * num_cus;
  return grid / kXcd >= 2 * kMaxHeadsPerXcd * (D / kFusedRows) ? grid : 0;
}

// The fused kernel hands every head to the XCD whose XCC_ID is h % 8 and
// counts on each XCD holding an equal share of the launch.  A one-time probe
// with the fused launch's size checks that the device deals workgroups that
// way: exactly ids 0-7, grid / 8 workgroups each (e.g. not a partition with
// fewer XCDs, whose ids would leave heads without workgroups).  Runs on the
// null stream and waits for it.
hipError_t fused_topology_ok(int grid, bool* ok) {
  *ok = false;
  uint32_t seen[16] = {};
  hipError_t e;
  if ((e = hipMemcpyToSymbol(HIP_SYMBOL(g_xcc_seen), seen, sizeof seen)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_xcc_probe, dim3((unsigned)grid), dim3(64), 0, nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = hipMemcpyFromSymbol(seen, HIP_SYMBOL(g_xcc_seen), sizeof seen)) != hipSuccess) return e;
  bool even = grid % kXcd == 0;
  for (int i = 0; i < 16; ++i) even = even && seen[i] == (i < kXcd ? (uint32_t)(grid / kXcd) : 0u);
  *ok = even;
  return hipSuccess;
}

const void* fused_error_word(const void* workspace) {
  return static_cast<const char*>(workspace) + offsetof(Ctrl, error);
}

hipError_t launch_fused(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* gamma,
                        const float* beta, const float* state_in, void* out, bool out_bf16,
                        float* state_out, void* workspace, int64_t heads, int64_t T, int S, float ks,
                        uint32_t spin_limit, int grid, hipStream_t st) {
  char* ws = static_cast<char*>(workspace);
  const int64_t group = kXcd * kMaxHeadsPerXcd;
  const int64_t ctrl_bytes = (int64_t)sizeof(Ctrl) + group * kFlagWords * 4;
  const int nwords = (int)(ctrl_bytes / 4);
  // heads are independent: groups of at most 16 heads, one launch each
  for (int64_t h0 = 0; h0 < heads; h0 += group) {
    const int64_t nh = heads - h0 < group ? heads - h0 : group;
    Args a;
    a.q = q + h0 * T * S * D;
    a.k = k + h0 * T * S * D;
    a.v = v + h0 * T * S * D;
    a.gamma = gamma + h0 * T;
    a.beta = beta + h0 * T;
    a.state_in = state_in ? state_in + h0 * D * D : nullptr;
    a.out = static_cast<char*>(out) + h0 * T * S * D * (out_bf16 ? 2 : 4);
    a.state_out = state_out + h0 * D * D;
    a.ctrl = reinterpret_cast<Ctrl*>(ws);
    a.flags = reinterpret_cast<uint32_t*>(ws + sizeof(Ctrl));
    a.ring = ws + ((ctrl_bytes + 255) & ~int64_t{255});
    a.heads = (int)nh;
    a.T = (int)T;
    a.S = S;
    a.ks = ks;
    a.spin_limit = spin_limit ? spin_limit : kSpinLimit;
    // the error word (word 0) is cleared for the first group only, so that
    // a wait that ran out in any group of the call stays reported
    const int skip = h0 == 0 ? 0 : 1;
    hipLaunchKernelGGL(k_fused_init, dim3((nwords + 255) / 256), dim3(256), 0, st,
                       reinterpret_cast<uint32_t*>(ws) + skip, nwords - skip);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    void* params[] = {&a};
    e = hipLaunchKernel(out_bf16 ? fused_kernel<true>() : fused_kernel<false>(), dim3((unsigned)grid), dim3(256),
                        params, 0, st);
    if (e != hipSuccess) {
      (void)hipGetLastError();  // do not leave the error for a later, unrelated check
      return e;
    }
  }
  return hipSuccess;
}

}  // namespace gdn
