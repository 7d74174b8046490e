// The whole frame-wise GDN forward (bf16 inputs, head dim 128) as one
// persistent kernel that overlaps the three stages:
//   build   G_t = K_t^T K_t, U_t = V_t^T K_t      (parallel over frames)
//   state   M_t = M_{t-1} gamma_t (I - beta_t G_t) + beta_t U_t   (sequential)
//   output  O_t = Q_t M_t^T                        (parallel over frames)
// (the recurrence of "SANA-WM: NVIDIA puts a one-minute world model on a
// single GPU", zhichai.net, section 1; one step per latent frame, bilibili
// cv49203711, fourth key point).
//
// Layout of the work.  MI355X has 8 XCDs, each with its own L2.  Head h is
// handled entirely by XCD h % 8: its state-pass workgroups and the workers
// that build its maps and form its outputs all run there, so every
// intermediate (G_t, U_t, M_t) passes between CUs through that XCD's L2 and
// never has to be written back to HBM.  A workgroup learns its XCD from the
// XCC_ID hardware register and takes a ticket from its XCD's counter: the
// first tickets become state-pass workgroups (kParts per head, each owning
// kRows rows of M, as in the standalone state pass), the rest become
// workers that pull build and output items from the XCD's queue.
//
// Hand-off between CUs of one XCD.  The L2 is shared by the XCD's CUs and
// the vector L1 is write-through, so a producer makes data visible by
// waiting for its stores to be acknowledged (s_waitcnt vmcnt(0)) and then
// setting a flag; a consumer reads the flag from L2 (device-scope relaxed
// load), invalidates its own L1 (buffer_inv sc0) and reads the data.
// Device-scope acquire/release would write back and invalidate whole L2s,
// which costs far more than the data itself, and is not needed within one
// XCD.
//
// Rings.  Per head: kWG slots for G_t/U_t and kWM slots for M_t, with
// monotonic per-slot flags (frame index + 1).  The queue order puts build
// items kLag frames ahead of the matching output items; with kLag > kPrefetch
// and enough slots, every wait depends only on items earlier in the queue
// or on state-pass progress that needs only such items, so the pipeline
// cannot deadlock even with a single worker.  Every wait is bounded: a wait
// that runs out sets an error word, every other wait then gives up too, the
// state pass writes NaN to state_out, and the kernel ends.
#include "frame_build.h"
#include "frame_output.h"
#include "gdn_common.h"
#include "gdn_launch.h"
#include "gdn_packed.h"

#include <type_traits>
#include <utility>

namespace gdn {
namespace {

constexpr int D = 128;
constexpr int kXcd = 8;
constexpr int kRows = 32;             // rows of M per state-pass workgroup
constexpr int kParts = D / kRows;     // state-pass workgroups per head
constexpr int kRB = kRows / 16;
constexpr int kPrefetch = 2;          // frames the state pass loads ahead
constexpr int kWG = 6;                // G/U ring slots per head
constexpr int kWM = 8;                // M ring slots per head
constexpr int kLag = 4;               // queue distance from build(t) to output(t)
constexpr int kMaxHeadsPerXcd = 2;
constexpr int kLdsW = D + 8;
constexpr uint32_t kSpinLimit = 1u << 22;  // polls (a few seconds) before a wait gives up

static_assert(kLag > kPrefetch && kWG >= kPrefetch + 2, "pipeline would stall");

// Control block (zeroed before every launch) followed by per-head flags.
struct Ctrl {
  uint32_t error;
  uint32_t pad0[31];
  uint32_t ticket[kXcd];
  uint32_t pad1[24];
  uint32_t queue[kXcd];
  uint32_t pad2[24];
};
// Per-head flag block.  The state pass publishes per wave (kParts x 4
// waves), so no extra barrier is needed to publish.
constexpr int kChainWaves = 4;
constexpr int kFlagGReady = 0;     // [kWG]                        frame + 1 of the G/U in the slot
constexpr int kFlagConsumed = 16;  // [kParts][kChainWaves]        frames whose G/U the wave has loaded
constexpr int kFlagMReady = 32;    // [kWM][kParts][kChainWaves]   frame + 1 of the wave's M rows in the slot
constexpr int kFlagOutDone = 160;  // [kWM]                        frame + 1 whose M the output has staged
constexpr int kFlagWords = 256;
static_assert(kFlagConsumed + kParts * kChainWaves <= kFlagMReady &&
              kFlagMReady + kWM * kParts * kChainWaves <= kFlagOutDone && kFlagOutDone + kWM <= kFlagWords,
              "flag block overlaps");

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

// Spin (one thread) until pred() holds; false if it never did or another
// wait already failed.
template <typename Pred>
__device__ bool spin_until(Ctrl* ctrl, Pred pred) {
  for (uint32_t i = 0; i < kSpinLimit; ++i) {
    if (pred()) return true;
    if ((i & 63) == 63 && flag_load(&ctrl->error)) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  __hip_atomic_store(&ctrl->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return false;
}

struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* gamma;
  const float* beta;
  const float* state_in;
  void* out;
  float* state_out;
  char* ring;       // per head: kWG x (Gp, Up) then kWM x Mp, 64 KB each
  Ctrl* ctrl;
  uint32_t* flags;  // per head kFlagWords
  int heads, T, S;
};

__host__ __device__ constexpr int64_t ring_head_bytes() { return int64_t{2 * kWG + kWM} * packed::kFrameBytes; }

struct Item {
  int kind;  // 0 build, 1 output
  int hl;    // head index within the XCD
  int t;     // frame
};

// Item i of an XCD with nh heads.  Slot k = i / nh holds one item per head:
// builds of frames 0..L-1, then alternately output(f) and build(f + L), then
// the last L outputs.
__device__ Item decode_item(int i, int nh, int T) {
  const int L = T < kLag ? T : kLag;
  const int k = i / nh, hl = i % nh;
  if (k < L) return {0, hl, k};
  const int j = k - L;
  if (j < 2 * (T - L)) return (j & 1) ? Item{0, hl, L + (j >> 1)} : Item{1, hl, j >> 1};
  return {1, hl, T - L + (j - 2 * (T - L))};
}

union __attribute__((aligned(16))) Lds {
  u32x4 build[build_lds_bytes<true>() / 16];
  uint16_t out[2][D][kOutLdsW];
  uint16_t chain[2][2][kRows][kLdsW];
};

// ---------------------------------------------------------------------------
// state pass: one workgroup owns rows [r0, r0 + kRows) of one head's M
// ---------------------------------------------------------------------------
// Each of the 4 waves keeps its own flags: at the top of step t it waits
// only for memory operations it issued during step t-1 (M_{t-1} stores, the
// loads of frame t-1+kPrefetch and the flag loads for this step), publishes
// M_{t-1} and its progress, and checks the flags it loaded a step ahead.
// The only barrier per step is the LDS hand-off of M between the waves.  A
// wave whose wait fails sets `abort` in LDS; after the barrier every wave
// sees it and all leave together.
__device__ void state_role(const Args& a, Lds& lds, uint32_t* bcast, int head, int part) {
  uint16_t (*Ml)[2][kRows][kLdsW] = lds.chain;
  const int T = a.T;
  const int r0 = part * kRows;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int n = l & 15, g = l >> 4;
  uint32_t* fl = a.flags + (int64_t)head * kFlagWords;
  char* ring = a.ring + head * ring_head_bytes();
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
  if (tid == 0) bcast[0] = 0;  // abort word

  // gamma/beta windows (see the standalone state pass)
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

  u32x4 rgh[kPrefetch][2][4], rgl[kPrefetch][2][4];
  f32x4 ru[kPrefetch][2][kRB];
  auto load_frame = [&](auto jc, int t) {
    constexpr int j = decltype(jc)::value;
    if (t >= T) return;
    const char* Gp = gp_slot(t);
    const char* Up = up_slot(t);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int unit = ((2 * w + cb) * 4 + kb) * 2;
        rgh[j][cb][kb] = *reinterpret_cast<const u32x4*>(Gp + (unit << 10) + 16 * l);
        rgl[j][cb][kb] = *reinterpret_cast<const u32x4*>(Gp + ((unit + 1) << 10) + 16 * l);
      }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
        ru[j][cb][rb] = *reinterpret_cast<const f32x4*>(Up + ((((r0 >> 4) + rb) * 8 + 2 * w + cb) << 10) + 16 * l);
  };

  // Prologue: wait for the first kPrefetch builds (every wave for itself).
  bool ok = true;
  if (l == 0) {
    const int need = T < kPrefetch ? T : kPrefetch;
    for (int u = 0; u < need && ok; ++u)
      ok = spin_until(a.ctrl, [&] { return flag_load(fl + kFlagGReady + u % kWG) >= (uint32_t)(u + 1); });
  }
  ok = __builtin_amdgcn_readfirstlane((int)ok) != 0;
  if (!ok) bcast[0] = 1;
  invalidate_l1();
  [&]<int... js>(std::integer_sequence<int, js...>) {
    (load_frame(std::integral_constant<int, js>{}, js), ...);
  }(std::make_integer_sequence<int, kPrefetch>{});
  // flags for step 0, loaded ahead (lane 0)
  uint32_t gflag = 0, oflag = 0;
  if (l == 0 && kPrefetch < T) gflag = flag_load(fl + kFlagGReady + kPrefetch % kWG);
  lds_barrier();
  ok = bcast[0] == 0;

  auto step = [&](auto jc, int t) {
    constexpr int j = decltype(jc)::value;
    // Everything this wave issued in step t-1 is complete after this wait.
    wait_stores();
    bool good = true;
    if (l == 0) {
      if (t > 0) flag_store(my_mready(t - 1), (uint32_t)t);
      flag_store(my_consumed, (uint32_t)(t + kPrefetch < T ? t + kPrefetch : T));
      const int tn = t + kPrefetch;
      if (tn < T && gflag < (uint32_t)(tn + 1))
        good = spin_until(a.ctrl, [&] { return flag_load(fl + kFlagGReady + tn % kWG) >= (uint32_t)(tn + 1); });
      if (good && t >= kWM && oflag < (uint32_t)(t - kWM + 1))
        good = spin_until(a.ctrl, [&] { return flag_load(fl + kFlagOutDone + t % kWM) >= (uint32_t)(t - kWM + 1); });
      // flags for step t + 1, in flight during this step
      if (t + 1 + kPrefetch < T) gflag = flag_load(fl + kFlagGReady + (t + 1 + kPrefetch) % kWG);
      if (t + 1 >= kWM) oflag = flag_load(fl + kFlagOutDone + (t + 1) % kWM);
    }
    good = __builtin_amdgcn_readfirstlane((int)good) != 0;
    if (good) {
      const int buf = t & 1;
      const int tw = t & 63;
      const float gm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gwin), tw));
      const float bt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bwin), tw));
      if (tw == 63) {
        gwin = gnxt;
        bwin = bnxt;
        win_load(t + 65, gnxt, bnxt);
      }
      u32x4 ahi[2][4], alo[2][4];
      f32x4 ureg[2][kRB];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          ahi[cb][kb] = rgh[j][cb][kb];
          alo[cb][kb] = rgl[j][cb][kb];
        }
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) ureg[cb][rb] = ru[j][cb][rb];
      }
      // refill this ring entry with frame t + kPrefetch (its build is done)
      invalidate_l1();
      load_frame(jc, t + kPrefetch);

      f32x4 acc[2][kRB];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) acc[cb][rb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        u32x4 bhi[kRB], blo[kRB];
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
          bhi[rb] = *reinterpret_cast<const u32x4*>(&Ml[buf][0][16 * rb + n][32 * kb + 8 * g]);
          blo[rb] = *reinterpret_cast<const u32x4*>(&Ml[buf][1][16 * rb + n][32 * kb + 8 * g]);
        }
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) acc[cb][rb] = mfma16x16x32(ahi[cb][kb], bhi[rb], acc[cb][rb]);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) acc[cb][rb] = mfma16x16x32(alo[cb][kb], bhi[rb], acc[cb][rb]);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) acc[cb][rb] = mfma16x16x32(ahi[cb][kb], blo[rb], acc[cb][rb]);
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
  };

  for (int t0 = 0; t0 < T && ok; t0 += kPrefetch) {
    [&]<int... js>(std::integer_sequence<int, js...>) {
      ((ok && t0 + js < T ? step(std::integral_constant<int, js>{}, t0 + js) : void()), ...);
    }(std::make_integer_sequence<int, kPrefetch>{});
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
template <bool kOutBf16>
__device__ void worker_role(const Args& a, Lds& lds, uint32_t* bcast, int xcd, int nh) {
  const int T = a.T, S = a.S;
  const int total = 2 * nh * T;
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
    char* ring = a.ring + head * ring_head_bytes();
    const int64_t fr = (int64_t)head * T + it.t;
    if (it.kind == 0) {
      // build(t): its G/U slot must have been loaded by every state-pass part
      if (tid == 0) {
        const uint32_t need = it.t >= kWG ? (uint32_t)(it.t - kWG + 1) : 0u;
        bcast[3] = spin_until(a.ctrl, [&] {
          uint32_t m = 0xffffffffu;
#pragma unroll
          for (int p = 0; p < kParts * kChainWaves; ++p) {
            const uint32_t c = flag_load(fl + kFlagConsumed + p);
            m = c < m ? c : m;
          }
          return m >= need;
        });
      }
      __syncthreads();
      if (!bcast[3]) return;
      char* gp = ring + (int64_t)(2 * (it.t % kWG)) * packed::kFrameBytes;
      float* up = reinterpret_cast<float*>(ring + (int64_t)(2 * (it.t % kWG) + 1) * packed::kFrameBytes);
      build_frame<true, 1>(a.k + fr * S * D, a.v + fr * S * D, S, lds.build, gp, up);
      wait_stores();
      __syncthreads();
      if (tid == 0) flag_store(fl + kFlagGReady + it.t % kWG, (uint32_t)(it.t + 1));
    } else {
      // output(t): every part's rows of M_t must be in the ring
      if (tid == 0) {
        bcast[3] = spin_until(a.ctrl, [&] {
          uint32_t m = 0xffffffffu;
#pragma unroll
          for (int p = 0; p < kParts * kChainWaves; ++p) {
            const uint32_t c = flag_load(fl + kFlagMReady + (it.t % kWM) * kParts * kChainWaves + p);
            m = c < m ? c : m;
          }
          return m >= (uint32_t)(it.t + 1);
        });
      }
      __syncthreads();
      if (!bcast[3]) return;
      invalidate_l1();
      const char* mp = ring + (int64_t)(2 * kWG + it.t % kWM) * packed::kFrameBytes;
      void* of = static_cast<char*>(a.out) + fr * S * D * (kOutBf16 ? 2 : 4);
      output_frame<true, kOutBf16, 2>(a.q + fr * S * D, mp, of, S, lds.out, [&] {
        if (tid == 0) flag_store(fl + kFlagOutDone + it.t % kWM, (uint32_t)(it.t + 1));
      });
    }
  }
}

template <bool kOutBf16>
__global__ __launch_bounds__(256, 1) void k_pipeline(Args a) {
  __shared__ Lds lds;
  __shared__ uint32_t bcast[4];
  const uint32_t xcd = xcc_id();
  if (xcd >= (uint32_t)kXcd) return;  // not an MI355X XCD id: take no part
  const int nh = (int)xcd < a.heads ? (a.heads - (int)xcd + kXcd - 1) / kXcd : 0;
  if (threadIdx.x == 0) {
    bcast[0] = 1;
    bcast[1] = atomicAdd(&a.ctrl->ticket[xcd], 1u);
  }
  __syncthreads();
  const int ticket = (int)bcast[1];
  __syncthreads();
  if (nh == 0) return;
  if (ticket < nh * kParts) {
    state_role(a, lds, bcast, (ticket / kParts) * kXcd + (int)xcd, ticket % kParts);
  } else {
    worker_role<kOutBf16>(a, lds, bcast, (int)xcd, nh);
  }
}

__global__ void k_pipeline_init(uint32_t* words, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) words[i] = 0;
}

}  // namespace

int64_t pipeline_workspace_bytes(int64_t heads) {
  return (int64_t)sizeof(Ctrl) + heads * kFlagWords * 4 + 256 + heads * ring_head_bytes();
}

bool pipeline_supported(int64_t heads, int64_t S) {
  return heads >= 1 && heads <= int64_t{kXcd} * kMaxHeadsPerXcd && S >= 1;
}

hipError_t launch_pipeline(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* gamma,
                           const float* beta, const float* state_in, void* out, bool out_bf16,
                           float* state_out, void* workspace, int64_t heads, int64_t T, int S,
                           int num_cus, hipStream_t st, hipEvent_t* ev) {
  char* ws = static_cast<char*>(workspace);
  Args a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.gamma = gamma;
  a.beta = beta;
  a.state_in = state_in;
  a.out = out;
  a.state_out = state_out;
  a.ctrl = reinterpret_cast<Ctrl*>(ws);
  a.flags = reinterpret_cast<uint32_t*>(ws + sizeof(Ctrl));
  const int64_t ctrl_bytes = (int64_t)sizeof(Ctrl) + heads * kFlagWords * 4;
  a.ring = ws + ((ctrl_bytes + 255) & ~int64_t{255});
  a.heads = (int)heads;
  a.T = (int)T;
  a.S = S;
  const int nwords = (int)(ctrl_bytes / 4);
  if (ev && hipEventRecord(ev[0], st) != hipSuccess) return hipErrorUnknown;
  hipLaunchKernelGGL(k_pipeline_init, dim3((nwords + 255) / 256), dim3(256), 0, st,
                     reinterpret_cast<uint32_t*>(ws), nwords);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev && hipEventRecord(ev[1], st) != hipSuccess) return hipErrorUnknown;
  // one workgroup per CU: every role must be resident at once
  const unsigned grid = (unsigned)num_cus;
  if (out_bf16)
    hipLaunchKernelGGL(k_pipeline<true>, dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_pipeline<false>, dim3(grid), dim3(256), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev && (hipEventRecord(ev[2], st) != hipSuccess || hipEventRecord(ev[3], st) != hipSuccess))
    return hipErrorUnknown;
  return hipSuccess;
}

}  // namespace gdn
