// State pass of the frame-wise GDN, head dim 128:
//   M_t = M_{t-1} gamma_t (I - beta_t G_t) + beta_t U_t = gamma_t (M_{t-1} - beta_t X_t) + beta_t U_t,
//   X_t = M_{t-1} G_t,
// sequential over frames, float32 state (the decay gate multiplies the
// previous state and the delta rule corrects the residual: "SANA-WM: NVIDIA
// puts a one-minute world model on a single GPU", zhichai.net, section 1).
//
// Rows of M evolve independently (row i of M_t needs only row i of M_{t-1}),
// so each head's 128 rows are split over D/kRows workgroups that never talk
// to each other.  A workgroup keeps its rows of M in registers (float32
// master copy) and in LDS as a bf16 hi/lo pair, double-buffered.  The
// product X = M G runs on bf16 MFMA as three passes, Ghi*Mhi + Glo*Mhi +
// Ghi*Mlo, each split term exact to about 2^-17 relative, with float32
// accumulation; the dropped lo*lo term is ~2^-16 of a term that is itself a
// few per cent of M.  Computed transposed, X^T = G M^T (G_t = K_t^T K_t is
// symmetric, so its rows serve as its columns): wave w owns rows
// 32w .. 32w+31 of G (= columns of X) and all of the workgroup's rows of M,
// so each lane ends up owning 4 consecutive columns of one row of M.
//
// Two data forms.  Packed (gdn_packed.h): G_t, U_t and M_t in the order
// the waves read or write them, each wave access one contiguous block; this
// is what gdn_frame_fwd uses.  Plain: float32 row-major (the stage entry
// point); the bf16 split of G_t then happens here.  The backward pass reads
// packed G_t, U_t and writes M_t as float32 (kMf32).
//
// The per-frame data (this wave's G_t rows and U_t elements) streams
// through a ring of kDepth register buffers: frame t + kDepth is requested
// as soon as frame t's buffer is consumed.  The per-frame barrier only waits
// for LDS traffic, so those loads stay in flight across it.  Workgroups of
// one head are placed on one XCD (dispatch is round-robin over the 8 XCDs),
// so the G_t they all read comes from one L2.
//
// A launch covers frames [tb, te) of every head (a segment of the
// overlapped schedule, or all frames), starting from the state after frame
// tb - 1 in state_in and leaving the state after frame te - 1 in
// state_out; the float32 state is carried exactly, so a sequence cut into
// segments gives the same bits as one launch.
#include "gdn_common.h"
#include "gdn_launch.h"
#include "gdn_packed.h"

#include <type_traits>
#include <utility>

namespace gdn {
namespace {

constexpr int D = 128;
constexpr int kLdsW = D + 8;  // padded LDS row (bf16 elements)

template <int kRows, bool kPacked, int kDepth, bool kMf32>
__global__ __launch_bounds__(256, 1) void k2_state_d128(
    const void* __restrict__ Gin, const float* __restrict__ U, const float* __restrict__ gamma,
    const float* __restrict__ beta, const float* state_in, void* __restrict__ Mout,
    float* state_out, int heads, int T, int tb, int te, int64_t mT, int64_t mt0) {
  constexpr int kRB = kRows / 16;     // 16-row blocks of M per workgroup
  constexpr int kParts = D / kRows;   // workgroups per head
  // [buffer][hi|lo][row][col]
  __shared__ uint16_t Ml[2][2][kRows][kLdsW];

  const int id = blockIdx.x;
  const int xcd = id & 7, slot = id >> 3;
  const int part = slot % kParts;
  const int head = (slot / kParts) * 8 + xcd;
  if (head >= heads) return;
  const int r0 = part * kRows;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int n = l & 15, g = l >> 4;

  // This lane's elements of M: row r0 + 16rb + n, columns 32w + 16cb + 4g .. +3.
  auto row_of = [&](int rb) { return r0 + 16 * rb + n; };
  auto col_of = [&](int cb) { return 32 * w + 16 * cb + 4 * g; };

  const int64_t hoff = (int64_t)head * D * D;
  f32x4 Mreg[2][kRB];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
      Mreg[cb][rb] = state_in ? *reinterpret_cast<const f32x4*>(state_in + hoff + row_of(rb) * D + col_of(cb))
                              : (f32x4){0.f, 0.f, 0.f, 0.f};

  // hi/lo words of this lane's M elements (4 consecutive columns each)
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

  // Ring of per-frame register buffers: the A-operand fragments of G_t
  // (packed: hi/lo words; plain: raw floats) and this lane's U_t elements.
  u32x4 rgh[kDepth][2][4], rgl[kDepth][2][4];
  f32x4 rg32[kDepth][2][4][2];
  f32x4 ru[kDepth][2][kRB];

  auto load_frame = [&](auto jc, int t) {
    constexpr int j = decltype(jc)::value;
    if (t >= te) return;
    const int64_t fo = ((int64_t)head * mT + t - mt0) * D * D;  // map slot of frame t
    if constexpr (kPacked) {
      const char* Gp = static_cast<const char*>(Gin) + fo * 4;
      const char* Up = reinterpret_cast<const char*>(U) + fo * 4;
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
    } else {
      const float* Gt = static_cast<const float*>(Gin) + fo;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const float* p = Gt + (32 * w + 16 * cb + n) * D + 32 * kb + 8 * g;
          rg32[j][cb][kb][0] = *reinterpret_cast<const f32x4*>(p);
          rg32[j][cb][kb][1] = *reinterpret_cast<const f32x4*>(p + 4);
        }
      const float* Ut = U + fo;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          ru[j][cb][rb] = *reinterpret_cast<const f32x4*>(Ut + row_of(rb) * D + col_of(cb));
    }
  };

  // gamma_t, beta_t arrive through vector loads, a 64-frame window per lane
  // (lane i holds frame t0 + i) fetched one window ahead, and are read with
  // readlane.  Scalar loads here would share the LDS wait counter and stall
  // every frame's first LDS read on an L2 round trip.
  const float* gh = gamma + (int64_t)head * T;
  const float* bh = beta + (int64_t)head * T;
  auto win_load = [&](int t0, float& gv, float& bv) {
    const int tt = t0 + l;
    gv = tt < te ? gh[tt] : 0.f;
    bv = tt < te ? bh[tt] : 0.f;
  };
  float gwin, bwin, gnxt, bnxt;
  win_load(tb, gwin, bwin);
  win_load(tb + 64, gnxt, bnxt);

  [&]<int... js>(std::integer_sequence<int, js...>) {
    (load_frame(std::integral_constant<int, js>{}, tb + js), ...);
  }(std::make_integer_sequence<int, kDepth>{});
  lds_barrier();

  auto step = [&](auto jc, int t) {
    constexpr int j = decltype(jc)::value;
    const int buf = (t - tb) & 1;
    const int tw = (t - tb) & 63;
    const float gm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gwin), tw));
    const float bt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bwin), tw));
    if (tw == 63) {  // move to the next window and fetch the one after it
      gwin = gnxt;
      bwin = bnxt;
      win_load(t + 65, gnxt, bnxt);
    }

    u32x4 ahi[2][4], alo[2][4];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if constexpr (kPacked) {
          ahi[cb][kb] = rgh[j][cb][kb];
          alo[cb][kb] = rgl[j][cb][kb];
        } else {
          const u32x2 p0 = split2(rg32[j][cb][kb][0][0], rg32[j][cb][kb][0][1]);
          const u32x2 p1 = split2(rg32[j][cb][kb][0][2], rg32[j][cb][kb][0][3]);
          const u32x2 p2 = split2(rg32[j][cb][kb][1][0], rg32[j][cb][kb][1][1]);
          const u32x2 p3 = split2(rg32[j][cb][kb][1][2], rg32[j][cb][kb][1][3]);
          ahi[cb][kb] = (u32x4){p0.x, p1.x, p2.x, p3.x};
          alo[cb][kb] = (u32x4){p0.y, p1.y, p2.y, p3.y};
        }
      }
    f32x4 ureg[2][kRB];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) ureg[cb][rb] = ru[j][cb][rb];
    load_frame(jc, t + kDepth);  // refill this ring slot kDepth frames ahead

    f32x4 acc[2][kRB];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) acc[cb][rb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      // B operand: row 16rb + n of this workgroup's M (as M^T column), 8 bf16 at column 32kb + 8g.
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

    // acc[cb][rb][i] = X[row_of(rb)][col_of(cb) + i]
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

    if (Mout) {
      const int64_t fo = ((int64_t)head * mT + t - mt0) * D * D;  // map slot of frame t
      if constexpr (!kMf32) {
        char* Mp = static_cast<char*>(Mout) + fo * 4;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb) {
            *reinterpret_cast<u32x2*>(Mp + packed::m_chunk(row_of(rb), col_of(cb), 0)) = mh[cb][rb];
            *reinterpret_cast<u32x2*>(Mp + packed::m_chunk(row_of(rb), col_of(cb), 1)) = ml[cb][rb];
          }
      } else {
        float* Mt = static_cast<float*>(Mout) + fo;
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb)
            *reinterpret_cast<f32x4*>(Mt + row_of(rb) * D + col_of(cb)) = Mreg[cb][rb];
      }
    }
    lds_barrier();
  };

  for (int t0 = tb; t0 < te; t0 += kDepth) {
    [&]<int... js>(std::integer_sequence<int, js...>) {
      ((t0 + js < te ? step(std::integral_constant<int, js>{}, t0 + js) : void()), ...);
    }(std::make_integer_sequence<int, kDepth>{});
  }

#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
      *reinterpret_cast<f32x4*>(state_out + hoff + row_of(rb) * D + col_of(cb)) = Mreg[cb][rb];
}

template <int kRows, bool kPacked, int kDepth, bool kMf32>
hipError_t launch_rows(const void* G, const float* U, const float* gamma, const float* beta,
                       const float* state_in, void* M_out, float* state_out, int64_t heads,
                       int64_t T, int64_t tb, int64_t te, MapLayout ml, hipStream_t st) {
  // Workgroup ids are grouped so that the workgroups of a head share id % 8.
  const int64_t groups = (heads + 7) / 8;
  const unsigned grid = (unsigned)(groups * 8 * (D / kRows));
  hipLaunchKernelGGL((k2_state_d128<kRows, kPacked, kDepth, kMf32>), dim3(grid), dim3(256), 0, st, G, U, gamma,
                     beta, state_in, M_out, state_out, (int)heads, (int)T, (int)tb, (int)te, ml.T, ml.t0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_state_d128(const void* G, bool packed, const float* U, const float* gamma,
                             const float* beta, const float* state_in, void* M_out, bool m_f32,
                             float* state_out, int64_t heads, int64_t T, int64_t tb, int64_t te,
                             MapLayout ml, hipStream_t st) {
  if (!packed)
    return launch_rows<32, false, 2, true>(G, U, gamma, beta, state_in, M_out, state_out, heads, T, tb, te, ml, st);
  if (m_f32)
    return launch_rows<16, true, 2, true>(G, U, gamma, beta, state_in, M_out, state_out, heads, T, tb, te, ml, st);
  return launch_rows<16, true, 2, false>(G, U, gamma, beta, state_in, M_out, state_out, heads, T, tb, te, ml, st);
}

}  // namespace gdn
