// Backward pass of the frame-wise GDN, head dim 128: the reverse-time state
// pass, the reduction of its dgamma/dbeta partial sums, and the key and
// value gradients (with the symmetric G-gradient term).  dq and
// P_t = dO_t^T Q_t reuse the forward's output and build kernels;
// gdn_api.cpp orders the launches.  Every launcher covers frames [t0, t1)
// of every head, so the schedule can cut the sequence into segments; results
// do not depend on the cut.
//
// Reverse-time state pass.  The forward
// M_t = gamma_t (M_{t-1} - beta_t M_{t-1} G_t) + beta_t U_t, O_t = Q_t M_t^T
// (the recurrence of "SANA-WM: NVIDIA puts a one-minute world model on a
// single GPU", zhichai.net, section 1) has, for the total gradient Lambda_t
// reaching M_t,
//   Lambda_t = L_t + P_t,          P_t = dO_t^T Q_t,  L_{T-1} = dM_T,
//   X_t      = Lambda_t G_t,
//   L_{t-1}  = gamma_t (Lambda_t - beta_t X_t)      (G_t is symmetric),
// and the gradient of the initial state is L_{-1}.  A launch over frames
// [tb, te) starts from L_{te-1} in d_state_out and leaves L_{tb-1} in
// d_state_in (P_{tb-1} not yet added: the next launch adds it).  Per frame it
// also writes LB_t = beta_t Lambda_t (the frame's dU_t, which the gradient
// kernel uses) and, over its rows, partial sums of
//   dgamma_t = < Lambda_t - beta_t X_t, M_{t-1} >,
//   dbeta_t  = < Lambda_t, U_t > - gamma_t < X_t, M_{t-1} >.
// It runs like the forward state pass, frames in reverse: rows of Lambda
// evolve independently (row i of L_{t-1} needs only row i of Lambda_t), so
// each head's 128 rows are split over workgroups of kBwdRows rows.
// X = Lambda G runs on bf16 MFMA in three passes (Ghi*Lhi + Glo*Lhi +
// Ghi*Llo; G_t and U_t in the forward's packed forms) with the float32
// running value in registers and its hi/lo pair in LDS; the per-frame inputs
// (this wave's G_t rows, and the workgroup's rows of U_t, M_{t-1} and
// P_{t-1}) stream through a two-frame register ring.  The partial sums are
// kept per 16-row block and reduced in a fixed order (lanes, then waves,
// then blocks), so the results are deterministic and do not depend on
// kBwdRows.
#include "frame_output.h"
#include "gdn_common.h"
#include "gdn_backward.h"
#include "gdn_launch.h"
#include "gdn_packed.h"

#include <type_traits>
#include <utility>

namespace gdn {
namespace {

constexpr int D = 128;
constexpr int kLdsW = D + 8;
constexpr int kDepth = 2;
// rows of the state gradient per workgroup of the reverse-time pass (32 rows,
// half the workgroups, measured slower: the pass is on the critical path)
constexpr int kBwdRows = 16;
// waves per workgroup of the key/value-gradient kernel (its LDS allows one
// workgroup per CU; 8 waves must fit 256 registers, spill and are slower)
constexpr int kDkvWaves = 4;
static_assert(kBwdParts == D / 16, "partial sums are kept per 16-row block");

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// a * b rounded, then + c rounded: kept apart (no fused multiply-add)
__device__ __forceinline__ float mul_then_add(float a, float b, float c) {
#pragma clang fp contract(off)
  return a * b + c;
}

template <int kRows>
__global__ __launch_bounds__(256, 1) void k2_state_bwd_d128(
    const float* __restrict__ G, const float* __restrict__ U, const float* __restrict__ P,
    const float* __restrict__ M_all, const float* m0, const float* __restrict__ gamma,
    const float* __restrict__ beta, const float* d_state_out, float* __restrict__ LB,
    float* __restrict__ partials, float* d_state_in, int heads, int T, int tb, int te) {
  constexpr int kRB = kRows / 16;    // 16-row blocks per workgroup
  constexpr int kParts = D / kRows;  // workgroups per head
  __shared__ uint16_t Ml[2][2][kRows][kLdsW];  // [buffer][hi|lo][row][col]
  __shared__ float red[2][4][kRB][2];         // [buffer][wave][row block][dgamma, dbeta]

  const int id = blockIdx.x;
  const int xcd = id & 7, slot = id >> 3;
  const int part = slot % kParts;
  const int head = (slot / kParts) * 8 + xcd;
  if (head >= heads) return;
  const int r0 = part * kRows;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int n = l & 15, g = l >> 4;
  // this lane's elements: rows row_of(rb), columns col_of(cb) .. +3
  auto row_of = [&](int rb) { return r0 + 16 * rb + n; };
  auto col_of = [&](int cb) { return 32 * w + 16 * cb + 4 * g; };
  const int64_t hoff = (int64_t)head * D * D;
  auto frame = [&](int t) { return ((int64_t)head * T + t) * D * D; };

  f32x4 Lr[2][kRB];  // the running gradient
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const int e = row_of(rb) * D + col_of(cb);
      const f32x4 d0 = d_state_out ? *reinterpret_cast<const f32x4*>(d_state_out + hoff + e)
                                   : (f32x4){0.f, 0.f, 0.f, 0.f};
      Lr[cb][rb] = d0 + *reinterpret_cast<const f32x4*>(P + frame(te - 1) + e);  // Lambda_{te-1}
    }
  auto put_lds = [&](int buf) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        const u32x2 p0 = split2(Lr[cb][rb][0], Lr[cb][rb][1]), p1 = split2(Lr[cb][rb][2], Lr[cb][rb][3]);
        *reinterpret_cast<u32x2*>(&Ml[buf][0][16 * rb + n][col_of(cb)]) = (u32x2){p0.x, p1.x};
        *reinterpret_cast<u32x2*>(&Ml[buf][1][16 * rb + n][col_of(cb)]) = (u32x2){p0.y, p1.y};
      }
  };
  put_lds(0);

  // Ring: this wave's G_t rows 32w .. 32w+31 (the A operand, hi/lo words of
  // the packed form) and the workgroup's rows of U_t (packed form), M_{t-1}
  // and P_{t-1} (this lane's elements; gdn_packed.h gives the packed units).
  u32x4 rgh[kDepth][2][4], rgl[kDepth][2][4];
  f32x4 ru[kDepth][2][kRB], rm[kDepth][2][kRB], rp[kDepth][2][kRB];
  auto load_frame = [&](auto jc, int t) {
    constexpr int j = decltype(jc)::value;
    if (t < tb) return;
    const char* Gp = reinterpret_cast<const char*>(G + frame(t));
    const char* Up = reinterpret_cast<const char*>(U + frame(t));
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int unit = ((2 * w + cb) * 4 + kb) * 2;
        rgh[j][cb][kb] = *reinterpret_cast<const u32x4*>(Gp + (unit << 10) + 16 * l);
        rgl[j][cb][kb] = *reinterpret_cast<const u32x4*>(Gp + ((unit + 1) << 10) + 16 * l);
      }
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const float* Mp = t > 0 ? M_all + frame(t - 1) : (m0 ? m0 + hoff : nullptr);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        const int e = row_of(rb) * D + col_of(cb);
        ru[j][cb][rb] = *reinterpret_cast<const f32x4*>(Up + ((((r0 >> 4) + rb) * 8 + 2 * w + cb) << 10) + 16 * l);
        rm[j][cb][rb] = Mp ? *reinterpret_cast<const f32x4*>(Mp + e) : zero;
        rp[j][cb][rb] = t > tb ? *reinterpret_cast<const f32x4*>(P + frame(t - 1) + e) : zero;
      }
  };

  // gamma/beta: lane i holds frame te-1-(64k+i) of window k (vector loads,
  // read with readlane; scalar loads would share the LDS wait counter)
  const float* gh = gamma + (int64_t)head * T;
  const float* bh = beta + (int64_t)head * T;
  auto win_load = [&](int i0, float& gv, float& bv) {
    const int t = te - 1 - (i0 + l);
    gv = t >= tb ? gh[t] : 0.f;
    bv = t >= tb ? bh[t] : 0.f;
  };
  float gwin, bwin, gnxt, bnxt;
  win_load(0, gwin, bwin);
  win_load(64, gnxt, bnxt);

  [&]<int... js>(std::integer_sequence<int, js...>) {
    (load_frame(std::integral_constant<int, js>{}, te - 1 - js), ...);
  }(std::make_integer_sequence<int, kDepth>{});
  lds_barrier();

  auto step = [&](auto jc, int i) {
    constexpr int j = decltype(jc)::value;
    const int t = te - 1 - i;
    const int buf = i & 1;
    const int iw = i & 63;
    const float gm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gwin), iw));
    const float bt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bwin), iw));
    if (iw == 63) {
      gwin = gnxt;
      bwin = bnxt;
      win_load(i + 65, gnxt, bnxt);
    }

    u32x4 ahi[2][4], alo[2][4];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        ahi[cb][kb] = rgh[j][cb][kb];
        alo[cb][kb] = rgl[j][cb][kb];
      }
    f32x4 uu[2][kRB], mm[2][kRB], pp[2][kRB];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        uu[cb][rb] = ru[j][cb][rb];
        mm[cb][rb] = rm[j][cb][rb];
        pp[cb][rb] = rp[j][cb][rb];
      }
    load_frame(jc, t - kDepth);  // refill this ring slot kDepth frames ahead

    // X^T = G Lambda^T: acc[cb][rb][i] = X[row_of(rb)][col_of(cb) + i]
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

    float* LBt = LB + frame(t);
    float dg[kRB], db[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      dg[rb] = 0.f;
      db[rb] = 0.f;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        f32x4 lb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lam = Lr[cb][rb][e], x = acc[cb][rb][e];
          lb[e] = bt * lam;
          dg[rb] = fmaf(fmaf(-bt, x, lam), mm[cb][rb][e], dg[rb]);
          db[rb] = fmaf(lam, uu[cb][rb][e], fmaf(-gm * x, mm[cb][rb][e], db[rb]));
          // L_{t-1} = gamma (Lambda - beta X), rounded, then + P_{t-1} (zero at
          // t = tb): the same two roundings as when a sequence is cut here and
          // the next launch or call adds P_{t-1} to the state gradient it is given
          Lr[cb][rb][e] = mul_then_add(gm, fmaf(-bt, x, lam), pp[cb][rb][e]);
        }
        *reinterpret_cast<f32x4*>(LBt + row_of(rb) * D + col_of(cb)) = lb;
      }
      dg[rb] = wave_sum(dg[rb]);
      db[rb] = wave_sum(db[rb]);
    }
    if (l == 0) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        red[buf][w][rb][0] = dg[rb];
        red[buf][w][rb][1] = db[rb];
      }
    }
    put_lds(buf ^ 1);
    lds_barrier();
    if (tid < kRB) {  // one partial pair per 16-row block, whatever the workgroup size
      const int rb = tid;
      float* pr = partials + (((int64_t)head * T + t) * kBwdParts + (r0 >> 4) + rb) * 2;
      pr[0] = ((red[buf][0][rb][0] + red[buf][1][rb][0]) + red[buf][2][rb][0]) + red[buf][3][rb][0];
      pr[1] = ((red[buf][0][rb][1] + red[buf][1][rb][1]) + red[buf][2][rb][1]) + red[buf][3][rb][1];
    }
  };

  const int nf = te - tb;
  for (int i0 = 0; i0 < nf; i0 += kDepth) {
    [&]<int... js>(std::integer_sequence<int, js...>) {
      ((i0 + js < nf ? step(std::integral_constant<int, js>{}, i0 + js) : void()), ...);
    }(std::make_integer_sequence<int, kDepth>{});
  }
  // after frame tb the running value is L_{tb-1} (the gradient of the
  // initial state when tb = 0)
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
      *reinterpret_cast<f32x4*>(d_state_in + hoff + row_of(rb) * D + col_of(cb)) = Lr[cb][rb];
}

__global__ void k_bwd_reduce(const float* __restrict__ partials, float* __restrict__ dgamma,
                             float* __restrict__ dbeta, int64_t frames) {
  const int64_t f = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (f >= frames) return;
  const float* p = partials + f * kBwdParts * 2;
  float sg = 0.f, sb = 0.f;
  for (int i = 0; i < kBwdParts; ++i) {
    sg += p[2 * i];
    sb += p[2 * i + 1];
  }
  dgamma[f] = sg;
  dbeta[f] = sb;
}

// Key and value gradients for the tokens of one frame (or one token part of
// it, in launches of a few frames):
//   dk_t = V_t LB_t + K_t S_t,   dv_t = K_t LB_t^T,
//   S_t = -gamma_t (A + A^T),    A = M_{t-1}^T LB_t
// for keys used as given; when the forward scaled them by ks inside its
// build, the gradients with respect to the unscaled keys are
// dk_t = ks V_t LB_t + ks^2 K_t S_t and dv_t = ks K_t LB_t^T: ks LB_t is
// staged in place of LB_t (so A and the S_t formed from it pick up one ks)
// and S_t is multiplied by ks once more.
// (K_t S_t is K_t (dG_t + dG_t^T) with dG_t = -gamma_t beta_t M_{t-1}^T Lambda_t;
// LB_t = beta_t Lambda_t carries beta).  LDS holds two 128 x 128 matrices as
// bf16 hi/lo planes (2 x 69.6 KB, so one workgroup per CU), which carry them
// to about 2^-17 relative: LB_t^T throughout, and in the second slot first
// M_{t-1}, then S_t.
//  * A on bf16 MFMA in three passes (Mhi*LBhi + Mlo*LBhi + Mhi*LBlo), each
//    wave taking 128 / kWaves rows: its A operand (M_{t-1} read down columns)
//    comes from transposed LDS reads of the row-major staged M, its B operand
//    from rows of the staged LB^T.  A then goes through LDS (as float32, in
//    the slot of M) for A + A^T, and S_t is split and staged.  With a zero
//    initial state, S_0 = 0.
//  * dk: one 256-term reduction per element, 128 terms over the rows of LB_t
//    (A = V tile, B = staged LB^T rows) and then 128 over those of S_t
//    (A = K tile, B = staged S rows), in one accumulator; output column
//    sigma(nb, n) as in the output kernel (frame_output.h), 16-byte stores.
//  * dv, computed transposed as dv^T = LB_t K_t^T: A = rows of LB_t, which
//    are columns of the staged LB^T, fetched with transposed LDS reads (two
//    per fragment), and B = the K tile already in registers for dk.  A lane
//    then holds 4 consecutive value dims of one token: 16-byte stores.
// The token tiling and global access patterns are the output kernel's: a
// wave takes 32-token tiles of V and K rows as MFMA operands.
template <int kDepth, int kWaves>
__global__ __launch_bounds__(64 * kWaves, 1) void k_dkv_d128(const uint16_t* __restrict__ V,
                                                   const uint16_t* __restrict__ K, const float* __restrict__ LB,
                                                   const float* __restrict__ M_all, const float* m0,
                                                   const float* __restrict__ gamma, float ks, float* __restrict__ dk,
                                                   float* __restrict__ dv, int S, int64_t T, int t0, int nt,
                                                   int nsplit) {
  // [LB^T | M_{t-1}, then S][hi | lo][LDS row][column]
  __shared__ __attribute__((aligned(16))) uint16_t Ml[2][2][D][kOutLdsW];
  constexpr int kThreads = 64 * kWaves;
  constexpr int kAB = 8 / kWaves;  // 16-row blocks of A per wave
  static_assert(kWaves == 4 || kWaves == 8, "4 or 8 waves");
  const int jf = blockIdx.x / nsplit, part = blockIdx.x % nsplit;
  const int head = jf / nt, t = t0 + jf % nt;
  const int64_t f = (int64_t)head * T + t;
  const int s0 = (int)((int64_t)part * S / nsplit), s1 = (int)((int64_t)(part + 1) * S / nsplit);
  const int ns = s1 - s0;
  const int64_t in_off = (f * (int64_t)S + s0) * D;
  const uint16_t* Vf = V + in_off;
  const uint16_t* Kf = K + in_off;
  float* dkf = dk + in_off;
  float* dvf = dv + in_off;
  const float* LBt = LB + f * D * D;
  const float* Mp = t > 0 ? M_all + (f - 1) * D * D : (m0 ? m0 + (int64_t)head * D * D : nullptr);
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int n = l & 15, g = l >> 4;

  // LDS row lds_row(r) of a staged matrix holds its row r (output column
  // sigma, as in the output kernel): staged LB^T row c is column c of LB.
  // M_{t-1} is staged row-major with natural rows.  All 16-byte loads of
  // LB_t and M_{t-1} are issued before the first is used.
  constexpr int kLoads = D * D / 4 / kThreads;
  f32x4 lvs[kLoads], mvs[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) lvs[i] = *reinterpret_cast<const f32x4*>(LBt + 4 * (tid + kThreads * i));
  if (Mp) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) mvs[i] = *reinterpret_cast<const f32x4*>(Mp + 4 * (tid + kThreads * i));
  }
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int idx = tid + kThreads * i;
    const int r = idx >> 5, c4 = (idx & 31) * 4;
    const f32x4 lv = lvs[i] * ks;
    const u32x2 p0 = split2(lv[0], lv[1]), p1 = split2(lv[2], lv[3]);
    const uint32_t hi[2] = {p0.x, p1.x}, lo[2] = {p0.y, p1.y};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rho = lds_row<false>(c4 + e);
      Ml[0][0][rho][r] = (uint16_t)(hi[e >> 1] >> (16 * (e & 1)));
      Ml[0][1][rho][r] = (uint16_t)(lo[e >> 1] >> (16 * (e & 1)));
    }
    if (Mp) {
      const f32x4 mv = mvs[i];
      const u32x2 q0 = split2(mv[0], mv[1]), q1 = split2(mv[2], mv[3]);
      *reinterpret_cast<u32x2*>(&Ml[1][0][r][c4]) = (u32x2){q0.x, q1.x};
      *reinterpret_cast<u32x2*>(&Ml[1][1][r][c4]) = (u32x2){q0.y, q1.y};
    } else {
      const int rs = lds_row<false>(r);  // S_0 = 0
      *reinterpret_cast<u32x2*>(&Ml[1][0][rs][c4]) = (u32x2){0u, 0u};
      *reinterpret_cast<u32x2*>(&Ml[1][1][rs][c4]) = (u32x2){0u, 0u};
    }
  }
  __syncthreads();
  if (Mp) {
    // A = M^T LB: wave w takes the row blocks kAB w .. kAB w + kAB - 1; lane
    // (n, g) of block (ab, bb) ends with A[16(kAB w + ab) + 4g + i][16bb + n]
    f32x4 acc[kAB][8];
#pragma unroll
    for (int ab = 0; ab < kAB; ++ab)
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) acc[ab][bb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      // A operand (ab, kb): lane (m, g) needs M[32kb + 8g + j][16(kAB w + ab) + m],
      // j = 0..7; as a source of the transposed read, lane (n, g) names row
      // 32kb + 8g + 4h + n/4 at columns 16(kAB w + ab) + 4(n%4) .. +3.
      u32x4 ah[kAB], al[kAB];
#pragma unroll
      for (int ab = 0; ab < kAB; ++ab) {
        const int r0 = 32 * kb + 8 * g + (n >> 2), c = 16 * (kAB * w + ab) + 4 * (n & 3);
        const u32x2 h0 = lds_read_tr16(&Ml[1][0][r0][c]), h1 = lds_read_tr16(&Ml[1][0][r0 + 4][c]);
        const u32x2 l0 = lds_read_tr16(&Ml[1][1][r0][c]), l1 = lds_read_tr16(&Ml[1][1][r0 + 4][c]);
        ah[ab] = (u32x4){h0.x, h0.y, h1.x, h1.y};
        al[ab] = (u32x4){l0.x, l0.y, l1.x, l1.y};
      }
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) {
        // B operand (kb, bb): lane (n, g) needs LB[32kb + 8g + j][16bb + n], a row of LB^T
        const int rho = lds_row<false>(16 * bb + n);
        const u32x4 bh = *reinterpret_cast<const u32x4*>(&Ml[0][0][rho][32 * kb + 8 * g]);
        const u32x4 bl = *reinterpret_cast<const u32x4*>(&Ml[0][1][rho][32 * kb + 8 * g]);
#pragma unroll
        for (int ab = 0; ab < kAB; ++ab) {
          acc[ab][bb] = mfma16x16x32(ah[ab], bh, acc[ab][bb]);
          acc[ab][bb] = mfma16x16x32(al[ab], bh, acc[ab][bb]);
          acc[ab][bb] = mfma16x16x32(ah[ab], bl, acc[ab][bb]);
        }
      }
    }
    __syncthreads();  // every wave is done with M: A takes its slot as float32
    constexpr int kAw = D + 4;  // 16-byte rows (128 x 528 B fit in the 69.6 KB slot)
    float (*As)[kAw] = reinterpret_cast<float (*)[kAw]>(&Ml[1][0][0][0]);
#pragma unroll
    for (int ab = 0; ab < kAB; ++ab)
#pragma unroll
      for (int bb = 0; bb < 8; ++bb)
#pragma unroll
        for (int i = 0; i < 4; ++i) As[16 * (kAB * w + ab) + 4 * g + i][16 * bb + n] = acc[ab][bb][i];
    __syncthreads();
    const float ng = ks * -gamma[f];  // staged LB carries one ks already: S picks up ks^2
    u32x2 sh[D * D / 4 / kThreads], sl[D * D / 4 / kThreads];
#pragma unroll
    for (int jj = 0; jj < D * D / 4 / kThreads; ++jj) {
      const int idx = tid + kThreads * jj, r = idx >> 5, c4 = (idx & 31) * 4;
      const f32x4 ar = *reinterpret_cast<const f32x4*>(&As[r][c4]);
      float sv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[e] = ng * (ar[e] + As[c4 + e][r]);
      const u32x2 q0 = split2(sv[0], sv[1]), q1 = split2(sv[2], sv[3]);
      sh[jj] = (u32x2){q0.x, q1.x};
      sl[jj] = (u32x2){q0.y, q1.y};
    }
    __syncthreads();  // A is read: S takes the slot
#pragma unroll
    for (int jj = 0; jj < D * D / 4 / kThreads; ++jj) {
      const int idx = tid + kThreads * jj, r = idx >> 5, c4 = (idx & 31) * 4;
      const int rs = lds_row<false>(r);
      *reinterpret_cast<u32x2*>(&Ml[1][0][rs][c4]) = sh[jj];
      *reinterpret_cast<u32x2*>(&Ml[1][1][rs][c4]) = sl[jj];
    }
    __syncthreads();
  }

  constexpr int kTile = kOutTile;
  const int ntiles = (ns + kTile - 1) / kTile;
  // A operands of a 32-token tile: lane (m, g) holds tokens tok0 + 16rb + m,
  // dims 32kb + 8g .. +7 of V (av) and of K (ak)
  auto load_a = [&](int tile, u32x4 (&av)[2][4], u32x4 (&ak)[2][4]) {
    const int tok0 = tile * kTile;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int s = tok0 + 16 * rb + n;
      const bool in = tile < ntiles && s < ns;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int64_t o = (int64_t)s * D + 32 * kb + 8 * g;
        av[rb][kb] = in ? *reinterpret_cast<const u32x4*>(Vf + o) : (u32x4){0u, 0u, 0u, 0u};
        ak[rb][kb] = in ? *reinterpret_cast<const u32x4*>(Kf + o) : (u32x4){0u, 0u, 0u, 0u};
      }
    }
  };
  constexpr int kRing = kDepth + 1;
  u32x4 rv[kRing][2][4], rk[kRing][2][4];
  auto tile_body = [&](auto jc, int tile) {
    constexpr int jb = decltype(jc)::value;
    const int tok0 = tile * kTile;
    load_a(tile + kWaves * kDepth, rv[(jb + kDepth) % kRing], rk[(jb + kDepth) % kRing]);
    {  // dk = V LB + K S
      f32x4 acc[2][8];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) acc[rb][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          u32x4(&a)[2][4] = m == 0 ? rv[jb] : rk[jb];
          u32x4 bh[4], bl[4];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            bh[kb] = *reinterpret_cast<const u32x4*>(&Ml[m][0][nb * 16 + n][32 * kb + 8 * g]);
            bl[kb] = *reinterpret_cast<const u32x4*>(&Ml[m][1][nb * 16 + n][32 * kb + 8 * g]);
          }
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
              acc[rb][nb] = mfma16x16x32(a[rb][kb], bh[kb], acc[rb][nb]);
              acc[rb][nb] = mfma16x16x32(a[rb][kb], bl[kb], acc[rb][nb]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // lane (n, g), register i of block nb: dk[tok0 + 16rb + 4g + i][sigma(nb, n)]
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = tok0 + 16 * rb + 4 * g + i;
          if (s >= ns) continue;
          float* o = dkf + (int64_t)s * D + 4 * n;
          st_nt(reinterpret_cast<f32x4*>(o), (f32x4){acc[rb][0][i], acc[rb][1][i], acc[rb][2][i], acc[rb][3][i]});
          st_nt(reinterpret_cast<f32x4*>(o + 64),
                (f32x4){acc[rb][4][i], acc[rb][5][i], acc[rb][6][i], acc[rb][7][i]});
        }
    }
    {  // dv^T = LB K^T
      f32x4 acc[2][8];  // [token block rb][value-dim block ib]
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int ib = 0; ib < 8; ++ib) acc[rb][ib] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ib = 0; ib < 8; ++ib) {
        // A fragment (ib, kb): lane (m, g) needs LB[16ib + m][32kb + 8g + j],
        // j = 0..7, i.e. staged LB^T rows 32kb + 8g + j at column 16ib + m.
        // As a source of the transposed read, lane (n, g) names row
        // 32kb + 8g + 4h + n/4 at columns 16ib + 4(n%4) .. +3 (h: j = 4h .. 4h+3).
        u32x4 ah[4], al[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const int r0 = lds_row<false>(32 * kb + 8 * g + (n >> 2));
          const int r1 = lds_row<false>(32 * kb + 8 * g + 4 + (n >> 2));
          const int c = 16 * ib + 4 * (n & 3);
          const u32x2 h0 = lds_read_tr16(&Ml[0][0][r0][c]), h1 = lds_read_tr16(&Ml[0][0][r1][c]);
          const u32x2 l0 = lds_read_tr16(&Ml[0][1][r0][c]), l1 = lds_read_tr16(&Ml[0][1][r1][c]);
          ah[kb] = (u32x4){h0.x, h0.y, h1.x, h1.y};
          al[kb] = (u32x4){l0.x, l0.y, l1.x, l1.y};
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            acc[rb][ib] = mfma16x16x32(ah[kb], rk[jb][rb][kb], acc[rb][ib]);
            acc[rb][ib] = mfma16x16x32(al[kb], rk[jb][rb][kb], acc[rb][ib]);
          }
        __builtin_amdgcn_sched_barrier(0);
      }
      // lane (n, g) holds dv^T[16ib + 4g + i][tok0 + 16rb + n] in acc[rb][ib][i]
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int s = tok0 + 16 * rb + n;
        if (s >= ns) continue;
#pragma unroll
        for (int ib = 0; ib < 8; ++ib)
          st_nt(reinterpret_cast<f32x4*>(dvf + (int64_t)s * D + 16 * ib + 4 * g), acc[rb][ib]);
      }
    }
  };
  [&]<int... js>(std::integer_sequence<int, js...>) {
    (load_a(w + kWaves * js, rv[js], rk[js]), ...);
  }(std::make_integer_sequence<int, kDepth>{});
  for (int tile0 = w; tile0 < ntiles; tile0 += kWaves * kRing) {
    [&]<int... js>(std::integer_sequence<int, js...>) {
      ((tile0 + kWaves * js < ntiles ? tile_body(std::integral_constant<int, js>{}, tile0 + kWaves * js) : void()), ...);
    }(std::make_integer_sequence<int, kRing>{});
  }
}

}  // namespace

hipError_t launch_dkv_bwd_d128(const uint16_t* v, const uint16_t* k, const float* LB, const float* M_all,
                               const float* m0, const float* gamma, float ks, float* dk, float* dv, int64_t heads,
                               int64_t T, int64_t t0, int64_t t1, int S, hipStream_t st) {
  const int64_t nt = t1 - t0, frames = heads * nt;
  const int nsplit = token_split(frames, S);
  hipLaunchKernelGGL((k_dkv_d128<1, kDkvWaves>), dim3((unsigned)(frames * nsplit)), dim3(64 * kDkvWaves), 0, st, v, k,
                     LB, M_all, m0, gamma, ks, dk, dv, S, T, (int)t0, (int)nt, nsplit);
  return hipGetLastError();
}

hipError_t launch_state_bwd_d128(const float* G, const float* U, const float* P, const float* M_all,
                                 const float* m0, const float* gamma, const float* beta,
                                 const float* d_state_out, float* LB, float* partials, float* d_state_in,
                                 int64_t heads, int64_t T, int64_t t0, int64_t t1, hipStream_t st) {
  // workgroup ids grouped so that the parts of a head share id % 8 (one XCD)
  const unsigned grid = (unsigned)((heads + 7) / 8 * 8 * (D / kBwdRows));
  hipLaunchKernelGGL(k2_state_bwd_d128<kBwdRows>, dim3(grid), dim3(256), 0, st, G, U, P, M_all, m0, gamma, beta,
                     d_state_out, LB, partials, d_state_in, (int)heads, (int)T, (int)t0, (int)t1);
  return hipGetLastError();
}

hipError_t launch_bwd_reduce(const float* partials, float* dgamma, float* dbeta, int64_t frames,
                             hipStream_t st) {
  hipLaunchKernelGGL(k_bwd_reduce, dim3((unsigned)((frames + 255) / 256)), dim3(256), 0, st, partials, dgamma,
                     dbeta, frames);
  return hipGetLastError();
}

}  // namespace gdn
