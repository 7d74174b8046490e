// Backward pass of the frame-wise GDN, head dim 128: the reverse-time state
// pass, the reduction of its dgamma/dbeta partial sums, and the symmetric
// G-gradient term.  (The contractions over tokens reuse the forward's build
// and output kernels; see gdn_api.cpp.)
//
// Reverse-time state pass.
//
// The forward M_t = gamma_t (M_{t-1} - beta_t M_{t-1} G_t) + beta_t U_t with
// O_t = Q_t M_t^T (the recurrence of "SANA-WM: NVIDIA puts a one-minute world
// model on a single GPU", zhichai.net, section 1) has, for the total gradient
// Lambda_t reaching M_t,
//   Lambda_t = L_t + P_t,          P_t = dO_t^T Q_t,  L_{T-1} = dM_T,
//   X_t      = Lambda_t G_t,
//   L_{t-1}  = gamma_t (Lambda_t - beta_t X_t)      (G_t is symmetric),
// and the gradient of the initial state is L_{-1}.  Per frame this kernel
// also writes LB_t = beta_t Lambda_t (the frame's dU_t, which the gradient
// kernels use) and, over its rows, partial sums of
//   dgamma_t = < Lambda_t - beta_t X_t, M_{t-1} >,
//   dbeta_t  = < Lambda_t, U_t > - gamma_t < X_t, M_{t-1} >.
//
// It runs like the forward state pass, frames in reverse: rows of Lambda
// evolve independently (row i of L_{t-1} needs only row i of Lambda_t), so
// each head's 128 rows are split over 8 workgroups of 16 rows; X = Lambda G
// runs on bf16 MFMA in three passes (Ghi*Lhi + Glo*Lhi + Ghi*Llo) with the
// float32 running value in registers and its hi/lo pair in LDS; the
// per-frame inputs (this wave's G_t rows, and the workgroup's rows of U_t,
// M_{t-1} and P_{t-1}) stream through a two-frame register ring.  The
// partial sums are reduced in a fixed order (lanes, then waves), so the
// results are deterministic.
#include "gdn_common.h"
#include "gdn_launch.h"

#include <type_traits>
#include <utility>

namespace gdn {
namespace {

constexpr int D = 128;
constexpr int kLdsW = D + 8;
constexpr int kRows = D / kBwdParts;  // 16
constexpr int kDepth = 2;

static_assert(kRows == 16, "one 16-row MFMA block per workgroup");

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

__global__ __launch_bounds__(256, 1) void k2_state_bwd_d128(
    const float* __restrict__ G, const float* __restrict__ U, const float* __restrict__ P,
    const float* __restrict__ M_all, const float* m0, const float* __restrict__ gamma,
    const float* __restrict__ beta, const float* d_state_out, float* __restrict__ LB,
    float* __restrict__ partials, float* d_state_in, int heads, int T) {
  __shared__ uint16_t Ml[2][2][kRows][kLdsW];  // [buffer][hi|lo][row][col]
  __shared__ float red[2][4][2];              // [buffer][wave][dgamma, dbeta]

  const int id = blockIdx.x;
  const int xcd = id & 7, slot = id >> 3;
  const int part = slot % kBwdParts;
  const int head = (slot / kBwdParts) * 8 + xcd;
  if (head >= heads) return;
  const int r0 = part * kRows;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int n = l & 15, g = l >> 4;
  const int row = r0 + n;
  auto col_of = [&](int cb) { return 32 * w + 16 * cb + 4 * g; };
  const int64_t hoff = (int64_t)head * D * D;
  auto frame = [&](int t) { return ((int64_t)head * T + t) * D * D; };

  // running gradient, this lane's 8 elements: row `row`, columns col_of(cb) .. +3
  f32x4 Lr[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const f32x4 d0 = d_state_out ? *reinterpret_cast<const f32x4*>(d_state_out + hoff + row * D + col_of(cb))
                                 : (f32x4){0.f, 0.f, 0.f, 0.f};
    Lr[cb] = d0 + *reinterpret_cast<const f32x4*>(P + frame(T - 1) + row * D + col_of(cb));  // Lambda_{T-1}
  }
  auto put_lds = [&](int buf) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const u32x2 p0 = split2(Lr[cb][0], Lr[cb][1]), p1 = split2(Lr[cb][2], Lr[cb][3]);
      *reinterpret_cast<u32x2*>(&Ml[buf][0][n][col_of(cb)]) = (u32x2){p0.x, p1.x};
      *reinterpret_cast<u32x2*>(&Ml[buf][1][n][col_of(cb)]) = (u32x2){p0.y, p1.y};
    }
  };
  put_lds(0);

  // Ring: this wave's G_t rows 32w .. 32w+31 (the A operand, float32) and
  // the workgroup's rows of U_t, M_{t-1} and P_{t-1} (this lane's elements).
  f32x4 rg[kDepth][2][4][2];
  f32x4 ru[kDepth][2], rm[kDepth][2], rp[kDepth][2];
  auto load_frame = [&](auto jc, int t) {
    constexpr int j = decltype(jc)::value;
    if (t < 0) return;
    const float* Gt = G + frame(t);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float* p = Gt + (32 * w + 16 * cb + n) * D + 32 * kb + 8 * g;
        rg[j][cb][kb][0] = *reinterpret_cast<const f32x4*>(p);
        rg[j][cb][kb][1] = *reinterpret_cast<const f32x4*>(p + 4);
      }
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const float* Mp = t > 0 ? M_all + frame(t - 1) : (m0 ? m0 + hoff : nullptr);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int e = row * D + col_of(cb);
      ru[j][cb] = *reinterpret_cast<const f32x4*>(U + frame(t) + e);
      rm[j][cb] = Mp ? *reinterpret_cast<const f32x4*>(Mp + e) : zero;
      rp[j][cb] = t > 0 ? *reinterpret_cast<const f32x4*>(P + frame(t - 1) + e) : zero;
    }
  };

  // gamma/beta: lane i holds frame T-1-(64k+i) of window k (vector loads,
  // read with readlane; scalar loads would share the LDS wait counter)
  const float* gh = gamma + (int64_t)head * T;
  const float* bh = beta + (int64_t)head * T;
  auto win_load = [&](int i0, float& gv, float& bv) {
    const int t = T - 1 - (i0 + l);
    gv = t >= 0 ? gh[t] : 0.f;
    bv = t >= 0 ? bh[t] : 0.f;
  };
  float gwin, bwin, gnxt, bnxt;
  win_load(0, gwin, bwin);
  win_load(64, gnxt, bnxt);

  [&]<int... js>(std::integer_sequence<int, js...>) {
    (load_frame(std::integral_constant<int, js>{}, T - 1 - js), ...);
  }(std::make_integer_sequence<int, kDepth>{});
  lds_barrier();

  auto step = [&](auto jc, int i) {
    constexpr int j = decltype(jc)::value;
    const int t = T - 1 - i;
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
        const u32x2 p0 = split2(rg[j][cb][kb][0][0], rg[j][cb][kb][0][1]);
        const u32x2 p1 = split2(rg[j][cb][kb][0][2], rg[j][cb][kb][0][3]);
        const u32x2 p2 = split2(rg[j][cb][kb][1][0], rg[j][cb][kb][1][1]);
        const u32x2 p3 = split2(rg[j][cb][kb][1][2], rg[j][cb][kb][1][3]);
        ahi[cb][kb] = (u32x4){p0.x, p1.x, p2.x, p3.x};
        alo[cb][kb] = (u32x4){p0.y, p1.y, p2.y, p3.y};
      }
    f32x4 uu[2], mm[2], pp[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      uu[cb] = ru[j][cb];
      mm[cb] = rm[j][cb];
      pp[cb] = rp[j][cb];
    }
    load_frame(jc, t - kDepth);  // refill this ring slot kDepth frames ahead

    // X^T = G Lambda^T: acc[cb][i] = X[row][col_of(cb) + i]
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const u32x4 bhi = *reinterpret_cast<const u32x4*>(&Ml[buf][0][n][32 * kb + 8 * g]);
      const u32x4 blo = *reinterpret_cast<const u32x4*>(&Ml[buf][1][n][32 * kb + 8 * g]);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) acc[cb] = mfma16x16x32(ahi[cb][kb], bhi, acc[cb]);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) acc[cb] = mfma16x16x32(alo[cb][kb], bhi, acc[cb]);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) acc[cb] = mfma16x16x32(ahi[cb][kb], blo, acc[cb]);
    }

    float dg = 0.f, db = 0.f;
    float* LBt = LB + frame(t);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      f32x4 lb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lam = Lr[cb][e], x = acc[cb][e];
        lb[e] = bt * lam;
        dg = fmaf(fmaf(-bt, x, lam), mm[cb][e], dg);
        db = fmaf(lam, uu[cb][e], fmaf(-gm * x, mm[cb][e], db));
        // L_{t-1} = gamma (Lambda - beta X), rounded, then + P_{t-1} (zero at
        // t = 0): the same two roundings as when a sequence is cut here and
        // the next call adds P_{t-1} to the state gradient it is given
        Lr[cb][e] = mul_then_add(gm, fmaf(-bt, x, lam), pp[cb][e]);
      }
      *reinterpret_cast<f32x4*>(LBt + row * D + col_of(cb)) = lb;
    }
    dg = wave_sum(dg);
    db = wave_sum(db);
    if (l == 0) {
      red[buf][w][0] = dg;
      red[buf][w][1] = db;
    }
    put_lds(buf ^ 1);
    lds_barrier();
    if (tid == 0) {
      float* pr = partials + (((int64_t)head * T + t) * kBwdParts + part) * 2;
      pr[0] = ((red[buf][0][0] + red[buf][1][0]) + red[buf][2][0]) + red[buf][3][0];
      pr[1] = ((red[buf][0][1] + red[buf][1][1]) + red[buf][2][1]) + red[buf][3][1];
    }
  };

  for (int i0 = 0; i0 < T; i0 += kDepth) {
    [&]<int... js>(std::integer_sequence<int, js...>) {
      ((i0 + js < T ? step(std::integral_constant<int, js>{}, i0 + js) : void()), ...);
    }(std::make_integer_sequence<int, kDepth>{});
  }
  // after frame 0 the running value is the gradient of the initial state
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
    *reinterpret_cast<f32x4*>(d_state_in + hoff + row * D + col_of(cb)) = Lr[cb];
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

// S_t = -gamma_t (A + A^T), A = M_{t-1}^T LB_t (both float32 row-major), one
// workgroup per frame.  The gradient of G_t = K_t^T K_t is
// dG_t = -gamma_t beta_t M_{t-1}^T Lambda_t, and K_t receives K_t (dG + dG^T);
// LB_t = beta_t Lambda_t already carries beta.  Thread (ta, tb) accumulates
// the 8 x 8 block A[8ta .. 8ta+7][8tb .. 8tb+7] over 32-row chunks of M and
// LB staged in LDS; A then goes through LDS once more to be symmetrized.
__global__ __launch_bounds__(256, 1) void k_sym_bwd_d128(const float* __restrict__ M_all, const float* m0,
                                                       const float* __restrict__ LB,
                                                       const float* __restrict__ gamma,
                                                       float* __restrict__ Sout, int T) {
  constexpr int kChunk = 32;
  __shared__ float Ms[kChunk][D];
  __shared__ float Ls[kChunk][D];
  __shared__ float As[D][D + 1];
  const int64_t f = blockIdx.x;
  const int head = (int)(f / T), t = (int)(f % T);
  const float* Mp = t > 0 ? M_all + (f - 1) * D * D : (m0 ? m0 + (int64_t)head * D * D : nullptr);
  const float* Lt = LB + f * D * D;
  float* St = Sout + f * D * D;
  const int tid = threadIdx.x;
  const int ta = tid >> 4, tb = tid & 15;
  if (!Mp) {  // zero initial state: M_{-1} = 0, so S_0 = 0
    for (int i = tid; i < D * D / 4; i += 256) reinterpret_cast<f32x4*>(St)[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    return;
  }
  float acc[8][8];
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int y = 0; y < 8; ++y) acc[x][y] = 0.f;
  for (int i0 = 0; i0 < D; i0 += kChunk) {
    __syncthreads();
    for (int e = tid; e < kChunk * D / 4; e += 256) {
      const int r = e / (D / 4), c = (e % (D / 4)) * 4;
      *reinterpret_cast<f32x4*>(&Ms[r][c]) = *reinterpret_cast<const f32x4*>(Mp + (i0 + r) * D + c);
      *reinterpret_cast<f32x4*>(&Ls[r][c]) = *reinterpret_cast<const f32x4*>(Lt + (i0 + r) * D + c);
    }
    __syncthreads();
    for (int i = 0; i < kChunk; ++i) {
      const f32x4 m0v = *reinterpret_cast<const f32x4*>(&Ms[i][8 * ta]);
      const f32x4 m1v = *reinterpret_cast<const f32x4*>(&Ms[i][8 * ta + 4]);
      const f32x4 l0v = *reinterpret_cast<const f32x4*>(&Ls[i][8 * tb]);
      const f32x4 l1v = *reinterpret_cast<const f32x4*>(&Ls[i][8 * tb + 4]);
      const float mv[8] = {m0v[0], m0v[1], m0v[2], m0v[3], m1v[0], m1v[1], m1v[2], m1v[3]};
      const float lv[8] = {l0v[0], l0v[1], l0v[2], l0v[3], l1v[0], l1v[1], l1v[2], l1v[3]};
#pragma unroll
      for (int x = 0; x < 8; ++x)
#pragma unroll
        for (int y = 0; y < 8; ++y) acc[x][y] = fmaf(mv[x], lv[y], acc[x][y]);
    }
  }
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int y = 0; y < 8; ++y) As[8 * ta + x][8 * tb + y] = acc[x][y];
  __syncthreads();
  const float ng = -gamma[f];
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    const int a = 8 * ta + x;
    f32x4 s0, s1;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      s0[y] = ng * (acc[x][y] + As[8 * tb + y][a]);
      s1[y] = ng * (acc[x][y + 4] + As[8 * tb + y + 4][a]);
    }
    *reinterpret_cast<f32x4*>(St + a * D + 8 * tb) = s0;
    *reinterpret_cast<f32x4*>(St + a * D + 8 * tb + 4) = s1;
  }
}

}  // namespace

hipError_t launch_sym_bwd_d128(const float* M_all, const float* m0, const float* LB, const float* gamma,
                               float* Sout, int64_t heads, int64_t T, hipStream_t st) {
  hipLaunchKernelGGL(k_sym_bwd_d128, dim3((unsigned)(heads * T)), dim3(256), 0, st, M_all, m0, LB, gamma, Sout,
                     (int)T);
  return hipGetLastError();
}

hipError_t launch_state_bwd_d128(const float* G, const float* U, const float* P, const float* M_all,
                                 const float* m0, const float* gamma, const float* beta,
                                 const float* d_state_out, float* LB, float* partials, float* d_state_in,
                                 int64_t heads, int64_t T, hipStream_t st) {
  // workgroup ids grouped so that the parts of a head share id % 8 (one XCD)
  const unsigned grid = (unsigned)((heads + 7) / 8 * 8 * kBwdParts);
  hipLaunchKernelGGL(k2_state_bwd_d128, dim3(grid), dim3(256), 0, st, G, U, P, M_all, m0, gamma, beta,
                     d_state_out, LB, partials, d_state_in, (int)heads, (int)T);
  return hipGetLastError();
}

hipError_t launch_bwd_reduce(const float* partials, float* dgamma, float* dbeta, int64_t frames,
                             hipStream_t st) {
  hipLaunchKernelGGL(k_bwd_reduce, dim3((unsigned)((frames + 255) / 256)), dim3(256), 0, st, partials, dgamma,
                     dbeta, frames);
  return hipGetLastError();
}

}  // namespace gdn
