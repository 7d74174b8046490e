// State pass of the frame-wise GDN, head dim 128:
//   M_t = M_{t-1} gamma_t (I - beta_t G_t) + beta_t U_t = gamma_t (M_{t-1} - beta_t X_t) + beta_t U_t,
//   X_t = M_{t-1} G_t,
// sequential over frames, float32 state (the decay gate multiplies the
// previous state and the delta rule corrects the residual: "SANA-WM: NVIDIA
// puts a one-minute world model on a single GPU", zhichai.net, section 1).
//
// Rows of M evolve independently (row i of M_t needs only row i of M_{t-1}),
// so each head's 128 rows are split over kParts workgroups that never talk
// to each other.  A workgroup keeps its rows of M in registers (float32
// master copy) and in LDS as a bf16 hi/lo pair, double-buffered.  The
// product X = M G runs on bf16 MFMA as three passes, Ghi*Mhi + Glo*Mhi +
// Ghi*Mlo, each split term exact to about 2^-17 relative, with float32
// accumulation; the dropped lo*lo term is ~2^-16 of a term that is itself a
// few per cent of M.  Computed transposed, X^T = G M^T (G_t = K_t^T K_t is
// symmetric, so its rows serve as its columns), so that each lane ends up
// owning 4 consecutive columns of one row of M.
//
// Workgroups of one head are placed on one XCD (dispatch is round-robin over
// the 8 XCDs), so the G_t and U_t rows they share come from one L2.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int D = 128;
constexpr int kRows = 64;              // rows of M per workgroup
constexpr int kParts = D / kRows;      // workgroups per head
constexpr int kLdsW = D + 8;           // padded LDS row (bf16 elements)

__global__ __launch_bounds__(256, 1) void k2_state_d128(
    const float* __restrict__ G, const float* __restrict__ U, const float* __restrict__ gamma,
    const float* __restrict__ beta, const float* state_in, float* __restrict__ M_all,
    float* state_out, int heads, int T) {
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
  f32x4 Mreg[2][4];
  const int64_t hoff = (int64_t)head * D * D;
  auto elem_off = [&](int cb, int rb) { return (r0 + 16 * rb + n) * D + 32 * w + 16 * cb + 4 * g; };

  auto put_lds = [&](int buf) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        uint32_t h[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) split_bf16(Mreg[cb][rb][i], h[i], lo[i]);
        const int row = 16 * rb + n, col = 32 * w + 16 * cb + 4 * g;
        *reinterpret_cast<u32x2*>(&Ml[buf][0][row][col]) = (u32x2){pack2(h[0], h[1]), pack2(h[2], h[3])};
        *reinterpret_cast<u32x2*>(&Ml[buf][1][row][col]) = (u32x2){pack2(lo[0], lo[1]), pack2(lo[2], lo[3])};
      }
  };

#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
      Mreg[cb][rb] = state_in ? *reinterpret_cast<const f32x4*>(state_in + hoff + elem_off(cb, rb))
                              : (f32x4){0.f, 0.f, 0.f, 0.f};
  put_lds(0);

  // A operand: rows 32w + 16cb + m of G_t (m = l%16), 8 floats at column 32kb + 8g.
  const int m = n;
  f32x4 graw[2][4][2];
  auto load_g = [&](int t) {
    const float* Gt = G + ((int64_t)head * T + t) * D * D;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const f32x4* p = reinterpret_cast<const f32x4*>(Gt + (32 * w + 16 * cb + m) * D + 32 * kb + 8 * g);
        graw[cb][kb][0] = p[0];
        graw[cb][kb][1] = p[1];
      }
  };
  load_g(0);
  __syncthreads();

  for (int t = 0; t < T; ++t) {
    const int buf = t & 1;
    const float gm = gamma[(int64_t)head * T + t];
    const float bt = beta[(int64_t)head * T + t];

    u32x4 ahi[2][4], alo[2][4];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        uint32_t h[8], lo[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          split_bf16(graw[cb][kb][0][e], h[e], lo[e]);
          split_bf16(graw[cb][kb][1][e], h[4 + e], lo[4 + e]);
        }
        ahi[cb][kb] = (u32x4){pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
        alo[cb][kb] = (u32x4){pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(lo[4], lo[5]), pack2(lo[6], lo[7])};
      }
    if (t + 1 < T) load_g(t + 1);

    f32x4 ureg[2][4];
    const float* Ut = U + ((int64_t)head * T + t) * D * D;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        ureg[cb][rb] = *reinterpret_cast<const f32x4*>(Ut + elem_off(cb, rb));

    f32x4 acc[2][4];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) acc[cb][rb] = (f32x4){0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        // B operand: row r0 + 16rb + n of M (as M^T column), 8 bf16 at column 32kb + 8g.
        const u32x4 bhi = *reinterpret_cast<const u32x4*>(&Ml[buf][0][16 * rb + n][32 * kb + 8 * g]);
        const u32x4 blo = *reinterpret_cast<const u32x4*>(&Ml[buf][1][16 * rb + n][32 * kb + 8 * g]);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          acc[cb][rb] = mfma16x16x32(ahi[cb][kb], bhi, acc[cb][rb]);
          acc[cb][rb] = mfma16x16x32(alo[cb][kb], bhi, acc[cb][rb]);
          acc[cb][rb] = mfma16x16x32(ahi[cb][kb], blo, acc[cb][rb]);
        }
      }

    // acc[cb][rb][i] = X[r0 + 16rb + n][32w + 16cb + 4g + i]
    const float gb = gm * bt;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Mreg[cb][rb][i] = fmaf(gm, Mreg[cb][rb][i], fmaf(-gb, acc[cb][rb][i], bt * ureg[cb][rb][i]));

    if (M_all) {
      float* Mt = M_all + ((int64_t)head * T + t) * D * D;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) *reinterpret_cast<f32x4*>(Mt + elem_off(cb, rb)) = Mreg[cb][rb];
    }
    put_lds(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
      *reinterpret_cast<f32x4*>(state_out + hoff + elem_off(cb, rb)) = Mreg[cb][rb];
}

}  // namespace

hipError_t launch_state_d128(const float* G, const float* U, const float* gamma,
                             const float* beta, const float* state_in, float* M_all,
                             float* state_out, int64_t heads, int64_t T, hipStream_t st) {
  // Workgroup ids are grouped so that the kParts workgroups of a head share id % 8.
  const int64_t groups = (heads + 7) / 8;
  const unsigned grid = (unsigned)(groups * 8 * kParts);
  hipLaunchKernelGGL(k2_state_d128, dim3(grid), dim3(256), 0, st, G, U, gamma, beta, state_in,
                     M_all, state_out, (int)heads, (int)T);
  return hipGetLastError();
}

}  // namespace gdn
