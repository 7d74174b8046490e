// Output of the frame-wise GDN on bf16 MFMA (gfx950), head dim 128:
//   O_t = Q_t M_t^T        (Q_t: S x 128 bf16, M_t: 128 x 128 float32)
// M_t enters the MFMA as a bf16 hi/lo pair (two passes, Q*Mhi + Q*Mlo); the
// pair carries M_t to about 2^-17 relative, so O keeps float32 accuracy.
//
// One workgroup per frame.  M_t is split into hi/lo once and kept in LDS.
// Two index permutations make every global access a contiguous run:
//  * the reduction (key) index: MFMA k-slot (kb, g, e) is key dim
//    32g + 8kb + e, so lane (m, g) reads 64 contiguous bytes of its Q row;
//  * the value index: column n of output block nb is value dim sigma(nb, n).
//    For a float32 output sigma = 64(nb / 4) + 4n + nb % 4, so one store of
//    blocks 0-3 (4-7) from 16 lanes is the first (second) 256 bytes of a
//    row; for a bf16 output sigma = 8n + nb and one store covers the row.
// LDS row nb*16 + n holds M row sigma(nb, n), which makes the B-operand reads
// of 16 lanes land on 16 distinct 4-bank groups.
#include "gdn_common.h"
#include "gdn_launch.h"
#include "gdn_packed.h"

namespace gdn {
namespace {

constexpr int D = 128;
constexpr int kLdsW = D + 8;
constexpr int kTile = 32;  // tokens per wave iteration

// LDS row holding M row r (the inverse of sigma above).
template <bool kOutBf16>
__device__ __forceinline__ int lds_row(int r) {
  if constexpr (kOutBf16) return (r & 7) * 16 + (r >> 3);
  else return (((r >> 6) << 2) + (r & 3)) * 16 + ((r & 63) >> 2);
}

// kPackedM: M_t arrives packed (bf16 hi/lo, gdn_packed.h), as the state pass
// writes it inside gdn_frame_fwd, instead of float32 row-major.
template <bool kPackedM, bool kOutBf16>
__global__ __launch_bounds__(256, 2) void k3_output_bf16_d128(
    const uint16_t* __restrict__ Q, const void* __restrict__ M_all, void* __restrict__ out, int S) {
  __shared__ uint16_t Ml[2][D][kLdsW];  // [hi|lo][permuted row][key dim]

  const int64_t f = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int n = l & 15, g = l >> 4;

  if constexpr (kPackedM) {
    // 8-byte chunk q: unit q / 64 = (row block, column block, plane), lane q % 64
    const char* Mp = static_cast<const char*>(M_all) + f * packed::kFrameBytes;
    for (int q = tid; q < D * D * 2 / 4; q += 256) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(Mp + 8 * q);
      const int unit = q >> 6, ln = q & 63;
      const int plane = unit & 1, rb = unit >> 4, cb = (unit >> 1) & 7;
      const int r = 16 * rb + (ln & 15), c = 16 * cb + 4 * (ln >> 4);
      *reinterpret_cast<u32x2*>(&Ml[plane][lds_row<kOutBf16>(r)][c]) = v;
    }
  } else {
    const float* Mt = static_cast<const float*>(M_all) + f * (int64_t)D * D;
    for (int idx = tid; idx < D * D / 4; idx += 256) {
      const int r = idx >> 5, c4 = (idx & 31) * 4;
      const f32x4 mv = *reinterpret_cast<const f32x4*>(Mt + r * D + c4);
      const u32x2 p0 = split2(mv[0], mv[1]), p1 = split2(mv[2], mv[3]);
      const int rho = lds_row<kOutBf16>(r);
      *reinterpret_cast<u32x2*>(&Ml[0][rho][c4]) = (u32x2){p0.x, p1.x};
      *reinterpret_cast<u32x2*>(&Ml[1][rho][c4]) = (u32x2){p0.y, p1.y};
    }
  }
  __syncthreads();

  const uint16_t* Qf = Q + f * (int64_t)S * D;
  const int ntiles = (S + kTile - 1) / kTile;
  // A operand of a 32-token tile: lane (m, g) holds tokens tok0 + 16rb + m,
  // key dims 32g + 8kb .. +7 (64 contiguous bytes per row and rb).
  auto load_a = [&](int tile, u32x4 (&a)[2][4]) {
    const int tok0 = tile * kTile;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int s = tok0 + 16 * rb + n;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        a[rb][kb] = (tile < ntiles && s < S)
                        ? ld_nt(reinterpret_cast<const u32x4*>(Qf + (int64_t)s * D + 32 * g + 8 * kb))
                        : (u32x4){0u, 0u, 0u, 0u};
    }
  };
  u32x4 a[2][4], an[2][4];
  load_a(w, a);
  for (int tile = w; tile < ntiles; tile += 4) {
    const int tok0 = tile * kTile;
    load_a(tile + 4, an);  // next tile's Q in flight during this tile's MFMAs
    f32x4 acc[2][8];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) acc[rb][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      u32x4 bh[4], bl[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        bh[kb] = *reinterpret_cast<const u32x4*>(&Ml[0][nb * 16 + n][32 * g + 8 * kb]);
        bl[kb] = *reinterpret_cast<const u32x4*>(&Ml[1][nb * 16 + n][32 * g + 8 * kb]);
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          acc[rb][nb] = mfma16x16x32(a[rb][kb], bh[kb], acc[rb][nb]);
          acc[rb][nb] = mfma16x16x32(a[rb][kb], bl[kb], acc[rb][nb]);
        }
      // keep the scheduler from hoisting later blocks' LDS reads (register pressure)
      __builtin_amdgcn_sched_barrier(0);
    }

    // Lane (n, g), register i of block nb: O[tok0 + 16rb + 4g + i][sigma(nb, n)].
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = tok0 + 16 * rb + 4 * g + i;
        if (s >= S) continue;
        const int64_t row = (f * (int64_t)S + s) * D;
        if constexpr (kOutBf16) {
          u32x4 pk;
#pragma unroll
          for (int p = 0; p < 4; ++p) pk[p] = cvt2bf(acc[rb][2 * p][i], acc[rb][2 * p + 1][i]);
          st_nt(reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + row + 8 * n), pk);
        } else {
          float* o = static_cast<float*>(out) + row + 4 * n;
          st_nt(reinterpret_cast<f32x4*>(o), (f32x4){acc[rb][0][i], acc[rb][1][i], acc[rb][2][i], acc[rb][3][i]});
          st_nt(reinterpret_cast<f32x4*>(o + 64), (f32x4){acc[rb][4][i], acc[rb][5][i], acc[rb][6][i], acc[rb][7][i]});
        }
      }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) a[rb][kb] = an[rb][kb];
  }
}

}  // namespace

template <bool kPackedM>
hipError_t launch_out(const uint16_t* q, const void* M_all, void* out, bool out_bf16, int64_t frames,
                      int S, hipStream_t st) {
  if (out_bf16)
    hipLaunchKernelGGL((k3_output_bf16_d128<kPackedM, true>), dim3((unsigned)frames), dim3(256), 0, st, q,
                       M_all, out, S);
  else
    hipLaunchKernelGGL((k3_output_bf16_d128<kPackedM, false>), dim3((unsigned)frames), dim3(256), 0, st, q,
                       M_all, out, S);
  return hipGetLastError();
}

hipError_t launch_output_bf16_d128(const uint16_t* q, const void* M_all, bool packed_m, void* out,
                                   bool out_bf16, int64_t frames, int S, hipStream_t st) {
  return packed_m ? launch_out<true>(q, M_all, out, out_bf16, frames, S, st)
                 : launch_out<false>(q, M_all, out, out_bf16, frames, S, st);
}

}  // namespace gdn
