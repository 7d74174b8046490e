// Output of the frame-wise GDN on bf16 MFMA (gfx950), head dim 128, one frame
// per call of output_frame by a 256-thread workgroup:
//   O_t = Q_t M_t^T        (Q_t: S x 128 bf16, M_t: 128 x 128 float32)
// M_t enters the MFMA as a bf16 hi/lo pair (two passes, Q*Mhi + Q*Mlo); the
// pair carries M_t to about 2^-17 relative, so O keeps float32 accuracy.
//
// M_t is split into hi/lo once and kept in LDS.
// Global accesses:
//  * Q: MFMA k-slot (kb, g, e) is key dim 32kb + 8g + e, so one load
//    instruction (fixed kb) reads 64 contiguous bytes of 16 rows, and the
//    instructions for kb and kb + 1 complete each 128-byte line.  These are
//    ordinary (temporal) loads: the second half of a line then hits in L2,
//    where a non-temporal load could re-fetch it from HBM;
//  * O: column n of output block nb is value dim sigma(nb, n).
//    For a float32 output sigma = 64(nb / 4) + 4n + nb % 4, so one store of
//    blocks 0-3 (4-7) from 16 lanes is the first (second) 256 bytes of a
//    row; for a bf16 output sigma = 8n + nb and one store covers the row.
// LDS row nb*16 + n holds M row sigma(nb, n), which makes the B-operand reads
// of 16 lanes land on 16 distinct 4-bank groups.
#pragma once

#include "gdn_common.h"
#include "gdn_packed.h"

#include <type_traits>
#include <utility>

namespace gdn {

constexpr int kOutLdsW = 128 + 8;  // padded LDS row (bf16 elements)
constexpr int kOutTile = 32;       // tokens per wave iteration

// LDS the output needs: M_t as bf16 hi and lo planes, 128 padded rows each.
constexpr int output_lds_bytes() { return 2 * 128 * kOutLdsW * 2; }

// LDS row holding M row r (the inverse of sigma above).
template <bool kOutBf16>
__device__ __forceinline__ int lds_row(int r) {
  if constexpr (kOutBf16) return (r & 7) * 16 + (r >> 3);
  else return (((r >> 6) << 2) + (r & 3)) * 16 + ((r & 63) >> 2);
}

// O_t = Q_t M_t^T for one frame.  Qf: the frame's [S, 128] bf16 rows; Mt_in:
// M_t packed (kPackedM, gdn_packed.h) or float32 row-major; Of: the frame's
// [S, 128] output rows (bf16 when kOutBf16, else float32).  Ml: LDS of
// output_lds_bytes().  on_staged() runs on every thread once M_t has been
// copied into LDS (the caller may then release M_t's buffer).  kDepth: token
// tiles each wave loads ahead.  All 256 threads of the workgroup must call it.
// With the float32 form of M_t, kTransM stages M_t^T instead of M_t (so the
// frame gets Q_t M_t; used by the backward pass).  M_t is read with all
// sixteen 16-byte loads of a thread in flight at once (one memory round trip,
// not sixteen).
template <bool kPackedM, bool kOutBf16, int kDepth = 1, bool kTransM = false, typename OnStaged>
__device__ __forceinline__ void output_frame(const uint16_t* __restrict__ Qf, const void* __restrict__ Mt_in,
                                             void* __restrict__ Of, int S, uint16_t (*Ml)[128][kOutLdsW],
                                             OnStaged on_staged) {
  constexpr int D = 128;
  constexpr int kTile = kOutTile;
  static_assert(!(kPackedM && kTransM), "option not available for this form");
  // An opaque copy of the thread index: lane-dependent addresses are then
  // computed at each call instead of being hoisted out of a caller's loop
  // and kept live (in registers) across the whole call.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int w = tid >> 6, l = tid & 63;
  const int n = l & 15, g = l >> 4;

  // M_t is 64 KiB in either form: 16 loads of 16 bytes per thread, all
  // issued before the first is used (one memory round trip, not sixteen).
  constexpr int kLoads = D * D * 4 / 16 / 256;
  if constexpr (kPackedM) {
    // 8-byte chunk q of the packed form: unit q / 64 = (row block, column
    // block, plane), lane q % 64; load i of this thread holds chunks 2j and
    // 2j + 1, j = tid + 256 i
    const char* Mp = static_cast<const char*>(Mt_in);
    u32x4 mv[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) mv[i] = *reinterpret_cast<const u32x4*>(Mp + 16 * (tid + 256 * i));
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int q = 2 * (tid + 256 * i) + h;
        const int unit = q >> 6, ln = q & 63;
        const int plane = unit & 1, rb = unit >> 4, cb = (unit >> 1) & 7;
        const int r = 16 * rb + (ln & 15), c = 16 * cb + 4 * (ln >> 4);
        *reinterpret_cast<u32x2*>(&Ml[plane][lds_row<kOutBf16>(r)][c]) =
            h ? (u32x2){mv[i][2], mv[i][3]} : (u32x2){mv[i][0], mv[i][1]};
      }
  } else {
    const float* Mt = static_cast<const float*>(Mt_in);
    f32x4 mvs[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) mvs[i] = *reinterpret_cast<const f32x4*>(Mt + 4 * (tid + 256 * i));
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 5, c4 = (idx & 31) * 4;
      const f32x4 mv = mvs[i];
      const u32x2 p0 = split2(mv[0], mv[1]), p1 = split2(mv[2], mv[3]);
      if constexpr (kTransM) {
        // element (r, c4 + e) of M is element (c4 + e, r) of the staged matrix
        const uint32_t hi[2] = {p0.x, p1.x}, lo[2] = {p0.y, p1.y};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rho = lds_row<kOutBf16>(c4 + e);
          Ml[0][rho][r] = (uint16_t)(hi[e >> 1] >> (16 * (e & 1)));
          Ml[1][rho][r] = (uint16_t)(lo[e >> 1] >> (16 * (e & 1)));
        }
        continue;
      }
      const int rho = lds_row<kOutBf16>(r);
      *reinterpret_cast<u32x2*>(&Ml[0][rho][c4]) = (u32x2){p0.x, p1.x};
      *reinterpret_cast<u32x2*>(&Ml[1][rho][c4]) = (u32x2){p0.y, p1.y};
    }
  }
  __syncthreads();
  on_staged();

  const int ntiles = (S + kTile - 1) / kTile;
  // A operand of a 32-token tile: lane (m, g) holds tokens tok0 + 16rb + m,
  // key dims 32kb + 8g .. +7.
  auto load_a = [&](int tile, u32x4 (&a)[2][4]) {
    const int tok0 = tile * kTile;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int s = tok0 + 16 * rb + n;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        a[rb][kb] = (tile < ntiles && s < S)
                        ? *reinterpret_cast<const u32x4*>(Qf + (int64_t)s * D + 32 * kb + 8 * g)
                        : (u32x4){0u, 0u, 0u, 0u};
    }
  };
  constexpr int kRing = kDepth + 1;
  u32x4 ar[kRing][2][4];
  auto tile_body = [&](auto jc, int tile) {
    constexpr int jb = decltype(jc)::value;
    const int tok0 = tile * kTile;
    // tile + 4 * kDepth goes into the ring entry this tile's predecessor used
    load_a(tile + 4 * kDepth, ar[(jb + kDepth) % kRing]);
    u32x4 (&a)[2][4] = ar[jb];
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
        bh[kb] = *reinterpret_cast<const u32x4*>(&Ml[0][nb * 16 + n][32 * kb + 8 * g]);
        bl[kb] = *reinterpret_cast<const u32x4*>(&Ml[1][nb * 16 + n][32 * kb + 8 * g]);
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
        const int64_t row = (int64_t)s * D;
        if constexpr (kOutBf16) {
          u32x4 pk;
#pragma unroll
          for (int p = 0; p < 4; ++p) pk[p] = cvt2bf(acc[rb][2 * p][i], acc[rb][2 * p + 1][i]);
          st_nt(reinterpret_cast<u32x4*>(static_cast<uint16_t*>(Of) + row + 8 * n), pk);
        } else {
          float* o = static_cast<float*>(Of) + row + 4 * n;
          const f32x4 v0 = {acc[rb][0][i], acc[rb][1][i], acc[rb][2][i], acc[rb][3][i]};
          const f32x4 v1 = {acc[rb][4][i], acc[rb][5][i], acc[rb][6][i], acc[rb][7][i]};
          st_nt(reinterpret_cast<f32x4*>(o), v0);
          st_nt(reinterpret_cast<f32x4*>(o + 64), v1);
        }
      }
  };
  [&]<int... js>(std::integer_sequence<int, js...>) {
    (load_a(w + 4 * js, ar[js]), ...);
  }(std::make_integer_sequence<int, kDepth>{});
  for (int tile0 = w; tile0 < ntiles; tile0 += 4 * kRing) {
    [&]<int... js>(std::integer_sequence<int, js...>) {
      ((tile0 + 4 * js < ntiles ? tile_body(std::integral_constant<int, js>{}, tile0 + 4 * js) : void()), ...);
    }(std::make_integer_sequence<int, kRing>{});
  }
}

}  // namespace gdn
