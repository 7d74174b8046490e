// Per-frame maps of the frame-wise GDN on bf16 MFMA (gfx950), head dim 128,
// one frame per call of build_frame by a 256-thread workgroup:
//   G_t = K_t^T K_t   and   U_t = V_t^T K_t,
// both reducing over the S tokens of one latent frame (one recurrent step
// consumes a whole frame: bilibili cv49203711, fourth key point).  Products
// of two bf16 numbers are exact in float32; accumulation is float32.
//
// One workgroup (4 waves) per frame.  The reduction index (tokens) is the
// slow index of the [S, 128] storage while an MFMA operand wants 8
// consecutive reduction values per lane, so every wave loads a 32-token x
// 128-dim slab with 16-byte loads (lane = token group g = l/16 of 8 tokens,
// dim group c = l%16 of 8 dims) and transposes 8x8 bf16 blocks in registers.
// That yields 8 operand fragments per slab; fragment j holds, in lane
// (g, c), the 8 tokens of group g at dim 8c + j, so MFMA row m of fragment j
// is dim 8m + j.  Fragments go to LDS once and every wave reads the ones it
// needs.  Wave w owns the output rows {8m + j : j in {2w, 2w+1}} of both G and
// U (32 accumulators of 16x16), which makes every lane's final row segment 8
// contiguous floats.
#pragma once

#include "gdn_common.h"
#include "gdn_packed.h"

#include <type_traits>
#include <utility>

namespace gdn {

constexpr int kBuildIterTok = 64;  // tokens per loop iteration: two 32-token slabs of K and of V

// LDS the build needs: 64 KB when kPacked (the output is staged there), else 32 KB.
template <bool kPacked>
constexpr int build_lds_bytes() { return kPacked ? 65536 : 32768; }

// G_t = K_t^T K_t and U_t = V_t^T K_t of one frame.  Kf, Vf: the frame's
// [S, 128] bf16 rows.  ks scales the keys: the maps are written as
// ks^2 G_t and ks U_t (the float32 sums times ks^2 or ks, one rounding;
// ks = 1 leaves them unchanged).  kPacked: Gout receives the packed bf16 hi/lo form
// and Uout the packed float32 form (gdn_packed.h); otherwise both are
// float32 row-major 128 x 128, and Gout may be null (only U_t is written).
// `lds` must hold build_lds_bytes<kPacked>().
// kDepth: token iterations loaded ahead (register buffers of 32 VGPRs each).
// kUpperG (packed only): of G_t, only the halves of the packed units that
// lie on or above the diagonal in 16 x 16 blocks are written (G_t is
// symmetric bit for bit: both entries of a pair are the same products
// summed in the same order).
// kWithG = false (float32 output only, Gout null): G_t is not formed at all,
// half the MFMAs (the backward's P_t = dO_t^T Q_t needs only the second map).
// All 256 threads of the workgroup must call it.  On return this thread's
// stores are issued, not necessarily complete.
template <bool kPacked, int kDepth = 1, bool kUpperG = false, bool kWithG = true>
__device__ __forceinline__ void build_frame(const uint16_t* __restrict__ Kf, const uint16_t* __restrict__ Vf,
                                            int S, u32x4* __restrict__ lds, void* __restrict__ Gout,
                                            float* __restrict__ Uout, float ks) {
  constexpr int D = 128;
  constexpr int kIterTok = kBuildIterTok;
  // During the token loop: frag[unit][j][lane] (32 KB); unit 0,1 = K slab 0,1;
  // unit 2,3 = V slab 0,1.  Afterwards the whole buffer (64 KB) stages the
  // packed output so that it leaves in contiguous 4 KB rows of stores.
  u32x4 (*frag)[8][kWave] = reinterpret_cast<u32x4 (*)[8][kWave]>(lds);

  // An opaque copy of the thread index: lane-dependent addresses are then
  // computed at each call instead of being hoisted out of a caller's loop
  // and kept live (in registers) across the whole call.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int w = tid >> 6, l = tid & 63;
  const int g = l >> 4, c = l & 15;
  const uint16_t* src = w < 2 ? Kf : Vf;
  const int slab = w & 1;

  u32x4 x[kDepth][8];
  auto load = [&](auto jc, int it) {
    constexpr int jb = decltype(jc)::value;
    const int base = it * kIterTok + slab * 32 + 8 * g;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = base + i;
      if (s < S)
        x[jb][i] = ld_nt(reinterpret_cast<const u32x4*>(src + (int64_t)s * D + 8 * c));
      else
        x[jb][i] = (u32x4){0u, 0u, 0u, 0u};
    }
  };

  f32x4 accG[2][8], accU[2][8];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      accG[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
      accU[a][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }

  const int iters = (S + kIterTok - 1) / kIterTok;
  auto iteration = [&](auto jc, int it) {
    constexpr int jb = decltype(jc)::value;
    __syncthreads();  // every wave is done reading the previous fragments
    // 8x8 transpose: fragment j, dword p = (token 2p, token 2p+1) at dim 8c+j.
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x4 o;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t a = x[jb][2 * p][j >> 1], b = x[jb][2 * p + 1][j >> 1];
        o[p] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
      }
      frag[w][j][l] = o;
    }
    __syncthreads();
    if (it + kDepth < iters) load(jc, it + kDepth);  // in flight during the MFMAs

#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      u32x4 kf[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) kf[j] = frag[sl][j][l];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const u32x4 kr = frag[sl][2 * w + jj][l];
        const u32x4 vr = frag[2 + sl][2 * w + jj][l];
#pragma unroll
        for (int jp = 0; jp < 8; ++jp) {
          if constexpr (kWithG) accG[jj][jp] = mfma16x16x32(kr, kf[jp], accG[jj][jp]);
          accU[jj][jp] = mfma16x16x32(vr, kf[jp], accU[jj][jp]);
        }
      }
    }
  };
  [&]<int... js>(std::integer_sequence<int, js...>) {
    ((js < iters ? load(std::integral_constant<int, js>{}, js) : void()), ...);
  }(std::make_integer_sequence<int, kDepth>{});
  for (int it0 = 0; it0 < iters; it0 += kDepth) {
    [&]<int... js>(std::integer_sequence<int, js...>) {
      ((it0 + js < iters ? iteration(std::integral_constant<int, js>{}, it0 + js) : void()), ...);
    }(std::make_integer_sequence<int, kDepth>{});
  }

  // the key scale: G_t picks up ks twice, U_t once
  const float ks2 = ks * ks;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      if constexpr (kWithG) accG[a][b] *= ks2;
      accU[a][b] *= ks;
    }

  // Lane (g, c), register i of block (j, jp) holds X[32g + 8i + j][8c + jp].
  if constexpr (kPacked) {
    char* stage = reinterpret_cast<char*>(lds);
    // pass 0: G_t as bf16 hi/lo (Gp); pass 1: U_t as float32 (Up)
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      __syncthreads();  // previous readers of the LDS buffer are done
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * w + jj;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 32 * g + 8 * i + j;
          if (pass == 0) {
            const u32x2 p0 = split2(accG[jj][0][i], accG[jj][1][i]), p1 = split2(accG[jj][2][i], accG[jj][3][i]);
            const u32x2 p2 = split2(accG[jj][4][i], accG[jj][5][i]), p3 = split2(accG[jj][6][i], accG[jj][7][i]);
            *reinterpret_cast<u32x4*>(stage + packed::g_chunk(row, 8 * c, 0)) = (u32x4){p0.x, p1.x, p2.x, p3.x};
            *reinterpret_cast<u32x4*>(stage + packed::g_chunk(row, 8 * c, 1)) = (u32x4){p0.y, p1.y, p2.y, p3.y};
          } else {
            *reinterpret_cast<f32x4*>(stage + packed::u_chunk(row, 8 * c)) =
                (f32x4){accU[jj][0][i], accU[jj][1][i], accU[jj][2][i], accU[jj][3][i]};
            *reinterpret_cast<f32x4*>(stage + packed::u_chunk(row, 8 * c + 4)) =
                (f32x4){accU[jj][4][i], accU[jj][5][i], accU[jj][6][i], accU[jj][7][i]};
          }
        }
      }
      __syncthreads();
      u32x4* dst = reinterpret_cast<u32x4*>(pass == 0 ? static_cast<char*>(Gout) : reinterpret_cast<char*>(Uout));
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        // chunk k * 256 + tid: packed unit 4k + tid / 64, half (tid % 64) / 32
        const int unit = 4 * k + (tid >> 6), half = (tid & 63) >> 5;
        const bool lower = (unit >> 3) > 2 * ((unit >> 1) & 3) + half;  // row block > column block
        if (!(kUpperG && pass == 0 && lower)) dst[k * 256 + tid] = lds[k * 256 + tid];
      }
    }
  } else {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * w + jj;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 32 * g + 8 * i + j;
        f32x4* gp = reinterpret_cast<f32x4*>(static_cast<float*>(Gout) + row * D + 8 * c);
        f32x4* up = reinterpret_cast<f32x4*>(Uout + row * D + 8 * c);
        if (kWithG && Gout) {
          gp[0] = (f32x4){accG[jj][0][i], accG[jj][1][i], accG[jj][2][i], accG[jj][3][i]};
          gp[1] = (f32x4){accG[jj][4][i], accG[jj][5][i], accG[jj][6][i], accG[jj][7][i]};
        }
        up[0] = (f32x4){accU[jj][0][i], accU[jj][1][i], accU[jj][2][i], accU[jj][3][i]};
        up[1] = (f32x4){accU[jj][4][i], accU[jj][5][i], accU[jj][6][i], accU[jj][7][i]};
      }
    }
  }
}

// A quarter of build_frame's work (packed forms), for spreading one frame
// over four workgroups: part q (0..3) computes the rows {8m + j : j in
// {2q, 2q+1}} of G_t and U_t (the rows wave q owns in build_frame), its wave
// w the 8 accumulators of G_t (w < 2) or U_t (w >= 2) at j = 2q + w % 2.
// It loads and transposes all of the frame's K and V slabs as build_frame
// does, so each accumulator receives the same MFMAs on the same operands in
// the same order: every element it writes is bit-identical to build_frame's,
// and a wave's serial MFMA chain is a quarter as long.  Gout and Uout
// receive the part's whole rows of the packed forms (for G both triangles);
// stores go straight from registers.  `frag` is 32 KB of LDS; kDepth token
// iterations are loaded ahead.  All 256 threads must call it; on return this
// thread's stores are issued, not necessarily complete.
template <int kDepth>
__device__ __forceinline__ void build_frame_part(const uint16_t* __restrict__ Kf, const uint16_t* __restrict__ Vf,
                                                 int S, u32x4 (*__restrict__ frag)[8][kWave],
                                                 char* __restrict__ Gout, char* __restrict__ Uout, float ks,
                                                 int q) {
  constexpr int D = 128;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));  // opaque, as in build_frame
  const int w = tid >> 6, l = tid & 63;
  const int g = l >> 4, c = l & 15;
  const uint16_t* src = w < 2 ? Kf : Vf;
  const int slab = w & 1;
  const int j = 2 * q + (w & 1);   // the MFMA row fragment this wave accumulates
  const int au = w < 2 ? 0 : 2;    // A operand from the K units (G) or the V units (U)

  u32x4 x[kDepth][8];
  auto load = [&](auto jc, int it) {
    constexpr int jb = decltype(jc)::value;
    const int base = it * kBuildIterTok + slab * 32 + 8 * g;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int s = base + r;
      x[jb][r] = s < S ? *reinterpret_cast<const u32x4*>(src + (int64_t)s * D + 8 * c) : (u32x4){0u, 0u, 0u, 0u};
    }
  };
  f32x4 acc[8];
#pragma unroll
  for (int jp = 0; jp < 8; ++jp) acc[jp] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int iters = (S + kBuildIterTok - 1) / kBuildIterTok;
  auto iteration = [&](auto jc, int it) {
    constexpr int jb = decltype(jc)::value;
    __syncthreads();  // every wave is done reading the previous fragments
#pragma unroll
    for (int jf = 0; jf < 8; ++jf) {
      u32x4 o;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t lo = x[jb][2 * p][jf >> 1], hi = x[jb][2 * p + 1][jf >> 1];
        o[p] = (jf & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      frag[w][jf][l] = o;
    }
    __syncthreads();
    if (it + kDepth < iters) load(jc, it + kDepth);
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      u32x4 kf[8];
#pragma unroll
      for (int jp = 0; jp < 8; ++jp) kf[jp] = frag[sl][jp][l];
      const u32x4 a = frag[au + sl][j][l];
#pragma unroll
      for (int jp = 0; jp < 8; ++jp) acc[jp] = mfma16x16x32(a, kf[jp], acc[jp]);
    }
  };
  [&]<int... js>(std::integer_sequence<int, js...>) {
    ((js < iters ? load(std::integral_constant<int, js>{}, js) : void()), ...);
  }(std::make_integer_sequence<int, kDepth>{});
  for (int it0 = 0; it0 < iters; it0 += kDepth) {
    [&]<int... js>(std::integer_sequence<int, js...>) {
      ((it0 + js < iters ? iteration(std::integral_constant<int, js>{}, it0 + js) : void()), ...);
    }(std::make_integer_sequence<int, kDepth>{});
  }

  // lane (g, c), register r of accumulator jp holds X[32g + 8r + j][8c + jp];
  // each lane's 8 columns are one 16-byte chunk of the packed form
  if (w < 2) {
    const float ks2 = ks * ks;
#pragma unroll
    for (int jp = 0; jp < 8; ++jp) acc[jp] *= ks2;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 32 * g + 8 * r + j;
      const u32x2 p0 = split2(acc[0][r], acc[1][r]), p1 = split2(acc[2][r], acc[3][r]);
      const u32x2 p2 = split2(acc[4][r], acc[5][r]), p3 = split2(acc[6][r], acc[7][r]);
      *reinterpret_cast<u32x4*>(Gout + packed::g_chunk(row, 8 * c, 0)) = (u32x4){p0.x, p1.x, p2.x, p3.x};
      *reinterpret_cast<u32x4*>(Gout + packed::g_chunk(row, 8 * c, 1)) = (u32x4){p0.y, p1.y, p2.y, p3.y};
    }
  } else {
#pragma unroll
    for (int jp = 0; jp < 8; ++jp) acc[jp] *= ks;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 32 * g + 8 * r + j;
      *reinterpret_cast<f32x4*>(Uout + packed::u_chunk(row, 8 * c)) =
          (f32x4){acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
      *reinterpret_cast<f32x4*>(Uout + packed::u_chunk(row, 8 * c + 4)) =
          (f32x4){acc[4][r], acc[5][r], acc[6][r], acc[7][r]};
    }
  }
}

}  // namespace gdn
