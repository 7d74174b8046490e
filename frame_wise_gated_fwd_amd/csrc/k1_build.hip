// Per-frame maps of the frame-wise GDN on bf16 MFMA (gfx950), head dim 128,
// one workgroup per frame:
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
#include "frame_build.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

template <bool kPacked>
__global__ __launch_bounds__(256, 2) void k1_build_bf16_d128(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, void* __restrict__ Gout,
    float* __restrict__ Uout, int S, int64_t T, int t0, int nt, float ks) {
  constexpr int D = 128;
  __shared__ u32x4 lds[build_lds_bytes<kPacked>() / 16];
  // workgroup i: frame t0 + i % nt of head i / nt (frames are [head][T])
  const int64_t f = (int64_t)(blockIdx.x / nt) * T + t0 + blockIdx.x % nt;
  const int64_t in_off = f * (int64_t)S * D, mat_off = f * (int64_t)D * D;
  build_frame<kPacked>(K + in_off, V + in_off, S, lds, Gout ? static_cast<char*>(Gout) + mat_off * 4 : nullptr,
                       Uout + mat_off, ks);
}

// The same maps for launches too small to fill the GPU (a few frames): the
// maps of one frame are split over kParts = 4 workgroups.  Part q computes
// the rows {8m + j : j in {2q, 2q+1}} of G_t and U_t (the rows wave q owns
// above), its wave w the 8 accumulators of G_t (w < 2) or U_t (w >= 2) at
// j = 2q + w % 2.  Every part loads and transposes all of the frame's K and
// V slabs exactly as above, so each accumulator receives the same MFMAs on
// the same operands in the same order: the results are bit-identical, and a
// wave's serial MFMA chain, which bounds a lone workgroup, is a quarter as
// long.  Four token iterations are in flight per wave.  The four parts of a
// frame get workgroup ids 8 apart, so that they share one XCD (workgroups
// are dealt to the 8 XCDs in turn) and its L2 serves the repeated loads.
constexpr int kParts = 4;
constexpr int kSplitDepth = 4;

__global__ __launch_bounds__(256, 2) void k1_build_bf16_d128_split(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, char* __restrict__ Gout,
    float* __restrict__ Uout, int S, int64_t T, int t0, int nt, int frames, float ks) {
  constexpr int D = 128;
  __shared__ u32x4 frag[4][8][kWave];  // unit 0,1 = K slab 0,1; unit 2,3 = V slab 0,1
  // workgroup b = 32 (i / 8) + 8 q + i % 8 holds part q of frame i
  const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
  const int q = slot & (kParts - 1), i = (slot / kParts) * 8 + xcd;
  if (i >= frames) return;
  const int64_t f = (int64_t)(i / nt) * T + t0 + i % nt;
  const uint16_t* Kf = K + f * (int64_t)S * D;
  const uint16_t* Vf = V + f * (int64_t)S * D;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int g = l >> 4, c = l & 15;
  const uint16_t* src = w < 2 ? Kf : Vf;
  const int slab = w & 1;
  const int j = 2 * q + (w & 1);   // the MFMA row fragment this wave accumulates
  const int au = w < 2 ? 0 : 2;    // A operand from the K units (G) or the V units (U)

  u32x4 x[kSplitDepth][8];
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
    if (it + kSplitDepth < iters) load(jc, it + kSplitDepth);
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
  }(std::make_integer_sequence<int, kSplitDepth>{});
  for (int it0 = 0; it0 < iters; it0 += kSplitDepth) {
    [&]<int... js>(std::integer_sequence<int, js...>) {
      ((it0 + js < iters ? iteration(std::integral_constant<int, js>{}, it0 + js) : void()), ...);
    }(std::make_integer_sequence<int, kSplitDepth>{});
  }

  // lane (g, c), register r of accumulator jp holds X[32g + 8r + j][8c + jp];
  // each lane's 8 columns are one 16-byte chunk of the packed form
  const int64_t mat_off = f * (int64_t)D * D * 4;
  if (w < 2) {
    const float ks2 = ks * ks;
#pragma unroll
    for (int jp = 0; jp < 8; ++jp) acc[jp] *= ks2;
    char* gp = Gout + mat_off;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 32 * g + 8 * r + j;
      const u32x2 p0 = split2(acc[0][r], acc[1][r]), p1 = split2(acc[2][r], acc[3][r]);
      const u32x2 p2 = split2(acc[4][r], acc[5][r]), p3 = split2(acc[6][r], acc[7][r]);
      *reinterpret_cast<u32x4*>(gp + packed::g_chunk(row, 8 * c, 0)) = (u32x4){p0.x, p1.x, p2.x, p3.x};
      *reinterpret_cast<u32x4*>(gp + packed::g_chunk(row, 8 * c, 1)) = (u32x4){p0.y, p1.y, p2.y, p3.y};
    }
  } else {
#pragma unroll
    for (int jp = 0; jp < 8; ++jp) acc[jp] *= ks;
    char* up = reinterpret_cast<char*>(Uout) + mat_off;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 32 * g + 8 * r + j;
      *reinterpret_cast<f32x4*>(up + packed::u_chunk(row, 8 * c)) =
          (f32x4){acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
      *reinterpret_cast<f32x4*>(up + packed::u_chunk(row, 8 * c + 4)) =
          (f32x4){acc[4][r], acc[5][r], acc[6][r], acc[7][r]};
    }
  }
}

}  // namespace

hipError_t launch_build_bf16_d128(const uint16_t* k, const uint16_t* v, void* G, bool packed_out,
                                  float* U, int64_t heads, int64_t T, int64_t t0, int64_t t1, int S, float ks,
                                  hipStream_t st) {
  const int nt = (int)(t1 - t0);
  const dim3 grid((unsigned)(heads * nt));
  if (packed_out && !G) return hipErrorInvalidValue;  // the packed form always writes G
  if (packed_out && heads * nt <= kFewFrames) {
    const int frames = (int)(heads * nt);
    const dim3 split((unsigned)((frames + 7) / 8 * 8 * kParts));
    hipLaunchKernelGGL(k1_build_bf16_d128_split, split, dim3(256), 0, st, k, v, static_cast<char*>(G), U, S, T,
                       (int)t0, nt, frames, ks);
  } else if (packed_out)
    hipLaunchKernelGGL(k1_build_bf16_d128<true>, grid, dim3(256), 0, st, k, v, G, U, S, T, (int)t0, nt, ks);
  else
    hipLaunchKernelGGL(k1_build_bf16_d128<false>, grid, dim3(256), 0, st, k, v, G, U, S, T, (int)t0, nt, ks);
  return hipGetLastError();
}

}  // namespace gdn
