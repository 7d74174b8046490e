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

template <bool kPacked, bool kWithG>
__global__ __launch_bounds__(256, 2) void k1_build_bf16_d128(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, void* __restrict__ Gout,
    float* __restrict__ Uout, int S, int64_t T, int t0, int nt, float ks, int64_t mT, int64_t mt0) {
  constexpr int D = 128;
  __shared__ u32x4 lds[build_lds_bytes<kPacked>() / 16];
  // workgroup i: frame t0 + i % nt of head i / nt (frames are [head][T];
  // its maps go to slot head * mT + t - mt0)
  const int64_t head = blockIdx.x / nt, t = t0 + blockIdx.x % nt;
  const int64_t f = head * T + t, mf = head * mT + t - mt0;
  const int64_t in_off = f * (int64_t)S * D, mat_off = mf * (int64_t)D * D;
  build_frame<kPacked, 1, false, kWithG>(K + in_off, V + in_off, S, lds,
                                         Gout ? static_cast<char*>(Gout) + mat_off * 4 : nullptr, Uout + mat_off, ks);
}

// The same maps for launches too small to fill the GPU (a few frames): the
// maps of one frame are split over kParts = 4 workgroups (build_frame_part),
// each with a quarter of the MFMA chain that bounds a lone workgroup; the
// results are bit-identical.  The four parts of a frame get workgroup ids 8
// apart, so that they share one XCD (workgroups are dealt to the 8 XCDs in
// turn) and its L2 serves the repeated loads.
constexpr int kParts = 4;
constexpr int kSplitDepth = 4;  // token iterations in flight per wave

__global__ __launch_bounds__(256, 2) void k1_build_bf16_d128_split(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, char* __restrict__ Gout,
    float* __restrict__ Uout, int S, int64_t T, int t0, int nt, int frames, float ks, int64_t mT, int64_t mt0) {
  constexpr int D = 128;
  __shared__ u32x4 frag[4][8][kWave];
  // workgroup b = 32 (i / 8) + 8 q + i % 8 holds part q of frame i
  const int b = blockIdx.x, xcd = b & 7, slot = b >> 3;
  const int q = slot & (kParts - 1), i = (slot / kParts) * 8 + xcd;
  if (i >= frames) return;
  const int64_t head = i / nt, t = t0 + i % nt;
  const int64_t f = head * T + t, mf = head * mT + t - mt0;
  const int64_t in_off = f * (int64_t)S * D, mat_off = mf * (int64_t)D * D * 4;
  build_frame_part<kSplitDepth>(K + in_off, V + in_off, S, frag, Gout + mat_off,
                                reinterpret_cast<char*>(Uout) + mat_off, ks, q);
}

}  // namespace

hipError_t launch_build_bf16_d128(const uint16_t* k, const uint16_t* v, void* G, bool packed_out,
                                  float* U, int64_t heads, int64_t T, int64_t t0, int64_t t1, int S, float ks,
                                  MapLayout ml, hipStream_t st) {
  const int nt = (int)(t1 - t0);
  const dim3 grid((unsigned)(heads * nt));
  if (packed_out && !G) return hipErrorInvalidValue;  // the packed form always writes G
  if (packed_out && heads * nt <= kFewFrames) {
    const int frames = (int)(heads * nt);
    const dim3 split((unsigned)((frames + 7) / 8 * 8 * kParts));
    hipLaunchKernelGGL(k1_build_bf16_d128_split, split, dim3(256), 0, st, k, v, static_cast<char*>(G), U, S, T,
                       (int)t0, nt, frames, ks, ml.T, ml.t0);
  } else if (packed_out)
    hipLaunchKernelGGL((k1_build_bf16_d128<true, true>), grid, dim3(256), 0, st, k, v, G, U, S, T, (int)t0, nt, ks,
                       ml.T, ml.t0);
  else if (G)
    hipLaunchKernelGGL((k1_build_bf16_d128<false, true>), grid, dim3(256), 0, st, k, v, G, U, S, T, (int)t0, nt, ks,
                       ml.T, ml.t0);
  else  // U_t only (the backward's P_t): G_t is not formed
    hipLaunchKernelGGL((k1_build_bf16_d128<false, false>), grid, dim3(256), 0, st, k, v, G, U, S, T, (int)t0, nt, ks,
                       ml.T, ml.t0);
  return hipGetLastError();
}

}  // namespace gdn
