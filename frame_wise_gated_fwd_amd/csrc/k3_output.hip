// Output of the frame-wise GDN on bf16 MFMA (gfx950), head dim 128, one
// workgroup per frame:
//   O_t = Q_t M_t^T        (Q_t: S x 128 bf16, M_t: 128 x 128 float32)
// M_t enters the MFMA as a bf16 hi/lo pair (two passes, Q*Mhi + Q*Mlo); the
// pair carries M_t to about 2^-17 relative, so O keeps float32 accuracy.
//
// One workgroup per frame (frame_output.h has the tiling and the access
// patterns), or per token part of a frame when a launch has only a few
// frames; frames [t0, t0 + nt) of every head per launch.  The backward pass
// uses it as well, with M_t given as float32 and optionally transposed (see
// output_frame).
#include "frame_output.h"
#include "gdn_backward.h"
#include "gdn_launch.h"

#include <algorithm>

namespace gdn {
namespace {

template <bool kPackedM, bool kOutBf16, bool kTransM = false>
__global__ __launch_bounds__(256, 2) void k3_output_bf16_d128(
    const uint16_t* __restrict__ Q, const void* __restrict__ M_all, void* __restrict__ out, int S,
    int64_t T, int t0, int nt, int nsplit, int64_t mT, int64_t mt0) {
  constexpr int D = 128;
  __shared__ uint16_t Ml[2][D][kOutLdsW];
  // workgroup i: token part i % nsplit of frame t0 + j % nt of head j / nt,
  // j = i / nsplit (frames are [head][T])
  const int j = blockIdx.x / nsplit, part = blockIdx.x % nsplit;
  const int64_t head = j / nt, t = t0 + j % nt;
  const int64_t f = head * T + t, mf = head * mT + t - mt0;  // M_t in slot mf
  const int s0 = (int)((int64_t)part * S / nsplit), s1 = (int)((int64_t)(part + 1) * S / nsplit);
  const int64_t in_off = (f * (int64_t)S + s0) * D;
  const char* Mt = static_cast<const char*>(M_all) + mf * packed::kFrameBytes;
  void* Of = static_cast<char*>(out) + in_off * (kOutBf16 ? 2 : 4);
  output_frame<kPackedM, kOutBf16, 1, kTransM>(Q + in_off, Mt, Of, s1 - s0, Ml, [] {});
}

}  // namespace

// A launch of a few frames splits each frame's tokens over up to 8
// workgroups (each token's arithmetic is unchanged).
int token_split(int64_t frames, int S) {
  return frames <= kFewFrames ? (int)std::min<int64_t>({8, 512 / frames, S}) : 1;
}

template <bool kPackedM>
hipError_t launch_out(const uint16_t* q, const void* M_all, void* out, bool out_bf16, int64_t heads,
                      int64_t T, int64_t t0, int64_t t1, int S, MapLayout ml, hipStream_t st) {
  const int nt = (int)(t1 - t0);
  const int64_t frames = heads * nt;
  const int nsplit = token_split(frames, S);
  const dim3 grid((unsigned)(frames * nsplit));
  if (out_bf16)
    hipLaunchKernelGGL((k3_output_bf16_d128<kPackedM, true>), grid, dim3(256), 0, st, q, M_all, out, S, T,
                       (int)t0, nt, nsplit, ml.T, ml.t0);
  else
    hipLaunchKernelGGL((k3_output_bf16_d128<kPackedM, false>), grid, dim3(256), 0, st, q, M_all, out, S, T,
                       (int)t0, nt, nsplit, ml.T, ml.t0);
  return hipGetLastError();
}

template <bool kTransM>
hipError_t launch_out_bwd(const uint16_t* q, const float* M_all, float* out, int64_t heads, int64_t T, int64_t t0,
                          int64_t t1, int S, hipStream_t st) {
  const int nt = (int)(t1 - t0);
  const int64_t frames = heads * nt;
  const int nsplit = token_split(frames, S);
  hipLaunchKernelGGL((k3_output_bf16_d128<false, false, kTransM>), dim3((unsigned)(frames * nsplit)), dim3(256),
                     0, st, q, M_all, out, S, T, (int)t0, nt, nsplit, T, int64_t{0});
  return hipGetLastError();
}

hipError_t launch_output_bwd_d128(const uint16_t* q, const float* M_all, float* out, bool trans_m, int64_t heads,
                                  int64_t T, int64_t t0, int64_t t1, int S, hipStream_t st) {
  return trans_m ? launch_out_bwd<true>(q, M_all, out, heads, T, t0, t1, S, st)
                 : launch_out_bwd<false>(q, M_all, out, heads, T, t0, t1, S, st);
}

hipError_t launch_output_bf16_d128(const uint16_t* q, const void* M_all, bool packed_m, void* out,
                                   bool out_bf16, int64_t heads, int64_t T, int64_t t0, int64_t t1, int S,
                                   MapLayout ml, hipStream_t st) {
  return packed_m ? launch_out<true>(q, M_all, out, out_bf16, heads, T, t0, t1, S, ml, st)
                 : launch_out<false>(q, M_all, out, out_bf16, heads, T, t0, t1, S, ml, st);
}

}  // namespace gdn
