// The gates of one frame of the frame-wise GDN, computed from activations:
//   gamma_t = exp(-exp(A_log) * softplus(mean_s a[t, s] + dt_bias)),
//   beta_t  = sigmoid(mean_s b[t, s]),
// a, b: the per-token gate pre-activations the layer's projections give for
// this head; A_log, dt_bias: the head's learned parameters.  The pages call
// gamma a learned decay scalar and beta the delta-rule strength ("SANA-WM:
// NVIDIA puts a one-minute world model on a single GPU", zhichai.net,
// section 1) and fuse the gate operations into the scan kernels (training
// pipeline); the parameterisation itself is not on the pages (a gated
// linear recurrence's per-head log-rate, pooled over the frame because one
// step consumes a whole frame).
//
// The token sums are reduced in a fixed order (per thread, then a butterfly
// inside each wave, then the four waves in order), so the gates of a frame
// are the same float32 values whatever launch computes them.
#pragma once

#include "gdn_common.h"

namespace gdn {

struct Gates {
  float gamma, beta;
};

// Sum over the 64 lanes of a wave by an xor butterfly: every lane ends with
// the same bits (each step adds the same two values in either order).
__device__ __forceinline__ float wave_sum_butterfly(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// The gates from the frame's token sums ta, tb (over its S tokens).
__device__ __forceinline__ Gates gates_from_sums(float ta, float tb, int S, float A_log, float dt_bias) {
  const float x = ta / (float)S + dt_bias;
  const float sp = x > 20.f ? x : log1pf(expf(x));  // softplus; above 20 it equals x in float32
  return {expf(-expf(A_log) * sp), 1.f / (1.f + expf(-(tb / (float)S)))};
}

// All 256 threads of the workgroup call it with the same arguments; `red`
// is 8 floats of LDS.  S >= 1.  Returns the frame's gates in every thread.
// Order of the token sums: thread i adds tokens i, i + 256, i + 512, ... in
// that order, starting from 0; then the butterfly in each wave; then the
// four waves' sums as ((w0 + w1) + w2) + w3.
__device__ inline Gates frame_gates(const float* __restrict__ a, const float* __restrict__ b, int S, float A_log,
                                    float dt_bias, float* red) {
  float sa = 0.f, sb = 0.f;
  for (int s = threadIdx.x; s < S; s += 256) {
    sa += a[s];
    sb += b[s];
  }
  sa = wave_sum_butterfly(sa);
  sb = wave_sum_butterfly(sb);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[w] = sa;
    red[4 + w] = sb;
  }
  __syncthreads();
  const float ta = ((red[0] + red[1]) + red[2]) + red[3];
  const float tb = ((red[4] + red[5]) + red[6]) + red[7];
  __syncthreads();  // `red` may be written again after this
  return gates_from_sums(ta, tb, S, A_log, dt_bias);
}

}  // namespace gdn
