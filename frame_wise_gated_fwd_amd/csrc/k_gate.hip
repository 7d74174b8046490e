// The gates of every frame from activations (frame_gate.h), one workgroup
// per frame, before the frame-wise GDN on every path.  (Computed inside the
// fused kernel instead, by its build items or by its state pass, the same
// call measured 8 % and 27 % slower: the build items set the kernel's
// throughput and the state pass its chain; this pass costs about 1 %.)
#include "frame_gate.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

__global__ __launch_bounds__(256) void k_frame_gates(const float* __restrict__ a, const float* __restrict__ b,
                                                    const float* __restrict__ A_log,
                                                    const float* __restrict__ dt_bias, float* gamma, float* beta,
                                                    int H, int T, int S) {
  __shared__ float red[8];
  const int64_t f = blockIdx.x;  // frame index in [B, H, T] order
  const int h = (int)((f / T) % H);
  const Gates gt = frame_gates(a + f * S, b + f * S, S, A_log[h], dt_bias[h], red);
  if (threadIdx.x == 0) {
    gamma[f] = gt.gamma;
    beta[f] = gt.beta;
  }
}

}  // namespace

hipError_t launch_frame_gates(const float* a, const float* b, const float* A_log, const float* dt_bias, float* gamma,
                              float* beta, int64_t frames, int H, int T, int S, hipStream_t st) {
  hipLaunchKernelGGL(k_frame_gates, dim3((unsigned)frames), dim3(256), 0, st, a, b, A_log, dt_bias, gamma, beta, H, T,
                     S);
  return hipGetLastError();
}

}  // namespace gdn
