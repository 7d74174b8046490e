// Degenerate shapes of the frame-wise GDN: no frames (T = 0) or frames with
// no tokens (S = 0).  The recurrence of "SANA-WM: NVIDIA puts a one-minute
// world model on a single GPU" (zhichai.net, section 1) still defines the
// state there:
//   T = 0:  no step is taken, so M_T = M_0 (state_in, zeros when NULL);
//   S = 0:  a frame without tokens has G_t = K_t^T K_t = 0 and U_t = 0, so
//           each step only decays the state: M_t = gamma_t M_{t-1}.
// Its backward, for the loss <dM_T, M_T> (no output when S = 0):
//   Lambda_t = (prod_{u>t} gamma_u) dM_T, M_{t-1} = (prod_{u<t} gamma_u) M_0,
//   dgamma_t = <Lambda_t, M_{t-1}> = (prod_{u != t} gamma_u) <dM_T, M_0>,
//   dbeta_t = <Lambda_t, U_t> - gamma_t <Lambda_t G_t, M_{t-1}> = 0,
//   d(state_in) = (prod_u gamma_u) dM_T.
// Plain float32 kernels; every thread owns one state element.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;

// dst = src, or zeros when src is null.
__global__ __launch_bounds__(kThreads) void e_fill(const float* __restrict__ src, float* __restrict__ dst,
                                                   int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.f;
}

// M_t = gamma_t M_{t-1}, one float32 product per frame in frame order.
// Block b covers elements [c * 256, c * 256 + 256) of head h = b / chunks's
// D x D state, c = b % chunks; state_out may equal state_in (each thread
// reads its element first).
__global__ __launch_bounds__(kThreads) void e_decay(const float* gamma, const float* state_in,
                                                    float* state_out, int64_t T, int dd, int chunks) {
  const int64_t h = blockIdx.x / chunks;
  const int e = (int)(blockIdx.x % chunks) * kThreads + threadIdx.x;
  if (e >= dd) return;
  const int64_t i = h * dd + e;
  float m = state_in ? state_in[i] : 0.f;
  const float* gh = gamma + h * T;
  for (int64_t t = 0; t < T; ++t) m = gh[t] * m;
  state_out[i] = m;
}

// The backward above, one workgroup per head.  d_state_in may equal
// d_state_out: every read of d_state_out precedes the barrier after which
// d_state_in is written.
__global__ __launch_bounds__(kThreads) void e_decay_bwd(const float* gamma, const float* state_in,
                                                        const float* d_state_out, float* dgamma, float* dbeta,
                                                        float* d_state_in, int64_t T, int dd) {
  __shared__ float part[kThreads];
  __shared__ float total_decay;
  const int64_t h = blockIdx.x;
  const int tid = threadIdx.x;
  const float* m0 = state_in ? state_in + h * dd : nullptr;
  const float* dm = d_state_out ? d_state_out + h * dd : nullptr;
  // <dM_T, M_0>: per-thread sums in element order, then a fixed tree
  float acc = 0.f;
  if (m0 && dm)
    for (int e = tid; e < dd; e += kThreads) acc = fmaf(dm[e], m0[e], acc);
  part[tid] = acc;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) part[tid] += part[tid + w];
    __syncthreads();
  }
  const float dot = part[0];
  float* dg = dgamma + h * T;
  float* db = dbeta + h * T;
  const float* gh = gamma + h * T;
  if (tid == 0) {
    // suffix products first (dg[t] = prod_{u>t} gamma_u), then the prefix
    float s = 1.f;
    for (int64_t t = T - 1; t >= 0; --t) {
      dg[t] = s;
      s = s * gh[t];
    }
    total_decay = s;
    float p = 1.f;
    for (int64_t t = 0; t < T; ++t) {
      dg[t] = dot * (p * dg[t]);
      p = p * gh[t];
    }
  }
  for (int64_t t = tid; t < T; t += kThreads) db[t] = 0.f;
  __syncthreads();
  const float c = total_decay;
  for (int e = tid; e < dd; e += kThreads) d_state_in[h * dd + e] = dm ? c * dm[e] : 0.f;
}

}  // namespace

hipError_t launch_state_fill(const float* src, float* dst, int64_t n, hipStream_t st) {
  if (n <= 0 || src == dst) return hipSuccess;
  hipLaunchKernelGGL(e_fill, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, st, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_decay(const float* gamma, const float* state_in, float* state_out, int64_t heads, int64_t T,
                        int D, hipStream_t st) {
  const int dd = D * D, chunks = (dd + kThreads - 1) / kThreads;
  if (heads <= 0) return hipSuccess;
  hipLaunchKernelGGL(e_decay, dim3((unsigned)(heads * chunks)), dim3(kThreads), 0, st, gamma, state_in, state_out,
                     T, dd, chunks);
  return hipGetLastError();
}

hipError_t launch_decay_bwd(const float* gamma, const float* state_in, const float* d_state_out, float* dgamma,
                            float* dbeta, float* d_state_in, int64_t heads, int64_t T, int D, hipStream_t st) {
  if (heads <= 0) return hipSuccess;
  hipLaunchKernelGGL(e_decay_bwd, dim3((unsigned)heads), dim3(kThreads), 0, st, gamma, state_in, d_state_out,
                     dgamma, dbeta, d_state_in, T, D * D);
  return hipGetLastError();
}

}  // namespace gdn
