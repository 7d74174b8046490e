// Launchers of the backward-pass kernels (bf16 inputs, D == 128), kept apart
// from gdn_launch.h so that the forward kernels do not depend on them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Each launcher covers frames [t0, t1) of every head; per-frame matrices are
// float32 row-major [head][T][D][D].
//
// out_t = Q_t X_t^T, X_t = M_t (or M_t^T when trans_m).  (dq = dO M uses it.)
hipError_t launch_output_bwd_d128(const uint16_t* q, const float* M_all, float* out, bool trans_m,
                                  int64_t heads, int64_t T, int64_t t0, int64_t t1, int S, hipStream_t st);
// Reverse-time state pass of the backward: from G_t, U_t (packed forms),
// P_t = dO_t^T Q_t, the forward states M_all and the forward initial state
// m0 (null = zero), starting from the gradient reaching M_{t1-1} from later
// frames in d_state_out (null = zero), writes LB_t = beta_t Lambda_t,
// partial sums of dgamma_t and dbeta_t per 16-row block of the state
// (partials[head][T][kBwdParts][2]) and the gradient reaching M_{t0-1} in
// d_state_in (may equal d_state_out).
constexpr int kBwdParts = 8;
hipError_t launch_state_bwd_d128(const float* G, const float* U, const float* P, const float* M_all,
                                 const float* m0, const float* gamma, const float* beta,
                                 const float* d_state_out, float* LB, float* partials, float* d_state_in,
                                 int64_t heads, int64_t T, int64_t t0, int64_t t1, hipStream_t st);
// dgamma, dbeta [head][T] from the partial sums (fixed summation order).
hipError_t launch_bwd_reduce(const float* partials, float* dgamma, float* dbeta, int64_t frames,
                             hipStream_t st);
// dk_t = ks V_t LB_t + ks^2 K_t S_t and dv_t = ks K_t LB_t^T, float32 out,
// with S_t = -gamma_t (M_{t-1}^T LB_t + LB_t^T M_{t-1}) formed in the kernel
// (M_{-1} = m0, null = zero) and ks the forward's key scale (1 for none).
hipError_t launch_dkv_bwd_d128(const uint16_t* v, const uint16_t* k, const float* LB, const float* M_all,
                               const float* m0, const float* gamma, float ks, float* dk, float* dv, int64_t heads,
                               int64_t T, int64_t t0, int64_t t1, int S, hipStream_t st);

}  // namespace gdn
