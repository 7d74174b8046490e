// Internal launchers (host side).  Arguments are validated by gdn_api.cpp
// before any of these is called; each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// ---- MFMA path: bf16 inputs, D == 128 --------------------------------------
// G_t = K_t^T K_t, U_t = V_t^T K_t for `frames` frames of S tokens.
hipError_t launch_build_bf16_d128(const uint16_t* k, const uint16_t* v, float* G, float* U,
                                  int64_t frames, int S, hipStream_t st);
// State pass over T frames for `heads` heads; M_all may be null.
hipError_t launch_state_d128(const float* G, const float* U, const float* gamma,
                             const float* beta, const float* state_in, float* M_all,
                             float* state_out, int64_t heads, int64_t T, hipStream_t st);
// O_t = Q_t M_t^T; out_bf16 selects the output dtype.
hipError_t launch_output_bf16_d128(const uint16_t* q, const float* M_all, void* out,
                                   bool out_bf16, int64_t frames, int S, hipStream_t st);

// ---- plain float32 path: any supported D, f32 or bf16 inputs ---------------
hipError_t launch_build_generic(const void* k, const void* v, bool in_bf16, float* G, float* U,
                                int64_t frames, int S, int D, hipStream_t st);
hipError_t launch_state_generic(const float* G, const float* U, const float* gamma,
                                const float* beta, const float* state_in, float* M_all,
                                float* state_out, int64_t heads, int64_t T, int D,
                                hipStream_t st);
hipError_t launch_output_generic(const void* q, bool in_bf16, const float* M_all, void* out,
                                 bool out_bf16, int64_t frames, int S, int D, hipStream_t st);

}  // namespace gdn
