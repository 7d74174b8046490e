// Plain float32 path of the frame-wise GDN for every supported head dim
// (multiples of 16 up to 128) and for float32 inputs: the same three stages
// as the MFMA path, written with LDS tiles and register-blocked float32 FMA.
//   build:  G_t = ks^2 K_t^T K_t, U_t = ks V_t^T K_t (ks: the key scale)
//   state:  M_t = gamma_t (M_{t-1} - beta_t M_{t-1} G_t) + beta_t U_t
//   output: O_t = Q_t M_t^T
// A 256-thread workgroup is a 16 x 16 grid; thread (ty, tx) owns the entries
// (ty + 16p, tx + 16q) of each D x D result, p, q < D/16.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kMaxD = 128;
constexpr int kMaxB = kMaxD / 16;  // entries per thread along one axis
constexpr int kTokTile = 32;

template <bool kBf16>
__device__ __forceinline__ float load_in(const void* p, int64_t i) {
  if constexpr (kBf16)
    return bf2f(static_cast<const uint16_t*>(p)[i]);
  else
    return static_cast<const float*>(p)[i];
}

template <bool kBf16>
__global__ __launch_bounds__(256) void g_build(const void* __restrict__ K, const void* __restrict__ V,
                                               float* __restrict__ G, float* __restrict__ U, int S, int D,
                                               float ks) {
  __shared__ float Ks[kTokTile][kMaxD + 1];
  __shared__ float Vs[kTokTile][kMaxD + 1];
  const int64_t f = blockIdx.x;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int nb = D / 16;
  float ag[kMaxB][kMaxB], au[kMaxB][kMaxB];
#pragma unroll
  for (int p = 0; p < kMaxB; ++p)
#pragma unroll
    for (int q = 0; q < kMaxB; ++q) ag[p][q] = au[p][q] = 0.f;

  const int64_t base = f * (int64_t)S * D;
  for (int s0 = 0; s0 < S; s0 += kTokTile) {
    __syncthreads();
    for (int idx = tid; idx < kTokTile * D; idx += 256) {
      const int s = idx / D, d = idx % D;
      const bool ok = s0 + s < S;
      Ks[s][d] = ok ? load_in<kBf16>(K, base + (int64_t)(s0 + s) * D + d) : 0.f;
      Vs[s][d] = ok ? load_in<kBf16>(V, base + (int64_t)(s0 + s) * D + d) : 0.f;
    }
    __syncthreads();
    for (int s = 0; s < kTokTile; ++s) {
      float ka[kMaxB], kb[kMaxB], va[kMaxB];
#pragma unroll
      for (int p = 0; p < kMaxB; ++p) {
        if (p < nb) {
          ka[p] = Ks[s][ty + 16 * p];
          va[p] = Vs[s][ty + 16 * p];
          kb[p] = Ks[s][tx + 16 * p];
        }
      }
#pragma unroll
      for (int p = 0; p < kMaxB; ++p)
#pragma unroll
        for (int q = 0; q < kMaxB; ++q)
          if (p < nb && q < nb) {
            ag[p][q] = fmaf(ka[p], kb[q], ag[p][q]);
            au[p][q] = fmaf(va[p], kb[q], au[p][q]);
          }
    }
  }
  float* Gf = G + f * (int64_t)D * D;
  float* Uf = U + f * (int64_t)D * D;
#pragma unroll
  for (int p = 0; p < kMaxB; ++p)
#pragma unroll
    for (int q = 0; q < kMaxB; ++q)
      if (p < nb && q < nb) {
        const int i = ty + 16 * p, j = tx + 16 * q;
        Gf[i * D + j] = ag[p][q] * (ks * ks);  // the key scale: twice in G, once in U
        Uf[i * D + j] = au[p][q] * ks;
      }
}

// One workgroup per head; M and G_t live in LDS.
__global__ __launch_bounds__(256) void g_state(const float* __restrict__ G, const float* __restrict__ U,
                                               const float* __restrict__ gamma, const float* __restrict__ beta,
                                               const float* state_in, float* __restrict__ M_all,
                                               float* state_out, int T, int D) {
  __shared__ float Ms[kMaxD][kMaxD + 1];
  __shared__ float Gs[kMaxD][kMaxD + 1];
  const int64_t h = blockIdx.x;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int nb = D / 16;
  const int64_t DD = (int64_t)D * D;

  float mreg[kMaxB][kMaxB];
#pragma unroll
  for (int p = 0; p < kMaxB; ++p)
#pragma unroll
    for (int q = 0; q < kMaxB; ++q)
      if (p < nb && q < nb) {
        const int i = ty + 16 * p, j = tx + 16 * q;
        mreg[p][q] = state_in ? state_in[h * DD + i * D + j] : 0.f;
        Ms[i][j] = mreg[p][q];
      }

  for (int t = 0; t < T; ++t) {
    const float* Gt = G + (h * T + t) * DD;
    for (int idx = tid; idx < D * D; idx += 256) Gs[idx / D][idx % D] = Gt[idx];
    __syncthreads();
    float acc[kMaxB][kMaxB];
#pragma unroll
    for (int p = 0; p < kMaxB; ++p)
#pragma unroll
      for (int q = 0; q < kMaxB; ++q) acc[p][q] = 0.f;
    for (int k = 0; k < D; ++k) {
      float mv[kMaxB], gv[kMaxB];
#pragma unroll
      for (int p = 0; p < kMaxB; ++p)
        if (p < nb) {
          mv[p] = Ms[ty + 16 * p][k];
          gv[p] = Gs[k][tx + 16 * p];
        }
#pragma unroll
      for (int p = 0; p < kMaxB; ++p)
#pragma unroll
        for (int q = 0; q < kMaxB; ++q)
          if (p < nb && q < nb) acc[p][q] = fmaf(mv[p], gv[q], acc[p][q]);
    }
    const float gm = gamma[h * T + t], bt = beta[h * T + t];
    const float* Ut = U + (h * T + t) * DD;
    float* Mt = M_all ? M_all + (h * T + t) * DD : nullptr;
#pragma unroll
    for (int p = 0; p < kMaxB; ++p)
#pragma unroll
      for (int q = 0; q < kMaxB; ++q)
        if (p < nb && q < nb) {
          const int i = ty + 16 * p, j = tx + 16 * q;
          mreg[p][q] = fmaf(gm, mreg[p][q], fmaf(-gm * bt, acc[p][q], bt * Ut[i * D + j]));
          if (Mt) Mt[i * D + j] = mreg[p][q];
        }
    __syncthreads();  // all reads of Ms and Gs for this frame are done
#pragma unroll
    for (int p = 0; p < kMaxB; ++p)
#pragma unroll
      for (int q = 0; q < kMaxB; ++q)
        if (p < nb && q < nb) Ms[ty + 16 * p][tx + 16 * q] = mreg[p][q];
  }
#pragma unroll
  for (int p = 0; p < kMaxB; ++p)
#pragma unroll
    for (int q = 0; q < kMaxB; ++q)
      if (p < nb && q < nb) state_out[h * DD + (ty + 16 * p) * D + tx + 16 * q] = mreg[p][q];
}

constexpr int kOutTok = 64;

// One workgroup per (frame, 64-token tile).
template <bool kInBf16, bool kOutBf16>
__global__ __launch_bounds__(256) void g_output(const void* __restrict__ Q, const float* __restrict__ M_all,
                                                void* __restrict__ out, int S, int D, int tiles) {
  __shared__ float Ms[kMaxD][kMaxD + 1];
  __shared__ float Qs[kOutTok][kMaxD + 1];
  const int64_t f = blockIdx.x / tiles;
  const int s0 = (blockIdx.x % tiles) * kOutTok;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int nb = D / 16;
  const float* Mt = M_all + f * (int64_t)D * D;
  for (int idx = tid; idx < D * D; idx += 256) Ms[idx / D][idx % D] = Mt[idx];
  const int64_t qbase = f * (int64_t)S * D;
  for (int idx = tid; idx < kOutTok * D; idx += 256) {
    const int s = idx / D, d = idx % D;
    Qs[s][d] = s0 + s < S ? load_in<kInBf16>(Q, qbase + (int64_t)(s0 + s) * D + d) : 0.f;
  }
  __syncthreads();
  // thread (ty, tx): tokens ty + 16p (p < 4), value dims tx + 16q (q < nb)
  float acc[4][kMaxB];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int q = 0; q < kMaxB; ++q) acc[p][q] = 0.f;
  for (int j = 0; j < D; ++j) {
    float qv[4], mv[kMaxB];
#pragma unroll
    for (int p = 0; p < 4; ++p) qv[p] = Qs[ty + 16 * p][j];
#pragma unroll
    for (int q = 0; q < kMaxB; ++q)
      if (q < nb) mv[q] = Ms[tx + 16 * q][j];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int q = 0; q < kMaxB; ++q)
        if (q < nb) acc[p][q] = fmaf(qv[p], mv[q], acc[p][q]);
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int s = s0 + ty + 16 * p;
    if (s >= S) continue;
#pragma unroll
    for (int q = 0; q < kMaxB; ++q)
      if (q < nb) {
        const int64_t o = qbase + (int64_t)s * D + tx + 16 * q;
        if constexpr (kOutBf16)
          static_cast<uint16_t*>(out)[o] = (uint16_t)f2bf(acc[p][q]);
        else
          static_cast<float*>(out)[o] = acc[p][q];
      }
  }
}

}  // namespace

hipError_t launch_build_generic(const void* k, const void* v, bool in_bf16, float* G, float* U,
                                int64_t frames, int S, int D, float ks, hipStream_t st) {
  if (in_bf16)
    hipLaunchKernelGGL(g_build<true>, dim3((unsigned)frames), dim3(256), 0, st, k, v, G, U, S, D, ks);
  else
    hipLaunchKernelGGL(g_build<false>, dim3((unsigned)frames), dim3(256), 0, st, k, v, G, U, S, D, ks);
  return hipGetLastError();
}

hipError_t launch_state_generic(const float* G, const float* U, const float* gamma,
                                const float* beta, const float* state_in, float* M_all,
                                float* state_out, int64_t heads, int64_t T, int D,
                                hipStream_t st) {
  hipLaunchKernelGGL(g_state, dim3((unsigned)heads), dim3(256), 0, st, G, U, gamma, beta, state_in,
                     M_all, state_out, (int)T, D);
  return hipGetLastError();
}

hipError_t launch_output_generic(const void* q, bool in_bf16, const float* M_all, void* out,
                                 bool out_bf16, int64_t frames, int S, int D, hipStream_t st) {
  const int tiles = (S + kOutTok - 1) / kOutTok;
  if (frames * tiles > (int64_t{1} << 31) / 256) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(frames * tiles));
  if (in_bf16) {
    if (out_bf16)
      hipLaunchKernelGGL((g_output<true, true>), grid, dim3(256), 0, st, q, M_all, out, S, D, tiles);
    else
      hipLaunchKernelGGL((g_output<true, false>), grid, dim3(256), 0, st, q, M_all, out, S, D, tiles);
  } else {
    if (out_bf16)
      hipLaunchKernelGGL((g_output<false, true>), grid, dim3(256), 0, st, q, M_all, out, S, D, tiles);
    else
      hipLaunchKernelGGL((g_output<false, false>), grid, dim3(256), 0, st, q, M_all, out, S, D, tiles);
  }
  return hipGetLastError();
}

}  // namespace gdn
