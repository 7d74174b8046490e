// Softmax attention of the chunk-causal variant with attention sinks and a
// local temporal window, bf16 inputs, head dim 128, on bf16 MFMA (gfx950).
//
// The pages put 5 softmax attention blocks among the 20 blocks of the model
// for exact long-range recall ("SANA-WM: NVIDIA puts a one-minute world
// model on a single GPU", zhichai.net, section 1), and give their
// chunk-causal autoregressive variant attention-sink tokens and local
// temporal windows so that memory stays constant over a long rollout (same
// page, training pipeline, Stage 4).  Per head, over T latent frames of S
// tokens grouped into generation chunks (chunk 0: the first `first_chunk`
// frames, then `chunk` frames each), a query of chunk c attends to every
// token of chunks c - window + 1 .. c and of the first `sink` frames that
// lie in chunks up to c:
//     O = softmax(Q K^T / sqrt(128)) V  over those keys,  lse = ln sum exp.
//
// One workgroup per 128 queries of one chunk (all of them see the same keys,
// so no per-element mask is needed except past the end of a key range).
// Key tiles of 64 tokens are staged through LDS (double-buffered, loaded a
// tile ahead through registers).  Each wave owns 32 queries and computes
//   S^T = K Q^T   (A = K rows from LDS, B = Q held in registers),
// so that every lane holds scores of one query, n = lane % 16 of its
// 16-query block, for keys 4g .. 4g+3 (g = lane / 16) of each 16-key block.
// That is already the B operand of O^T = V^T P^T for a 32-key step whose
// reduction slot (g, e) is key 4g + e (e < 4) or 16 + 4g + e - 4 (e >= 4),
// so the probabilities never move between lanes; the A operand V^T comes
// from gfx950's transposed LDS read.  The online softmax's row maximum is
// combined over the four lanes of a query; row sums stay per lane until the
// end.  P enters the MFMA as a bf16 hi/lo pair (two passes), which keeps the
// weights to about 2^-17 relative, so O has float32 accuracy.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int D = 128;
constexpr int kQTile = 128;        // queries per workgroup, 32 per wave
constexpr int kKTile = 64;         // keys per step
constexpr int kLdsW = D + 16;      // padded LDS row (bf16): 288 bytes
constexpr int kXcd = 8;

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* out;
  float* lse;              // may be null
  int T, S;
  int sink, first_chunk, chunk, window;
  int tiles0, tilesc;      // query tiles of chunk 0 and of a full later chunk
  int tiles_per_head;
  int64_t total_tiles;
  int64_t per_xcd;         // logical tiles per XCD
  float scale_log2;        // log2(e) / sqrt(D)
};

// frames [f0, f1) of chunk c
__device__ __forceinline__ void chunk_frames(const AttnArgs& a, int c, int& f0, int& f1) {
  if (c == 0) {
    f0 = 0;
    f1 = a.first_chunk < a.T ? a.first_chunk : a.T;
  } else {
    f0 = a.first_chunk + (c - 1) * a.chunk;
    f1 = f0 + a.chunk < a.T ? f0 + a.chunk : a.T;
  }
}

// Reductions over the four lanes of a query (n, n + 16, n + 32, n + 48)
// with gfx950's row swaps, in registers: v_permlane16_swap exchanges the odd
// 16-lane rows of one operand with the even rows of the other, so with both
// operands x each lane ends with the pair (x of its even row, x of its odd
// row); v_permlane32_swap does the same for the two halves.  Combining the
// two results gives every lane of a pair the same value.
__device__ __forceinline__ float pair16(float x, bool mx) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return mx ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float pair32(float x, bool mx) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return mx ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float wave_max4(float x) { return pair32(pair16(x, true), true); }
__device__ __forceinline__ float wave_sum4(float x) { return pair32(pair16(x, false), false); }

__global__ __launch_bounds__(256, 2) void k_attn_d128(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kKTile][kLdsW];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kKTile][kLdsW];

  // XCD-aware order: the workgroups of one XCD (id % 8) take a contiguous
  // run of (head, chunk, tile) items, so consecutive chunks of a head, which
  // share most of their keys, are served by one L2.
  const int64_t L = (int64_t)(blockIdx.x % kXcd) * a.per_xcd + blockIdx.x / kXcd;
  if (L >= a.total_tiles) return;
  const int head = (int)(L / a.tiles_per_head);
  int r = (int)(L % a.tiles_per_head);
  int c, j;
  if (r < a.tiles0) {
    c = 0;
    j = r;
  } else {
    r -= a.tiles0;
    c = 1 + r / a.tilesc;
    j = r % a.tilesc;
  }
  int qf0, qf1;
  chunk_frames(a, c, qf0, qf1);
  const int S = a.S;
  const int64_t hbase = (int64_t)head * a.T * S;  // first token of the head
  const int q_lo = qf0 * S + j * kQTile;          // this tile's queries, head-relative tokens
  const int q_hi = min(q_lo + kQTile, qf1 * S);

  // visible key ranges (head-relative tokens): sinks up to this chunk and the window
  const int lo_chunk = c - a.window + 1 > 0 ? c - a.window + 1 : 0;
  int wf0, wf1;
  chunk_frames(a, lo_chunk, wf0, wf1);
  const int sink_end = a.sink < qf1 ? a.sink : qf1;  // sink frames in chunks <= c
  int r0a, r0b, r1a, r1b;                           // ranges [r0a, r0b) and [r1a, r1b)
  if (sink_end >= wf0) {
    r0a = 0, r0b = qf1 * S, r1a = r1b = 0;
  } else {
    r0a = 0, r0b = sink_end * S, r1a = wf0 * S, r1b = qf1 * S;
  }
  const int n0 = (r0b - r0a + kKTile - 1) / kKTile, n1 = (r1b - r1a + kKTile - 1) / kKTile;
  const int nsteps = n0 + n1;
  auto step_base = [&](int s, int& base, int& end) {
    if (s < n0) base = r0a + s * kKTile, end = r0b;
    else base = r1a + (s - n0) * kKTile, end = r1b;
  };

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int n = l & 15, g = l >> 4;

  // Q of this wave as B operands: lane (n, g) holds query 16 qb + n, dims 32 kb + 8g .. +7
  const int qw = q_lo + 32 * w;
  u32x4 qop[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = qw + 16 * qb + n;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      qop[qb][kb] = qi < q_hi ? *reinterpret_cast<const u32x4*>(a.q + (hbase + qi) * D + 32 * kb + 8 * g)
                              : (u32x4){0u, 0u, 0u, 0u};
  }

  // staging: chunk i of a tile is row (tid + 256 i) / 16, 16-byte column (tid + 256 i) % 16
  u32x4 kst[4], vst[4];
  auto load_tile = [&](int s) {
    int base, end;
    step_base(s, base, end);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + 256 * i, row = ch >> 4, col = ch & 15;
      const int key = base + row;
      const bool ok = key < end;
      kst[i] = ok ? ld_nt(reinterpret_cast<const u32x4*>(a.k + (hbase + key) * D) + col) : (u32x4){0u, 0u, 0u, 0u};
      vst[i] = ok ? ld_nt(reinterpret_cast<const u32x4*>(a.v + (hbase + key) * D) + col) : (u32x4){0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + 256 * i, row = ch >> 4, col = ch & 15;
      *reinterpret_cast<u32x4*>(&Ks[buf][row][8 * col]) = kst[i];
      *reinterpret_cast<u32x4*>(&Vs[buf][row][8 * col]) = vst[i];
    }
  };

  f32x4 acc[8][2];  // O^T: d block db, query block qb; lane (n, g): dims 16db + 4g + i of query n
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) acc[db][qb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m[2] = {-__builtin_inff(), -__builtin_inff()};  // running max (log2 domain) of query n, per qb
  float lsum[2] = {0.f, 0.f};                             // this lane's part of the row sum

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) load_tile(s + 1);  // in flight during this step
    int base, end;
    step_base(s, base, end);

    // S^T = K Q^T for 64 keys x 32 queries
    f32x4 sc[4][2];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) sc[kk][qb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(&Ks[buf][16 * kk + n][32 * kb + 8 * g]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) sc[kk][qb] = mfma16x16x32(ka, qop[qb][kb], sc[kk][qb]);
      }

    // online softmax; lane (n, g) holds keys base + 16 kk + 4g + i of query n
    float p[4][2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool valid = base + 16 * kk + 4 * g + i < end;
          const float x = valid ? sc[kk][qb][i] * a.scale_log2 : -__builtin_inff();
          p[kk][qb][i] = x;
          mx = fmaxf(mx, x);
        }
      mx = wave_max4(mx);
      const float mn = fmaxf(m[qb], mx);  // finite: every step has a visible key
      const float alpha = __builtin_amdgcn_exp2f(m[qb] - mn);
      m[qb] = mn;
      float sum = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(p[kk][qb][i] - mn);
          p[kk][qb][i] = e;
          sum += e;
        }
      lsum[qb] = lsum[qb] * alpha + sum;
#pragma unroll
      for (int db = 0; db < 8; ++db) acc[db][qb] *= alpha;
    }

    // O^T += V^T P^T over two 32-key steps, P as bf16 hi + lo
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 phi[2], plo[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        u32x4 h, lo;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          // slot pair (2 e2, 2 e2 + 1): e < 4 from key block 2 ks, else 2 ks + 1
          const int kk = 2 * ks + (e2 >> 1), i0 = 2 * (e2 & 1);
          const u32x2 sp = split2(p[kk][qb][i0], p[kk][qb][i0 + 1]);
          h[e2] = sp.x;
          lo[e2] = sp.y;
        }
        phi[qb] = h;
        plo[qb] = lo;
      }
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        // lane (i, g) of the A operand: V[key(g, e)][16 db + i]; the addressing lane
        // 4e' + jj names key 32 ks + 4g + e' (+16 for the second read), columns 16 db + 4 jj
        const int e1 = n >> 2, jj = n & 3;
        const u32x2 v0 = lds_read_tr16(&Vs[buf][32 * ks + 4 * g + e1][16 * db + 4 * jj]);
        const u32x2 v1 = lds_read_tr16(&Vs[buf][32 * ks + 16 + 4 * g + e1][16 * db + 4 * jj]);
        const u32x4 vt = {v0.x, v0.y, v1.x, v1.y};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          acc[db][qb] = mfma16x16x32(vt, phi[qb], acc[db][qb]);
          acc[db][qb] = mfma16x16x32(vt, plo[qb], acc[db][qb]);
        }
      }
    }

    // buffer buf ^ 1 was last read in step s - 1, before the barrier that ended it
    if (s + 1 < nsteps) store_tile(buf ^ 1);
    __syncthreads();
  }

  // normalise and store: lane (n, g) writes dims 16 db + 4g .. +3 of query 16 qb + n
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float total = wave_sum4(lsum[qb]);
    const float inv = 1.f / total;
    const int qi = qw + 16 * qb + n;
    if (qi < q_hi) {
      float* orow = a.out + (hbase + qi) * D;
#pragma unroll
      for (int db = 0; db < 8; ++db) st_nt(reinterpret_cast<f32x4*>(orow + 16 * db + 4 * g), acc[db][qb] * inv);
      if (a.lse && g == 0) a.lse[hbase + qi] = (m[qb] + __log2f(total)) * 0.69314718055994531f;
    }
  }
}

}  // namespace

// Query tiles per head for T frames of S tokens: ceil(frames * S / 128) per chunk.
hipError_t launch_attn_d128(const uint16_t* q, const uint16_t* k, const uint16_t* v, float* out, float* lse,
                            int64_t heads, int T, int S, int sink, int first_chunk, int chunk, int window,
                            hipStream_t st) {
  AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.T = T;
  a.S = S;
  a.sink = sink;
  a.first_chunk = first_chunk;
  a.chunk = chunk;
  a.window = window;
  const int f0 = first_chunk < T ? first_chunk : T;
  a.tiles0 = (int)(((int64_t)f0 * S + kQTile - 1) / kQTile);
  a.tilesc = (int)(((int64_t)chunk * S + kQTile - 1) / kQTile);
  int64_t tiles = a.tiles0;
  if (T > first_chunk) {
    const int rest = T - first_chunk, full = rest / chunk, part = rest % chunk;
    tiles += (int64_t)full * a.tilesc + ((int64_t)part * S + kQTile - 1) / kQTile;
  }
  a.tiles_per_head = (int)tiles;
  a.total_tiles = tiles * heads;
  a.per_xcd = (a.total_tiles + kXcd - 1) / kXcd;
  a.scale_log2 = 1.4426950408889634f / sqrtf((float)D);
  const int64_t grid = a.per_xcd * kXcd;
  hipLaunchKernelGGL(k_attn_d128, dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace gdn
