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
// Key and value tiles of 64 tokens go to LDS by direct global-to-LDS loads,
// a step ahead (two buffers each).  Each wave owns 32 queries and computes
//   S^T = K Q^T   (A = K rows from LDS, B = Q held in registers),
// so that every lane holds scores of one query, n = lane % 16 of its
// 16-query block, for keys 4g .. 4g+3 (g = lane / 16) of each 16-key block.
// That is already the B operand of O^T = V^T P^T for a 32-key step whose
// reduction slot (g, e) is key 4g + e (e < 4) or 16 + 4g + e - 4 (e >= 4),
// so the probabilities never move between lanes; the A operand V^T comes
// from gfx950's transposed LDS read.  The online softmax's row maximum is
// combined over the four lanes of a query; row sums stay per lane until the
// end.  P enters the MFMA as a bf16 hi/lo pair (two passes), which keeps the
// weights to about 2^-17 relative, so O has float32 accuracy.  A step's
// scores come from the step before, so that its exponentials run beside the
// next tile's Q K^T and its own P V on the matrix cores.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int D = 128;
constexpr int kQTile = 128;        // queries per workgroup, 32 per wave
constexpr int kKTile = 64;         // keys per step
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

// Key and value tiles in LDS: 64 rows of 256 bytes, unpadded; the 16-byte
// slot c of row r holds the row's chunk c ^ rsw(r % 16), with the bits of
// rsw(r) = (r2, r0, r1, r2 ^ r3) for the bits r0 .. r3 of r.  Written by
// direct global-to-LDS loads (lane l of a load instruction fills bytes
// 16 l .. of its 1 KiB run).  The LDS serves 128 bytes a clock from 32
// four-byte banks: a 16-byte read in 8-lane groups (here 8 rows, one chunk
// each), an 8-byte read in 16-lane groups (here 4 rows, 32 bytes each).  The
// first needs rsw % 8 one-to-one on each run of 8 rows, the second
// rsw / 2 % 4 one-to-one on each aligned run of 4; rsw gives both, and also
// stays conflict-free for 64 banks and twice the group sizes (rsw one-to-one
// on all 16 rows, rsw / 2 on each run of 8).  The bank-conflict counter
// reads zero.
constexpr int kRowBytes = D * 2;
constexpr int kTileBytes = kKTile * kRowBytes;  // 16 KiB

// A key row of zeros: the V rows past the end of a key range are loaded from it.
__device__ __attribute__((aligned(256))) uint32_t g_zero_row[kRowBytes / 4];

__device__ __forceinline__ int rsw(int r) { return ((r >> 2) & 1) | ((r & 3) << 1) | ((((r >> 2) ^ (r >> 3)) & 1) << 3); }

// (a, b) as packed bf16 hi = bf16(x) and lo = bf16(x - hi); x - hi is exact
// in float32 and comes from one dot2 each: hi . (-1, 0) + a, hi . (0, -1) + b.
// The masks (-1, 0) and (0, -1) are passed in registers: as an operand
// constant the compiler encodes 0x0000bf80 as the inline constant -1.0, which
// this instruction reads as the float32 pattern 0xbf800000, i.e. (0, -1).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 split2_dot(float a, float b, uint32_t m_lo, uint32_t m_hi) {
  const uint32_t hi = cvt2bf(a, b);
  const bf16x2_t h = __builtin_bit_cast(bf16x2_t, hi);
  const float la = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2_t, m_lo), a, false);
  const float lb = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2_t, m_hi), b, false);
  return (u32x2){hi, cvt2bf(la, lb)};
}

__global__ __launch_bounds__(256, 2) void k_attn_d128(AttnArgs a) {
  // [2] K tiles and [2] V tiles
  __shared__ __attribute__((aligned(1024))) unsigned char lds[4 * kTileBytes];
  unsigned char* Kbuf = lds;
  unsigned char* Vbuf = lds + 2 * kTileBytes;

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
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;  // w: wave-uniform
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

  // Direct loads of step s's K or V tile into `dst`: instruction i of wave w
  // fills LDS chunks 256 i + 64 w + lane, i.e. row 16 i + 4 w + lane / 16,
  // slot lane % 16, which receives the row's chunk slot ^ rsw(row % 16).  The
  // lane's byte offset within a 16-row block is the same for every i, so a
  // full tile needs one address per instruction, uniform over the wave.  In
  // a range's last, partial tile the K rows past its end read the range's
  // last key (so the scores there repeat one of the range) and the V rows
  // past its end read a row of zeros (so those slots add nothing to O).
  const int lrow = 4 * w + (l >> 4);
  const unsigned loff = lrow * kRowBytes + (((l & 15) ^ rsw(lrow)) << 4);
  auto load_tile = [&](const uint16_t* src, unsigned char* dst, int s, bool is_v) {
    int base, end;
    step_base(s, base, end);
    const unsigned char* tile = reinterpret_cast<const unsigned char*>(src + (hbase + base) * D);
    if (end - base >= kKTile) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds(tile + i * 16 * kRowBytes + loff,
                                         (__attribute__((address_space(3))) void*)(dst + (256 * i + 64 * w) * 16), 16, 0, 0);
    } else {
      const int nvalid = end - base;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * i + lrow;
        const unsigned char* gp = row < nvalid ? tile + row * kRowBytes
                                  : is_v     ? reinterpret_cast<const unsigned char*>(g_zero_row)
                                             : tile + (nvalid - 1) * kRowBytes;
        __builtin_amdgcn_global_load_lds(gp + (loff & (kRowBytes - 1)),
                                         (__attribute__((address_space(3))) void*)(dst + (256 * i + 64 * w) * 16), 16, 0, 0);
      }
    }
  };

  // LDS read addresses.  K operand of key block kk, dim block kb: row 16 kk + n,
  // chunk 4 kb + g, in slot (4 kb + g) ^ rsw(n) = (4 kb) ^ (g ^ rsw(n)): the kb part
  // flips bits 6-7 of the byte address, the kk part adds whole rows.
  const int kaddr = n * kRowBytes + ((g ^ rsw(n)) << 4);
  // V^T operand of d block db: the addressing lane 4 e1 + jj (e1 = n / 4,
  // jj = n % 4) names key 4g + e1 (+16 for the second read, +32 ks for the
  // key step) and columns 16 db + 4 jj .. +3, which are bytes 8 (jj % 2) ..
  // of chunk 2 db + jj / 2 in slot (2 db) ^ (jj / 2 ^ rsw(row % 16)): the db part
  // flips bits 5-7, the key offsets add whole rows.
  const int vrow = 4 * g + (n >> 2);
  const int vaddr = vrow * kRowBytes + ((((n >> 1) & 1) ^ rsw(vrow)) << 4) + (n & 1) * 8;

  // (-1, 0) and (0, -1) as packed bf16, opaque to constant folding
  uint32_t m_lo = 0x0000bf80u, m_hi = 0xbf800000u;
  asm volatile("" : "+s"(m_lo), "+s"(m_hi));

  f32x4 acc[8][2];  // O^T: d block db, query block qb; lane (n, g): dims 16db + 4g + i of query n
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) acc[db][qb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m[2] = {-__builtin_inff(), -__builtin_inff()};  // running max (log2 domain) of query n, per qb
  float lsum[2] = {0.f, 0.f};                             // this lane's part of the row sum

  // S^T = K Q^T for 64 keys x 32 queries from a K tile in LDS
  auto qk = [&](const unsigned char* Kt, f32x4 (&sc)[4][2]) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) sc[kk][qb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(Kt + (kaddr ^ (kb << 6)) + kk * 16 * kRowBytes);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) sc[kk][qb] = mfma16x16x32(ka, qop[qb][kb], sc[kk][qb]);
      }
  };

  // Row maxima of a step's scores in the log2 domain: c = log2(e) / sqrt(D)
  // is positive, so scaling the raw maximum gives the maximum of the scaled
  // scores.  The slots past a range's end repeat one of its scores and leave
  // the maximum as it is.
  auto rowmax = [&](const f32x4(&x)[4][2], float(&mx)[2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float v = x[0][qb][0];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaxf(v, x[kk][qb][i]);
      mx[qb] = wave_max4(v) * a.scale_log2;
    }
  };

  // Pipeline: step s's scores and their row maxima are computed in step
  // s - 1, so that the softmax (vector ALU) overlaps the next tile's Q K^T
  // and this tile's P V (matrix cores).  Buffers: K tiles of steps s + 1
  // (read) and s + 2 (loading), V tiles of steps s (read) and s + 1
  // (loading); every overwrite waits for the barrier that ended the last
  // reads of that buffer.
  load_tile(a.k, Kbuf, 0, false);
  if (nsteps > 1) load_tile(a.k, Kbuf + kTileBytes, 1, false);
  load_tile(a.v, Vbuf, 0, true);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads have landed
  __syncthreads();
  f32x4 sc[4][2];
  float mx[2];
  qk(Kbuf, sc);
  rowmax(sc, mx);
  __syncthreads();  // every wave's reads of K buffer 0 are done before step 0 refills it

  for (int s = 0; s < nsteps; ++s) {
    const int cur = s & 1;
    if (s + 2 < nsteps) load_tile(a.k, Kbuf + cur * kTileBytes, s + 2, false);
    if (s + 1 < nsteps) load_tile(a.v, Vbuf + (cur ^ 1) * kTileBytes, s + 1, true);
    int base, end;
    step_base(s, base, end);

    // Online softmax of step s into weights p = 2^(x c - m); lane (n, g)
    // holds keys base + 16 kk + 4g + i of query n.  The running maximum m is
    // raised only when a row's new maximum exceeds it by more than 8 (then
    // for every row of the wave, each to its exact maximum): the weights stay
    // below 2^8, and O and the row sums need no rescale in the other steps.
    // The result is the same softmax.
    if (__builtin_amdgcn_ballot_w64(mx[0] > m[0] + 8.f || mx[1] > m[1] + 8.f)) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float mn = fmaxf(m[qb], mx[qb]);
        const float alpha = __builtin_amdgcn_exp2f(m[qb] - mn);
        m[qb] = mn;
        lsum[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db) acc[db][qb] *= alpha;
      }
    }
    float p[4][2][4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[kk][qb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kk][qb][i], a.scale_log2, -m[qb]));
    // slot (3, 3): past the end whenever any slot of this lane is
    const float pdup[2] = {p[3][0][3], p[3][1][3]};
    // the next step's scores, on the matrix cores while the exponentials run
    // (in the last step from a stale buffer, and never used)
    qk(Kbuf + (cur ^ 1) * kTileBytes, sc);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float sum = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) sum += p[kk][qb][i];
      lsum[qb] += sum;
    }

    // O^T += V^T P^T over two 32-key steps, P as bf16 hi + lo
    const unsigned char* Vt = Vbuf + cur * kTileBytes;
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
          const u32x2 sp = split2_dot(p[kk][qb][i0], p[kk][qb][i0 + 1], m_lo, m_hi);
          h[e2] = sp.x;
          lo[e2] = sp.y;
        }
        phi[qb] = h;
        plo[qb] = lo;
      }
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        // lane (i, g) of the A operand: V[key(g, e)][16 db + i]
        const unsigned char* vp = Vt + (vaddr ^ (db << 5)) + 32 * ks * kRowBytes;
        const u32x2 v0 = lds_read_tr16(reinterpret_cast<const uint16_t*>(vp));
        const u32x2 v1 = lds_read_tr16(reinterpret_cast<const uint16_t*>(vp + 16 * kRowBytes));
        const u32x4 vt = {v0.x, v0.y, v1.x, v1.y};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          acc[db][qb] = mfma16x16x32(vt, phi[qb], acc[db][qb]);
          acc[db][qb] = mfma16x16x32(vt, plo[qb], acc[db][qb]);
        }
      }
    }

    rowmax(sc, mx);  // of the next step's scores
    // The slots past the range's end carry one weight each, that of the
    // range's last key (the same score); their V rows are zero, so only the
    // row sums counted them.
    if (end - base < kKTile) {
      int past = 0;  // this lane's slots past the end: keys 16 kk + 4g + i >= end - base
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) past += 4 - min(max(end - base - 16 * kk - 4 * g, 0), 4);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) lsum[qb] -= (float)past * pdup[qb];
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads for the next steps have landed
    __syncthreads();               // and everyone's; the buffers read in this step are free
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
