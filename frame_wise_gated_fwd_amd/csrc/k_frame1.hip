// The forward of a single frame (T = 1; bf16 inputs, head dim 128), for
// frame-by-frame (chunk-causal) generation, where every call carries one
// latent frame (bilibili cv49203711, second key point; the zhichai.net page's
// Stage 4 rollout at constant memory).
//
// One step of the recurrence (zhichai.net, section 1: decay gate gamma,
// delta-rule correction beta),
//   M' = gamma (M - beta M G) + beta U,   G = K^T K,  U = V^T K,
// equals, with G and U written out as sums over the frame's tokens,
//   M' = gamma M + beta sum_s (v_s - gamma M k_s) k_s^T:
// every token adds the residual of its value against the decayed state's
// prediction (the delta rule) times its key.  Rows of M' then depend only on
// the same rows of M: row block r of M' needs M's rows in r, the values'
// columns in r and all keys.  Output columns in row block r need only the
// same rows of M': O[:, r] = Q M'_r^T.  So the step spreads over row blocks
// of 16 rows, 8 per head, with no reduction between row blocks.
//
// Token halves.  With at most 16 heads (8 x 16 row blocks: half the CUs) a
// row block is split over a pair of workgroups: half p takes the 64-token
// tiles t with t % 2 == p, sums its part P_p of P, and the two swap their
// parts, so that each has P = P_0 + P_1 and writes the output columns of its
// own tiles.  With more heads, or with no room for the swap in the workspace,
// one workgroup sums all the tiles and writes all of its columns.  The two
// forms add the tokens' products in different orders, so they agree to
// float32 rounding, not bit for bit; each is deterministic.
//
// The swap.  Head h's workgroups have ids h % 8 + 8 j, which the dispatcher
// deals to XCD h % 8 (the library uses this form only on a device where a
// probe has seen that dealing), so the two halves of a pair, 8 ids apart,
// share that XCD's L2, the point where its CUs' stores meet.  Per pair there
// is one 64-bit word and each half's partial sums.  A half stores its sums
// and waits for all of its memory operations (its reads of state_in included)
// before it touches the word; the workgroup that finds its partner already
// there is the second: it invalidates its L1, reads the partner's sums and
// alone writes the pair's rows of state_out (both halves have read state_in
// by then, so state_out may equal state_in).  The other is the first: it
// polls the word, a bounded number of times, until the second has been there,
// then reads the second's sums.  An eager call carries a new epoch from the
// host: each half exchanges the word for (epoch, half, XCD id) in one atomic
// operation, and a word of an earlier call never passes for this call's
// partner.  A captured graph replays its arguments, epoch included, so a
// captured call flips a tagged toggle with a compare-and-swap instead (idle
// to waiting, waiting to idle; a load and an atomic operation more on the
// second's path): each arrival flips it once, every call leaves it idle, and
// an untagged word (an eager call's, or fresh memory) reads as idle.  The
// halves wait only for each other and an XCD starts its workgroups in id
// order, so at most the last few pairs started on an XCD can be waiting on a
// partner while the others finish and make room.  A first half that still
// gives up (about a second by default) writes NaN to its output columns; the
// second, when it comes, writes the correct state.
//
// Arithmetic, per workgroup: for a tile, C = M_r K^T (M's 16 rows as a bf16
// hi/lo pair, about 2^-17 relative; the keys exact in bf16), the residuals
// R = V_r - (gamma ks) C in float32 (one rounding), then P_w += R^T K with R
// as a bf16 hi/lo pair, on 16x16x32 bf16 MFMA with float32 sums;
// M'_r = gamma M_r + (beta ks) P; then, over the tiles again,
// O[:, r] = Q M'_r^T with M'_r as a bf16 hi/lo pair.  The tokens are summed
// in another order than by the frame-parallel kernels, so results agree with
// theirs to rounding, not bit for bit; they are deterministic.
//
// Placement.  Head h's workgroups have ids h % 8 + 8 j, which the dispatcher
// deals to one XCD, so one fetch of the keys and queries from HBM serves all
// of them through that XCD's L2.  A workgroup takes a whole CU (160 KB of
// LDS).  Global loads are contiguous (a wave's 16-byte loads cover whole
// rows) and the MFMA operands are read from LDS: loading a 16-row operand
// layout straight from memory (each load instruction 16 rows x 64 bytes)
// moves a workgroup's 128 KB at about a third of the rate of contiguous
// loads.
//
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int D = 128;
constexpr int kXcd = 8;
constexpr int kTile = 64;        // tokens per MFMA tile
constexpr int kRowWgs = 8;       // row blocks per head, 16 rows of M' each
constexpr int kRowWaves = 8;     // waves per row workgroup

// Row blocks are split over two workgroups for at most this many heads
// (16 heads: 256 workgroups, one per CU).
constexpr int64_t kSplitMaxHeads = 16;
constexpr int64_t kPairWordBytes = 128;                 // one pair word per 128-byte line
constexpr int64_t kHalfSumBytes = kRowWaves * 64 * 16;  // a half's partial sums: 8 KB
constexpr int kPairSleep = 2;                            // s_sleep between polls (~128 clocks)
constexpr uint64_t kPairMagic = 0x9d3a61;               // tag of a pair word in use
constexpr uint32_t kPairSpinLimit = 1u << 20;            // default polls (about a second)

struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* gamma;
  const float* beta;
  const float* state_in;  // null: zero state
  void* out;
  float* state_out;
  int64_t heads;
  int S;
  float ks;
  uint64_t* words;  // pair words, kPairWordBytes apart; null: one workgroup per row block
  f32x4* sums;      // [pair][half][wave][lane] partial sums
  uint32_t epoch;   // eager calls: nonzero, new for every call; 0 under stream capture
  uint32_t spin_limit;
};

// This wave's LDS writes are done before its later LDS reads (the tiles a
// wave writes are read only by its own lanes).
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ uint32_t xcc_id() {
  // HW_REG_XCC_ID, bits [3:0]
  return __builtin_amdgcn_s_getreg((15 << 11) | (0 << 6) | 20) & 0xfu;
}

// A key tile in LDS: 64 token rows x 256 bytes.  Row s keeps its sixteen
// 16-byte chunks in the order c ^ swz(s): for 8 consecutive rows swz is a
// permutation of 0..7 (16-byte writes of one chunk from 8 rows hit 8
// distinct 4-bank groups), and for rows 4a .. 4a+3 it is 0, 2, 4, 6 or
// 1, 3, 5, 7, so the transposed 8-byte reads of a chunk pair from 4 rows
// cover all 32 banks once.
__device__ __forceinline__ int swz(int s) { return ((s & 3) << 1) | ((s >> 2) & 1); }
__device__ __forceinline__ int tile_off(int s, int c) { return s * 256 + ((c ^ swz(s)) << 4); }

// Rows of float32 M (row length 512 bytes) into LDS as bf16 hi and lo
// planes in the tile layout above (row stride 256 bytes per plane): float4
// q of row r (q = 0..31) goes to the 8-byte half q % 2 of chunk q / 2.
__device__ __forceinline__ void stage_m4(char* planes, int plane_bytes, int r, int q, f32x4 x) {
  const u32x2 p0 = split2(x[0], x[1]), p1 = split2(x[2], x[3]);
  const int off = tile_off(r, q >> 1) + 8 * (q & 1);
  *reinterpret_cast<u32x2*>(planes + off) = (u32x2){p0.x, p1.x};
  *reinterpret_cast<u32x2*>(planes + plane_bytes + off) = (u32x2){p0.y, p1.y};
}

// LDS of a row workgroup: per wave a key tile (16 KB) and its residuals as
// [token][16 rows] bf16, hi and lo planes (4 KB); after a token loop the
// same bytes hold the waves' sums for the reduction (8 KB per wave), the
// pair's hand-off words (past the reduction) and M' for the output.
constexpr int kWaveLds = kTile * 256 + 2 * kTile * 32;
constexpr int kRowLds = kRowWaves * kWaveLds;
constexpr int kRedBytes = kRowWaves * 8 * 64 * 16;
constexpr int kBcastOff = kRedBytes + 32 * 1024;  // clear of the reduction and of M' (at kRedBytes)
static_assert(kRowLds <= 160 * 1024, "a row workgroup's LDS fits a CU");
static_assert(kRowLds >= kRedBytes + 32 * 1024 + 16, "the reduction, M' and the hand-off reuse the tiles' LDS");

// ---------------------------------------------------------------------------
// rows [16rb, 16rb + 16) of head h and the output columns of the same index,
// over one or both token halves
// ---------------------------------------------------------------------------
template <bool kOutBf16>
__global__ __launch_bounds__(64 * kRowWaves, 1) void k_frame1(Args a) {
  __shared__ __attribute__((aligned(16))) char lds[kRowLds];
  // ids h % 8 + 8 j: head h's workgroups on one XCD when the dispatcher
  // deals ids to the 8 XCDs in turn; the two halves of a pair 8 ids apart
  const bool split = a.words != nullptr;
  const int per_head = split ? 2 * kRowWgs : kRowWgs;
  const int xs = blockIdx.x % kXcd, local = blockIdx.x / kXcd;
  const int64_t hl = xs + (int64_t)kXcd * (local / per_head);
  const int within = local % per_head;
  const int rb = split ? within >> 1 : within;
  const int half = split ? within & 1 : 0;
  if (hl >= a.heads) return;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, n = l & 15, g = l >> 4;
  const int S = a.S, r0 = 16 * rb;
  const int ntiles = (S + kTile - 1) / kTile;
  const uint16_t* Kh = a.k + hl * S * D;
  const uint16_t* Vh = a.v + hl * S * D;
  const uint16_t* Qh = a.q + hl * S * D;
  const float* Mi = a.state_in ? a.state_in + hl * D * D : nullptr;
  float* Mo = a.state_out + hl * D * D;
  char* Kt = lds + w * kWaveLds;
  char* Rt = Kt + kTile * 256;
  const float gks = a.gamma[hl] * a.ks;

  // this wave's tiles: i = (w + rb) % 8 + 8 j (tile tstep i + toff below), so
  // that the head's row blocks start on different tiles
  const int first = (w + rb) % kRowWaves;

  // a tile's keys, loaded row by row (load i of lane l: token 4i + l / 16,
  // 16-byte chunk l % 16), and this lane's values (token 16tb + n, dims
  // r0 + 4g .. +3).  Tokens past the frame load its last token and are
  // zeroed, so that all loads are issued at once.
  u32x4 kx[16];
  u32x2 vv[4];
  auto load_rows = [&](const uint16_t* X, int tile) {
    const int s0 = tile * kTile, last = S - 1;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      kx[i] = *reinterpret_cast<const u32x4*>(X + (int64_t)min(s0 + 4 * i + (l >> 4), last) * D + 8 * (l & 15));
  };
  auto load_tile = [&](int tile) {
    load_rows(Kh, tile);
    const int s0 = tile * kTile, last = S - 1;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
      vv[tb] = *reinterpret_cast<const u32x2*>(Vh + (int64_t)min(s0 + 16 * tb + n, last) * D + r0 + 4 * g);
  };
  // the tiles of this workgroup: all of them, or every second from `half`
  const int tstep = split ? 2 : 1, toff = split ? half : 0;
  const int nt = split ? (ntiles + 1 - half) >> 1 : ntiles;  // tiles tstep i + toff, i < nt
  if (first < nt) load_tile(tstep * first + toff);

  // M's rows r0 .. r0 + 15 as MFMA A operands (lane (m, g): row r0 + m,
  // columns 32kb + 8g .. +7, bf16 hi/lo), staged once through LDS: one
  // 16-byte load per thread
  u32x4 mh[4], ml[4];
  if (Mi) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(Mi + (r0 + (tid >> 5)) * D + 4 * (tid & 31));
    stage_m4(lds, 16 * 256, tid >> 5, tid & 31, x);
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      mh[kb] = *reinterpret_cast<const u32x4*>(lds + tile_off(n, 4 * kb + g));
      ml[kb] = *reinterpret_cast<const u32x4*>(lds + 16 * 256 + tile_off(n, 4 * kb + g));
    }
    __syncthreads();  // wave 0's tile overwrites the staging area
  }

  f32x4 acc[8];
#pragma unroll
  for (int jb = 0; jb < 8; ++jb) acc[jb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // the transposed reads: lane L = 4e + q of a 16-lane group names row
  // base + e, 4 columns from 4q
  const int tre = (l & 15) >> 2, trq = l & 3;

  for (int i = first; i < nt; i += kRowWaves) {
    const int tile = tstep * i + toff;
    const int cnt = min(kTile, S - tile * kTile);
    // the keys into LDS (rows past the frame as zeros)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 4 * r + (l >> 4);
      *reinterpret_cast<u32x4*>(Kt + tile_off(row, l & 15)) = row < cnt ? kx[r] : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
      if (16 * tb + n >= cnt) vv[tb] = (u32x2){0u, 0u};
    wave_lds_sync();
    // C^T = M_r K^T: lane (n, g) ends with (M k_s)[r0 + 4g + i], s = 16tb + n
    f32x4 c[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) c[tb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    if (Mi) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        // the keys as MFMA B operands: lane (n, g) token 16tb + n, dims 32kb + 8g .. +7
        u32x4 kf[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) kf[tb] = *reinterpret_cast<const u32x4*>(Kt + tile_off(16 * tb + n, 4 * kb + g));
        // the four accumulators in turn, so that no MFMA waits for the one
        // just before it
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) c[tb] = mfma16x16x32(mh[kb], kf[tb], c[tb]);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) c[tb] = mfma16x16x32(ml[kb], kf[tb], c[tb]);
      }
    }
    // residuals, one rounding each, into LDS as [token][row] hi/lo
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const float r0v = __builtin_fmaf(-gks, c[tb][0], bf2f(vv[tb].x & 0xffffu));
      const float r1v = __builtin_fmaf(-gks, c[tb][1], bf2f(vv[tb].x >> 16));
      const float r2v = __builtin_fmaf(-gks, c[tb][2], bf2f(vv[tb].y & 0xffffu));
      const float r3v = __builtin_fmaf(-gks, c[tb][3], bf2f(vv[tb].y >> 16));
      const u32x2 p0 = split2(r0v, r1v), p1 = split2(r2v, r3v);
      const int off = (16 * tb + n) * 32 + 8 * g;
      *reinterpret_cast<u32x2*>(Rt + off) = (u32x2){p0.x, p1.x};
      *reinterpret_cast<u32x2*>(Rt + kTile * 32 + off) = (u32x2){p0.y, p1.y};
    }
    // the next tile's loads are in flight during this tile's products
    if (i + kRowWaves < nt) load_tile(tstep * (i + kRowWaves) + toff);
    wave_lds_sync();
    // P_w += R^T K over the tile's tokens
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int row0 = 32 * kb + 8 * g + tre;
      u32x4 ra[2];
#pragma unroll
      for (int pl = 0; pl < 2; ++pl) {
        const u32x2 x0 = lds_read_tr16(reinterpret_cast<const uint16_t*>(Rt + pl * kTile * 32 + row0 * 32 + 8 * trq));
        const u32x2 x1 =
            lds_read_tr16(reinterpret_cast<const uint16_t*>(Rt + pl * kTile * 32 + (row0 + 4) * 32 + 8 * trq));
        ra[pl] = (u32x4){x0.x, x0.y, x1.x, x1.y};
      }
      u32x4 kt[8];
#pragma unroll
      for (int jb = 0; jb < 8; ++jb) {
        const int ch = 2 * jb + (trq >> 1), hf = 8 * (trq & 1);
        const u32x2 x0 = lds_read_tr16(reinterpret_cast<const uint16_t*>(Kt + tile_off(row0, ch) + hf));
        const u32x2 x1 = lds_read_tr16(reinterpret_cast<const uint16_t*>(Kt + tile_off(row0 + 4, ch) + hf));
        kt[jb] = (u32x4){x0.x, x0.y, x1.x, x1.y};
      }
      // all hi products, then all lo products: consecutive MFMAs update
      // different accumulators
#pragma unroll
      for (int jb = 0; jb < 8; ++jb) acc[jb] = mfma16x16x32(ra[0], kt[jb], acc[jb]);
#pragma unroll
      for (int jb = 0; jb < 8; ++jb) acc[jb] = mfma16x16x32(ra[1], kt[jb], acc[jb]);
    }
    wave_lds_sync();  // this tile's LDS reads are done before the next tile's writes
  }

  // the queries of this wave's first output tile: in flight during the
  // reduction (when split, during the swap below)
  if (!split && first < nt) load_rows(Qh, tstep * first + toff);

  // M's elements this lane updates: rows r0 + 4g + i, column 16 w + n
  // (wave w finishes column block w).  Only the workgroups of this row
  // block read or write M's rows r0 .. r0 + 15.
  float m_old[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) m_old[i] = Mi ? Mi[(r0 + 4 * g + i) * D + 16 * w + n] : 0.f;
  // the waves' sums, added in the order w = 0..7: lane (n, g) holds
  // P[r0 + 4g + i][16jb + n] in acc[jb]
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(lds);  // 64 KB
#pragma unroll
  for (int jb = 0; jb < 8; ++jb) red[(w * 8 + jb) * 64 + l] = acc[jb];
  __syncthreads();
  f32x4 sum = red[w * 64 + l];
#pragma unroll
  for (int v = 1; v < kRowWaves; ++v) sum += red[(v * 8 + w) * 64 + l];

  bool writer = true;
  if (split) {
    // the swap: this half's sums out, the word exchanged, the partner's in
    const int64_t pair = hl * kRowWgs + rb;
    a.sums[(pair * 2 + half) * (kRowWaves * 64) + w * 64 + l] = sum;
    // every earlier memory operation of this workgroup is done (its sums
    // are in the L2, its reads of state_in are over) before the exchange;
    // the queries of its first output tile, issued after them, stay in
    // flight (vector memory operations retire in issue order, and a query
    // tile is 16 loads)
    asm volatile("" ::: "memory");
    if (first < nt) {
      load_rows(Qh, tstep * first + toff);
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    uint32_t* bc = reinterpret_cast<uint32_t*>(lds + kBcastOff);
    if (tid == 0) {
      uint64_t* word = a.words + pair * (kPairWordBytes / 8);
      const uint64_t xcc = xcc_id();
      bool second, ok;
      uint64_t seen, from;  // the partner's value, and its XCD id
      if (a.epoch != 0) {
        // eager calls: one exchange.  The word: this call's epoch in bits
        // 0-31, the half in bit 32, the XCD id in bits 40-47.
        const uint64_t mine = (uint64_t)a.epoch | ((uint64_t)half << 32);
        const uint64_t want = (uint64_t)a.epoch | ((uint64_t)(1 - half) << 32);
        auto partner = [&](uint64_t x) { return (x & 0x1ffffffffull) == want && (x >> 40) < 256; };
        seen = __hip_atomic_exchange(word, mine | (xcc << 40), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        second = partner(seen);
        ok = second;
        for (uint32_t i = 0; !ok && i < a.spin_limit; ++i) {
          __builtin_amdgcn_s_sleep(kPairSleep);
          seen = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = partner(seen);
        }
        from = seen >> 40;
      } else {
        // captured calls (a graph replays its arguments, so no epoch): a
        // toggle.  The word: kPairMagic in bits 40-63 (anything else, an
        // epoch word or fresh memory, reads as idle), the XCD id of the
        // last workgroup to arrive in bits 32-39, bit 0 set while the first
        // of the pair waits.  Each arrival flips it once, so every call
        // leaves it idle.
        seen = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (;;) {
          second = (seen >> 40) == kPairMagic && (seen & 1u);
          const uint64_t next = (kPairMagic << 40) | (xcc << 32) | (second ? 0u : 1u);
          if (__hip_atomic_compare_exchange_strong(word, &seen, next, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT))
            break;
        }
        ok = second;
        for (uint32_t i = 0; !ok && i < a.spin_limit; ++i) {
          __builtin_amdgcn_s_sleep(kPairSleep);
          seen = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = !(seen & 1u);
        }
        from = (seen >> 32) & 0xffu;
      }
      bc[0] = second;
      bc[1] = ok && from == xcc;  // the partner's sums are in this XCD's L2
    }
    __syncthreads();
    writer = bc[0] != 0;
    if (bc[1] != 0) {
      asm volatile("buffer_inv sc0" ::: "memory");  // no stale line of the partner's sums in L1
      // P = P_0 + P_1: float addition is commutative, so both halves get
      // the same bits
      sum += a.sums[(pair * 2 + (1 - half)) * (kRowWaves * 64) + w * 64 + l];
    } else {
      // no partner in time (or, on a device that does not deal pairs to
      // one XCD, none whose sums this L2 holds): NaN, in this workgroup's
      // output columns and, when it is the second, in the pair's state rows
      sum = (f32x4){__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    }
  }

  // M'_r to state_out (by one workgroup of the row block, after every read
  // of state_in in it), and into LDS as bf16 hi/lo (after the reduction
  // buffer) for the output's A operands
  const float gam = a.gamma[hl], bks = a.beta[hl] * a.ks;
  char* Ms = lds + kRedBytes;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float mn = __builtin_fmaf(bks, sum[i], gam * m_old[i]);
    if (writer) Mo[(r0 + 4 * g + i) * D + 16 * w + n] = mn;
    const uint32_t hi = f2bf(mn), lo = f2bf(mn - bf2f(hi));
    const int off = tile_off(4 * g + i, 2 * w + (n >> 3)) + 2 * (n & 7);
    *reinterpret_cast<uint16_t*>(Ms + off) = (uint16_t)hi;
    *reinterpret_cast<uint16_t*>(Ms + 16 * 256 + off) = (uint16_t)lo;
  }
  __syncthreads();
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    mh[kb] = *reinterpret_cast<const u32x4*>(Ms + tile_off(n, 4 * kb + g));
    ml[kb] = *reinterpret_cast<const u32x4*>(Ms + 16 * 256 + tile_off(n, 4 * kb + g));
  }
  __syncthreads();  // the tiles below reuse the reduction buffer and the staging

  // O[:, r0 .. r0 + 15] = Q M'_r^T over this wave's output tiles: lane
  // (n, g) ends with O[s][r0 + 4g + i], s = 16tb + n
  constexpr int kOutB = kOutBf16 ? 2 : 4;
  char* Oh = static_cast<char*>(a.out) + hl * S * D * kOutB;
  for (int i = first; i < nt; i += kRowWaves) {
    const int s0 = (tstep * i + toff) * kTile;
#pragma unroll
    for (int r = 0; r < 16; ++r) *reinterpret_cast<u32x4*>(Kt + tile_off(4 * r + (l >> 4), l & 15)) = kx[r];
    wave_lds_sync();
    // the next tile's queries are in flight during this tile's products
    if (i + kRowWaves < nt) load_rows(Qh, tstep * (i + kRowWaves) + toff);
    f32x4 o[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) o[tb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      // B operands: lane (n, g) token 16tb + n, dims 32kb + 8g .. +7
      u32x4 qf[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) qf[tb] = *reinterpret_cast<const u32x4*>(Kt + tile_off(16 * tb + n, 4 * kb + g));
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) o[tb] = mfma16x16x32(mh[kb], qf[tb], o[tb]);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) o[tb] = mfma16x16x32(ml[kb], qf[tb], o[tb]);
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int s = s0 + 16 * tb + n;
      if (s >= S) continue;
      const int64_t e = (int64_t)s * D + r0 + 4 * g;
      if constexpr (kOutBf16)
        st_nt(reinterpret_cast<u32x2*>(Oh + e * 2), (u32x2){cvt2bf(o[tb][0], o[tb][1]), cvt2bf(o[tb][2], o[tb][3])});
      else
        st_nt(reinterpret_cast<f32x4*>(Oh + e * 4), o[tb]);
    }
    wave_lds_sync();  // this tile's LDS reads are done before the next tile's writes
  }
}

int64_t pair_words_bytes(int64_t heads) { return (heads * kRowWgs * kPairWordBytes + 255) & ~int64_t{255}; }

// XCC_ID seen by each workgroup of the largest split launch (the probe).
constexpr int kProbeWgs = 2 * kSplitMaxHeads * kRowWgs;
__device__ uint32_t g_pair_xcc[kProbeWgs];
__global__ void k_pair_probe() {
  if (threadIdx.x == 0) g_pair_xcc[blockIdx.x] = xcc_id();
}

}  // namespace

// Whether workgroups b and b + 8 of a launch run on one XCD (ids dealt to
// the 8 XCDs in turn), as the split form's swap needs: a probe launch of the
// split form's largest size records each workgroup's XCC_ID.  Runs on the
// null stream and waits for it.
hipError_t frame1_pairs_share_xcd(bool* ok) {
  *ok = false;
  hipLaunchKernelGGL(k_pair_probe, dim3(kProbeWgs), dim3(64 * kRowWaves), 0, nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  uint32_t seen[kProbeWgs];
  if ((e = hipMemcpyFromSymbol(seen, HIP_SYMBOL(g_pair_xcc), sizeof seen)) != hipSuccess) return e;
  bool same = true;
  for (int b = 0; b < kProbeWgs; ++b) same = same && seen[b] < (uint32_t)kXcd && seen[b] == seen[b % kXcd];
  *ok = same;
  return hipSuccess;
}

int64_t frame1_workspace_bytes(int64_t heads) {
  if (heads <= 0 || heads > kSplitMaxHeads) return 0;
  return pair_words_bytes(heads) + heads * kRowWgs * 2 * kHalfSumBytes;
}

hipError_t launch_frame1(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* gamma,
                         const float* beta, const float* state_in, void* out, bool out_bf16, float* state_out,
                         int64_t heads, int S, float ks, void* pair_ws, uint32_t epoch, uint32_t spin_limit,
                         hipStream_t st) {
  Args a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.gamma = gamma;
  a.beta = beta;
  a.state_in = state_in;
  a.out = out;
  a.state_out = state_out;
  a.heads = heads;
  a.S = S;
  a.ks = ks;
  const bool split = pair_ws && frame1_workspace_bytes(heads) > 0;
  a.words = split ? static_cast<uint64_t*>(pair_ws) : nullptr;
  a.sums = split ? reinterpret_cast<f32x4*>(static_cast<char*>(pair_ws) + pair_words_bytes(heads)) : nullptr;
  a.epoch = epoch;
  a.spin_limit = spin_limit ? spin_limit : kPairSpinLimit;
  const int64_t grid = (heads + kXcd - 1) / kXcd * kXcd * kRowWgs * (split ? 2 : 1);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (out_bf16)
    hipLaunchKernelGGL(k_frame1<true>, dim3((unsigned)grid), dim3(64 * kRowWaves), 0, st, a);
  else
    hipLaunchKernelGGL(k_frame1<false>, dim3((unsigned)grid), dim3(64 * kRowWaves), 0, st, a);
  return hipGetLastError();
}

}  // namespace gdn
