/*
 * gdn_attn.h -- C ABI of the softmax attention block of the chunk-causal
 * variant, with attention sinks and a local temporal window, on AMD Instinct
 * MI355X (gfx950).  Part of libgdn; status codes and gdn_shape are those of
 * gdn.h.
 *
 * What is computed.  The SANA-WM pages ("SANA-WM: NVIDIA puts a one-minute
 * world model on a single GPU", zhichai.net) interleave 5 softmax attention
 * blocks with the 15 frame-wise Gated DeltaNet blocks of the model (section
 * "1. Hybrid Linear Attention -- Gated DeltaNet + Softmax"), and give the
 * chunk-causal autoregressive variant's softmax layers attention-sink tokens
 * and local temporal windows so that memory stays constant over a long
 * rollout (training pipeline, Stage 4).  The pages state no sizes; the
 * layout below makes each one a parameter.  Per batch b and head h, the
 * T latent frames of S tokens are grouped into generation chunks: chunk 0 is
 * the first `first_chunk` frames, every later chunk `chunk` frames (the last
 * one may be shorter).  A query token in chunk c attends to
 *   - every token of chunks c - window + 1 .. c (the local window:
 *     bidirectional inside chunk c, causal across chunks), and
 *   - every token of the first `sink` frames that lie in chunks 0 .. c (the
 *     attention sinks; a sink is never in a query's future),
 * and to nothing else:
 *     O[q]   = sum_j softmax_j(q . k_j / sqrt(D)) v_j
 *     lse[q] = ln sum_j exp(q . k_j / sqrt(D))
 * over those keys j.
 *
 * Layout.  q, k, v: [B, H, T, S, D] bf16 (the GDN block's layout); out:
 * [B, H, T, S, D] float32; lse: [B, H, T, S] float32.  Row-major, innermost
 * index last.  Device pointers owned by the caller; no workspace.
 */
#ifndef GDN_ATTN_H_
#define GDN_ATTN_H_

#include "gdn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int64_t sink;         /* leading frames that act as attention sinks (>= 0)  */
  int64_t first_chunk;  /* frames of chunk 0 (>= 1)                           */
  int64_t chunk;        /* frames of every later chunk (>= 1)                 */
  int64_t window;       /* chunks in a query's window, its own included (>= 1) */
} gdn_attn_layout;

/*
 * The attention block above for in_dtype GDN_BF16 and D == 128 (otherwise
 * GDN_E_DTYPE or GDN_E_UNSUPPORTED_D).  lse may be NULL.  Asynchronous on
 * `stream` (a hipStream_t; NULL: the null stream); one kernel launch.
 * Argument errors return before any launch, writing nothing:
 * GDN_E_NULLPTR (shape, layout, q, k, v or out NULL), GDN_E_SHAPE (a
 * negative size, or T * S >= 2^30 tokens per head), GDN_E_VALUE (a layout
 * field out of its range), GDN_E_ALIAS (out or lse overlapping q, k, v or
 * each other).  B, H, T or S of 0: nothing to do, GDN_OK.  The softmax
 * weights enter the value product as a bf16 hi/lo pair, so out keeps float32
 * accuracy; the exponentials are the device's exp2.
 */
int gdn_attn_fwd(const gdn_shape* shape, int in_dtype, const gdn_attn_layout* layout,
                 const void* q, const void* k, const void* v, float* out, float* lse,
                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_ATTN_H_ */
