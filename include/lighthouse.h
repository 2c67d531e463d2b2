/*
 * lighthouse.h — C ABI of the Lighthouse attention layer for AMD Instinct
 * MI355X (gfx950).
 *
 * The layer wraps causal scaled-dot-product attention in a selection
 * pipeline (gist.science technical summary of the Lighthouse paper, §2 parts
 * A–C; bitsgeniais.com.br post, phases 1–4):
 *   pyramid -> score -> joint top-K -> causal gather -> subsequence attention
 *   -> scatter back to tokens, plus the backward through scatter, attention
 *   and gather/pooling.
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 *  - Tensors are caller-owned DEVICE memory, row-major with the head
 *    dimension fastest, contiguous unless lh_shape gives strides for the
 *    token tensors (see lh_shape).  The library never allocates device
 *    memory: scratch space comes from the `ws` argument, sized by
 *    lh_query_sizes().
 *  - Element type of q/k/v-like tensors is shape->dtype (LH_FP32: float,
 *    LH_BF16: bfloat16 bit patterns, 2 bytes).  Scores, lse and the
 *    subsequence gradients are float32; index tensors are int32.
 *  - Per (batch b, head h) with notation N_l = N / p^l:
 *      M        = sum_{l<L} N_l          entries of all levels
 *      n_coarse = N_{L-1}                entries of the coarsest level
 *      C        = M - n_coarse           top-K candidates (levels 0..L-2)
 *      K        = S - n_coarse           candidates selected
 *    Flat entry index: flat(l, j) = sum_{m<l} N_m + j (level-major); flat
 *    indices < N are tokens.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on that stream and returns without synchronising; outputs
 *    are ready when the stream reaches that point.  (lh_backward may also
 *    run part of its work on a side stream of the library, which that stream
 *    waits for within the call; see lh_backward.)
 *  - Inputs and outputs of one call must not overlap.
 *  - Errors: shapes and pointers are checked on the host before anything is
 *    launched.  A failed check returns LH_EINVAL / LH_EUNSUPPORTED /
 *    LH_EWORKSPACE and enqueues nothing; a launch failure returns LH_EHIP.
 *    lh_last_error() gives a message for the calling thread.
 *  - Determinism: identical inputs give bit-identical outputs (no floating
 *    point atomics anywhere).
 *  - Inputs are expected to be finite.  A NaN or infinity in q or k gives a
 *    non-finite score, which the top-K ranks by its bit pattern (as a value
 *    above every finite score); outputs touched by it are not meaningful.
 *  - Shape limits: 2 <= p <= 64, 1 <= L <= 16, N % p^(L-1) == 0,
 *    n_coarse <= S <= M, d in {64, 128}, B*H*M < 2^31, M*d < 2^31 (so one head's
 *    S*d*2 bytes stay below 2^32), B*H <= 65535 (p > 64 returns
 *    LH_EUNSUPPORTED: the pooling kernels stage a workgroup's positions in
 *    LDS sized for spans of at most 64 rows per pass).
 */
#ifndef LIGHTHOUSE_H
#define LIGHTHOUSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LH_OK = 0,
  LH_EINVAL = 1,        /* bad shape, null pointer, S out of range        */
  LH_EUNSUPPORTED = 2,  /* valid but not implemented (d, dtype, L > 16)   */
  LH_EWORKSPACE = 3,    /* ws_bytes smaller than lh_query_sizes() asks for */
  LH_EHIP = 4           /* a HIP runtime call or kernel launch failed      */
} lh_status;

typedef enum { LH_FP32 = 0, LH_BF16 = 1 } lh_dtype;

/* Scatter reading (how subsequence outputs go back to tokens, bitsgeniais
 * phase 4; gist.science technical summary §2.C and §3 item 1).
 *  LH_SCATTER_SPAN (0, the default): token t receives the outputs of its
 *    selected ancestors, the entries whose span holds t.  NOT causal: every
 *    token except the last of its coarsest span (1 - p^-(L-1) of all tokens)
 *    reads later tokens, up to p^(L-1) - 1 of them, through its coarsest
 *    ancestor (whose pooled q, k, v include them).  Not a drop-in for causal
 *    attention in language-model training, where it lets a position see the
 *    tokens it is to predict.
 *  LH_SCATTER_CAUSAL (1): entry (l, j) feeds the p^l tokens from its end
 *    token (j+1)*p^l - 1 on, so token t receives, per level, the entry
 *    (t+1)/p^l - 1 (integer division), the last one completed at or before t
 *    (level 0: t itself).  out[t] depends on tokens <= t only.  Tokens that
 *    no selected entry feeds (only possible for t < p^(L-1) - 1) get 0.
 * Both take the mean over the entries that feed the token. */
typedef enum { LH_SCATTER_SPAN = 0, LH_SCATTER_CAUSAL = 1 } lh_scatter_mode;

/* Problem shape.  p = pooling factor, L = number of pyramid levels (level 0 =
 * tokens), S = subsequence length.  L = 1 means S = N and the layer is plain
 * dense causal attention.
 *
 * Token-tensor layouts (optional).  The [B,H,N,d] token tensors may be
 * strided views, as a model's packed projections give them (e.g. q, k, v
 * inside one [B, N, 3, H, d] buffer): element (b, h, n, i) sits at
 * b*s[0] + h*s[1] + n*s[2] + i elements from the tensor's pointer.
 *   qkv_stride: q, k, v (lh_build_pyramid, lh_score, lh_gather, lh_forward)
 *               and the gradients dq, dk, dv (lh_gather_backward,
 *               lh_backward);
 *   out_stride: out (lh_scatter, lh_forward) and dout (lh_scatter_backward,
 *               lh_backward).
 * All three zero = the packed layout s = {H*N*d, N*d, d}.  Otherwise every
 * stride of a dimension longer than 1 is positive and a multiple of 16
 * bytes, and no two rows overlap (LH_EINVAL if not); the stride of a
 * dimension of extent 1 is ignored.  Tensor pointers must be 16-byte aligned.  Every other
 * tensor of the API (pyramid, scores, maps, subsequence tensors) is packed.
 * Zero-initialising the struct keeps the packed layout and the span scatter.
 *
 * scatter: lh_scatter_mode (LH_EINVAL for other values); it changes
 * lh_scatter, lh_scatter_backward and the fused calls, and the scatter
 * backward's workspace size. */
typedef struct {
  int64_t B, H, N, d;
  int32_t p, L;
  int64_t S;
  int32_t dtype; /* lh_dtype */
  int64_t qkv_stride[3];
  int64_t out_stride[3];
  int32_t scatter; /* lh_scatter_mode */
} lh_shape;

/* Derived sizes (per (b,h) counts; byte sizes are for all B*H heads). */
typedef struct {
  int64_t M, C, K, n_coarse;
  size_t bytes_qkv;      /* one [B,H,N,d] tensor                          */
  size_t bytes_pyramid;  /* one pooled tensor [B,H,M-N,d], levels 1..L-1  */
  size_t bytes_score;    /* float32 [B,H,M]                               */
  size_t bytes_sel;      /* int32   [B,H,K]                               */
  size_t bytes_sub_idx;  /* int32   [B,H,S]                               */
  size_t bytes_pos;      /* int32   [B,H,M]                               */
  size_t bytes_sub;      /* one subsequence tensor [B,H,S,d] (dtype)      */
  size_t bytes_sub_f32;  /* one float32 subsequence tensor [B,H,S,d] (os)  */
  size_t bytes_lse;      /* float32 [B,H,S]                               */
  size_t ws_build_pyramid, ws_score, ws_topk, ws_gather, ws_attention_backward,
      ws_scatter_backward, ws_forward, ws_backward;
} lh_sizes;

/* Buffers that lh_forward fills and lh_backward reads.  All caller-owned
 * device memory, sizes as in lh_sizes. */
typedef struct {
  void *pq, *pk, *pv;   /* pyramid levels 1..L-1, [B,H,M-N,d] dtype          */
  float *score;         /* [B,H,M]                                            */
  int32_t *sel;         /* [B,H,K] selected candidates, ascending flat index  */
  int32_t *sub_idx;     /* [B,H,S] flat index at each subsequence position    */
  int32_t *pos;         /* [B,H,M] subsequence position of each entry, or -1  */
  void *qs, *ks, *vs;   /* [B,H,S,d] gathered subsequence (dtype)             */
  float *os;            /* [B,H,S,d] float32 attention output on the subsequence */
  float *lse;           /* [B,H,S] natural-log softmax normaliser per row     */
} lh_buffers;

/* Sizes of every buffer and workspace for a shape.  Host only; no GPU call.
 * A workspace (ws) is caller-owned device memory of at least the stated
 * size, 16-byte aligned (LH_EINVAL otherwise), whose contents need not be
 * initialised and are not kept between calls.
 * Returns LH_EINVAL / LH_EUNSUPPORTED for shapes the library rejects. */
lh_status lh_query_sizes(const lh_shape *shape, lh_sizes *out);

/* Message describing the last failure on the calling thread ("" if none). */
const char *lh_last_error(void);

/* a1. Symmetric average pooling of Q, K and V into levels 1..L-1 (technical
 * summary §2.A; bitsgeniais phase 1): level-l entry j = mean of the p^l tokens
 * j*p^l .. (j+1)*p^l-1, computed hierarchically in float32 and rounded once
 * to dtype.  q,k,v: [B,H,N,d]; pq,pk,pv: [B,H,M-N,d] (row flat(l,j)-N).
 * ws: ws_build_pyramid bytes (float32 partial sums for deep pyramids). */
lh_status lh_build_pyramid(const lh_shape *shape, const void *q, const void *k, const void *v,
                           void *pq, void *pk, void *pv, void *ws, size_t ws_bytes,
                           void *stream);

/* a2. Parameter-free scores (technical summary §2.B; bitsgeniais phase 2):
 * score[flat(0,t)] = ||q_t|| + ||k_t|| in float32 (squares, halving-tree sum
 * y[i] += y[i+w/2] for w = d..2 without fused multiply-add, correctly rounded
 * sqrt); score[flat(l,j)] = max of its p children for l >= 1.
 * q,k: [B,H,N,d]; score: float32 [B,H,M].  ws: ws_score bytes. */
lh_status lh_score(const lh_shape *shape, const void *q, const void *k, float *score,
                   void *ws, size_t ws_bytes, void *stream);

/* a3. Joint top-K over levels 0..L-2 (technical summary §2.B; bitsgeniais
 * phase 2): the K = S - n_coarse candidates first under (score descending,
 * flat index ascending), written in ascending flat order.  The coarsest level
 * is not a candidate (it is always kept whole).  score: [B,H,M];
 * sel: int32 [B,H,K].  ws: ws_topk bytes. */
lh_status lh_topk(const lh_shape *shape, const float *score, int32_t *sel, void *ws,
                  size_t ws_bytes, void *stream);

/* lh_topk for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same selection, written to sel exactly as lh_topk writes it, with the
 * scratch space in a fixed 16 MiB device array of the library instead of a
 * workspace argument.  The array is per device and lives until the process
 * ends; the call allocates nothing and frees nothing.  Shapes whose top-K
 * scratch (lh_sizes.ws_topk) exceeds 16 MiB -- above about 30 heads of 98K
 * tokens or 5 heads of 1M tokens; heads of at most 16384 candidates need none
 * -- return LH_EWORKSPACE before anything is launched.  Every call on
 * one device shares that device's array: calls that overlap on one GPU (on
 * different streams, or from different threads) race and give undefined
 * results; calls ordered on one stream are safe, and each call clears what
 * it needs zeroed in a kernel.  The first call on a device looks the array's
 * address up (hipGetSymbolAddress); a failure there returns LH_EHIP. */
lh_status lh_topk_noalloc(const lh_shape *shape, const float *score, int32_t *sel,
                          void *stream);

/* a4. Causal gather (technical summary §2.C; bitsgeniais phase 3): the
 * selected candidates plus every coarsest-level entry, ordered by (end token,
 * level) ascending with end(l,j) = (j+1)*p^l - 1.  Writes sub_idx [B,H,S]
 * (flat index per position), pos [B,H,M] (position per entry, -1 if not
 * selected) and copies the rows of q/k/v (level 0) or pq/pk/pv (levels >= 1)
 * into qs,ks,vs [B,H,S,d].  sel must be strictly ascending within [0, C), as
 * lh_topk writes it; for any other sel the outputs are unspecified, but no
 * write leaves sub_idx, pos, qs, ks, vs.  ws: ws_gather bytes (may be 0). */
lh_status lh_gather(const lh_shape *shape, const int32_t *sel, const void *q, const void *k,
                    const void *v, const void *pq, const void *pk, const void *pv,
                    int32_t *sub_idx, int32_t *pos, void *qs, void *ks, void *vs, void *ws,
                    size_t ws_bytes, void *stream);

/* a5. Causal softmax attention on an S-long sequence (technical summary §2.C:
 * stock dense attention on the gathered subsequence), scale 1/sqrt(d):
 * os[i] = sum_{j<=i} softmax_j(qs[i].ks[j]/sqrt(d)) vs[j]; lse[i] = log of the
 * softmax normaliser.  qs,ks,vs: [B,H,S,d] dtype; os: float32 [B,H,S,d]
 * (kept in float32 so that the backward's rowsum(dO * O) is not perturbed by a
 * rounding of O); lse: float32 [B,H,S].  With L = 1 (S = N) and the raw q,k,v
 * this is dense causal attention. */
lh_status lh_attention(const lh_shape *shape, const void *qs, const void *ks, const void *vs,
                       float *os, float *lse, void *stream);

/* a6. Deterministic scatter back to tokens (technical summary §2.C;
 * bitsgeniais phase 4): out[t] = mean over the selected entries e that feed
 * token t (levels 0..L-1, summed in a fixed order) of os[pos(e)]; 0 if none.
 * Which entries feed t is shape->scatter's reading: t's ancestors
 * (LH_SCATTER_SPAN; reads later tokens, see lh_scatter_mode) or the last
 * completed entry of each level (LH_SCATTER_CAUSAL).
 * os: float32 [B,H,S,d]; pos: [B,H,M]; out: [B,H,N,d] dtype. */
lh_status lh_scatter(const lh_shape *shape, const float *os, const int32_t *pos, void *out,
                     void *stream);

/* a1..a6 in one call.  bufs: every field required; out: [B,H,N,d].
 * ws: ws_forward bytes.  Causal in the tokens only with
 * shape->scatter = LH_SCATTER_CAUSAL (see lh_scatter_mode).
 * With bf16 on grids small enough to leave the GPU's workgroup slots
 * unevenly loaded, the attention splits the key range of its heaviest query
 * blocks in two and merges the halves (partials in ws), so os and lse can
 * differ from lh_attention's in the last bits. */
lh_status lh_forward(const lh_shape *shape, const void *q, const void *k, const void *v,
                     void *out, const lh_buffers *bufs, void *ws, size_t ws_bytes,
                     void *stream);

/* a7. Backward of the scatter (technical summary §2.B: gradients flow through
 * scatter, attention and gather; selection gets none):
 * dos[pos(e)] = sum over the tokens t that e feeds of dout[t] / c_t, c_t =
 * number of selected entries feeding t (tokens with c_t = 0 add nothing);
 * "feeds" as in lh_scatter for shape->scatter.  Every row of dos is written.
 * dout: [B,H,N,d] dtype; dos: [B,H,S,d] dtype.  ws: ws_scatter_backward. */
lh_status lh_scatter_backward(const lh_shape *shape, const void *dout, const int32_t *pos,
                              void *dos, void *ws, size_t ws_bytes, void *stream);

/* a8. Backward of lh_attention: given qs,ks,vs (dtype), os (float32) and lse
 * of the forward and the output gradient dos (dtype), writes float32
 * gradients dqs,dks,dvs [B,H,S,d].  Deterministic (separate key-block and
 * query-block passes, no atomics).  ws: ws_attention_backward bytes. */
lh_status lh_attention_backward(const lh_shape *shape, const void *qs, const void *ks,
                                const void *vs, const float *os, const float *lse,
                                const void *dos, float *dqs, float *dks, float *dvs, void *ws,
                                size_t ws_bytes, void *stream);

/* a9. Backward of gather and pooling: dX[t] = sum over t's selected ancestors
 * e of dXs[pos(e)] / p^level(e), for X in {q,k,v}.  dqs,dks,dvs: float32
 * [B,H,S,d]; dq,dk,dv: [B,H,N,d] dtype. */
lh_status lh_gather_backward(const lh_shape *shape, const float *dqs, const float *dks,
                             const float *dvs, const int32_t *pos, void *dq, void *dk,
                             void *dv, void *stream);

/* a7..a9 in one call, from the buffers lh_forward filled (pos, qs, ks, vs,
 * os, lse are read).  dout: [B,H,N,d]; dq,dk,dv: [B,H,N,d] dtype.
 * ws: ws_backward bytes.
 * With bf16 and d = 64 the call forks part of its work onto a side stream
 * that the library keeps per host thread and device (made by the first such
 * call that is not inside a graph capture, kept until the process ends):
 * the gather backward of dq runs there beside the dK/dV pass, and `stream`
 * waits for it before the call's last work, so the outputs are ready, as
 * always, when `stream` reaches that point.  Under graph capture the side
 * stream joins the capture and rejoins `stream` within the call. */
lh_status lh_backward(const lh_shape *shape, const void *dout, const lh_buffers *bufs,
                      void *dq, void *dk, void *dv, void *ws, size_t ws_bytes,
                      void *stream);

/* Measurement aid (not part of the layer's computation): runs lh_forward and
 * then lh_backward once on `stream`, records a hipEvent after each stage and
 * writes the elapsed milliseconds of each stage to ms[0..LH_PROFILE_STAGES-1]:
 *   0 pyramid + scores   1 top-K            2 gather        3 attention
 *   4 scatter            5 scatter backward 6 rowsum(dO*O)  7 attention dK,dV
 *   8 attention dQ       9 gather+pool backward
 * With bf16 storage the dQ pass forms rowsum(dO*O) itself and runs before
 * the dK/dV pass, so stage 6 is empty (about 0 ms).
 * Arguments as for lh_forward / lh_backward; ws must hold
 * max(ws_forward, ws_backward) bytes.  Unlike every other entry point this
 * call waits for the stream before returning. */
#define LH_PROFILE_STAGES 10
lh_status lh_profile_step(const lh_shape *shape, const void *q, const void *k, const void *v,
                          void *out, const lh_buffers *bufs, const void *dout, void *dq, void *dk,
                          void *dv, void *ws, size_t ws_bytes, float *ms, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* LIGHTHOUSE_H */
