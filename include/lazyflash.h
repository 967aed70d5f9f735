/*
 * lazyflash.h -- C ABI of liblazyflash.so: LazyFlash-style attention on AMD
 * Instinct MI355X (gfx950).
 *
 * Method (the LazyFlash journal entry on gyom.fr, "LazyFlash allège la
 * rétropropagation de l'attention, 5,72 fois"):
 *   - the forward is ordinary exact FlashAttention and is left dense
 *     (section "Le passage arrière fait deux fois le travail du passage
 *     avant");
 *   - the backward ranks query blocks by the norm of their output gradient,
 *     keeps each block with a probability set by a budget delta on the
 *     discarded gradient mass, reweights kept blocks so the gradient stays
 *     unbiased in expectation, and never loads or computes the skipped tiles
 *     (section "Un budget sur la masse de gradient, et un tirage qui garde le
 *     gradient non biaisé");
 *   - the backward kernel consumes per-block weights directly (section
 *     "Trois tailles de modèle, 19 découpages sur 21").
 *
 * The exact keep rule implemented here (the pages fix the idea, not the rule):
 *   m[b,h,i] = ||dO[b,h,block i]||_F^2 in float64, summed by the halving tree
 *              over the row-major flattening of the block;
 *   p_i      = 0 if m_i == 0, else min(1, m_i / tau);
 *   tau      = root of sum_i (1 - p_i) m_i = delta * sum_i m_i per (b, h)
 *              (tau = smallest positive mass when delta == 0, +inf when every
 *              mass is zero, NaN when a mass is not finite: then every block
 *              is kept with weight 1);
 *   u_i      = (x0 >> 11) * 2^-53, x0 = first word of Philox4x64-10 with key
 *              (seed, 0) and counter (i, h, b, 0);
 *   keep_i   = u_i < p_i;   w_i = (float)(1.0 / p_i) if kept, else 0.
 * The sparse gradient equals the dense gradient of dO' = keep * w * dO.
 *
 * Conventions for every entry point:
 *   - Tensors are row-major and contiguous: Q, O, dO, dQ are [B, Hq, N, d],
 *     K, V, dK, dV are [B, Hkv, N, d] (d fastest); LSE and D are [B, Hq, N].
 *     Query head h reads key/value head h / (Hq / Hkv).
 *   - All tensor pointers are DEVICE pointers owned by the caller; outputs are
 *     fully overwritten (never accumulated into).  The library allocates
 *     nothing and keeps no state between calls; scratch memory, where an entry
 *     point needs it, is a caller-owned workspace argument.  The one exception
 *     is lf_attn_bwd_noalloc, for callers that cannot allocate: its scratch is
 *     a static device array of the library (one per GPU, loaded with the
 *     library's kernels).  Work is enqueued on `stream` (a hipStream_t; NULL =
 *     the default stream) and the call returns without waiting for it.
 *   - Alignment: the element tensors (Q, K, V, O, dO, dQ, dK, dV) and the
 *     workspace start on a 16-byte boundary (the kernels move them in 16-byte
 *     pieces); the other arrays on their element size (4 bytes; 8 for the
 *     double-precision mass and tau).  A misaligned pointer is LF_EINVAL.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     failed check returns LF_EINVAL (malformed) or LF_EUNSUPPORTED (valid
 *     but outside what the kernels implement) and launches nothing.  A failed
 *     launch returns LF_EHIP.  lf_last_error() describes the last failure of
 *     the calling thread.
 *   - An empty problem (batch == 0 or seqlen == 0) is valid and enqueues
 *     nothing; its tensor pointers may then be NULL.
 *   - Supported: dtype LF_BF16 or LF_F32, head_dim 64 or 128, block 64 or 128,
 *     ceil(seqlen / block) <= 4096, heads_q a multiple of heads_kv, finite
 *     scale.  seqlen need not be a multiple of block: the last query block of
 *     each head then has seqlen - (nqb - 1) * block rows (its mass sums those
 *     rows; the backward treats it like any block).
 */
#ifndef LAZYFLASH_H
#define LAZYFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LF_OK = 0,
    LF_EINVAL = 1,        /* malformed arguments (null pointer, bad shape, delta) */
    LF_EUNSUPPORTED = 2,  /* well-formed but not implemented (head_dim, block, ...) */
    LF_EHIP = 3,          /* the HIP runtime reported an error at launch */
    /* not a status: makes every int32_t value a valid lf_status, so a code
     * from a newer library or a caller's cast is safe to pass around */
    LF_STATUS_MAX_ENUM = 0x7fffffff
} lf_status;

/* LF_DTYPE_MAX_ENUM is not a dtype: it makes every int32_t value a valid
 * lf_dtype, so an unknown code in lf_shape is rejected, not undefined */
typedef enum { LF_BF16 = 0, LF_F32 = 1, LF_DTYPE_MAX_ENUM = 0x7fffffff } lf_dtype;

typedef struct {
    int32_t batch;      /* B */
    int32_t heads_q;    /* Hq: query heads */
    int32_t heads_kv;   /* Hkv: key/value heads, divides Hq */
    int32_t seqlen;     /* N: queries = keys (self-attention) */
    int32_t head_dim;   /* d */
    int32_t block;      /* query-block size of the selection, rows */
    int32_t causal;     /* nonzero: query i sees keys j <= i */
    float scale;        /* softmax scale, usually 1/sqrt(d) */
    int32_t dtype;      /* lf_dtype of Q, K, V, O, dO, dQ, dK, dV */
} lf_shape;

/*
 * Dense attention forward (FlashAttention tiling, exact softmax).
 * The forward is unchanged by the method: see the section "Le passage arrière
 * fait deux fois le travail du passage avant" of the LazyFlash entry, and the
 * FlashAttention course page on voce.life, section "Le mécanisme".
 *   q [B,Hq,N,d], k, v [B,Hkv,N,d]  (dtype)            in
 *   o [B,Hq,N,d] (dtype)                               out: softmax(scale q k^T) v
 *   lse [B,Hq,N] float32                               out: natural-log logsumexp
 *                                                           of each scaled score row
 */
lf_status lf_attn_fwd(const lf_shape* shape, const void* q, const void* k, const void* v,
                      void* o, float* lse, void* stream);

/*
 * Block selection: masses, budget tau, Philox draw, weights, compaction.
 * Section "Un budget sur la masse de gradient, et un tirage qui garde le
 * gradient non biaisé" of the LazyFlash entry; the rule is stated above.
 *   o, dout [B,Hq,N,d] (dtype)                         in
 *   delta in [0, 1), seed                              in
 *   D [B,Hq,N] float32                                 out: rowsum(dout * o) on the
 *                                                           rows of kept blocks, 0 on
 *                                                           the rows of skipped blocks
 *                                                           (the backward reads only
 *                                                           kept rows' D)
 *   mass [B,Hq,nqb] float64                            out: block masses (bit-exact)
 *   tau [B,Hq] float64                                 out: per-head threshold
 *   block_w [B,Hq,nqb] float32                         out: 1/p if kept, else 0
 *   kept_idx [B,Hq,nqb] int32                          out: kept blocks ascending,
 *                                                           then -1 padding
 *   kept_count [B,Hq] int32                            out: number of kept blocks
 * nqb = ceil(seqlen / block).  Returns LF_EINVAL for delta outside [0, 1) or NaN.
 */
lf_status lf_block_select(const lf_shape* shape, const void* o, const void* dout,
                          double delta, uint64_t seed, float* D, double* mass, double* tau,
                          float* block_w, int32_t* kept_idx, int32_t* kept_count,
                          void* stream);

/*
 * Block selection under another rule, for comparing rules at equal backward
 * time (section "Le choix des blocs pèse plus que la quantité sautée" of the
 * LazyFlash entry: the budget against a fixed fraction, chosen once where the
 * budget adapts, and top-k, which drops the same blocks at every step where
 * the budget's draw changes).  Same outputs, layouts and errors as
 * lf_block_select; the backward consumes them unchanged.  With n the number
 * of positive-mass blocks of a (batch, head):
 *   LF_SELECT_BUDGET    param = delta in [0, 1): exactly lf_block_select;
 *   LF_SELECT_FRACTION  param = f in (0, 1]: the budget's draw (Philox
 *                       uniform, keep iff u < p, w = 1/p) with p = min(1, m/tau)
 *                       and tau the root of sum_i p_i = f n, found on the
 *                       sorted masses like the budget's tau (f n >= n keeps
 *                       every positive block, tau = smallest positive mass);
 *   LF_SELECT_TOPK      param = f in (0, 1]: the ceil(f n) largest masses, ties
 *                       to the lower block index, weight 1, no draw (seed
 *                       unused); tau = the smallest kept mass.
 * Zero-mass blocks are never kept; a head with a non-finite mass keeps every
 * block with weight 1 and tau = NaN under every rule.  An unknown rule or a
 * parameter outside its range is LF_EINVAL.
 */
#define LF_SELECT_BUDGET 0
#define LF_SELECT_FRACTION 1
#define LF_SELECT_TOPK 2
lf_status lf_block_select_rule(const lf_shape* shape, const void* o, const void* dout,
                               int32_t rule, double param, uint64_t seed, float* D, double* mass,
                               double* tau, float* block_w, int32_t* kept_idx,
                               int32_t* kept_count, void* stream);

/*
 * Block-sparse attention backward over the kept query blocks only.
 * Sections "Un budget sur la masse de gradient..." (skipped tiles are never
 * loaded nor computed) and "Trois tailles de modèle, 19 découpages sur 21"
 * (the backward kernel consumes the per-block weights) of the LazyFlash entry.
 *   q, k, v, dout (dtype), lse, D (float32)            in: as above
 *   kept_idx, kept_count, block_w                      in: from lf_block_select
 *   dq [B,Hq,N,d], dk, dv [B,Hkv,N,d] (dtype)          out: gradient of dO' =
 *                                                           keep*w*dO; rows of
 *                                                           skipped blocks of dq
 *                                                           are exact zeros
 *   workspace, workspace_bytes                         scratch: device memory of at
 *                                                           least lf_bwd_workspace_size
 *                                                           bytes, owned by the caller
 * The result is deterministic: bit-identical on every call with the same
 * inputs (no floating-point atomics; partial sums are added in a fixed
 * order).  The workspace needs no initialisation and holds nothing useful
 * afterwards; calls that may overlap (other streams) need workspaces of their
 * own.  Too small a workspace, or NULL with a nonzero size requirement, is
 * LF_EINVAL.  Passing every block kept with weight 1 (lf_block_select with
 * delta = 0) gives the dense backward through the same kernels.
 */
lf_status lf_attn_bwd(const lf_shape* shape, const void* q, const void* k, const void* v,
                      const float* lse, const void* dout, const float* D,
                      const int32_t* kept_idx, const int32_t* kept_count, const float* block_w,
                      void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * Workspace bytes that lf_attn_bwd and lf_attn_bwd_phases need for `shape`
 * (written to *bytes).  It depends on the shape only: at most
 * 6144 * block * head_dim + 30 * B * Hq * nqb + 29 KiB, about 100 MB for
 * block = head_dim = 128, and 0 for LF_F32.  Shape errors as in lf_attn_bwd.
 */
lf_status lf_bwd_workspace_size(const lf_shape* shape, size_t* bytes);

/*
 * The two independent halves of lf_attn_bwd, selectable by a bit mask; all
 * bits together are exactly lf_attn_bwd.  They may run in either order or on
 * different streams (each reads only the inputs and writes only its own
 * outputs), which lets a caller overlap them with other work or time them.
 *   LF_BWD_DKDV  the key-tile walk over kept blocks: writes dk and dv
 *   LF_BWD_DQ    the query-block walk: writes dq (zeros for skipped blocks);
 *                the only half that uses the workspace
 * Unused output pointers of an unselected half, and the workspace when
 * LF_BWD_DQ is not selected, may be NULL.  An empty or unknown mask is
 * LF_EINVAL.
 */
#define LF_BWD_DKDV 1u
#define LF_BWD_DQ 2u
#define LF_BWD_ALL 3u
lf_status lf_attn_bwd_phases(const lf_shape* shape, const void* q, const void* k, const void* v,
                             const float* lse, const void* dout, const float* D,
                             const int32_t* kept_idx, const int32_t* kept_count,
                             const float* block_w, void* dq, void* dk, void* dv, void* workspace,
                             size_t workspace_bytes, uint32_t phases, void* stream);

/*
 * lf_attn_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same backward, with the dQ phase's workspace taken from a static device
 * array of the library (128 MiB per GPU, held until the process ends; the
 * headline shape B=1, Hq=32, N=32768, d=128, block=128 needs 96.3 MiB) instead
 * of a workspace argument.  Arguments, results and determinism are those of
 * lf_attn_bwd; nothing is allocated and nothing needs clearing.  The first call
 * on a GPU looks up that GPU's array address once (make it before capturing a
 * graph).  Every call on one GPU shares that GPU's array: calls that may
 * overlap on one GPU (other streams, other threads) race; serialise them or use
 * lf_attn_bwd with workspaces of their own.  A problem whose workspace
 * (lf_bwd_workspace_size) exceeds the array is LF_EUNSUPPORTED, before
 * anything is enqueued.
 */
lf_status lf_attn_bwd_noalloc(const lf_shape* shape, const void* q, const void* k, const void* v,
                              const float* lse, const void* dout, const float* D,
                              const int32_t* kept_idx, const int32_t* kept_count,
                              const float* block_w, void* dq, void* dk, void* dv, void* stream);

/*
 * Variable-length batches (a batch of sequences of different lengths, packed
 * without padding: the pages' workload is examples cut to each length, section
 * "À 32 000 tokens, 5,72 fois sur l'attention arrière" of the LazyFlash entry).
 * shape->batch is the number of sequences B; shape->seqlen is not used.
 * cu_seqlens is a HOST array of B + 1 token offsets: cu[0] = 0, nondecreasing,
 * sequence b has L_b = cu[b + 1] - cu[b] tokens (0 allowed).  Each sequence is
 * one fixed-length problem of batch 1 and length L_b (all rules above apply
 * per sequence, L_b need not be a multiple of block), stored as consecutive
 * slices of the packed buffers:
 *   q, o, dout, dq   [Hq, L_b, d] at element offset Hq * cu[b] * d
 *   k, v, dk, dv     [Hkv, L_b, d] at element offset Hkv * cu[b] * d
 *   lse, D           [Hq, L_b] at element offset Hq * cu[b]
 *   mass, block_w, kept_idx   [Hq, nqb_b] at element offset Hq * cb[b],
 *                    nqb_b = ceil(L_b / block), cb[b] = sum over j < b of nqb_j
 *   tau, kept_count  [Hq] at element offset Hq * b
 * The selection draw of block i of head h of sequence b is the draw of batch
 * entry b (counter (i, h, b, 0)), so sequences never share uniforms.  Every
 * sequence is checked before anything is enqueued; the work of the sequences
 * is enqueued one after the other on `stream` (the backward's sequences share
 * the workspace, which must hold lf_bwd_workspace_size_varlen bytes).  An
 * empty sequence gets tau = +inf and kept_count = 0 and nothing else.
 */
lf_status lf_attn_fwd_varlen(const lf_shape* shape, const int32_t* cu_seqlens, const void* q,
                             const void* k, const void* v, void* o, float* lse, void* stream);
lf_status lf_block_select_varlen(const lf_shape* shape, const int32_t* cu_seqlens,
                                 const void* o, const void* dout, int32_t rule, double param,
                                 uint64_t seed, float* D, double* mass, double* tau,
                                 float* block_w, int32_t* kept_idx, int32_t* kept_count,
                                 void* stream);
lf_status lf_bwd_workspace_size_varlen(const lf_shape* shape, const int32_t* cu_seqlens,
                                       size_t* bytes);
lf_status lf_attn_bwd_varlen(const lf_shape* shape, const int32_t* cu_seqlens, const void* q,
                             const void* k, const void* v, const float* lse, const void* dout,
                             const float* D, const int32_t* kept_idx, const int32_t* kept_count,
                             const float* block_w, void* dq, void* dk, void* dv, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Static, human-readable name of a status code. */
const char* lf_status_str(lf_status status);

/* Description of the last failure on the calling thread ("" if none).  The
 * string is owned by the library and valid until the thread's next call. */
const char* lf_last_error(void);

/* ABI version of this header, for run-time checks by bindings. */
int32_t lf_abi_version(void);

#define LF_ABI_VERSION 8  /* 8: misaligned pointers refused; 7: lf_attn_bwd_noalloc; 6: D on kept rows only */

#ifdef __cplusplus
}
#endif

#endif /* LAZYFLASH_H */
