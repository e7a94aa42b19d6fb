/*
 * gdn.h -- C ABI of the gated delta-rule layer on AMD Instinct MI355X (gfx950).
 *
 * The layer (gated-deltanet card, "Method"; per-key-channel decay as in GDN-2,
 * Marin note "Background") keeps a state S [Dk x Dv] per (batch, head) and,
 * for each token t, applies
 *     S <- diag(exp(g_t)) S;  m = S^T k_t;  d = beta_t (v_t - m);
 *     S <- S + k_t d^T;       o_t = scale * S^T q_t.
 * g_t is one log-decay per key channel (GDN_DECAY_PER_CHANNEL) or one scalar
 * per head broadcast over the channels (GDN_DECAY_PER_HEAD).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers are DEVICE pointers (hipMalloc'd or from a torch tensor), dense,
 * row-major, 16-byte aligned.  The caller owns every buffer; the library keeps
 * no allocation between calls and allocates nothing itself.  All work is
 * enqueued on `stream` (a hipStream_t; NULL = the null stream) with no host
 * synchronisation, so asynchronous faults surface at the caller's next sync.
 *
 * Tensor layouts (element types in brackets):
 *   q, k      [B, T, H, Dk]         (dtype: float32 or bf16)
 *   v, o, dO  [B, T, H, Dv]         (dtype)
 *   g         [B, T, H, Dk] per channel, or [B, T, H] per head   (float32)
 *   beta      [B, T, H]                                          (float32)
 *   states    h0, hT, dhT, dh0, decode state: [B, H, Dk, Dv]     (float32)
 *   dq, dk    [B, T, H, Dk] (dtype);  dv [B, T, H, Dv] (dtype)
 *   dg        like g (float32);  dbeta [B, T, H] (float32)
 * Grouped-query repetition of q/k heads is the caller's (gated-deltanet card,
 * "Requirements and limits").  q and k are used as given unless the shape's
 * qk_l2norm is set (the card's use_qk_l2norm, "Usage"): then every q and k row
 * (the Dk values of one token and head) is replaced inside the call by
 * x / sqrt(sum(x^2) + GDN_L2NORM_EPS) before the recurrence, and dq, dk are the
 * gradients with respect to the raw, unnormalised rows,
 * dx = r (dx_hat - x_hat (x_hat . dx_hat)) with r = 1 / sqrt(sum(x^2) + eps).
 * The card names the option but not its guard; 1e-6 inside the root is the
 * reading taken here.
 *
 * Errors: every call returns a status.  Bad shapes, NULL required pointers,
 * misaligned pointers and a too-small workspace are rejected before anything
 * is launched.  An unsupported (chunk, Dk, Dv) combination returns
 * GDN_ERR_UNSUPPORTED; there is no fallback path.  A failed launch returns
 * GDN_ERR_HIP.  Results are deterministic: repeated calls with the same inputs
 * are bitwise identical (gated-deltanet card, "Correctness").
 *
 * Supported sizes: chunked calls Dk = Dv in {64, 128} with chunk 64 (the
 * default) and Dk = Dv = 16 with chunk 16; decode Dk = Dv in {16, 32, 64, 128};
 * any T >= 0 (a ragged last chunk is processed as if padded with tokens that
 * have g = 0 and beta = 0, which leave the state exactly unchanged; their
 * outputs are not written); B, H >= 1, and for chunked calls
 * H * max(Dk, Dv) * chunk <= 2^28 (H <= 32768 at 128 x 128) and
 * B * H * ceil(T / chunk) * chunk < 2^27 (the token-heads of one call, the last
 * chunk counted whole; the largest launch has 32 work-items per token-head).
 * Anything else: GDN_ERR_UNSUPPORTED, before any launch.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1,
    GDN_ERR_UNSUPPORTED = 2,
    GDN_ERR_ALIGNMENT = 3,
    GDN_ERR_WORKSPACE = 4,
    GDN_ERR_HIP = 5
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;
typedef enum { GDN_DECAY_PER_HEAD = 0, GDN_DECAY_PER_CHANNEL = 1 } gdn_decay;

#define GDN_L2NORM_EPS 1e-6f

/* Stage boundaries of the chunked forward that the numerical-safety options act
 * on (atomic_ops card, "Features": chunk scores -> WY block solve -> recompute
 * -> inter-chunk scan): the scores P (unscaled) and A (with beta), the solve's
 * T, the recompute's U and W, the outputs o and the final state hT. */
enum {
    GDN_DIAG_P = 0,
    GDN_DIAG_A = 1,
    GDN_DIAG_T = 2,
    GDN_DIAG_U = 3,
    GDN_DIAG_W = 4,
    GDN_DIAG_O = 5,
    GDN_DIAG_HT = 6,
    GDN_DIAG_STAGES = 7
};
/* counters: word 2*stage counts non-finite values, word 2*stage+1 finite
 * values with |x| > 1e6 */
#define GDN_DIAG_WORDS (2 * GDN_DIAG_STAGES)

typedef struct {
    int B, T, H, Dk, Dv;
    int dtype;     /* gdn_dtype of q, k, v, o, dO, dq, dk, dv */
    int decay;     /* gdn_decay */
    float scale;   /* output scale; 0 means Dk^-0.5 (the atomic_ops card passes d^-0.5) */
    int chunk;     /* chunk length C of the chunked form: 16 or 64; 0 means 64 */
    int qk_l2norm; /* 1: L2-normalise q and k rows inside the call (see above); 0: as given.
                      A training pair (gdn_forward_train, gdn_backward_train) must pass the
                      same value to both calls. */
    /* Numerical-safety options of the chunked calls (atomic_ops card, "Features"
     * and "Debugging"); all zero = off.  Not supported by gdn_decode_step.  A
     * training pair must pass the same values to both calls. */
    float wy_eps;  /* >= 0: the WY block solve inverts (1 + wy_eps) I + A instead of
                      I + A (damping on the diagonal); results then depend on the chunk */
    float clip;    /* >= 0; > 0: at each stage boundary (GDN_DIAG_*) values are made
                      finite (NaN -> 0, +-inf -> +-clip) and clamped to [-clip, clip],
                      and so are dq, dk, dv, dg, dbeta, dh0; gradients take the clipping
                      as the identity */
    int diag;      /* 1: the forward counts, per stage boundary and before clipping,
                      non-finite values and finite values with |x| > 1e6 into counters
                      in the workspace (read with gdn_diag_read); never changes values */
} gdn_shape;

/*
 * gdn_new_state -- zero-fill a caller-allocated state buffer [B,H,Dk,Dv] float32.
 * The gated-deltanet card's new_state(batch, heads, key_dim, value_dim) gives a
 * fresh state for a sequence ("Usage"); zero is the state before any token.
 * Errors: GDN_ERR_INVALID_ARG for NULL state or non-positive sizes.
 */
gdn_status gdn_new_state(float *state, int B, int H, int Dk, int Dv, void *stream);

/*
 * gdn_workspace_bytes -- device scratch size that gdn_forward
 * (for_backward = 0) or gdn_backward (for_backward = 1) needs for `shape`.
 * Returns 0 for an invalid or unsupported shape.  The workspace is caller
 * memory, 256-byte aligned, contents on entry irrelevant.
 */
size_t gdn_workspace_bytes(const gdn_shape *shape, int for_backward);

/*
 * gdn_forward -- the whole layer over T tokens in chunked form.
 *
 * Within each chunk of C tokens the per-channel cumulative decay is formed
 * (Marin note, "Background"); query-key and key-key scores that span the two
 * halves of a block are computed with the decay split at the last token of
 * the earlier half, so the spanning scores are one dense matrix product per
 * block pair (Marin note, "Approach"); the split is repeated inside every
 * half down to single tokens, so every score comes from such a product; the
 * unit-lower-triangular delta system of the chunk is solved in WY form; and
 * the state is carried across chunks
 * (atomic_ops card, "Features": chunk scores, WY block solve, recompute,
 * inter-chunk scan).  The result equals the token recurrence above up to
 * floating-point rounding.
 *
 * h0 may be NULL (zero initial state).  hT may be NULL (not written) and may
 * alias h0 (the state carries in place across calls, as in the gated-deltanet
 * card's "Usage").  o must not alias any input.  ws must hold
 * gdn_workspace_bytes(shape, 0) bytes (GDN_ERR_WORKSPACE otherwise).
 */
gdn_status gdn_forward(const gdn_shape *shape, const void *q, const void *k, const void *v,
                       const float *g, const float *beta, const float *h0, void *o, float *hT,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * gdn_forward_noalloc -- gdn_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation and results (bitwise), with the
 * workspace taken from a static device array of GDN_NOALLOC_SCRATCH_BYTES that
 * every device holds from the library's first use on it until the process
 * ends.  The call allocates nothing.  Every call on one device shares that
 * device's array, so calls that overlap on one device (concurrent streams or
 * host threads) race and must be serialised by the caller; consecutive calls on
 * one stream are safe.  The shape must have diag = 0 (the stage counters would
 * sit in the shared array, out of the caller's reach).
 * Errors: as gdn_forward; GDN_ERR_WORKSPACE when gdn_workspace_bytes(shape, 0)
 * exceeds GDN_NOALLOC_SCRATCH_BYTES (64 MiB: at 128 x 128 with chunk 64 about
 * 450 chunk-heads, e.g. B = 1, H = 6, T = 4096); GDN_ERR_UNSUPPORTED for diag = 1;
 * GDN_ERR_HIP if the array's device address cannot be obtained.
 */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)
gdn_status gdn_forward_noalloc(const gdn_shape *shape, const void *q, const void *k,
                               const void *v, const float *g, const float *beta, const float *h0,
                               void *o, float *hT, void *stream);

/*
 * gdn_backward -- gradients of the chunked forward with respect to q, k, v, g,
 * beta and h0, given dO = dL/do and dhT = dL/dhT (NULL = zero).  The forward
 * intermediates are recomputed from the inputs (nothing is kept between
 * calls); the backward runs a reverse scan over chunks followed by a
 * chunk-parallel gradient stage (atomic_ops card, "Features": fused backward).
 * dh0 may be NULL (not written).  Every other output is required.
 * ws must hold gdn_workspace_bytes(shape, 1) bytes.
 */
gdn_status gdn_backward(const gdn_shape *shape, const void *q, const void *k, const void *v,
                        const float *g, const float *beta, const float *h0, const void *dO,
                        const float *dhT, void *dq, void *dk, void *dv, float *dg, float *dbeta,
                        float *dh0, void *ws, size_t ws_bytes, void *stream);

/*
 * gdn_forward_train / gdn_backward_train -- the same forward and backward for
 * training, where the backward reuses what the forward computed instead of
 * recomputing it (atomic_ops card, "Features": the backward reuses forward
 * residuals).  gdn_forward_train writes o and hT exactly as gdn_forward and
 * also leaves its chunk intermediates and the state at the start of every
 * chunk in `ws`, which must hold gdn_workspace_bytes(shape, 1) bytes.
 * gdn_backward_train then reads them from the same `ws`: it must be called
 * with the same shape, the same q, k, v, g, beta contents and the workspace
 * untouched in between (the library cannot check this; a mismatch gives
 * wrong gradients, not an error).  Results equal gdn_backward's bitwise.
 * Errors as gdn_forward / gdn_backward.
 */
gdn_status gdn_forward_train(const gdn_shape *shape, const void *q, const void *k, const void *v,
                             const float *g, const float *beta, const float *h0, void *o,
                             float *hT, void *ws, size_t ws_bytes, void *stream);
gdn_status gdn_backward_train(const gdn_shape *shape, const void *q, const void *k,
                              const void *v, const float *g, const float *beta, const void *dO,
                              const float *dhT, void *dq, void *dk, void *dv, float *dg,
                              float *dbeta, float *dh0, void *ws, size_t ws_bytes, void *stream);

/*
 * gdn_decode_step -- one token of the recurrence for every (batch, head), with
 * the state updated in place: each state is read once and written once
 * (gated-deltanet card, "Method": the state is the whole cost).  shape->T must
 * be 1; q, k [B,1,H,Dk]; v, o [B,1,H,Dv]; g [B,1,H,Dk] or [B,1,H];
 * beta [B,1,H]; state [B,H,Dk,Dv] float32 (read and overwritten).
 * Decoding token by token equals the chunked forward up to rounding.
 */
gdn_status gdn_decode_step(const gdn_shape *shape, const void *q, const void *k, const void *v,
                           const float *g, const float *beta, float *state, void *o,
                           void *stream);

/*
 * Decode with a checkpoint and a buffer of recent tokens (the ReplaySSM idea:
 * news digest "Gated DeltaNet", the blurb on state traffic in SSM decoding).
 * The state of each (batch, head) is a checkpoint `ckpt` [B,H,Dk,Dv] fp32 plus
 * up to `depth` (1..16) buffered tokens (their key, accumulated log-decay and
 * delta).  gdn_replay_step reads the checkpoint, computes the token's output
 * and delta directly (no state write), and appends to the buffer; when the
 * buffer fills it folds it into the checkpoint.  Outputs and, after
 * gdn_replay_fold, the state are those of gdn_decode_step (same recurrence,
 * reassociated; equal up to fp32 rounding).  Shapes as gdn_decode_step
 * (T == 1, no numerical-safety options); `buf` is caller-owned device memory of
 * gdn_replay_buffer_bytes(shape, depth) bytes, emptied by gdn_replay_reset
 * before first use.  Every call must pass the same depth and decay kind.
 * Errors: GDN_ERR_INVALID_ARG for a bad shape or depth or a NULL pointer,
 * GDN_ERR_ALIGNMENT, GDN_ERR_UNSUPPORTED for sizes gdn_decode_step refuses.
 */
size_t gdn_replay_buffer_bytes(const gdn_shape *shape, int depth);
gdn_status gdn_replay_reset(const gdn_shape *shape, void *buf, int depth, void *stream);
gdn_status gdn_replay_step(const gdn_shape *shape, const void *q, const void *k, const void *v,
                           const float *g, const float *beta, float *ckpt, void *buf, int depth,
                           void *o, void *stream);
/* gdn_replay_fold -- fold the buffer into the checkpoint (ckpt becomes the
 * current state) and empty it; q, k, v, g, beta are not read. */
gdn_status gdn_replay_fold(const gdn_shape *shape, float *ckpt, void *buf, int depth,
                           void *stream);

/*
 * gdn_diag_read -- copy the stage counters of the last chunked forward pass run
 * in `ws` (gdn_forward, gdn_forward_train, or the recompute inside gdn_backward,
 * which has no o / hT stage) to host memory: counts[GDN_DIAG_WORDS].  The
 * shape must have diag = 1 and match the call that ran.  Synchronises `stream`
 * (atomic_ops card, "Debugging": per-stage reports of non-finite or > 1e6
 * values; diagnostic only).
 * Errors: GDN_ERR_INVALID_ARG for a bad shape, diag = 0, NULL ws or counts;
 * GDN_ERR_HIP if the copy fails.
 */
gdn_status gdn_diag_read(const gdn_shape *shape, const void *ws, unsigned int *counts,
                         void *stream);

/* gdn_status_string -- static, human-readable name of a status code. */
const char *gdn_status_string(gdn_status status);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
