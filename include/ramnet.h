/*
 * ramnet.h: C ABI of the RAM-Net layer recurrence on AMD Instinct MI355X
 * (gfx950).
 *
 * The layer (RAM-Net project page, muoncat.github.io/ramnet_web, "RAM-Net:
 * Linear-Time Sequence Modeling with Sparsely Addressable State"):
 *   1. Address Decoder, Product Softmax ("Product Softmax", "Soft Radix
 *      Address" paragraphs): a key or query carries U blocks of d_p logits;
 *      a softmax over each block is one base-d_p digit's distribution and a
 *      slot's weight is the product of its U digit probabilities, over
 *      M = d_p^U slots.  The K heaviest slots are found exactly by a
 *      level-by-level prefix search (the exact Top-K paragraph after
 *      "Waveform Modulation").  Block u is digit u counted from the most
 *      significant one.  Weights are the raw products (not renormalised).
 *      Equal weights rank by the smaller slot index.  The ranking is that
 *      of the exact weights: a weight is exp(sum of the slot's digit logits
 *      - sum of the blocks' log-normalisers), the normalisers are common to
 *      every slot, so slots rank by their logit sums, which the decoders
 *      form exactly (bf16 logits; fp64 sums for fp32 logits), and ties are
 *      exact ties.  Returned weights are exp(...) in fp64, rounded to fp32.
 *   2. CAPE ("Cyclic Address Positional Embedding" paragraphs): a token at
 *      position P moves every digit of its read and write slots by
 *      (P mod d_p), cyclically within d_p values.  Weights are unchanged.
 *   3. Gated Sparse Update ("Gated Sparse Update" paragraphs, four steps),
 *      for each of the K write slots i with weight w at a token with gate
 *      gamma and value v:
 *          alpha = (1 - w)^(exp(gamma))      (retention; 0 when w >= 1)
 *          m_i   = alpha * m_i + w           (mass, stored fp32)
 *          lam   = w / (m_i + eps_gsu)       (rate)
 *          S_i   = S_i + lam * (v - S_i)     (content, stored in state dtype)
 *      A slot with w = 0, and every slot that is not addressed, keeps its
 *      content and mass bit-for-bit.
 *   4. Read ("three stages" paragraph): after the token's K writes,
 *      r = sum_j rho_j * S_{r_j} over the K read slots, then RMSNorm over d_v
 *      (eps_norm, optional weight omega) and the output gate sigmoid(g):
 *          out = r / sqrt(mean(r^2) + eps_norm) * omega * sigmoid(g)
 *      (out = 0 for an all-zero read with eps_norm = 0).
 *
 * Conventions for every entry point:
 *   - Tensors are contiguous, row-major, in DEVICE memory, caller-owned.
 *     The library allocates no device memory; scratch space comes from the
 *     caller's `workspace` (size from ramnet_workspace_bytes or
 *     ramnet_layer_workspace_bytes).  The one exception: the first
 *     projection call on a device creates that device's hipBLASLt handle,
 *     which lives until the process ends.
 *   - Every device pointer must be 16-byte aligned.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*; NULL is the null stream).  Validation runs synchronously on the
 *     host before anything is enqueued; on any error nothing is enqueued and
 *     no buffer is touched.
 *   - Errors are returned as ramnet_status; ramnet_last_error() gives a
 *     message for the calling thread's last failure.
 *   - S and mass are updated in place.  Inputs are never written.  `out`
 *     and the address outputs must not overlap any other buffer.
 *   - Calls that share S/mass must be ordered by the caller (same stream).
 *     Calls on different buffers may run concurrently; the only global state
 *     is the per-device hipBLASLt handle and its per-shape algorithm cache
 *     (guarded by a lock).
 */
#ifndef RAMNET_H
#define RAMNET_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RAMNET_VERSION 6
/* Largest supported K (Top-K per address). */
#define RAMNET_KMAX 64

typedef enum {
    RAMNET_OK = 0,
    RAMNET_EINVAL = -1,       /* bad shape, NULL or misaligned pointer, overlap */
    RAMNET_EUNSUPPORTED = -2, /* valid request this build does not implement */
    RAMNET_EWORKSPACE = -3,   /* workspace missing or too small */
    RAMNET_EHIP = -4          /* the HIP runtime reported an error */
} ramnet_status;

typedef enum { RAMNET_F32 = 0, RAMNET_BF16 = 1 } ramnet_dtype;

typedef enum {
    RAMNET_OP_DECODE = 0,
    RAMNET_OP_PREFILL = 1,
    RAMNET_OP_STEP = 2,
    RAMNET_OP_BACKWARD = 3
} ramnet_op;

typedef struct {
    int32_t B, T, H;      /* batch, tokens per sequence, heads; T = 1 for a step */
    int32_t d_p, U;       /* digit base and digit count; 2 <= d_p <= 8 */
    int64_t M;            /* slots per head; must equal d_p^U, <= 2^30 */
    int32_t K;            /* slots per read/write, 1 <= K <= min(M, RAMNET_KMAX) */
    int32_t d_v;          /* value channels; 64, 128, 192 or 256 */
    int32_t in_dtype;     /* ramnet_dtype of q, k, v, gamma, g */
    int32_t state_dtype;  /* ramnet_dtype of S and out (mass is always fp32) */
    int32_t cape;         /* CAPE (project page, CAPE paragraph, which leaves the exact
                           * shift open): 0 content-only addresses; at position P,
                           * 1 every digit advances by P mod d_p; 2 digit u advances
                           * by digit u of P in base d_p (no carry); 3 the slot index
                           * advances by P, wrapping over the M slots */
    float eps_gsu;        /* epsilon of the update rate; >= 0 (1e-6 typical) */
    float eps_norm;       /* epsilon of the RMSNorm; >= 0 (1e-6 typical) */
    uint64_t content_heads; /* bit h set: head h uses content-only addresses
                             * (the page mixes CAPE and content heads); heads
                             * 63 and above follow bit 63.  0: every head
                             * uses `cape`. */
} ramnet_params;

/* Sparse addresses, each [B,T,H,K] (a step: [B,H,K]).  Slots are post-CAPE
 * indices in [0, M).  Per address the K entries are ordered by weight
 * (heaviest first), equal weights by the smaller pre-CAPE slot index. */
typedef struct {
    int32_t *w_idx;   /* write slots (from the key) */
    float *w_wt;      /* write weights */
    int32_t *r_idx;   /* read slots (from the query) */
    float *r_wt;      /* read weights */
} ramnet_addr;

/* Address Decoder + CAPE only (steps 1-2 above).
 *   q, k  [B,T,H,U*d_p] in in_dtype: query and key logits.
 *   pos0  [B] int32 or NULL (= 0): position of token t is pos0[b] + t.
 *   out   all four arrays required.
 * The decision follows step 1's rule (fp64 logit sums); weights are
 * returned rounded to fp32.  The prefill decodes bf16 logits in exact
 * fixed point instead and takes the same decisions. */
ramnet_status ramnet_decode_addresses(const ramnet_params *p, const void *q,
                                      const void *k, const int32_t *pos0,
                                      const ramnet_addr *out, void *stream);

/* Bytes of workspace `op` needs for `p` (0 for an invalid p): enough for any
 * call with these parameters.  (A call that exports its addresses through
 * addr_out, or takes them from addr_in, needs less; the call reports
 * RAMNET_EWORKSPACE with the exact figure if given too little.) */
size_t ramnet_workspace_bytes(const ramnet_params *p, int32_t op);

/* Prefill (project page, GPU-execution paragraphs: addresses for all tokens
 * in parallel, then the recurrence in causal order): steps 1-4 for every
 * token of B sequences of T tokens, H heads each.
 *   q, k      [B,T,H,U*d_p] in_dtype      v, g   [B,T,H,d_v] in_dtype
 *   gamma     [B,T,H] in_dtype            norm_w [d_v] fp32 or NULL (= 1)
 *   pos0      [B] int32 or NULL (= 0)
 *   S         [B,H,M,d_v] state_dtype, in/out
 *   mass      [B,H,M] fp32, in/out
 *   out       [B,T,H,d_v] state_dtype
 *   addr_in   NULL: decode q, k.  Otherwise the addresses to use (post-CAPE
 *             slots and weights); q, k and pos0 are then ignored.  Slots must
 *             be distinct within an address; a slot outside [0, M) is
 *             skipped (treated as weight 0).
 *   addr_out  NULL, or where to export the addresses used.
 *   workspace ramnet_workspace_bytes(p, RAMNET_OP_PREFILL) bytes.  It holds
 *             the decoded addresses (unless addr_out is given), the
 *             decoder's per-wave fallback marks (K <= 32) and, on the
 *             slot-grouped path (T >= 32, M <= 2^22, K <= 63), the per-chunk
 *             slot-grouping plans, the un-normalised reads and per-token sums
 *             of squares (M <= 1024), or the per-range partial reads and
 *             spilled version rows (larger M).  Its contents on entry do not
 *             matter.
 * Results are deterministic: every sum is taken in a fixed order, so repeated
 * calls on the same inputs give the same bits. */
ramnet_status ramnet_scan_prefill(const ramnet_params *p, const void *q,
                                  const void *k, const void *v,
                                  const void *gamma, const void *g,
                                  const float *norm_w, const int32_t *pos0,
                                  void *S, float *mass, void *out,
                                  const ramnet_addr *addr_in,
                                  const ramnet_addr *addr_out, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * prefill as ramnet_scan_prefill, with the same arguments except that there
 * is no workspace.  Its scratch is a static device array of
 * RAMNET_NOALLOC_SCRATCH_BYTES bytes (64 MiB) that every GPU the library
 * runs on holds from when the library is loaded until the process ends; the
 * call itself allocates nothing (no hipMalloc, no allocating library call).
 *   - A prefill whose scratch need exceeds that size is refused with
 *     RAMNET_EWORKSPACE before anything is enqueued (the need is at most
 *     ramnet_workspace_bytes(p, RAMNET_OP_PREFILL); exporting addresses
 *     through addr_out, or giving addr_in, lowers it).
 *   - Every call on one GPU uses that GPU's one array, whose contents on
 *     entry do not matter.  Calls that may overlap in time on one GPU
 *     (other streams, other host threads) race on it: serialise them, e.g.
 *     on one stream.
 * Results are bit-identical to ramnet_scan_prefill's on the same inputs. */
#define RAMNET_NOALLOC_SCRATCH_BYTES (64u << 20)
ramnet_status ramnet_scan_prefill_noalloc(const ramnet_params *p, const void *q,
                                          const void *k, const void *v,
                                          const void *gamma, const void *g,
                                          const float *norm_w, const int32_t *pos0,
                                          void *S, float *mass, void *out,
                                          const ramnet_addr *addr_in,
                                          const ramnet_addr *addr_out, void *stream);

/* One decoding step (project page, decoding paragraph: the current token's
 * slots are accessed directly, without a pass over the state): steps 1-4
 * for one token of each of B sequences.  p->T must be 1.
 *   q, k [B,H,U*d_p]; v, g [B,H,d_v]; gamma [B,H] (in_dtype)
 *   pos  [B] int32: position of this token; required when p->cape != 0
 *   S, mass as for prefill; out [B,H,d_v] state_dtype
 *   addr_out NULL or [B,H,K] each. */
ramnet_status ramnet_step_decode(const ramnet_params *p, const void *q,
                                 const void *k, const void *v,
                                 const void *gamma, const void *g,
                                 const float *norm_w, const int32_t *pos,
                                 void *S, float *mass, void *out,
                                 const ramnet_addr *addr_out, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * A tiered slot state for decoding loops (AI Radio page, deployment remark:
 * the sparse access lets only the frequently accessed slots be cached in
 * VRAM, so the state need not fit the GPU's memory).  The rows live in
 * host memory; each (batch, head) unit caches at most C of them in device
 * memory.  The masses stay in device memory ([B,H,M] fp32, 1/16 to 1/128 of
 * the rows' bytes).  All buffers are the caller's:
 *   S_host     [B,H,M,d_v] state_dtype, pinned host memory that the device
 *              addresses at its host address (ramnet_host_alloc): the row of
 *              every slot that is
 *              not cached; a cached slot's row here is stale until
 *              ramnet_tier_flush
 *   cache      [B,H,C,d_v] state_dtype, device: the cached rows (line i of
 *              unit u holds the row of slot line_slot[u][i])
 *   line_slot  [B,H,C] int32, device: slot of each line, -1 for an empty line
 *   slot_line  [B,H,M] int32, device: line of each slot, -1 if not cached
 *   hits       [B,H,M] uint32, device: accesses (a token's write and read
 *              slots, after CAPE) since the last rebalance, halved by it
 *   C          lines per unit, 1 <= C <= min(M, RAMNET_TIER_CMAX)
 * The step gives bit-identical results to ramnet_step_decode on the same
 * state; only where the rows live differs.  Calls on one tiered state must
 * be ordered (one stream). */
#define RAMNET_TIER_CMAX 16384
typedef struct {
    void *S_host;
    void *cache;
    int32_t *line_slot;
    int32_t *slot_line;
    uint32_t *hits;
    int32_t C;
} ramnet_tiered_state;

/* Pinned host memory for S_host (hipHostMalloc, mapped and portable), whose
 * device address is checked to equal its host address; freed with
 * ramnet_host_free.  The only calls that allocate. */
ramnet_status ramnet_host_alloc(size_t bytes, void **ptr);
ramnet_status ramnet_host_free(void *ptr);

/* Empties the cache (every line empty, every slot uncached) and zeroes the
 * counts; S_host must then hold the whole state.  Rows are not moved. */
ramnet_status ramnet_tier_reset(const ramnet_params *p, const ramnet_tiered_state *ts,
                                void *stream);

/* One decoding step as ramnet_step_decode, the rows read and written where
 * they live (a cached slot in its line, any other in S_host, over the host
 * link), and each accessed slot's count raised.  No workspace.  Only the
 * fused step's shapes (K <= 32, d_p <= 8, d_v 64..256 as the step takes
 * them) are supported; RAMNET_EUNSUPPORTED otherwise. */
ramnet_status ramnet_step_decode_tiered(const ramnet_params *p, const void *q,
                                        const void *k, const void *v,
                                        const void *gamma, const void *g,
                                        const float *norm_w, const int32_t *pos,
                                        const ramnet_tiered_state *ts, float *mass,
                                        void *out, const ramnet_addr *addr_out,
                                        void *stream);

/* Re-chooses each unit's cached slots: the C slots with the highest key
 * 2 * hits + (1 if cached), the key capped at 255, ties to the smaller
 * slot, slots with key 0 never cached.  Rows leaving the cache are written
 * back to S_host; rows entering it are copied from S_host; slots that stay
 * keep their line; entering slots take the free lines in line order, in
 * slot order.  Then every count is halved. */
ramnet_status ramnet_tier_rebalance(const ramnet_params *p, const ramnet_tiered_state *ts,
                                    void *stream);

/* Writes every cached row back to S_host (the cache keeps it), so that
 * S_host alone holds the whole state. */
ramnet_status ramnet_tier_flush(const ramnet_params *p, const ramnet_tiered_state *ts,
                                void *stream);

/* Backward pass of a prefill (training; the project page's GPU-execution
 * paragraph treats training and prefill alike).  The pages give no backward
 * formulas: this is the exact derivative of steps 1-4 with the Top-K
 * selection held fixed (it is piecewise constant), the power-decay retention
 * differentiated exactly (the AI Radio page's proxy gradient is not defined
 * there and is not used), and each fp32 storage rounding passing its
 * gradient through.  The gradients are those of
 *   sum(out * dout) + sum(S_final * dS_final) + sum(mass_final * dmass_final)
 * with respect to the inputs and the state the forward started from.
 * Built for every d_v and M the forward takes, with U*d_p <= 64
 * (RAMNET_EUNSUPPORTED otherwise); the state may be fp32 or bf16 (the replay
 * rounds it as the forward does), the gradients are fp32.  d_v = 64 with
 * M <= 1024 keeps each slot's row and adjoint on chip; every other shape
 * walks slot ranges chunk by chunk with the replayed state in the workspace
 * and the adjoint accumulated in dS0 and dmass0 (which then start as
 * dS_final and dmass_final).  Both group each chunk's events by slot.  A
 * token may write one slot twice (caller-given addresses): the writes apply
 * in address order, as in the forward.
 *   q, k, v, gamma, g, norm_w, pos0   the forward's inputs (q, k only read
 *             when dq, dk are given)
 *   S0, mass0 [B,H,M,d_v] state_dtype, [B,H,M] fp32: the state before the
 *             forward
 *   addr      the forward's addresses (its addr_out), [B,T,H,K] each
 *   dout      [B,T,H,d_v] fp32; dS_final, dmass_final fp32 or NULL (= 0)
 *   dq, dk    [B,T,H,U*d_p] fp32 or NULL; dv, dg [B,T,H,d_v] fp32;
 *   dgamma    [B,T,H] fp32; dnorm_w [d_v] fp32 or NULL; dS0 [B,H,M,d_v]
 *             fp32, dmass0 [B,H,M] fp32
 *   workspace ramnet_workspace_bytes(p, RAMNET_OP_BACKWARD) bytes: the
 *             forward is replayed from S0 and, per token-head, each write's
 *             row and mass before it and each read's row are recorded
 *             ((2 K d_v + 3 K) fp32); the token walk adds a copy of S0 and
 *             mass0.
 * Every sum is taken in a fixed order: repeated calls give the same bits. */
ramnet_status ramnet_scan_backward(const ramnet_params *p, const void *q,
                                   const void *k, const void *v,
                                   const void *gamma, const void *g,
                                   const float *norm_w, const int32_t *pos0,
                                   const void *S0, const float *mass0,
                                   const ramnet_addr *addr, const float *dout,
                                   const float *dS_final,
                                   const float *dmass_final, float *dq,
                                   float *dk, float *dv, float *dgamma,
                                   float *dg, float *dnorm_w, float *dS0,
                                   float *dmass0, void *workspace,
                                   size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * A whole layer: the dense projections either side of the recurrence (RAM-Net
 * project page, layer outline: the token is projected to key, query and
 * value, the GSU's gamma comes from the token by a learned projection, and
 * the gated read is projected out), with the address weights re-parameterised
 * as W = e^alpha * W' per head (AI Radio page, stability of the decoder: alpha
 * sets the temperature of the Product Softmax).
 *
 * All weights are bf16, [out, in] row-major (one output's weights contiguous
 * over its inputs, as a linear layer y = x W^T stores them), d_model = D:
 *   w_q, w_k   [H*U*d_p, D]  W' of the query / key logits; row h*U*d_p + j
 *              gives logit j of head h.  The GEMM uses W = bf16(t_h * W'),
 *              with t_h = fp32(e^alpha[h]), rounded once from the exact
 *              product.
 *   w_v, w_g   [H*d_v, D]    values and output-gate logits (row h*d_v + c)
 *   w_gamma    [H, D]        the GSU's gamma, one per head
 *   w_o        [D, H*d_v]    output projection of the layer output
 *   alpha      [H] fp32 or NULL (= 0, W = W')
 *   w_in_packed  NULL, or the five input weights packed by
 *              ramnet_pack_weights (then w_q .. w_gamma and alpha are not
 *              read).  Packing once saves re-packing on every call, which
 *              matters for decoding steps.
 * The five input projections are one GEMM against the packed [N, D] matrix
 * (rows: q, k, v, g, gamma; each block starts at a multiple of 8 rows, zero
 * padding between); the layer reads its inputs in place from the packed
 * result [B*T, N].  Each product is accumulated in fp32 and rounded to bf16
 * (hipBLASLt on the matrix cores); the layer output is rounded to bf16
 * before w_o.  p->in_dtype must be RAMNET_BF16 (q, k, v, gamma, g are the
 * bf16 projections).
 * GEMM algorithms: by default hipBLASLt's first heuristic choice, so these
 * calls stay asynchronous and give the same bits in every process.  With
 * RAMNET_GEMM_TUNE=1 in the environment, the first call of each GEMM shape
 * in a process (outside graph capture) instead times up to 24 candidates on
 * its own operands and keeps the fastest: that call SYNCHRONISES THE HOST
 * with the stream, its bits can differ from another process's (a different
 * algorithm sums in another order), and a timing failure of the output GEMM
 * is reported after the recurrence has already been enqueued (S and mass
 * then hold the updated state).
 */
typedef struct {
    int32_t d_model;
    const void *w_q, *w_k, *w_v, *w_g, *w_gamma, *w_o;
    const float *alpha;
    const void *w_in_packed;
} ramnet_proj;

/* Bytes of the packed input weights for `p` and d_model (0 if invalid). */
size_t ramnet_packed_weights_bytes(const ramnet_params *p, int32_t d_model);

/* Packs w->w_q, w_k (as W = bf16(t_h * W')), w_v, w_g, w_gamma into
 * `packed` (ramnet_packed_weights_bytes bytes, bf16 [N, d_model]).  w->w_o
 * and w->w_in_packed are not read. */
ramnet_status ramnet_pack_weights(const ramnet_params *p, const ramnet_proj *w,
                                  void *packed, size_t packed_bytes,
                                  void *stream);

/* Workspace bytes of ramnet_layer_forward / ramnet_layer_step /
 * ramnet_project_inputs for `p` and d_model (0 if either is invalid). */
size_t ramnet_layer_workspace_bytes(const ramnet_params *p, int32_t d_model);

/* The five input projections of x [B,T,D] bf16 into q, k [B,T,H,U*d_p],
 * v, g [B,T,H,d_v] and gamma [B,T,H], all bf16, exactly as
 * ramnet_layer_forward computes them. */
ramnet_status ramnet_project_inputs(const ramnet_params *p, const ramnet_proj *w,
                                    const void *x, void *q, void *k, void *v,
                                    void *gamma, void *g, void *workspace,
                                    size_t workspace_bytes, void *stream);

/* Prefill of a whole layer: x [B,T,D] bf16 -> y [B,T,D] bf16.  Projections,
 * then ramnet_scan_prefill on them (norm_w, pos0, S, mass, addr_out as
 * there), then the output projection.  workspace:
 * ramnet_layer_workspace_bytes(p, D) bytes; it also holds the projected
 * inputs and the layer output. */
ramnet_status ramnet_layer_forward(const ramnet_params *p, const ramnet_proj *w,
                                   const void *x, const float *norm_w,
                                   const int32_t *pos0, void *S, float *mass,
                                   void *y, const ramnet_addr *addr_out,
                                   void *workspace, size_t workspace_bytes,
                                   void *stream);

/* One decoding step of a whole layer (p->T == 1): x [B,D] -> y [B,D], bf16,
 * through ramnet_step_decode (pos, S, mass, addr_out as there). */
ramnet_status ramnet_layer_step(const ramnet_params *p, const ramnet_proj *w,
                                const void *x, const float *norm_w,
                                const int32_t *pos, void *S, float *mass,
                                void *y, const ramnet_addr *addr_out,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

const char *ramnet_status_str(ramnet_status s);
const char *ramnet_last_error(void);
int32_t ramnet_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RAMNET_H */
