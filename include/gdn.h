/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet token-mixer library (libgdn.so).
 *
 * The operation (explainer page "論文解説: Qwen3.8-Next の設計", ta-paperlens.web.app,
 * section "GDNの中身: 足すのではなく、消してから書く", Eq. (1)): every head keeps a
 * matrix state S of dk x dv fp32 values that maps keys to values.  For each token t
 *
 *     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t                      (read from the updated state)
 *
 * alpha_t in (0,1] is the decay gate that scales the whole memory, passed in log space
 * as g_t = log(alpha_t) <= 0; beta_t in [0,1] is the write strength.  q and k are
 * expected to be L2-normalised by the caller (the library does not renormalise).
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, row-major (innermost index last), in device memory.
 *     Alignment: states 16 bytes; prefill q, k, v, o 16 bytes; beta, g and all decode
 *     inputs/outputs one element; the workspace 256 bytes.  B = batch, T = tokens,
 *     Hk = q/k heads, Hv = value heads, dk = key/query head size, dv = value head size.
 *   - Grouped heads: Hv must be a multiple of Hk; value head hv reads q/k head
 *     hv / (Hv/Hk) (groups of consecutive value heads share one q/k head).  beta and
 *     g are per value head.
 *   - The state layout is [B, Hv, dk, dv] fp32 (dv contiguous): S[b][hv][i][j] is the
 *     entry for key coordinate i and value coordinate j.
 *   - Ownership: the caller owns every buffer.  No call allocates device memory,
 *     keeps state between calls (apart from gdn_chunk_fwd_noalloc's static scratch), or
 *     synchronises the host; every call only enqueues kernels on `stream` (a hipStream_t;
 *     NULL = the null stream) and returns.
 *   - Errors: arguments are validated on the host before anything is enqueued; on an
 *     error nothing is launched and no output is touched.  Faults inside a kernel
 *     surface at the caller's next synchronisation of the stream.  NaN and Inf in the
 *     inputs propagate; they are not checked.
 *   - Results are deterministic: the same inputs, sizes and stream give bit-identical
 *     outputs (no floating-point atomics; the only atomics are integer counts in LDS).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 5

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1, /* null required pointer, negative size, misalignment, Hv % Hk != 0,
                                o aliasing an input, workspace too small */
    GDN_ERR_UNSUPPORTED = 2, /* valid but not implemented: head sizes, chunk size or dtype pair */
    GDN_ERR_HIP = 3,         /* the HIP runtime refused a launch */
    GDN_ERR_SCRATCH_TOO_SMALL = 4, /* gdn_chunk_fwd_noalloc: even one chunk per segment needs
                                      more workspace than its static scratch holds
                                      (GDN_NOALLOC_SCRATCH_BYTES) */
    GDN_STATUS_MAX_ = 0x7fffffff   /* not a status: makes every int a valid value in C++ */
} gdn_status_t;

typedef enum gdn_dtype {
    GDN_F32 = 0,
    GDN_BF16 = 1,
    GDN_DTYPE_MAX_ = 0x7fffffff    /* not a dtype: any int a caller passes is rejected, not UB */
} gdn_dtype_t;

/*
 * Input prologue flags (gdn_chunk_fwd_varlen, gdn_decode_tokens): the library applies these
 * to the inputs as it reads them, so no separate pass over q, k, beta, g is needed.
 *   GDN_QK_L2NORM   q and k are L2-normalised per token and head: x / max(||x||_2, 1e-6),
 *                   computed in fp32 from the stored values
 *   GDN_BETA_LOGIT  beta holds logits: beta = sigmoid(x)
 *   GDN_G_LOGIT     g holds logits of alpha: log alpha = log sigmoid(x) (instead of log alpha)
 */
#define GDN_QK_L2NORM 1u
#define GDN_BETA_LOGIT 2u
#define GDN_G_LOGIT 4u

/*
 * Plan hint (gdn_chunk_fwd_varlen and gdn_chunk_fwd_varlen_workspace_size only): run the
 * "split" plan whenever it takes the sizes (bf16 inputs, dk = dv in {64, 128}, chunk 32 or
 * 64), whatever the number of chains.  Meant for packed batches of very uneven lengths (one
 * long prompt among short ones): the single-pass kernel's time follows the longest sequence,
 * the split plan's the total number of chunks.  The host never reads the offsets, so the
 * library cannot tell such a batch from an even one by itself.  Results agree with the other
 * plans to the stated precision; the workspace size must be queried with the same flags.
 */
#define GDN_PREFER_SPLIT 8u

/* Returns GDN_ABI_VERSION of the built library. */
int gdn_abi_version(void);

/* Returns a static, human-readable name for a status code (never NULL). */
const char *gdn_status_string(gdn_status_t status);

/*
 * Bytes of device workspace gdn_chunk_fwd needs for these sizes (0 means none; pass
 * workspace = NULL then).  Returns 0 for sizes gdn_chunk_fwd would reject.  The "split" plan
 * keeps per-chunk records there for a segment of chunks: at most 2 GiB of them (or the
 * number of bytes the environment variable GDN_SPLIT_RECORD_BYTES gives), plus 256 B and one
 * fp32 state per chain.  Longer sequences run segment after segment, with the state carried
 * between them and the same results bit for bit, so the size stays bounded for any T.  The
 * "segmented" plan keeps three fp32 dk x dv matrices per (chain, segment) there: each
 * segment's transition M and state N (all but the last segment) and its entry state; with at
 * most 256 (chain, segment) units that is at most 48 MiB at dk = dv = 128, whatever T.  After
 * them it keeps every chunk's (I + A)^-1 (the unit-lower-triangular inverse of the chunk's
 * WY/UT transform) as fp16, its (chunk/16)(chunk/16 + 1)/2 lower 16 x 16 blocks of 512 B
 * (5 KiB at chunk 64), in ceil(rows / chunk) + B slots per value head (rows = B T, or T for
 * packed sequences): the transition pass stores it and the output pass reads it instead of
 * forming it again (320 MiB for 262,144 tokens x 16 heads).  Where those records would exceed
 * 2 GiB (beyond about 1.7 million tokens x 16 heads at chunk 64), or with the environment variable
 * GDN_SEG_NO_TM=1, both passes form it and the size is the maps' alone: the segmented plan's
 * workspace stays bounded for any T.
 */
size_t gdn_chunk_fwd_workspace_size(int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                                    gdn_dtype_t in_dtype);

/*
 * Which kernels gdn_chunk_fwd runs for these sizes: "fused" (one kernel per chain: 128 chains
 * or more), "segmented" (fewer, long chains: every chain cut into segments of at least 8 chunks,
 * at most 256 (chain, segment) units; a transition pass gives each segment's affine state map
 * S_out = M S_in + N -- Eq. (1) is affine in the state -- a combine pass chains the maps into
 * every segment's entry state in fp32, and the single-pass kernel then runs all segments from
 * their entry states), "split" (fewer, shorter chains: a prep kernel parallel over chunks,
 * whose per-chunk operands go through the workspace, then a state-scan kernel per chain and
 * 16-column state tile that also forms the outputs), "recurrent" (token by token; the fp32
 * path) or "invalid".  Packed sequences (gdn_chunk_fwd_varlen with offsets) run "segmented"
 * with every (sequence, head) chain in 256 / chains segments formed on the device from its own
 * length, when the mean sequence (T / num_seqs, since the host does not read the offsets)
 * gives segments of at least 8 chunks; GDN_PREFER_SPLIT keeps the split plan.  Static string.
 */
const char *gdn_chunk_fwd_plan(int B, int T, int Hk, int Hv, int dk, int dv, int chunk,
                               gdn_dtype_t in_dtype);

/*
 * Prefill: run Eq. (1) over T tokens for every (b, hv) chain, chunk by chunk.
 *
 *   q, k           [B, T, Hk, dk]  in_dtype     (read only; q may equal k)
 *   v              [B, T, Hv, dv]  in_dtype
 *   beta, g        [B, T, Hv]      in_dtype     beta in [0,1]; g = log(alpha) <= 0
 *   initial_state  [B, Hv, dk, dv] fp32, or NULL for a zero state
 *   o              [B, T, Hv, dv]  out_dtype    fully overwritten; must not overlap any input
 *   final_state    [B, Hv, dk, dv] fp32, or NULL to skip; may be the same pointer as
 *                  initial_state (updated in place); fully overwritten when given
 *   chunk          tokens per chunk of the chunk-parallel form: 16, 32 or 64 (the result
 *                  does not depend on it beyond rounding); T need not be a multiple
 *   scale          multiplies every output (1.0 for the plain rule)
 *   in_dtype       GDN_F32 or GDN_BF16;  out_dtype  GDN_F32 or GDN_BF16
 *   workspace      device buffer of at least gdn_chunk_fwd_workspace_size(...) bytes
 *
 * Supported: dk, dv in {16, 32, 64, 128}.  T = 0 writes final_state = initial_state
 * (or zeros) and nothing else.  B = 0 is a no-op.
 *
 * Precision: bf16 inputs run on the matrix cores with fp16 (or bf16) operands and fp32
 * accumulation.  q and k are taken as fp16 copies (exact for unit rows, whose entries are at
 * most 1 in magnitude; rows far from unit norm with entries beyond fp16 range are outside the
 * method's use and would overflow).  Derived operands (U, W, the state S, Delta, P) are
 * rounded to fp16 for each product; every sum and the fp32 state itself are never rounded.
 * The value side (v, U, Delta, S, o) is linear in (v, initial_state), so its fp16 copies carry
 * a power of two, chosen per chunk and taken back out of the fp32 results exactly: v and the
 * state may have any magnitude that fp32 holds, and scaling v and initial_state by 2^n scales
 * o and final_state by exactly 2^n.  The single-pass and segmented plans take the scale of
 * each value column (and of each column of a segment's transition M) from its largest
 * magnitude in the chunk, and the segmented plan chains its segments in fp32; the split plan
 * takes one scale per 16 value columns from a bound on the state's column norms that holds
 * for keys of norm at most 1 (beta |k|^2 <= 2; unit keys rounded to bf16 qualify), so keys
 * far above unit norm may overflow there -- pass GDN_QK_L2NORM (gdn_chunk_fwd_varlen) when the
 * keys are not normalised.  fp32 inputs run the token-recurrent kernel in fp32.
 */
gdn_status_t gdn_chunk_fwd(const void *q, const void *k, const void *v, const void *beta,
                           const void *g, const float *initial_state, void *o,
                           float *final_state, int B, int T, int Hk, int Hv, int dk, int dv,
                           int chunk, float scale, gdn_dtype_t in_dtype, gdn_dtype_t out_dtype,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_chunk_fwd for callers that cannot allocate device memory -- code being captured into a
 * HIP graph, tight serving loops, harnesses that forbid hipMalloc: the same arguments without
 * the workspace, the same plan, and the same results bit for bit wherever the plan's whole
 * workspace fits the scratch.  Where the plan needs a
 * workspace (gdn_chunk_fwd_workspace_size(...) > 0) it uses a static scratch buffer of
 * GDN_NOALLOC_SCRATCH_BYTES that the library holds in every GPU's memory from its load until
 * the process ends; the call itself allocates nothing (no hipMalloc, no allocating library
 * routine).  The segmented plan's maps and entry states always fit the scratch; where its
 * per-chunk (I + A)^-1 records do not fit beside them, both of its passes form that inverse
 * instead (results to the same precision bar, not the same bits).  The split
 * plan runs in segments of as many chunks as the scratch holds
 * (about 1,000 chunk-heads at dk = dv = 128 and chunk 64, e.g. 64 chunks of 16 heads): the
 * same results, bit for bit, at any T, and slower than one pass for long sequences.  A size
 * whose smallest workspace (one chunk per segment) exceeded GDN_NOALLOC_SCRATCH_BYTES would
 * return GDN_ERR_SCRATCH_TOO_SMALL before anything is launched; no size the plans take comes
 * near it.  Every call on one GPU shares that GPU's scratch and leaves its contents behind:
 * calls that can run at the same time on one GPU (different streams without ordering between
 * them, or different host threads) race and must be serialised by the caller.  The first
 * call on each device looks up the scratch's device address once (hipGetSymbolAddress, with
 * that device current), under a lock.
 */
#define GDN_NOALLOC_SCRATCH_BYTES (80ull << 20)
gdn_status_t gdn_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const void *beta,
                                   const void *g, const float *initial_state, void *o,
                                   float *final_state, int B, int T, int Hk, int Hv, int dk,
                                   int dv, int chunk, float scale, gdn_dtype_t in_dtype,
                                   gdn_dtype_t out_dtype, void *stream);

/*
 * Decode: apply one token of Eq. (1) to every state in place and read it out.
 *
 *   q, k      [B, Hk, dk]      in_dtype
 *   v         [B, Hv, dv]      in_dtype
 *   beta, g   [B, Hv]          in_dtype
 *   state     [B, Hv, dk, dv]  fp32, read and overwritten with the updated state
 *   o         [B, Hv, dv]      out_dtype, o = scale * S_new^T q; must not overlap any input
 *
 * Each state is read once and written once (a streaming, memory-bound update).
 * Supported: dk, dv in {16, 32, 64, 128}.  B = 0 is a no-op.
 */
gdn_status_t gdn_decode_step(const void *q, const void *k, const void *v, const void *beta,
                             const void *g, float *state, void *o, int B, int Hk, int Hv,
                             int dk, int dv, float scale, gdn_dtype_t in_dtype,
                             gdn_dtype_t out_dtype, void *stream);

/*
 * Decode several tokens per sequence in one pass over the state: apply T consecutive tokens
 * of Eq. (1) to every state and read out every one of them, e.g. T drafted tokens being
 * verified (multi-token prediction) or a short continuation.  Each state is read once and
 * written once for all T tokens; T = 1 is gdn_decode_step.
 *
 *   q, k       [B, T, Hk, dk]   in_dtype     token t of sequence b at row b*T + t
 *   v          [B, T, Hv, dv]   in_dtype
 *   beta, g    [B, T, Hv]       in_dtype
 *   state_in   [B, Hv, dk, dv]  fp32, the state before the T tokens, or NULL for zeros
 *   state_out  [B, Hv, dk, dv]  fp32, written with the state after the T tokens; either the
 *                               same pointer as state_in (update in place) or not
 *                               overlapping it.  Keeping state_in intact lets a verifier that
 *                               accepts only the first m < T tokens re-apply those m.
 *   o          [B, T, Hv, dv]   out_dtype, o_t = scale * S_t^T q_t; must not overlap any
 *                               input or either state
 *
 * T = 0 copies state_in (or zeros) to state_out and touches nothing else.  Any T >= 0 is
 * accepted.  Up to T = 4 (and for fp32 inputs, dk != dv, head sizes other than 64 and 128,
 * or q, k, v not 16-byte aligned) the tokens are applied one after the other in fp32, exactly
 * the arithmetic of T gdn_decode_step calls.  From T = 5 on, bf16 inputs with dk = dv in
 * {64, 128} take the chunk form of Eq. (1) over chunks of up to 16 tokens: products with the
 * state on the matrix cores from fp16 copies (power-of-two scaled per column, so v and the
 * state may have any magnitude; |q|, |k| < 65504), the state itself updated in fp32; the
 * precision is that of the bf16 chunk-parallel prefill.  Long runs still belong to
 * gdn_chunk_fwd.
 * flags: the input prologue (GDN_QK_L2NORM | GDN_BETA_LOGIT | GDN_G_LOGIT, or 0).
 * Supported: dk, dv in {16, 32, 64, 128}.  B = 0 is a no-op.
 */
gdn_status_t gdn_decode_tokens(const void *q, const void *k, const void *v, const void *beta,
                               const void *g, const float *state_in, float *state_out, void *o,
                               int B, int T, int Hk, int Hv, int dk, int dv, float scale,
                               unsigned flags, gdn_dtype_t in_dtype, gdn_dtype_t out_dtype,
                               void *stream);

/*
 * Prefill with the input prologue and, optionally, packed sequences of different lengths
 * (the serving layout: one tensor of all the batch's tokens, no padding).
 *
 *   cu_seqlens   NULL: dense batches, exactly as gdn_chunk_fwd with B = num_seqs and T
 *                tokens per sequence.
 *                Otherwise DEVICE memory, num_seqs + 1 int32 offsets, nondecreasing, from 0
 *                to T: sequence i is rows cu_seqlens[i] .. cu_seqlens[i+1]-1 of
 *                  q, k       [T, Hk, dk]  in_dtype
 *                  v          [T, Hv, dv]  in_dtype
 *                  beta, g    [T, Hv]      in_dtype
 *                  o          [T, Hv, dv]  out_dtype
 *                and has its own state: initial_state / final_state [num_seqs, Hv, dk, dv]
 *                fp32.  Chunks never cross a sequence boundary; a sequence of length 0 gets
 *                final = initial.  The offsets are not read on the host: offsets outside
 *                [0, T] or decreasing are clamped on the device (wrong results for the
 *                sequences concerned, but no access outside the tensors or the workspace).
 *   flags        GDN_QK_L2NORM | GDN_BETA_LOGIT | GDN_G_LOGIT | GDN_PREFER_SPLIT (or 0);
 *                other bits are invalid
 *
 * Every other argument, alignment rule and error is as for gdn_chunk_fwd.  Packed sequences
 * run the plan that gdn_chunk_fwd_plan names for B = num_seqs and the same T (the total),
 * or "split" with GDN_PREFER_SPLIT where it takes the sizes:
 * "split" for few (sequence, head) chains -- its workspace holds one record per chunk
 * plus at most one unused record per sequence and head -- else "fused", or "recurrent" for
 * fp32 inputs and head sizes the chunked kernels do not take.
 */
gdn_status_t gdn_chunk_fwd_varlen(const void *q, const void *k, const void *v, const void *beta,
                                  const void *g, const float *initial_state, void *o,
                                  float *final_state, const int32_t *cu_seqlens, int num_seqs,
                                  int T, int Hk, int Hv, int dk, int dv, int chunk, float scale,
                                  unsigned flags, gdn_dtype_t in_dtype, gdn_dtype_t out_dtype,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Workspace bytes of gdn_chunk_fwd_varlen (0 means none): packed != 0 for cu_seqlens != NULL;
 * flags: those of the call (only GDN_PREFER_SPLIT changes the size).  The packed size depends
 * on num_seqs and the total T only, not on the offsets.
 */
size_t gdn_chunk_fwd_varlen_workspace_size(int num_seqs, int T, int Hk, int Hv, int dk, int dv,
                                           int chunk, gdn_dtype_t in_dtype, int packed,
                                           unsigned flags);

/*
 * Backward: the gradients of Eq. (1) over T tokens for every (b, hv) chain (training).
 * Inputs are the forward inputs of gdn_chunk_fwd (already in the form the recurrence takes:
 * unit q/k, beta, g = log alpha; the input prologue is not differentiated here) plus
 *   d_o            [B, T, Hv, dv]   dout_dtype   gradient of the outputs o
 *   d_final_state  [B, Hv, dk, dv]  fp32, gradient of the final state, or NULL for zero
 * and it writes, all fp32, fully overwritten:
 *   dq, dk         [B, T, Hk, dk]   (a q/k head's gradient sums over its Hv/Hk value heads)
 *   dv             [B, T, Hv, dv]
 *   dbeta, dg      [B, T, Hv]       (dg: gradient w.r.t. g = log alpha)
 *   d_initial_state [B, Hv, dk, dv] or NULL to skip
 * Outputs must not overlap each other or any input.  The workspace (at least
 * gdn_backward_workspace_size(...) bytes, 256-byte aligned) holds the intermediate results:
 * for dk, dv in {64, 128} with 16-byte-aligned q, k, v and d_o, the chunk-parallel path's
 * per-chunk records, chunk-start states and chunk-end gradients; otherwise the token-recurrent
 * path's state checkpoints every 64 tokens, one block of recomputed states per chain and the
 * per-slice parts of dq, dk, dbeta and dg.  Supported: dk, dv in {16, 32, 64, 128}; in_dtype
 * and dout_dtype GDN_F32 or GDN_BF16.  Deterministic (no atomics).  B = 0 is a no-op.
 * Precision: fp32 inputs compute in fp32 throughout.  bf16 inputs on the chunk-parallel path
 * keep the per-chunk records in fp16 and take fp16 operands with fp32 accumulation on the
 * matrix cores (values must lie within fp16 range); the states, e^gamma_last and every sum
 * stay fp32.
 */
size_t gdn_backward_workspace_size(int B, int T, int Hk, int Hv, int dk, int dv);
gdn_status_t gdn_backward(const void *q, const void *k, const void *v, const void *beta,
                          const void *g, const float *initial_state, const void *d_o,
                          const float *d_final_state, float *dq, float *dk, float *dv,
                          float *dbeta, float *dg, float *d_initial_state, int B, int T, int Hk,
                          int Hv, int dk_dim, int dv_dim, float scale, gdn_dtype_t in_dtype,
                          gdn_dtype_t dout_dtype, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * QSA compressed indexer (explainer page "論文解説: Qwen3.8-Next の設計", section "部品②: QSA"):
 * for every query token, the key blocks its sparse attention keeps.  The indexer is
 * multi-query attention with Hq = 4 query heads over one shared key head.  Keys are averaged
 * over blocks of r tokens before the position encoding, and each block is rotated at the
 * position of its first token; scoring then costs one product per (query, block) instead of
 * per (query, key).
 *
 *   q            [B, T, 4, d]   in_dtype   indexer queries (query at position t = row t)
 *   k            [B, T, d]      in_dtype   indexer keys
 *   sel          [B, T, nsel]   int32 out  kept block indices of each query, ascending, padded
 *                                          with -1 when fewer than nsel blocks are eligible;
 *                                          block j stands for tokens j*r .. min((j+1)r, T)-1
 *   importance   [B, T, nb]     fp32 out   (nb = ceil(T/r)) the importance of every block for
 *                                          every query, 0 where not eligible; NULL to skip
 *   r            tokens per block (the compression rate; 4 on the page)
 *   nsel         blocks kept per query (the token budget / r; 2048 / 4 = 512 on the page)
 *   rope_dims    leading dimensions rotated (rotate-half pairs (i, i + rope_dims/2), angle
 *                pos * rope_base^(-2i/rope_dims)); 0..d, even (64 of 128 on the page)
 *   scale        score scale (1/sqrt(d) for the usual attention temperature)
 *
 * Block j is eligible for the query at t when all its tokens are at or before t (the block
 * still being filled is not scored).  Its importance is the sum over the 4 heads of the
 * softmax over the eligible blocks of scale * rope(q_{t,h}, t) . rope(mean(k in j), j*r).
 * The kept blocks are the nsel most important eligible ones, ties to the lower index.  The
 * scores are computed from fp16 copies of the rotated queries and pooled keys (power-of-two
 * scaled per row and per batch, so no range is lost) with fp32 accumulation; the selection is
 * exact for the fp32 importance values this produces.
 *
 * Supported: Hq = 4; d in {64, 128}; in_dtype GDN_F32 or GDN_BF16.  The workspace (at least
 * gdn_qsa_workspace_size(...) bytes, 256-byte aligned) holds the fp16 queries and pooled keys.
 * Outputs must not overlap the inputs, each other or the workspace.  B = 0 or T = 0 is a
 * no-op.  Deterministic.
 */
size_t gdn_qsa_workspace_size(int B, int T, int Hq, int d, int r);
gdn_status_t gdn_qsa_index(const void *q, const void *k, int32_t *sel, float *importance, int B,
                           int T, int Hq, int d, int r, int nsel, int rope_dims, float rope_base,
                           float scale, gdn_dtype_t in_dtype, void *workspace,
                           size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
