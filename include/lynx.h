/*
 * lynx.h — C ABI of liblynx: the Lynx split-stream KV codec and anchor-only
 * decode attention, hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [Review] "Lynx: Progressive Speculative KV Cache Transfer for Disaggregated
 *            LLM Inference" (technical review of arXiv 2607.01831).
 *   [Digest] "Lynx: Progressive Speculative Quantization for accelerating KV
 *            Transfer in Long-Context Inference" (paper digest), Method.
 *
 * Conventions for every entry point
 *   - Pointers named *_dev are device pointers (hipMalloc'd or torch CUDA
 *     tensors), owned by the caller, 16-byte aligned.  The library allocates no
 *     device memory and is re-entrant; its only state is the per-GPU partial-result
 *     buffer of lynx_attn_anchor_noalloc (a static device array, and its address per
 *     GPU once looked up).  lynx_encode_to_host creates and destroys four HIP events
 *     per call to order its two streams.
 *   - `hip_stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *     enqueued asynchronously on it; the host is never synchronised.  Calls on
 *     different streams may run at once (give each its own output buffers): many
 *     small calls, such as one per layer tensor, keep the GPU fuller when they
 *     alternate over two streams than when they queue on one.
 *   - Argument errors are detected on the host and returned BEFORE anything
 *     is launched; nothing is written in that case.  A failed launch returns
 *     LYNX_ELAUNCH.  No C++ exception crosses this boundary.
 *   - KV input must be finite BF16.  NaN/Inf inputs give unspecified codes.
 *
 * KV page and channel
 *   A page is `page_tokens` (P) consecutive tokens of one KV tensor, stored
 *   token-major as BF16 [P][kv_heads][head_dim] ([Review] Mechanism 1: the
 *   page block X in R^{H x P}).  A channel is one (kv_head, head_dim) pair,
 *   H = kv_heads*head_dim channels per page; channel index c = h*head_dim + d.
 *   Per-channel statistics run over the page's tokens; chunk k covers tokens
 *   k*C .. k*C+C-1 ([Review] Mechanism 1, Stage 2).  K and V are encoded
 *   identically.
 *
 * Stream layout (per page; pages are contiguous and page-major)
 *   anchor segment  = [anchor nibbles : P*H/2 bytes]
 *                     [gamma_min   : float32[H]]
 *                     [gamma_scale : float32[H]]
 *                     [mu          : float32[P/C][H]]
 *                     [sigma       : float32[P/C][H]]
 *   residual segment = [residual nibbles : P*H/2 bytes]
 *   Anchor codes and their metadata are contiguous so one copy moves the whole
 *   high-priority stream ([Review] Mechanism 2, prefill-side workflow).  Codes
 *   are ordered [kv_head][channel block][token][channel in block] inside a page,
 *   the 128 channels of a head split into two blocks of 64 (so a code row is 32
 *   bytes: element (t, h, d) is nibble ((h*2 + d/64)*P + t)*64 + d%64 of the
 *   stream); two 4-bit codes share a byte, the even element in the low nibble
 *   ([Review] Implementation Notes).
 *   A 4-bit code q in [-8, 7] is stored as the nibble q & 0xF.
 *   Metadata count = H*(2 + 2P/C) float32 scalars ([Review] Deep Dive).
 *
 * Readings of the pages this ABI implements (where the pages are silent or
 * inconsistent):
 *   eps = 1e-6 in both normalisation stages; metadata stored as float32 and the
 *   stored values used by every later stage; sigma = max |X_n - mu| over the
 *   chunk; sign S taken from X_final (S(0) = +1); Round = nearest-even;
 *   Stage 4 with the +7 bias applied at reconstruction:
 *     V_mag = I >> 4, V_recon = 16*V_mag + 7, V_res = V_recon - I in [-8, 7],
 *     Q_anc = V_mag*S + min(S, 0) in [-8, 7] (Eq. 9), Q_res = V_res;
 *   anchor-only decode uses I = 16*V_mag + 7, full decode I = V_recon - V_res.
 */
#ifndef LYNX_H
#define LYNX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define LYNX_OK            0
#define LYNX_EINVAL       -1   /* bad size, count, chunk, alpha, selector or dtype */
#define LYNX_EALIGN       -2   /* a pointer is NULL where data is required, or misaligned (16 bytes for
                                   data buffers, 4 bytes for block tables and length arrays) */
#define LYNX_EUNSUPPORTED -3   /* a valid shape this library does not implement (e.g. head_dim != 128) */
#define LYNX_ENOSPACE     -4   /* workspace or staging buffer smaller than its *_bytes() query */
#define LYNX_ELAUNCH      -5   /* the HIP runtime rejected a kernel launch */

/* ---- selectors ---------------------------------------------------------- */
#define LYNX_SEL_ANCHOR   1u   /* encode: write the anchor segments (codes + metadata); required */
#define LYNX_SEL_RESIDUAL 2u   /* encode: also write the residual segments */
#define LYNX_OUT_BF16     0    /* decoders / attention: BF16 output, round to nearest even */
#define LYNX_OUT_F32      1    /* decoders / attention: float32 output */

/* Human-readable text for a status code (static storage; never NULL). */
const char* lynx_strerror(int status);

/*
 * Bytes of one page's anchor segment (P*H/2 + 4*H*(2 + 2P/C)) and residual
 * segment (P*H/2).  Pure host arithmetic.  Returns LYNX_EINVAL for
 * non-positive sizes, P % C != 0, or odd P*H.
 */
int lynx_stream_sizes(int page_tokens, int kv_heads, int head_dim, int chunk,
                      size_t* anchor_seg_bytes, size_t* residual_seg_bytes);

/*
 * Encode ([Review] Mechanism 1, Algorithm 1, Stages 1-4; [Digest] Method 1-4).
 *   kv_dev      : BF16 [n_pages*P][kv_heads][head_dim], read only.
 *   n_pages     : >= 0; 0 is a no-op returning LYNX_OK.
 *   page_tokens : P, a multiple of `chunk`.
 *   chunk       : C, a power of two in [8, 256] dividing P.
 *   alpha       : finite, > 0 (alpha-law parameter of Eq. 7).
 *   sel         : LYNX_SEL_ANCHOR, optionally | LYNX_SEL_RESIDUAL.
 *   anchor_dev  : n_pages anchor segments (see lynx_stream_sizes), written.
 *   residual_dev: n_pages residual segments, written when selected (may be
 *                 NULL otherwise).
 * Per element: X_n = (X - gamma_min)/(gamma_scale + eps);
 * X_f = (X_n - mu)/(sigma + eps); Y = 127*ln(1 + alpha|X_f|)/ln(1 + alpha);
 * I = Round(Y); S = sign(X_f); then the split above.
 * Pages longer than 256 tokens are encoded by three launches on the stream (the
 * page extremes per 256-token tile, gamma, then the tiles); until they have run,
 * the anchor segments' mu / sigma rows hold intermediate values.
 * Supported by this library: head_dim == 128 (else LYNX_EUNSUPPORTED).
 */
int lynx_encode(const void* kv_dev, int n_pages, int page_tokens, int kv_heads, int head_dim,
                int chunk, float alpha, unsigned sel, void* anchor_dev, void* residual_dev,
                void* hip_stream);

/*
 * Anchor-only decode: Q_approx = dequant(Q_anc, gamma, mu, sigma)
 * ([Review] Mechanism 2, decode-side anchor phase; Eq. 8 and the worked
 * example's anchor-only reconstruction, Eq. 14).
 *   anchor_dev : n_pages anchor segments, read only.
 *   out_dtype  : LYNX_OUT_BF16 or LYNX_OUT_F32.
 *   out_dev    : [n_pages*P][kv_heads][head_dim] of out_dtype, written.
 * x_hat = ((S*|x|)*(sigma + eps) + mu)*(gamma_scale + eps) + gamma_min with
 * |x| = ((1 + alpha)^(I/127) - 1)/alpha and I = 16*V_mag + 7.
 * Other arguments and errors as lynx_encode.
 */
int lynx_decode_anchor(const void* anchor_dev, int n_pages, int page_tokens, int kv_heads,
                       int head_dim, int chunk, float alpha, int out_dtype, void* out_dev,
                       void* hip_stream);

/*
 * Full decode from Anchor + Residual: Q_full = dequant(Q_anc + Q_res)
 * ([Review] Mechanism 2, decode-side residual phase; worked example, Eq. 15):
 * the exact 7-bit code I = V_recon - V_res, then as lynx_decode_anchor.
 *   residual_dev : n_pages residual segments, read only.
 */
int lynx_decode_full(const void* anchor_dev, const void* residual_dev, int n_pages,
                     int page_tokens, int kv_heads, int head_dim, int chunk, float alpha,
                     int out_dtype, void* out_dev, void* hip_stream);

/*
 * Workspace bytes lynx_attn_anchor needs for the given shape (split-context
 * partial results); 0 for shapes it would reject.
 */
size_t lynx_attn_workspace_bytes(int batch, int ctx_tokens, int q_heads, int kv_heads,
                                 int head_dim, int page_tokens, int chunk);

/*
 * Single-token decode attention over anchor-only codes, the speculative draft
 * path ([Review] Prerequisites §1, Eq. 1 evaluated on Q_approx of Mechanism 2),
 * fused with the anchor decode: O = softmax(q K^T * sm_scale) V where K and V
 * are the anchor-only reconstructions of the given segments.
 *   q_dev        : BF16 [batch][q_heads][head_dim].
 *   k_anchor_dev, v_anchor_dev : anchor segments; sequence b's context is the
 *                  ctx_tokens/page_tokens consecutive segments starting at
 *                  segment b*(ctx_tokens/page_tokens), with kv_heads heads.
 *   q_heads      : a multiple of kv_heads; query head hq reads kv head
 *                  hq / (q_heads/kv_heads).  Group size q_heads/kv_heads <= 16
 *                  (else LYNX_EUNSUPPORTED).
 *   ctx_tokens   : a positive multiple of page_tokens.
 *   chunk        : a multiple of 64; or 32; or 16 with page_tokens a multiple of 64;
 *                  or 8 with page_tokens a multiple of 32 (else LYNX_EUNSUPPORTED).
 *                  A wave step covers a 64-token tile (one chunk of 64 or more, or two
 *                  / four chunks of 32 / 16), or a 32-token tile (one chunk of 32 in
 *                  pages of an odd number of chunks, or four chunks of 8).
 *   sm_scale     : > 0, or <= 0 to use 1/sqrt(head_dim).
 *   workspace_dev, ws_bytes : at least lynx_attn_workspace_bytes(...) bytes.
 *   out_dtype    : LYNX_OUT_BF16 or LYNX_OUT_F32.
 *   out_dev      : [batch][q_heads][head_dim] of out_dtype, written.
 * Supported by this library: head_dim == 128.
 * Range: the key map folded into the query is carried in float16 with a power-of-two
 * exponent chosen per tile, so keys of any BF16 range are scored correctly; the scores
 * themselves (q . k * sm_scale) and the output must be finite in float32.
 */
int lynx_attn_anchor(const void* q_dev, const void* k_anchor_dev, const void* v_anchor_dev,
                     int batch, int ctx_tokens, int q_heads, int kv_heads, int head_dim,
                     int page_tokens, int chunk, float alpha, float sm_scale,
                     void* workspace_dev, size_t ws_bytes, int out_dtype, void* out_dev,
                     void* hip_stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): lynx_attn_anchor without a workspace argument.  Its
 * split-context partial results go to a library-owned device buffer of LYNX_ATTN_SCRATCH_BYTES,
 * one per GPU, held from the library's first use on that GPU until the process ends; the call
 * allocates and frees nothing (the buffer's device address is looked up once per GPU, on the
 * first call made with that GPU current).
 *   Arguments and results as lynx_attn_anchor, without workspace_dev / ws_bytes.
 *   Errors: those of lynx_attn_anchor; LYNX_ENOSPACE when the shape needs more than
 *   LYNX_ATTN_SCRATCH_BYTES of partial results (lynx_attn_workspace_bytes(...) says how much);
 *   LYNX_ELAUNCH when the buffer's address cannot be obtained.
 *   Calls that overlap on one GPU (different streams, or different host threads) share the
 *   buffer and race: order them on one stream.
 */
#define LYNX_ATTN_SCRATCH_BYTES (32u << 20)
int lynx_attn_anchor_noalloc(const void* q_dev, const void* k_anchor_dev, const void* v_anchor_dev,
                             int batch, int ctx_tokens, int q_heads, int kv_heads, int head_dim,
                             int page_tokens, int chunk, float alpha, float sm_scale, int out_dtype,
                             void* out_dev, void* hip_stream);

/*
 * Staging bytes lynx_encode_to_host needs for groups of group_pages pages: two groups'
 * anchor + residual segments.  0 for an invalid geometry.
 */
size_t lynx_encode_to_host_staging_bytes(int group_pages, int page_tokens, int kv_heads, int head_dim, int chunk);

/*
 * Encode a request page group by page group and copy each group's streams to host memory
 * while the next group is encoded ([Review] Implementation Notes: ping-pong double
 * buffering, quantisation of one buffer while the other is transferred; Mechanism 2:
 * the anchor stream is sent ahead of the residual stream).
 *   kv_dev        : BF16 [n_pages * page_tokens][kv_heads][head_dim], as for lynx_encode.
 *   group_pages   : pages per group (> 0); the last group may be shorter.
 *   staging_dev   : device buffer of at least lynx_encode_to_host_staging_bytes(min(group_pages,
 *                   n_pages), ...) bytes, 16-byte aligned; the two group buffers alternate.
 *   anchor_host   : n_pages anchor segments, written in page order; residual_host likewise.
 *                   Page-locked (pinned) host memory makes the copies asynchronous.
 *   compute_stream: encodes run here; copy_stream: the copies (anchor segments of a group,
 *                   then its residual segments) run here, each group after its encode.
 *                   The two may be the same stream (no overlap).
 * Asynchronous: the host buffers are complete once copy_stream's work so far has finished.
 * The first encodes wait for the work already queued on copy_stream, so back-to-back calls
 * may share one staging buffer.  Measured on ROCm 7 with 16 groups per call: queueing
 * several calls ahead without waiting for copy_stream slowed the copies down up to ~4x;
 * waiting between requests keeps them at the copy engine's rate.
 * Errors: those of lynx_encode (checked once for the whole request); LYNX_EINVAL for
 * group_pages <= 0 or a null host pointer; LYNX_EALIGN; LYNX_ENOSPACE for a small staging
 * buffer; LYNX_ELAUNCH if a HIP call fails (work already enqueued stays enqueued).
 */
int lynx_encode_to_host(const void* kv_dev, int n_pages, int page_tokens, int kv_heads, int head_dim, int chunk,
                        float alpha, int group_pages, void* staging_dev, size_t staging_bytes, void* anchor_host,
                        void* residual_host, void* compute_stream, void* copy_stream);

/*
 * lynx_attn_anchor over a paged cache with per-sequence lengths (the paged-attention
 * block layout of the serving engines the pages integrate with, [Review] Implementation
 * Notes: KV page granularity of 256 tokens as in paged attention).
 *   k_anchor_pool_dev, v_anchor_pool_dev : n_pool_pages anchor segments each (one page of
 *                  page_tokens tokens per segment, as lynx_encode writes them).
 *   block_table_dev : int32 [batch][max_pages_per_seq], device; entry (b, p) is the pool
 *                  segment holding page p of sequence b.  Entries past a sequence's last
 *                  page are not read; an entry outside [0, n_pool_pages) is clamped into it
 *                  (no out-of-range access; the result for that sequence is then unspecified).
 *   seq_lens_dev : int32 [batch], device; sequence b attends to its first seq_lens[b] tokens
 *                  (clamped into [0, max_pages_per_seq * page_tokens]); the tail of its last
 *                  page is masked.  A zero length gives an output of 0.
 * The other arguments are those of lynx_attn_anchor, with ctx_tokens replaced by
 * max_pages_per_seq * page_tokens; the workspace size is
 * lynx_attn_workspace_bytes(batch, max_pages_per_seq * page_tokens, ...).
 * Errors: those of lynx_attn_anchor; LYNX_EINVAL for n_pool_pages or max_pages_per_seq <= 0;
 * LYNX_EALIGN for a null or misaligned block_table_dev / seq_lens_dev.
 */
int lynx_attn_anchor_paged(const void* q_dev, const void* k_anchor_pool_dev, const void* v_anchor_pool_dev,
                           int n_pool_pages, const int32_t* block_table_dev, const int32_t* seq_lens_dev, int batch,
                           int max_pages_per_seq, int q_heads, int kv_heads, int head_dim, int page_tokens,
                           int chunk, float alpha, float sm_scale, void* workspace_dev, size_t ws_bytes,
                           int out_dtype, void* out_dev, void* hip_stream);

/*
 * Bytes of workspace lynx_attn_verify needs for this shape, or 0 if the shape is
 * not supported (see lynx_attn_verify).
 */
size_t lynx_attn_verify_workspace_bytes(int batch, int n_query, int ctx_tokens, int q_heads,
                                        int kv_heads, int head_dim, int page_tokens, int chunk);

/*
 * The verification pass over full codes ([Review] Mechanism 3, single parallel
 * verification pass; Mechanism 2, residual phase; Eq. 1): each of the n_query draft
 * tokens of a sequence attends, per query head, to the sequence's ctx_tokens context
 * tokens, whose K and V are the full (anchor + residual) reconstruction:
 *   O[b,m,hq] = softmax(q[b,m,hq] K^T * sm_scale) V,  lse[b,m,hq] = log(sum_t exp(s_t)).
 * The draft tokens' own keys and values are not in the compressed cache: a caller
 * merges O with the attention over them through lse (natural logarithm).
 *   q_dev        : BF16 [batch][n_query][q_heads][head_dim].
 *   k_anchor_dev, k_residual_dev, v_anchor_dev, v_residual_dev : anchor and residual
 *                  segments; sequence b's context is the ctx_tokens/page_tokens
 *                  consecutive segments starting at segment b*(ctx_tokens/page_tokens).
 *   q_heads      : a multiple of kv_heads (query head hq reads kv head hq / (q_heads/kv_heads)).
 *   chunk        : a multiple of 64, or 32 or 16 with page_tokens a multiple of 64, in this
 *                  library (else LYNX_EUNSUPPORTED).
 *   sm_scale     : > 0, or <= 0 to use 1/sqrt(head_dim).
 *   workspace_dev, ws_bytes : at least lynx_attn_verify_workspace_bytes(...) bytes.
 *   out_dtype    : LYNX_OUT_BF16 or LYNX_OUT_F32; out_dev [batch][n_query][q_heads][head_dim].
 *   lse_dev      : float32 [batch][n_query][q_heads], written; may be NULL.
 * Keys are formed in float32 and carried as BF16 high + low parts (~16 significant
 * bits); values are formed in float32 and carried in float16 after a power-of-two range
 * scaling (so values beyond float16's range are supported), with float32 accumulation.
 * Supported by this library: head_dim == 128.  Asynchronous on hip_stream.
 */
int lynx_attn_verify(const void* q_dev, const void* k_anchor_dev, const void* k_residual_dev,
                     const void* v_anchor_dev, const void* v_residual_dev, int batch, int n_query,
                     int ctx_tokens, int q_heads, int kv_heads, int head_dim, int page_tokens,
                     int chunk, float alpha, float sm_scale, void* workspace_dev, size_t ws_bytes,
                     int out_dtype, void* out_dev, float* lse_dev, void* hip_stream);

/*
 * lynx_attn_verify over a paged cache with per-sequence lengths (as lynx_attn_anchor_paged):
 * the anchor and residual pools hold n_pool_pages segments each, and pool segment s of both
 * streams is the same page.  block_table_dev int32 [batch][max_pages_per_seq] and seq_lens_dev
 * int32 [batch] as for lynx_attn_anchor_paged (clamped entries; a sequence's tail is masked;
 * an empty context gives O = 0 and LSE = -inf).  Workspace:
 * lynx_attn_verify_workspace_bytes(batch, n_query, max_pages_per_seq * page_tokens, ...).
 * Errors: those of lynx_attn_verify; LYNX_EINVAL for n_pool_pages or max_pages_per_seq <= 0;
 * LYNX_EALIGN for a null or misaligned block table or length array.
 */
int lynx_attn_verify_paged(const void* q_dev, const void* k_anchor_pool_dev, const void* k_residual_pool_dev,
                           const void* v_anchor_pool_dev, const void* v_residual_pool_dev, int n_pool_pages,
                           const int32_t* block_table_dev, const int32_t* seq_lens_dev, int batch, int n_query,
                           int max_pages_per_seq, int q_heads, int kv_heads, int head_dim, int page_tokens, int chunk,
                           float alpha, float sm_scale, void* workspace_dev, size_t ws_bytes, int out_dtype,
                           void* out_dev, float* lse_dev, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* LYNX_H */
