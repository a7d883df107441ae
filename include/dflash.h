/*
 * dflash.h -- C ABI of the MI355X (gfx950) DFlash2 block-drafting hot path.
 *
 * Entry points, each a stream-ordered sequence of hand-written HIP kernels:
 *
 *   dflash_context_fuse  fuse tapped target hidden states into the context
 *                        representation H_t and append every draft layer's
 *                        context K/V rows to per-sequence ring buffers;
 *   dflash_block_attn    block-draft attention of one draft layer;
 *   dflash_topk          per-position top-k candidates, log-normaliser and
 *                        drafted token of the drafter's logits;
 *   spec_verify          lossless verification of one drafted block.
 *   dflash_select_path   the candidate selector's walk through the top-k
 *                        candidates of each block position.
 *   dflash_two_tap_conv  the two-tap dynamic convolution inside a block.
 *   dflash_top_p_mask    top-p (nucleus) truncation of logits rows, for
 *                        sampling and verifying with top-p;
 *   dflash_top_p_cut     the same nucleus as one cut per row, which
 *                        dflash_topk and spec_verify apply in their scans.
 *   dflash_lm_head_topk  the drafter's LM head with top-k, log-normaliser and
 *                        drafted token computed in the GEMM epilogue (the
 *                        logits never reach memory).
 *
 * Sources (web pages, cited by title and section):
 *   "DFlash vs DFlash 2" (blog): "The problem: one expensive token at a time",
 *       "DFlash: generate the block all at once", "Conditioning on the target
 *       model", "The candidate selector".
 *   "Beam 1.0 DFlash2" (model card): "Model", "Evaluation".
 *   "Speculative decoding" (Reflection docs): "How it works".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument is a DEVICE pointer (memory visible to the GPU that
 *   `stream` belongs to), except where a comment says otherwise.  bf16 values
 *   are passed as uint16_t bit patterns.  All tensors are dense, row-major, in
 *   the index order written next to them.
 * - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *   enqueues work on it and returns; nothing is synchronised.  The calls make
 *   no allocation, memset or host synchronisation, so a caller may record them
 *   into a HIP graph (stream capture) and replay it.
 * - The caller owns every buffer.  The library never allocates or frees
 *   memory and keeps no state between calls; scratch space comes only from
 *   the caller's `workspace` (device memory of at least the size the matching
 *   *_workspace_size() query returns, 256-byte aligned).  Two calls may run
 *   concurrently if their workspaces and outputs do not overlap.
 * - Inputs are read-only.  Outputs are fully overwritten, except the ring
 *   buffer of dflash_context_fuse, of which only the addressed slots change.
 * - Every argument the host can check is checked BEFORE any HIP call; a
 *   rejected call enqueues nothing.  Device-side data (token ids, lengths) are
 *   preconditions stated per call: out-of-range values there are undefined
 *   behaviour (they are clamped where clamping is cheap, never trapped).
 * - Temperatures: T == 0 selects greedy behaviour; T > 0 samples.
 * - Random numbers: one Philox4x64-10 block (Salmon et al., SC'11) per draw,
 *   key = (seed[b], 0), counter = (step, b, row, purpose), uniform =
 *   (first output word >> 11) * 2^-53.  Purposes: 0 draft draw, 1 accept test,
 *   2 correction or bonus draw.  `row` is the 0-based position in the block.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
#define DFLASH_OK                0
#define DFLASH_ERR_NULL         -1  /* a required pointer is NULL               */
#define DFLASH_ERR_SHAPE        -2  /* a size or scalar argument is invalid     */
#define DFLASH_ERR_UNSUPPORTED  -3  /* valid, but outside what this build runs  */
#define DFLASH_ERR_WORKSPACE    -4  /* workspace NULL, misaligned or too small  */
#define DFLASH_ERR_HIP          -5  /* a HIP launch failed                      */
#define DFLASH_ERR_TOO_LARGE    -6  /* needs more scratch than the static array holds */

/* Element types of dflash_block_attn's Q/K/V/output tensors. */
#define DFLASH_DTYPE_BF16 0
#define DFLASH_DTYPE_FP32 1

/* Static description of a status code (never NULL). */
const char* dflash_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int dflash_version(void);

/* ------------------------------------------------------------------------
 * dflash_block_attn -- block-draft attention of one draft layer.
 *
 * "DFlash vs DFlash 2", "DFlash: generate the block all at once" and
 * "Conditioning on the target model" (equation for Q_i, K_i, V_i): the
 * queries come from the block of gamma positions (anchor + masks) only; keys
 * and values are the target-context rows followed by the block's own rows;
 * positions inside the block attend to one another without a causal mask.
 * "Speculative decoding", "How it works" / "Beam 1.0 DFlash2", "Model": the
 * context is a sliding window of the most recent `window` (4,096) tokens;
 * 40 query heads share 8 KV heads of dimension 128.
 *
 * For each sequence b, query head h (KV head h / (n_q / n_kv)) and block row r:
 *   out[b,r,h,:] = sum_j softmax_j(scale * <q[b,r,h,:], k_j>) v_j
 * over the key set { ring slots 0 .. n_b-1 } U { block rows 0 .. gamma-1 },
 * n_b = min(ctx_len[b], window).  The ring is a set: slot order is irrelevant
 * (a writer puts absolute position p at slot p mod window).  Q and K arrive
 * already projected (and rotated, if the model rotates them).
 *
 *   q       [batch, gamma, n_q,  d_head]   dtype
 *   k_blk   [batch, gamma, n_kv, d_head]   dtype
 *   v_blk   [batch, gamma, n_kv, d_head]   dtype
 *   k_ring  [batch, n_kv, window, d_head]  dtype  (slots >= n_b are never read)
 *   v_ring  [batch, n_kv, window, d_head]  dtype
 *   ctx_len [batch] int64, >= 0 (precondition)
 *   out     [batch, gamma, n_q, d_head]    dtype (bf16 rounded to nearest even)
 *   lse     [batch, gamma, n_q] float32, natural-log normaliser of the scaled
 *           scores; may be NULL.
 * Supported: n_q % n_kv == 0; 1 <= gamma <= 32; window % 64 == 0,
 *   64 <= window <= 2^28, batch*gamma*n_q <= 2^28; d_head in {64, 128}
 *   (bf16) or 1 <= d_head <= 128 (fp32).
 * Accuracy: fp32 softmax and accumulation; bf16 products (bf16) or fp32
 *   fused multiply-adds (fp32).
 * ------------------------------------------------------------------------ */
size_t dflash_block_attn_workspace_size(int batch, int gamma, int n_q, int n_kv,
                                        int d_head, int window, int dtype);
int dflash_block_attn(const void* q, const void* k_blk, const void* v_blk,
                      const void* k_ring, const void* v_ring, const int64_t* ctx_len,
                      float scale, void* out, float* lse, int dtype,
                      int batch, int gamma, int n_q, int n_kv, int d_head, int window,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * A top-p nucleus of one logits row, named by its last entry in the rank
 * order (logit descending, index ascending; -0.0 and +0.0 are equal):
 * entry v, logit z_v, is in the nucleus iff z_v > logit, or z_v == logit
 * and v <= index.  {-inf, INT32_MAX} keeps every entry.  Written by
 * dflash_top_p_cut; dflash_topk and spec_verify take one per row and treat
 * every entry outside it as -inf, exactly as on rows masked by
 * dflash_top_p_mask, without a masked copy of the rows.
 * ------------------------------------------------------------------------ */
typedef struct dflash_nucleus_cut {
    float logit;
    int32_t index;
} dflash_nucleus_cut;

/* ------------------------------------------------------------------------
 * dflash_topk -- drafter side of one block: per-position top-k candidates,
 * log-normaliser and drafted token.
 *
 * "DFlash vs DFlash 2", "The candidate selector": keep the top k candidates
 * of each position's draft logits.  "The problem: one expensive token at a
 * time": the drafter proposes token y from its distribution q.
 *
 *   logits   [batch, gamma, vocab] float32, finite or -inf (results are
 *            unspecified for rows holding NaN or +inf); row r is the
 *            drafter's logits of block position r+1 (the token after
 *            anchor + r masks).
 *   cut      [batch, gamma] nucleus cuts (top-p sampling), or NULL: every
 *            output below is that of the row with the entries outside its
 *            nucleus set to -inf.
 *   topk_idx [batch, gamma, k] int32, topk_val [batch, gamma, k] float32:
 *            the k largest raw logits of each row, descending; equal logits
 *            in increasing index order.
 *   lse      [batch, gamma] float64, log sum_v exp(logit_v / T)  (T > 0;
 *            NaN when T == 0); may be NULL.
 *   draft    [batch, gamma] int32; may be NULL.  T == 0: the row's argmax
 *            (lowest index among equal maxima).  T > 0: a draw from
 *            softmax(logits / T) by inverse CDF in increasing vocabulary order
 *            with the purpose-0 uniform of (seeds[b], step, b, r).
 *   seeds    [batch] uint64 (device); may be NULL when T == 0.
 * Supported: 1 <= k <= 64, k <= vocab, vocab % 4 == 0, vocab <= 2^23 (the
 * row's segment statistics live in one workgroup's LDS), 1 <= gamma <= 32,
 * batch*gamma <= 2^20 (one 1,024-thread workgroup per row).
 * Workspace: none (dflash_topk_workspace_size returns 0; workspace may be
 * NULL and is ignored).  One workgroup per row does the whole row in one
 * launch.
 * ------------------------------------------------------------------------ */
size_t dflash_topk_workspace_size(int batch, int gamma, int vocab, int k);
int dflash_topk(const float* logits, const dflash_nucleus_cut* cut, int batch, int gamma,
                int vocab, int k,
                float temperature, const uint64_t* seeds, uint64_t step,
                int32_t* topk_idx, float* topk_val, double* lse, int32_t* draft,
                void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * spec_verify -- verification of one drafted block per sequence.
 *
 * "DFlash vs DFlash 2", "The problem: one expensive token at a time": the
 * target scores the whole block in one pass, keeps the longest valid prefix
 * and corrects the first rejection.  Greedy (T == 0): a draft survives while
 * it equals the target's argmax.  Sampled (T > 0): draft y at row r survives
 * if u < min(1, p_r(y) / q_r(y)) (u: purpose-1 uniform at row r); the first
 * rejected row j draws a correction from [p_j - q_j]_+ renormalised (from p_j
 * if that has no mass); if all gamma-1 drafts survive, a bonus token is
 * drawn from the target's last row p_{gamma-1}.  Draws are inverse CDF in
 * increasing vocabulary order with the purpose-2 uniform at the row drawn
 * from.  p_r = softmax(target_logits[b,r,:] / T),
 * q_r = softmax(draft_logits[b,r,:] / T).  "Beam 1.0 DFlash2",
 * "Evaluation": a block of 8 verifies 7 drafts.
 *
 *   target_logits [batch, gamma, vocab] float32, finite or -inf (as for
 *            draft_logits, results are unspecified for rows holding NaN or
 *            +inf); row r is the target's distribution for the token after
 *            anchor + drafts 0..r-1; rows 0..gamma-2 verify, row gamma-1
 *            gives the bonus.
 *   draft_logits  [batch, gamma, vocab] float32 (rows 0..gamma-2 are read),
 *            or NULL.  NULL with T > 0 means deterministic drafts (chosen by
 *            dflash_select_path, "The candidate selector"): q_r is the point
 *            mass at the draft, so a draft survives with probability p_r(y)
 *            and the correction is drawn from p_j with the rejected draft
 *            removed (still lossless).  Unused when T == 0.
 *   draft_tokens  [batch, gamma] int32 (as written by dflash_topk); entries
 *            0..gamma-2 are the drafts, in [0, vocab) (precondition); entry
 *            gamma-1 is ignored (so dflash_topk's output passes unchanged).
 *   draft_lse     [batch, gamma] float64 from dflash_topk at the same T (and
 *            the same draft_cut); may be NULL (then recomputed from
 *            draft_logits; unused with deterministic drafts).
 *   target_cut, draft_cut  [batch, gamma] nucleus cuts (top-p sampling), or
 *            NULL: p_r and q_r are then the softmax of the rows with the
 *            entries outside their nuclei set to -inf (the truncated
 *            distributions), exactly as on rows masked by dflash_top_p_mask.
 *            Unused when T == 0 (the argmax is always in the nucleus).
 *   seeds         [batch] uint64 (device); may be NULL when T == 0.
 *   accept_len    [batch] int32: j = accepted drafts (0..gamma-1);
 *                 tau = j + 1 tokens are committed.
 *   out_tokens    [batch, gamma] int32: drafts 0..j-1, then the correction
 *                 or bonus token, then -1.
 *   accepted      [batch, gamma-1] uint8 or NULL: the accept test of every
 *                 draft row (also rows after the first rejection).
 * Supported: 1 <= gamma <= 32, vocab % 4 == 0, vocab <= 2^29,
 * batch*gamma <= 2^20.
 * ------------------------------------------------------------------------ */
size_t spec_verify_workspace_size(int batch, int gamma, int vocab);
int spec_verify(const float* target_logits, const float* draft_logits,
                const int32_t* draft_tokens, const double* draft_lse,
                const dflash_nucleus_cut* target_cut, const dflash_nucleus_cut* draft_cut,
                float temperature, const uint64_t* seeds, uint64_t step,
                int32_t* accept_len, int32_t* out_tokens, uint8_t* accepted,
                int batch, int gamma, int vocab,
                void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * dflash_context_fuse -- context fusion and context K/V append.
 *
 * "DFlash vs DFlash 2", "Conditioning on the target model", equation for
 * H_t: the hidden states of five target layers ("Beam 1.0 DFlash2", "Model":
 * layers 4, 16, 28, 40, 46) are concatenated, projected by W_c and
 * RMS-normalised; equation for K_i, V_i: the context half of draft layer i's
 * keys and values is W_i^K H_t, W_i^V H_t, a read-only memory at every layer.
 *
 *   H_t[r,:] = g * y / sqrt(mean(y^2) + eps),  y = W_c x_r
 *   kv[r,c]  = sum_n H_t[r,n] * w_kv[c,n],  c = ((i*2 + t)*n_kv + h)*d_head + d
 *              (layer i, t = 0 key / 1 value, KV head h)
 *   kv_ring[i, t, row_seq[r], h, row_pos[r] % window, d] = bf16(kv[r,c])
 *
 *   taps     [rows, n_taps*d_tgt] bf16, the tapped states of each new token
 *   w_c      [d_model, n_taps*d_tgt] bf16, one row per output feature (the
 *            H_t equation's W_c applied to the concatenated column; both
 *            GEMM operands then have the reduction dimension contiguous)
 *   rms_gain [d_model] float32
 *   w_kv     [n_layers*2*n_kv*d_head, d_model] bf16, one row per output
 *            feature (W_i^K, W_i^V of every layer stacked)
 *   row_seq  [rows] int32 in [0, batch), row_pos [rows] int64 >= 0
 *            (preconditions; no two rows may address the same slot)
 *   kv_ring  [n_layers, 2, batch, n_kv, window, d_head] bf16, in/out
 *   h_t_out  [rows, d_model] bf16, or NULL
 * Supported: d_model % 128 == 0, (n_taps*d_tgt) % 64 == 0,
 *   (n_layers*2*n_kv*d_head) % 128 == 0, d_head % 4 == 0, 1 <= rows <= 65,535,
 *   d_model <= 8192, n_taps*d_tgt <= 2^30, n_layers*2*n_kv*d_head <= 2^30.
 * Accuracy: bf16 products, fp32 accumulation; H_t is rounded to bf16 before
 * the K/V projection.
 * ------------------------------------------------------------------------ */
size_t dflash_context_fuse_workspace_size(int rows, int n_taps, int d_tgt, int d_model,
                                          int n_layers, int n_kv, int d_head);
int dflash_context_fuse(const uint16_t* taps, const uint16_t* w_c, const float* rms_gain,
                        float eps, const uint16_t* w_kv, const int32_t* row_seq,
                        const int64_t* row_pos, uint16_t* kv_ring, uint16_t* h_t_out,
                        int rows, int n_taps, int d_tgt, int d_model, int n_layers,
                        int n_kv, int d_head, int window, int batch,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * dflash_select_path -- the candidate selector.
 *
 * "DFlash vs DFlash 2", "The candidate selector": each block position keeps
 * the top-k draft candidates and the transition from candidate a at the
 * preceding position to candidate b at position t scores
 *     S_t(a, b) = U_t(b) + sum_i A(a)_i * g_t,i * B(b)_i,
 * with U_t(b) the drafter's logit of b, A and B compact token embeddings and
 * g_t = H(h_t) the gate computed from the position's hidden state.  All
 * transition scores are computed in parallel; the walk is greedy: position 0
 * follows the anchor, each later position follows the token just chosen, and
 * equal scores go to the candidate listed first.  The resulting path is a set
 * of deterministic drafts for spec_verify with draft_logits == NULL.
 *
 *   cand_idx   [batch, gamma, k] int32 token ids (as dflash_topk writes)
 *   cand_score [batch, gamma, k] float32 U_t(b) (dflash_topk's values)
 *   emb_a, emb_b [vocab, r] bf16 (16-byte aligned)
 *   gate       [batch, gamma, r] bf16 (16-byte aligned)
 *   anchor     [batch] int32, the last verified token of each sequence
 *   path       [batch, gamma] int32 out: the chosen token of each position
 *   path_score [batch, gamma] float32 out or NULL: S_t(previous, chosen)
 * Token ids outside [0, vocab) are clamped (precondition: they are in range).
 * Supported: k <= 64, r % 8 == 0, r <= 4096, gamma <= 4096, batch <= 2^20.
 * Accuracy: every term is a product of three bf16 values (exact in fp64) and
 * the sum over i runs in increasing i in fp64, so the walk's choices are those
 * of the exact scores up to fp64 rounding of that sum.
 * All pointers are device memory owned by the caller; no workspace.
 * ------------------------------------------------------------------------ */
int dflash_select_path(const int32_t* cand_idx, const float* cand_score, const uint16_t* emb_a,
                       const uint16_t* emb_b, const uint16_t* gate, const int32_t* anchor,
                       int32_t* path, float* path_score, int batch, int gamma, int k, int vocab,
                       int r, void* stream);

/* ------------------------------------------------------------------------
 * dflash_two_tap_conv -- the two-tap dynamic convolution.
 *
 * "DFlash vs DFlash 2", "The two-tap dynamic convolution": each block
 * position mixes its representation with its immediate predecessor,
 *     y[b,t,c] = kern[b,t,0,g(c)] * x[b,t,c] + kern[b,t,1,g(c)] * x[b,t-1,c],
 * depthwise, with content-dependent kernel values shared by the channels of a
 * group (g(c) = c / (d / n_groups)), never across a block boundary.  Row 0 of
 * a block is the anchor's position: row t >= 1 reads row t - 1 (the first
 * drafted position reads the anchor), row 0 has no predecessor (zero).
 *
 *   x     [batch, gamma, d] bf16 (16-byte aligned)
 *   kern  [batch, gamma, 2, n_groups] float32 (computed from the content by
 *         the caller's projection)
 *   y     [batch, gamma, d] bf16 out (16-byte aligned; must not overlap x)
 * Supported: d % n_groups == 0, (d / n_groups) % 8 == 0, batch*gamma*d <= 2^34.
 * Accuracy: fp32 arithmetic, per channel one multiply (the predecessor term)
 * and one fused multiply-add (the own term added to it): two fp32
 * roundings, then the output is rounded to bf16, nearest even.
 * All pointers are device memory owned by the caller; no workspace.
 * ------------------------------------------------------------------------ */
int dflash_two_tap_conv(const uint16_t* x, const float* kern, uint16_t* y, int batch, int gamma,
                        int d, int n_groups, void* stream);

/* ------------------------------------------------------------------------
 * dflash_lm_head_topk -- the drafter's LM head, z = hidden W_head^T, with the
 * drafter-side outputs of dflash_topk computed from z in the GEMM's epilogue.
 *
 * "Beam 1.0 DFlash2" model card, "Model": the drafter reuses the target's LM
 * head over the shared 151,936-entry vocabulary; "DFlash vs DFlash 2", "The
 * candidate selector": top-k candidates of every block position, the
 * full-vocabulary LM-head pass being the costly step; "The problem: one
 * expensive token at a time": the drafter proposes y ~ softmax(z / T).
 *
 *   hidden   [rows, d_model] bf16 (16-byte aligned); row r is block position
 *            r % gamma of sequence r / gamma.
 *   w_head   [vocab, d_model] bf16 (16-byte aligned), one row per token.
 *   topk_idx [rows, k] int32, topk_val [rows, k] float32: the k largest
 *            logits of each row, descending; equal logits in increasing index
 *            order.
 *   lse      [rows] float64, log sum_v exp(z_v / T) (T > 0; NaN when T == 0);
 *            may be NULL.
 *   draft    [rows] int32; may be NULL.  T == 0: the row's argmax (lowest
 *            index among equal maxima).  T > 0: a draw from softmax(z / T) by
 *            inverse CDF over the whole row in increasing vocabulary order
 *            with the purpose-0 uniform of (seeds[b], step, b, r % gamma),
 *            b = r / gamma: the same rule, and with the same seeds the same
 *            token, as dflash_topk on these logits (up to the rounding of
 *            the logits).  The finalize recomputes the 16 logits of the
 *            group holding the crossing from hidden and w_head.
 *   seeds    [rows / gamma rounded up] uint64 (device); may be NULL when
 *            T == 0 or draft == NULL.
 * Work: the weights are streamed from HBM once per 256 rows of hidden.
 * Supported: 1 <= k <= 16, k <= vocab <= 1,048,576, d_model % 64 == 0,
 * d_model <= 65,536, rows <= 2^20 (DFLASH_ERR_UNSUPPORTED otherwise).
 * Accuracy: bf16 products, fp32 accumulation (the GEMM); fp32 exponentials
 * and segment sums, fp64 across segments.
 * Workspace: dflash_lm_head_topk_workspace_size bytes, 256-byte aligned.
 * ------------------------------------------------------------------------ */
size_t dflash_lm_head_topk_workspace_size(int rows, int d_model, int vocab, int k);
int dflash_lm_head_topk(const uint16_t* hidden, const uint16_t* w_head, int rows, int gamma,
                        int d_model, int vocab, int k, float temperature,
                        const uint64_t* seeds, uint64_t step, int32_t* topk_idx,
                        float* topk_val, double* lse, int32_t* draft, void* workspace,
                        size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * dflash_top_p_mask -- top-p (nucleus) truncation of logits rows.
 *
 * "Beam 1.0 DFlash2" model card, "Evaluation": sampled runs use temperature
 * 0.7 and top-p 0.99.  The nucleus of softmax(z / T) is the shortest prefix of
 * the row, in the order (logit descending, index ascending), whose
 * probability reaches top_p; every entry outside it is set to -inf.  Then
 * softmax(z / T) of the masked row is the renormalised truncation, and
 * dflash_topk (drafter rows) and spec_verify (target and drafter rows) run on
 * masked rows sample and verify top-p decoding losslessly ("DFlash vs DFlash
 * 2", "The problem: one expensive token at a time").
 *
 *   logits [rows, vocab] float32 (finite or -inf)
 *   out    [rows, vocab] float32; may equal logits (in place: only the masked
 *          entries are written)
 *   kept   [rows] int32 or NULL: the nucleus size of each row
 *   temperature > 0; 0 < top_p <= 1 (top_p == 1 keeps every entry)
 * Supported: vocab < 2^24 (a mass bin's 64-bit fixed-point sum stays
 * exact), rows <= 2^20; DFLASH_ERR_UNSUPPORTED otherwise.
 * Accuracy: weights 2^((z - max) log2(e)/T) from fp32 exponentials, grouped
 * in bins of 1/64 of a log2 unit and summed exactly in 31-bit fixed point
 * relative to the bin's top, bin masses added in fp64; the nucleus boundary
 * is exact up to that rounding of the cumulative mass (about 1e-7 of it).
 * No workspace; one workgroup per row.
 * ------------------------------------------------------------------------ */
int dflash_top_p_mask(const float* logits, float* out, int32_t* kept, int rows, int vocab,
                      float temperature, float top_p, void* stream);

/* ------------------------------------------------------------------------
 * dflash_top_p_cut -- the same nucleus as dflash_top_p_mask, returned as one
 * cut per row instead of a masked copy of the rows.
 *
 * "Beam 1.0 DFlash2" model card, "Evaluation" (temperature 0.7, top-p 0.99
 * for sampled runs); the cut is handed to dflash_topk and spec_verify, whose
 * row scans apply it, so top-p decoding reads each row three times here
 * (maximum, mass histogram, boundary gather) and writes nothing per entry.
 *
 *   logits [rows, vocab] float32 (finite or -inf)
 *   cut    [rows] out: the last nucleus entry (logit, index); {-inf,
 *          INT32_MAX} when top_p == 1 or the row is all -inf
 *   kept   [rows] int32 or NULL: the nucleus size of each row
 * Arguments, limits and accuracy as dflash_top_p_mask.
 * No workspace; one workgroup per row.
 * ------------------------------------------------------------------------ */
int dflash_top_p_cut(const float* logits, dflash_nucleus_cut* cut, int32_t* kept, int rows,
                     int vocab, float temperature, float top_p, void* stream);

/* ------------------------------------------------------------------------
 * spec_verify_noalloc -- spec_verify for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same operation, arguments and results as
 * spec_verify, with no workspace argument.
 *
 * The scratch is a fixed array of spec_verify_noalloc_max_scratch() bytes
 * (8 MiB) in device memory, one per GPU, allocated with the library's code
 * object and held until the process ends; the call itself allocates nothing.
 * A shape whose scratch (spec_verify_workspace_size) exceeds it returns
 * DFLASH_ERR_TOO_LARGE before any HIP call (B = 32, gamma = 8 at 151,936
 * entries needs about 0.5 MiB).  `stream` must belong to the device current
 * on the calling thread.  Every call on one GPU uses that GPU's array: calls
 * that overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  The first call on a device looks up the array's
 * device address (hipGetSymbolAddress); DFLASH_ERR_HIP if that fails.
 * ------------------------------------------------------------------------ */
size_t spec_verify_noalloc_max_scratch(void);
int spec_verify_noalloc(const float* target_logits, const float* draft_logits,
                        const int32_t* draft_tokens, const double* draft_lse,
                        const dflash_nucleus_cut* target_cut,
                        const dflash_nucleus_cut* draft_cut, float temperature, const uint64_t* seeds, uint64_t step,
                        int32_t* accept_len, int32_t* out_tokens, uint8_t* accepted,
                        int batch, int gamma, int vocab, void* stream);

/* ------------------------------------------------------------------------
 * Device-data preconditions.
 *
 * Values the library reads on the device (token ids, lengths, positions) are
 * preconditions: a release build does not check them (an out-of-range id is
 * clamped into range, a negative length counts as 0, a fused row with an
 * invalid sequence or position is skipped, so that no access leaves its
 * buffer, but the results are unspecified).  The library built with device
 * checks (libdflash_checked.so: the same sources compiled with
 * DFLASH_DEVICE_CHECKS=1, for debugging callers) computes the same results
 * and, in addition, records every violation it meets in a word per GPU:
 * ------------------------------------------------------------------------ */
#define DFLASH_VIOLATION_TOKEN    1u  /* a token id outside [0, vocab): spec_verify's
                                         drafts, dflash_select_path's candidates or anchor */
#define DFLASH_VIOLATION_CTX_LEN  2u  /* ctx_len < 0 (dflash_block_attn) */
#define DFLASH_VIOLATION_ROW      4u  /* row_seq outside [0, batch) or row_pos < 0
                                         (dflash_context_fuse) */
#define DFLASH_VIOLATION_SLOT     8u  /* two rows of one dflash_context_fuse call address
                                         the same (sequence, slot), e.g. more than `window`
                                         rows of one sequence */

/* 1 in the build with device checks, 0 in a release build. */
int dflash_device_checks(void);

/* The word of the GPU current on the calling thread: waits for `stream`,
 * ORs the violations recorded so far into *word (set to 0 first) and, if
 * `clear` is non-zero, resets them.  Synchronous; not for graph capture.
 * The read and the reset are two copies: a kernel still running on another
 * stream may record a violation between them, which the reset then drops
 * (synchronise the device first to see every one).
 * DFLASH_ERR_UNSUPPORTED in a release build (*word = 0), DFLASH_ERR_NULL
 * for a NULL word, DFLASH_ERR_HIP if a copy fails. */
int dflash_violations(uint32_t* word, int clear, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
