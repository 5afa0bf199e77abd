/*
 * spec_verify.h — C ABI of the greedy draft/verify step on MI355X (gfx950).
 *
 * One speculative cycle scores B sequences of k_s + 1 rows each against the target
 * model: row j of sequence s feeds position pos_s + j (row 0 carries the last
 * emitted token, rows 1..k_s the drafts). The library provides the four steps of
 * that verify pass that dominate its cost:
 *
 *   spec_verify_attn           KV append in place + paged causal attention
 *   spec_lm_head_argmax        lm_head contraction with the greedy argmax fused in
 *   spec_greedy_accept         greedy acceptance and position rollback
 *   spec_lm_head_argmax_accept the lm_head argmax and the greedy acceptance in one call
 *   spec_delta_verify_rollback Gated DeltaNet per-token state record and restore
 *
 * and, for drafts shaped as a tree (trie or star) instead of a chain:
 *
 *   spec_verify_attn_tree      the attention step over tree rows
 *   spec_tree_accept           the acceptance walk from the root
 *   spec_kv_compact            the accepted path's K/V moved to contiguous slots
 *
 * and, for sampled (temperature > 0) instead of greedy decoding:
 *
 *   spec_lm_head_sample        lm_head with softmax statistics and two draws fused in
 *   spec_sample_accept         the speculative-sampling chain walk
 *   spec_lm_head_sample_dense  the same pass for dense draft distributions (keeps z)
 *   spec_sample_accept_dense   the chain walk with a dense q and its residual draw
 *
 * and the pieces around them: spec_greedy_accept_stop and spec_truncate_stop (stop
 * tokens and a generation limit) and the host-side adaptive draft-depth policy
 * spec_kpolicy_*.
 *
 * The method follows the page "span-02 engine/crates/model/src/spec.rs"
 * (module doc: ONE batched verify forward of B(k+1) rows over each branch's own
 * pages, KV appended in place at pos..pos+k, greedy acceptance, rollback by
 * advancing pos only; rows past the new pos hold stale KV that no later row reads,
 * since each row's keys stop at its own position;
 * SpecReq: the KV slot of position p lives in page pages[p / 16]).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All pointers are DEVICE pointers unless marked "host". The caller owns every
 *    buffer; the library allocates nothing and keeps no state between calls.
 *  - bf16 values travel as their raw 16-bit patterns (spec_bf16).
 *  - Every call takes `stream` (a hipStream_t, NULL = the null stream), only
 *    enqueues work on it and never synchronises.
 *  - Return codes: SPEC_OK, or a negative SPEC_E* code for errors the host can see
 *    (bad scalar, bad pointer, workspace too small, launch failure); nothing is
 *    enqueued in that case, and spec_last_error() gives the message (thread-local).
 *  - Conditions only the device can see (a page id out of range, a position past
 *    the page table, row counts that do not add up, a draft id out of range) are
 *    reported per sequence in `seq_status` [B] (written for EVERY sequence on
 *    every call, 0 = fine, else an OR of SPEC_STATUS_* bits); such a sequence is
 *    skipped and its outputs are as documented per call.
 *  - Row packing: sequence s owns rows off_s .. off_s + k_s with
 *    off_s = sum_{s' < s} (k_{s'} + 1) (the chain packing of span-02's
 *    spec_build_verify, made ragged). The packing is defined only if every
 *    k_s >= 0 and sum_s (k_s + 1) == R; otherwise EVERY sequence is flagged
 *    SPEC_STATUS_BAD_ROWS.
 *  - Row invariance: no launch parameter, tile or reduction order depends on R, B,
 *    the k_s or on other rows, so each row's result bytes depend only on its own
 *    inputs, its absolute position and the shape arguments. A verify row is
 *    therefore byte-identical to a one-row decode at the same position (the
 *    exactness rule of span-02 set_row_invariant, DSSD fast.py _layers and memra
 *    full_attn_verify).
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t spec_bf16;

#define SPEC_PAGE_TOKENS 16

#define SPEC_OK 0
#define SPEC_EINVAL (-1)     /* bad scalar argument, null or misaligned pointer */
#define SPEC_ECAPACITY (-2)  /* a host-known size exceeds a documented limit     */
#define SPEC_EHIP (-3)       /* the HIP runtime refused a launch                 */
#define SPEC_EWORKSPACE (-4) /* workspace pointer null or smaller than required  */

#define SPEC_STATUS_BAD_PAGE 1  /* a page id the sequence needs is outside [0, n_pages)   */
#define SPEC_STATUS_BAD_POS 2   /* pos_s < 0, or (pos_s + k_s) / 16 >= max_pages         */
#define SPEC_STATUS_BAD_ROWS 4  /* packing undefined (see above), or k_s > kmax           */
#define SPEC_STATUS_BAD_TOKEN 8 /* draft id outside its vocabulary, or d2t entry >= V     */
#define SPEC_STATUS_BAD_TREE 16 /* tree calls: a parent not before its node, a bad path   */
#define SPEC_STATUS_BAD_LIMIT 32 /* stop call: a generation limit below one token          */

/* Library version (increases with any ABI or numerics change). */
int spec_version(void);

/* Message of the last error returned on the calling host thread ("" if none). */
const char* spec_last_error(void);

/* ---------------------------------------------------------------------------
 * spec_verify_attn — KV append + paged causal verify attention (one layer).
 *
 * Defined by: span-02 spec.rs module doc (KV appended in place at pos..pos+k;
 * kv_hi = position); memra-engine spec.rs full_attn_verify ("query row r attends
 * to keys [0 .. base_len + r + 1)", scale 1/sqrt(head_dim), per-row KV append);
 * DSSD fast.py _attention (per-row SDPA over keys [0, p+1) with grouped query
 * heads) and _layers (index_copy_ of the rows' K/V into the cache).
 *
 * For every valid sequence s and row j (position p = pos[s] + j, packed row r):
 *   1. K/V append: k_new[r, hk, :] and v_new[r, hk, :] are written to position p
 *      of every kv head hk (page page_table[s, p / 16], in-page token p % 16).
 *   2. Attention, for every query head h (kv head hk = h / (Hq / Hkv)):
 *        out[r, h, :] = sum_{t <= p} softmax_t(scale * q[r,h,:] . K_t[hk,:]) V_t[hk,:]
 *      over the sequence's positions 0..p after the append; bf16 output rounded
 *      to nearest-even from fp32 accumulation.
 *
 * Layouts (row-major, contiguous):
 *   q      [R][Hq][D]           bf16         k_new, v_new [R][Hkv][D] bf16
 *   k_pool, v_pool [n_pages][Hkv][16 * D] bf16: one block of 16 tokens x D channels
 *          per (page, kv head); inside a block, token t and channel d sit at
 *            K: (d/32)*512 + ((d%32)/8)*128 + t*8 + d%8
 *            V: (d/16)*256 + (t/4)*64 + (d%16)*4 + t%4
 *          (MFMA operand-fragment order: every wave access is contiguous)
 *   page_table [B][max_pages] int32 (entries past a sequence's last page unread)
 *   pos [B], k [B] int32         out [R][Hq][D] bf16      seq_status [B] int32
 * kmax: an upper bound on the k_s (a sequence with k_s > kmax is flagged
 * BAD_ROWS); it sizes the launch and never changes a row's result.
 * Pool pages shared by two sequences, or two rows mapping to one slot, give
 * unspecified results. Bytes of the pool other than the R x Hkv written slots
 * are never modified.
 *
 * Split-KV: each sequence's positions are cut into splits of kv_split_tokens
 * (a multiple of 64; 0 = spec_attn_split_tokens(max_pages)) at absolute
 * positions; a row's result depends on the split size, so decode and verify
 * calls that must agree use the same value.
 *
 * Limits: D in {64, 128, 256}; 1 <= Hkv <= Hq, Hq % Hkv == 0, Hq / Hkv <= 16;
 * 1 <= B <= 4096; R >= 1; scale > 0; 0 <= kmax <= 127 (so a kv head serves up to
 * (Hq / Hkv) * 128 = 2048 query rows of a sequence, 64 per workgroup); 16-byte
 * aligned q, k_new, v_new, k_pool, v_pool, out, workspace.
 * A flagged sequence writes nothing to the pool or to its out rows.
 * workspace: at least spec_verify_attn_workspace_bytes(...) bytes; no state is
 * carried between calls in it.
 * ------------------------------------------------------------------------- */
int32_t spec_attn_split_tokens(int32_t max_pages);
size_t spec_verify_attn_workspace_bytes(int32_t B, int32_t R, int32_t Hq, int32_t Hkv, int32_t D,
                                        int32_t max_pages, int32_t kv_split_tokens);
int spec_verify_attn(const spec_bf16* q, const spec_bf16* k_new, const spec_bf16* v_new,
                     spec_bf16* k_pool, spec_bf16* v_pool, int64_t n_pages,
                     const int32_t* page_table, int32_t max_pages, const int32_t* pos,
                     const int32_t* k, int32_t kmax, int32_t B, int32_t R, int32_t Hq, int32_t Hkv,
                     int32_t D, float scale, int32_t kv_split_tokens, spec_bf16* out, void* workspace,
                     size_t workspace_bytes, int32_t* seq_status, void* stream);

/* ---------------------------------------------------------------------------
 * spec_lm_head_argmax — lm_head contraction with the greedy argmax fused in.
 *
 * Defined by: span-02 spec.rs body_inner (lm_head_argmax writes the per-row
 * token g and its maximum am_val; logits are not materialised) and
 * greedy_logprob (the FIRST maximum wins); flashrt whole_step.py _gstep (argmax
 * on fp32 logits, not bf16); memra-engine spec.rs decode_step_t (lm_head on the
 * normed hidden rows).
 *
 *   logit[r, v] = sum_i w[v, i] * hidden[r, i]      (bf16 products, fp32 sums)
 *   argmax[r]   = smallest v with logit[r, v] == max_v logit[r, v]
 *   maxval[r]   = that maximum (fp32)                (maxval may be NULL)
 *
 * The weight is passed packed (see spec_lm_head_pack), the way the pages' engines
 * keep their weights in kernel-specific block formats; packing is a byte
 * permutation done once per weight, so every logit is the same.
 * Layouts: hidden [R][H] bf16, w_packed spec_lm_head_packed_bytes(V, H) bytes,
 * argmax [R] int32, maxval [R] fp32.
 * Limits: R >= 1, H % 256 == 0, 1 <= V < 2^31 - 1; 16-byte aligned hidden,
 * w_packed, workspace. NaN logits never win. workspace: at least
 * spec_lm_head_argmax_workspace_bytes(R, H, V) bytes: a ticket counter and one
 * 64-bit key per row, through which the workgroups merge their per-row maxima, and
 * for R <= 96, after the per-row keys padded to a multiple of 8, one 64-bit key per
 * (vocabulary workgroup, row) in rows of that padded length, through which a second
 * small kernel merges them instead (this call up to R = 64, spec_lm_head_argmax_accept
 * up to 96) (a workspace of at least the ticket
 * and per-row keys but too small for these makes the call take the first way: the
 * same result; smaller than that: SPEC_EWORKSPACE). The workspace must be all zero
 * the first time it is used; every call leaves it zero again, so a workspace is
 * zero-filled once and then reused, also for other row counts and across HIP graph
 * replays. Calls that may overlap in time must not share a workspace.
 * ------------------------------------------------------------------------- */
size_t spec_lm_head_argmax_workspace_bytes(int32_t R, int32_t H, int32_t V);
int spec_lm_head_argmax(const spec_bf16* hidden, const spec_bf16* w_packed, int32_t R, int32_t H,
                        int32_t V, int32_t* argmax, float* maxval, void* workspace,
                        size_t workspace_bytes, void* stream);

/* spec_lm_head_argmax_noalloc — spec_lm_head_argmax with no workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). It computes exactly what
 * spec_lm_head_argmax computes (the same tile kernel, so the same bytes; at R <= 64
 * it merges the per-row maxima through the per-row keys, as at larger R) and calls no
 * allocating routine: its ticket and per-row keys live in a library-owned device
 * array of SPEC_NOALLOC_SCRATCH_BYTES bytes per GPU, which holds them for rows
 * R <= SPEC_NOALLOC_MAX_ROWS (larger R: SPEC_ECAPACITY, nothing launched). Each call
 * first clears the part of the array it uses with a small fill kernel on the
 * caller's stream, then runs the lm_head. The array is shared by every call on one
 * GPU: calls that may overlap in time on the same GPU race and must be ordered by
 * the caller (e.g. one stream). Arguments, layouts and the other limits as
 * spec_lm_head_argmax. */
#define SPEC_NOALLOC_MAX_ROWS 8192
#define SPEC_NOALLOC_SCRATCH_BYTES (256 + 8 * SPEC_NOALLOC_MAX_ROWS)
int spec_lm_head_argmax_noalloc(const spec_bf16* hidden, const spec_bf16* w_packed, int32_t R, int32_t H,
                                int32_t V, int32_t* argmax, float* maxval, void* stream);

/* spec_lm_head_pack — one-time re-layout of a row-major lm_head weight w [V][H]
 * (bf16) into the packed form spec_lm_head_argmax reads. Vocabulary rows are
 * taken in groups of 128 and channels in K-blocks of 128; a group stores its
 * K-blocks in order, each K-block its 8 tiles of 16 rows, each tile its 4 k-steps
 * of 32 channels as 64 lanes x 8 bf16 in MFMA B-fragment order. Fragment
 *   f = (((g * H/128 + b) * 8 + t) * 4 + s) * 64 + lane
 * holds w[128g + 16t + lane % 16][128b + 32s + 8(lane / 16) .. +8]; rows past V
 * are zero. w_packed holds spec_lm_head_packed_bytes(V, H) = ceil(V/128) * 128 *
 * H * 2 bytes and must not overlap w. Limits as above. */
size_t spec_lm_head_packed_bytes(int32_t V, int32_t H);
int spec_lm_head_pack(const spec_bf16* w, int32_t V, int32_t H, spec_bf16* w_packed, void* stream);

/* ---------------------------------------------------------------------------
 * spec_greedy_accept — greedy acceptance and rollback bookkeeping.
 *
 * Defined by: span-02 spec.rs module doc (a draft survives only while it matches
 * the target's greedy choice at the row that verifies it; rollback moves pos past
 * the accepted tokens) and step_chunk (next pos = pos + a + 1, next token = last
 * emitted); DSSD fast.py generate_spec (first miss stops; target[len(committed)]
 * appended as correction or bonus); oxinfer qwen_mtp.rs speculative_accept
 * (greedy case: accept iff the draft is the target argmax, else emit the
 * argmax) and DraftHead (draft id i stands for target id d2t[i]); flashrt
 * generate_speculative (device prefix match, pos += j + 1).
 *
 * With map(x) = d2t ? d2t[x] : x and g = argmax (packed rows):
 *   a_s         = number of leading j < k_s with map(drafts[s, j]) == g[off_s + j]
 *   emit[s, :]  = map(drafts[s, 0..a_s)) ++ [g[off_s + a_s]], then -1 up to kmax + 1
 *   accept_len[s] = a_s, n_emit[s] = a_s + 1, next_tok[s] = g[off_s + a_s]
 *   pos_out[s]  = pos_in[s] + a_s + 1      (pos_out may alias pos_in)
 *
 * Layouts: argmax [R], drafts [B][kmax] (only the first k_s of a row are read),
 * k [B], d2t [n_draft_vocab] (NULL: drafts are target ids), pos_in, pos_out,
 * accept_len, n_emit, next_tok, seq_status [B], emit [B][kmax + 1]; all int32.
 * A flagged sequence gets accept_len = -1, n_emit = 0, next_tok = -1,
 * pos_out = pos_in and an all -1 emit row. Only the d2t entries that drafts
 * reference are checked. Limits: 1 <= B <= 8192, 0 <= kmax <= 1024, R >= 1, V >= 1.
 * ------------------------------------------------------------------------- */
int spec_greedy_accept(const int32_t* argmax, const int32_t* drafts, int32_t kmax,
                       const int32_t* k, const int32_t* d2t, int32_t n_draft_vocab, int32_t V,
                       int32_t B, int32_t R, const int32_t* pos_in, int32_t* pos_out,
                       int32_t* accept_len, int32_t* n_emit, int32_t* emit, int32_t* next_tok,
                       int32_t* seq_status, void* stream);

/* spec_lm_head_argmax_accept — spec_lm_head_argmax followed by spec_greedy_accept
 * on its argmax, as one call: the same outputs, bit for bit (argmax, maxval when
 * non-NULL, and every acceptance output and status), with the arguments of the two
 * calls (R, the packing of k and the workspace as there; the workspace is sized by
 * spec_lm_head_argmax_workspace_bytes(R, H, V), must be zero the first time it is
 * used and is left zero). Defined by the two passages cited for those calls; the
 * fusion is this library's: for R <= 96 with the full workspace the per-row maxima
 * over vocabulary groups are taken by the acceptance kernel itself (one workgroup
 * per sequence merges its own rows' keys, then one wave walks its drafts), which
 * saves the separate finalize of the few-row path and one launch. Otherwise it runs
 * the two calls' kernels in turn. Returns the first error of either call's checks
 * before launching anything that call would launch.
 * ------------------------------------------------------------------------- */
int spec_lm_head_argmax_accept(const spec_bf16* hidden, const spec_bf16* w_packed, int32_t R, int32_t H,
                               int32_t V, int32_t* argmax, float* maxval, const int32_t* drafts, int32_t kmax,
                               const int32_t* k, const int32_t* d2t, int32_t n_draft_vocab, int32_t B,
                               const int32_t* pos_in, int32_t* pos_out, int32_t* accept_len, int32_t* n_emit,
                               int32_t* emit, int32_t* next_tok, int32_t* seq_status, void* workspace,
                               size_t workspace_bytes, void* stream);

/* spec_greedy_accept_stop — spec_greedy_accept with stop tokens and a generation
 * limit (oxinfer step: an accepted stop token ends the round, the committed tokens
 * end at the first stop token and the session advances by the number committed;
 * DSSD _commit: truncation at a stop token or at max_new).
 * With out = map(drafts[s][0..a)) ++ [argmax[off_s + a]] (the greedy round):
 *   c = the length of out up to and including its first token in stop_ids (host
 *       count n_stop <= 16, device array), then min(c, remaining[s]);
 *   n_emit = c, emit = out[0..c) (-1 after), accept_len = min(a, c),
 *   next_tok = out[c - 1], pos_out = pos_in + c,
 *   done [B] int32 = 1 iff out[c - 1] is a stop token or c == remaining[s].
 * remaining [B] int32 (tokens the sequence may still emit) may be NULL (no limit);
 * remaining[s] < 1 sets SPEC_STATUS_BAD_LIMIT. Flagged sequences as
 * spec_greedy_accept, with done = 0. */
int spec_greedy_accept_stop(const int32_t* argmax, const int32_t* drafts, int32_t kmax, const int32_t* k,
                            const int32_t* d2t, int32_t n_draft_vocab, int32_t V, int32_t B, int32_t R,
                            const int32_t* stop_ids, int32_t n_stop, const int32_t* remaining,
                            const int32_t* pos_in, int32_t* pos_out, int32_t* accept_len, int32_t* n_emit,
                            int32_t* emit, int32_t* next_tok, int32_t* done, int32_t* seq_status, void* stream);

/* spec_truncate_stop — the same stop-token and limit rule, applied in place to the
 * outputs of any acceptance walk: spec_greedy_accept, spec_tree_accept (with its
 * path) or spec_sample_accept (oxinfer step and DSSD _commit as above; a tree or a
 * sampled round commits its emitted tokens in the same way).
 * In/out [B] int32: pos_out, accept_len, n_emit, next_tok, seq_status;
 * emit [B][kmax+1] and path [B][kmax] (NULL for chain walks) int32, in/out; pos_in
 * [B] the walk's input positions; done [B] int32 output. For each s with
 * seq_status[s] == 0 on entry, with out = emit[s][0 .. n_emit):
 *   c = the length of out up to and including its first token in stop_ids, then
 *       min(c, remaining[s]);
 *   n_emit = c, emit = out[0..c) (-1 after), accept_len = min(accept_len, c),
 *   path keeps its first accept_len entries (-1 after), next_tok = out[c - 1],
 *   pos_out = pos_in + c, done = 1 iff out[c - 1] is a stop token or
 *   c == remaining[s].
 * A tree round then calls spec_kv_compact with the truncated path and accept_len,
 * so that only committed nodes move. remaining may be NULL (no limit);
 * remaining[s] < 1 sets SPEC_STATUS_BAD_LIMIT, and n_emit outside 1 .. kmax + 1 or
 * accept_len outside 0 .. n_emit sets SPEC_STATUS_BAD_ROWS; such a sequence gets
 * the flagged outputs of its walk (accept_len -1, n_emit 0, next_tok -1,
 * pos_out = pos_in, emit and path all -1). Sequences flagged on entry are left as
 * they are, with done = 0. Applying the call twice gives the result of once.
 * Limits: B >= 1, 0 <= kmax <= 1024, 0 <= n_stop <= 16. */
int spec_truncate_stop(int32_t kmax, int32_t B, const int32_t* stop_ids, int32_t n_stop, const int32_t* remaining,
                       const int32_t* pos_in, int32_t* pos_out, int32_t* accept_len, int32_t* n_emit, int32_t* emit,
                       int32_t* next_tok, int32_t* path, int32_t* done, int32_t* seq_status, void* stream);

/* ---------------------------------------------------------------------------
 * spec_delta_verify_rollback — Gated DeltaNet verify with per-token state
 * recording, and rollback to the committed prefix.
 *
 * Defined by: oxinfer qwen_mtp.rs module doc (the Gated DeltaNet states are
 * recorded per token during the verify forward, so a partial acceptance
 * restores them exactly instead of re-running the accepted tokens); memra-engine
 * spec.rs decode_step_t_core_stream (per-column state clones) and
 * linear_attn_verify_t (one scan over T tokens equals T chained one-token
 * steps); flashrt whole_step.py (the gated-delta states roll back on a partial
 * accept). The update is the gated delta rule
 *   S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t (q_scale q_t)
 * with S [dv][dk] (row = value channel), fp32 state and arithmetic.
 *
 * mode 1 (RECORD):   from S_0 = state, run t = 1..T; rec[s, t-1, h] = S_t,
 *                    o[s, t-1, h] = o_t. state is not modified.
 * mode 2 (ROLLBACK): state[s, h] = rec[s, L[s]-1, h] when L[s] >= 1; L[s] = 0
 *                    leaves S_0. Bit-exact copy.
 * mode 3 (BOTH):     mode 1, then state <- S_{L[s]} in the same pass.
 * mode 4 (VERIFY):   from S_0 = state, run t = 1..T; o only (no record; state and
 *                    rec untouched, rec may be NULL).
 * mode 5 (RESCAN):   state <- S_{L[s]} by running t = 1..L[s] again from the
 *                    retained S_0 = state (L[s] = 0 leaves it); o and rec untouched.
 * Modes 4 + 5 are the input-stash alternative to 1 + 2 (memra-engine spec.rs: keep
 * the round's inputs and the pre-round state, and on a partial accept re-run the
 * accepted prefix): S_0 is read twice and S_L written, instead of T states recorded.
 * Iteration t does the same arithmetic in every mode, so mode 5 gives the bytes of
 * rec[L-1] from mode 1.
 * L[s] = committed tokens in 0..T (the greedy flow commits a_s + 1); values
 * outside 0..T are clamped.
 *
 * Layouts: q, k [B][T][Hd][dk] bf16; v [B][T][Hd][dv] bf16; a, b [B][T][Hd] fp32;
 * state [B][Hd][dv][dk] fp32; rec [B][T][Hd][dv][dk] fp32; L [B] int32 (may be
 * NULL in modes 1 and 4); o [B][T][Hd][dv] bf16 (may be NULL; unused in modes 2
 * and 5); rec may be NULL in modes 4 and 5.
 * Limits: dk == dv == 128, 1 <= T <= 64, B, Hd >= 1; 16-byte aligned state, rec.
 * ------------------------------------------------------------------------- */
#define SPEC_DELTA_RECORD 1
#define SPEC_DELTA_ROLLBACK 2
#define SPEC_DELTA_BOTH 3
#define SPEC_DELTA_VERIFY 4
#define SPEC_DELTA_RESCAN 5
int spec_delta_verify_rollback(int32_t mode, const spec_bf16* q, const spec_bf16* k,
                               const spec_bf16* v, const float* a, const float* b, float q_scale,
                               float* state, float* rec, const int32_t* L, int32_t B, int32_t T,
                               int32_t Hd, int32_t dk, int32_t dv, spec_bf16* o, void* stream);

/* ---------------------------------------------------------------------------
 * Tree drafts (trie or star).
 *
 * Defined by: DSSD fast.py _set_rows (tree rows carry a position, a KV slot, the
 * length of the contiguous prefix they read and the slots of their path),
 * _tree_cycle (rows are the trie's nodes in creation order; node i sits at
 * position pos + depth(i), writes its K/V at slot pos + i and attends to slots
 * [0, pos] and to the slots of its own path; the walk from the root follows the
 * child whose token equals the current node's target; the accepted path's K/V is
 * compacted to slots pos + 1, ...) and _star_cycle (the depth-1 case: children at
 * position pos + 1 on slots pos + 1 + i; the first child whose token matches).
 *
 * The k_s + 1 rows of sequence s (packed as for the chain calls) are its tree's
 * nodes in creation order: row j is node j, node 0 the root (the last emitted
 * token), node i >= 1 carries drafts[s][i - 1]. parent [B][kmax + 1] int32 holds
 * parent[s][0] = -1 and parent[s][i] in [0, i) for 1 <= i <= k_s (entries past
 * k_s are unread); anything else flags the sequence SPEC_STATUS_BAD_TREE.
 * path(j) = the nodes from the root's child down to j (empty for the root).
 * The caller computes row j's position pos + depth(j) (for RoPE and the like)
 * from the same parent list; the library needs only slots.
 * A chain (parent[s][i] = i - 1) gives the results of the chain calls.
 * ------------------------------------------------------------------------- */

/* spec_verify_attn_tree — KV append + attention over tree rows (one layer).
 * As spec_verify_attn (same layouts, limits, split-KV rule, workspace rules,
 * status bits and skip behaviour), except that row j of sequence s appends at slot
 * pos[s] + j and attends, for query head h, to the key slots
 *   t in {0, ..., pos[s]}  followed by  {pos[s] + u : u in path(j)}
 * (ascending slot order, which is the path's root-to-leaf order), i.e.
 *   out[r, h, :] = sum_t softmax_t(scale * q[r,h,:] . K_t[hk,:]) V_t[hk,:].
 * Bytes: row j's output is bit-identical to spec_verify_attn's one-row decode of
 * the same query at position pos[s] + depth(j) (same kv_split_tokens) over a pool
 * whose slots pos[s] + 1 .. pos[s] + depth(j) hold path(j)'s K/V in order, i.e. to
 * its decode after the accepted path is compacted (DSSD fast.py _attention: one
 * query per row over its exact path). Inputs are finite.
 * Extra limits: kmax <= 127, and the workgroup's LDS (the 64-token tile, K and V
 * of kmax new rows, 20 bytes per node and 4 paths) must fit gfx950's 160 KB: at
 * D = 256 that means kmax <= 93 (SPEC_EINVAL otherwise).
 * workspace: spec_verify_attn_tree_workspace_bytes. */
size_t spec_verify_attn_tree_workspace_bytes(int32_t B, int32_t R, int32_t Hq, int32_t Hkv, int32_t D,
                                             int32_t max_pages, int32_t kv_split_tokens, int32_t kmax);
int spec_verify_attn_tree(const spec_bf16* q, const spec_bf16* k_new, const spec_bf16* v_new,
                          spec_bf16* k_pool, spec_bf16* v_pool, int64_t n_pages,
                          const int32_t* page_table, int32_t max_pages, const int32_t* pos,
                          const int32_t* k, const int32_t* parent, int32_t kmax, int32_t B, int32_t R,
                          int32_t Hq, int32_t Hkv, int32_t D, float scale, int32_t kv_split_tokens,
                          spec_bf16* out, void* workspace, size_t workspace_bytes, int32_t* seq_status,
                          void* stream);

/* spec_tree_accept — the greedy acceptance walk over a tree.
 * argmax [R] int32 (the greedy token of every row), drafts [B][kmax], d2t,
 * n_draft_vocab, V, pos_in and the outputs as spec_greedy_accept; parent as above;
 * path [B][kmax] int32 (output).
 * Walk: u = root; while some child c of u (parent[s][c] == u) has
 * map(drafts[s][c - 1]) == argmax[off_s + u], move to the lowest-index such c.
 * With accepted nodes u_1 .. u_a:
 *   accept_len = a, emit[s][0..a] = map(tokens of u_1..u_a), argmax[off_s + u_a]
 *   (-1 after), n_emit = a + 1, next_tok = argmax[off_s + u_a],
 *   pos_out = pos_in + a + 1, path[s] = u_1 .. u_a (-1 after).
 * A flagged sequence (status bits as spec_greedy_accept, plus BAD_TREE) gets
 * accept_len -1, n_emit 0, next_tok -1, pos_out = pos_in, emit and path all -1.
 * Limits: 1 <= B <= 8192, 0 <= kmax <= 127, R >= 1, V >= 1. */
int spec_tree_accept(const int32_t* argmax, const int32_t* drafts, int32_t kmax, const int32_t* k,
                     const int32_t* parent, const int32_t* d2t, int32_t n_draft_vocab, int32_t V, int32_t B,
                     int32_t R, const int32_t* pos_in, int32_t* pos_out, int32_t* accept_len,
                     int32_t* n_emit, int32_t* emit, int32_t* next_tok, int32_t* path, int32_t* seq_status,
                     void* stream);

/* spec_kv_compact — moves the accepted path's K/V to contiguous slots.
 * For every sequence with seq_status[s] == 0 on entry: for d = 0 .. accept_len[s]-1
 * the K and V of slot pos[s] + path[s][d] (every kv head) are copied to slot
 * pos[s] + 1 + d, with the result of doing so in ascending d. Afterwards slots
 * 0 .. pos + a hold what a chain of the accepted tokens would have written, and
 * the next cycle's pos is pos + a + 1. Call it with the pos_in, path and
 * accept_len of spec_tree_accept, once per layer's pool.
 * Checks before any write (then the sequence is flagged and nothing moves):
 * accept_len <= kmax, 1 <= path[d] <= kmax strictly increasing (BAD_TREE), pos >= 0
 * and every slot's page inside the page table (BAD_POS), page ids in [0, n_pages)
 * (BAD_PAGE). seq_status is in/out: nonzero entries are left as they are (the
 * sequence is skipped), zero entries receive these bits.
 * Layouts as spec_verify_attn. Limits: D in {64, 128, 256}, 1 <= Hkv <= 64,
 * B >= 1, 0 <= kmax <= 127; 16-byte aligned pools. */
int spec_kv_compact(spec_bf16* k_pool, spec_bf16* v_pool, int64_t n_pages, const int32_t* page_table,
                    int32_t max_pages, const int32_t* pos, const int32_t* path, const int32_t* accept_len,
                    int32_t kmax, int32_t B, int32_t Hkv, int32_t D, int32_t* seq_status, void* stream);

/* ---------------------------------------------------------------------------
 * Speculative-sampling verify.
 *
 * Defined by: DSSD fast.py _sample_verify (exact speculative sampling on a chain:
 * draft i is kept with probability min(1, p_i(x_i) / q_i(x_i)); at the first
 * rejection the token is drawn from norm(max(p_i - q_i, 0)); if every draft is kept
 * the bonus is drawn from p_n; p = softmax(logits / temperature)); oxinfer
 * speculative_accept (the same test, q given as (token, probability) pairs, the
 * resulting token distributed exactly as p); memra's sampled-spec note
 * (counter-based Philox keyed by seed and event, so that runs are reproducible).
 *
 * Random numbers: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, SC 2011) with key
 * (seed & 0xffffffff, seed >> 32); a word w gives u = (floor(w / 512) + 1/2) / 2^23.
 * Each row r carries two caller-chosen counter words row_ctr[r] = (a, b), e.g. the
 * row's position and a request id, so that a sequence's draws do not depend on the
 * batch it shares:
 *   Gumbel noise of entry v of row r:  G = -ln(-ln u), u from word v % 4 of
 *                                      counter (v / 4, a, b, 0)
 *   acceptance uniform of row r:       u from word 0 of counter (0, a, b, 1)
 * Draws use the Gumbel-max rule: the argmax of log-weight + G over the entries is a
 * draw from the normalised weights (ties to the smaller index).
 *
 * The draft distribution of row r (the row that verifies draft j of its sequence)
 * is sparse: up to NQ <= 8 support tokens q_tok[r][e] (-1 = unused) with masses
 * q_prob[r][e] (a point mass: one token with mass 1). Bonus rows have no support.
 * ------------------------------------------------------------------------- */

/* spec_lm_head_sample — for every row r of hidden [R][H] against the packed W:
 *   z_v = logit_v / temperature  (logit as in spec_lm_head_argmax, fp32)
 *   lse[r]        = ln sum_v exp(z_v)
 *   z_supp[r][e]  = z of q_tok[r][e] (NaN for unused entries)
 *   sample_p[r]   = argmax_v z_v + G_v                         (a draw from p)
 *   sample_res[r] = argmax_{v : p_v > q_v} ln(p_v - q_v) + G_v  (a draw from
 *                   norm(max(p - q, 0)); sample_p[r] if that set is empty)
 * with q_v the summed mass of v in the row's support. Logits never reach memory:
 * the tile kernel leaves one record per (row, vocabulary group) (softmax partials
 * and the best z + G outside the support as a packed 64-bit key) and the support
 * z's; a per-row kernel reduces the records in a fixed order and forms the draws.
 * workspace: spec_lm_head_sample_workspace_bytes(R, H, V) bytes, any contents
 * (every call writes the records it reads; calls sharing one must not overlap).
 * Limits as spec_lm_head_argmax; 0 <= NQ <= 8; temperature finite and > 0. */
size_t spec_lm_head_sample_workspace_bytes(int32_t R, int32_t H, int32_t V);
int spec_lm_head_sample(const spec_bf16* hidden, const spec_bf16* w_packed, int32_t R, int32_t H, int32_t V,
                        float temperature, const int32_t* q_tok, const float* q_prob, int32_t NQ,
                        const int32_t* row_ctr, uint64_t seed, float* lse, float* z_supp, int32_t* sample_p,
                        int32_t* sample_res, void* workspace, size_t workspace_bytes, void* stream);

/* spec_sample_accept — the chain walk. For sequence s (rows off_s .. off_s + k_s,
 * packed as for the greedy call) and j = 0 .. k_s - 1, row r = off_s + j, draft
 * x = map(drafts[s][j]) (d2t as in spec_greedy_accept), q_x = the summed mass of
 * the row's support entries holding x (the same q_v as the residual draw uses) and
 * e the first entry holding x:
 *   keep x iff u_r < exp(z_supp[r][e] - lse[r]) / q_x
 *   else emit sample_res[r] and stop;
 * if every draft is kept, emit sample_p[off_s + k_s]. Outputs as
 * spec_greedy_accept (accept_len, n_emit = accept_len + 1, emit [B][kmax + 1] with
 * -1 after the last token, next_tok = the drawn token, pos_out = pos_in +
 * accept_len + 1). A draft outside its row's support (q_x <= 0), or outside its
 * vocabulary, sets SPEC_STATUS_BAD_TOKEN; status bits and the outputs of a flagged sequence as
 * spec_greedy_accept. lse, z_supp, sample_p and sample_res are the outputs of
 * spec_lm_head_sample for the same rows, row_ctr and seed.
 * Limits: 1 <= B <= 8192, 0 <= kmax <= 1024, R >= 1, V >= 1, 0 <= NQ <= 8. */
int spec_sample_accept(const int32_t* drafts, int32_t kmax, const int32_t* k, const int32_t* d2t,
                       int32_t n_draft_vocab, int32_t V, int32_t B, int32_t R, const int32_t* q_tok,
                       const float* q_prob, int32_t NQ, const float* lse, const float* z_supp,
                       const int32_t* sample_p, const int32_t* sample_res, const int32_t* row_ctr, uint64_t seed,
                       const int32_t* pos_in, int32_t* pos_out, int32_t* accept_len, int32_t* n_emit,
                       int32_t* emit, int32_t* next_tok, int32_t* seq_status, void* stream);

/* Dense draft distributions (DSSD _sample_verify with the draft head's whole
 * distribution): q [R][V] fp32 gives q_r(v) for every target-vocabulary entry. The
 * residual of a rejected row, norm(max(p_r - q_r, 0)), then needs that row's whole
 * p, so the pass keeps every z (R * V * 4 bytes) and the walk draws the residual. */

/* spec_lm_head_sample_dense — spec_lm_head_sample with no support list: lse[r] and
 * sample_p[r] (a draw from p of every row) as there, and z [R][V] fp32 = z_v of every
 * entry (logit / temperature). Workspace, limits and temperature as
 * spec_lm_head_sample (the same workspace size). */
int spec_lm_head_sample_dense(const spec_bf16* hidden, const spec_bf16* w_packed, int32_t R, int32_t H, int32_t V,
                              float temperature, const int32_t* row_ctr, uint64_t seed, float* lse, int32_t* sample_p,
                              float* z, void* workspace, size_t workspace_bytes, void* stream);

/* spec_sample_accept_dense — the chain walk with q [R][V]. For sequence s and
 * j = 0 .. k_s - 1, row r = off_s + j, draft x = map(drafts[s][j]):
 *   q[r][x] <= 0 (a draft the draft distribution cannot produce) or x outside its
 *   vocabulary: SPEC_STATUS_BAD_TOKEN;
 *   keep x iff u_r < exp(z[r][x] - lse[r]) / q[r][x];
 *   else the token is argmax over {v : p_v > q_v} of ln(p_v - q_v) + G_v with
 *   p_v = exp(z[r][v] - lse[r]) and the row's Gumbel noise G (the first such v on
 *   a tie; sample_p[r] if that set is empty in fp32), and the walk stops;
 * if every draft is kept, emit sample_p[off_s + k_s]. Outputs, status bits and the
 * outputs of a flagged sequence as spec_sample_accept. z, lse and sample_p come from
 * spec_lm_head_sample_dense for the same rows, row_ctr and seed.
 * workspace: spec_sample_accept_dense_workspace_bytes(B) bytes (any contents; the
 * call initialises what it uses; calls sharing one must not overlap).
 * Limits: 1 <= B <= 8192, 0 <= kmax <= 1024, R >= 1, V >= 1. */
size_t spec_sample_accept_dense_workspace_bytes(int32_t B);
int spec_sample_accept_dense(const int32_t* drafts, int32_t kmax, const int32_t* k, const int32_t* d2t,
                             int32_t n_draft_vocab, int32_t V, int32_t B, int32_t R, const float* q, const float* z,
                             const float* lse, const int32_t* sample_p, const int32_t* row_ctr, uint64_t seed,
                             const int32_t* pos_in, int32_t* pos_out, int32_t* accept_len, int32_t* n_emit,
                             int32_t* emit, int32_t* next_tok, int32_t* seq_status, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Adaptive draft depth (host side; no GPU work, no allocation).
 *
 * Defined by: span-02 spec.rs KPolicy (a smoothed estimate of how often draft
 * position j is kept once every earlier position was, a verify cost that grows
 * piecewise linearly with the rows, and k picked for the least expected time per
 * emitted token) and oxinfer DraftCosts (the same trade-off from measured round
 * times and per-position acceptance rates). For positions j and depths k:
 *   p_j       = (kept[j] + prior_p * prior_n) / (tried[j] + prior_n)
 *   E(k)      = sum_{i=0..k} p_0 p_1 ... p_{i-1}   (kept drafts + the bonus; the
 *               i = 0 term is 1)
 *   verify(r) = the polyline through (0, 0) and the (cost_rows, cost_us) points,
 *               its last piece continued past the last point
 *   choose(B) = the smallest k in kmin .. kmax with the least
 *               (verify(B (k + 1)) + k draft_us) / E(k); with row_cap > 0 the top
 *               is lowered to max(row_cap / B - 1, kmin)
 *   update(k, a): tried[j] += 1 for j < min(k, a + 1); kept[j] += 1 for j < min(k, a)
 * The caller owns the struct (plain data; copy it freely).
 * ------------------------------------------------------------------------- */
#define SPEC_KPOLICY_MAXK 64
#define SPEC_KPOLICY_MAXPTS 32
typedef struct {
    int32_t kmin, kmax;
    double prior_p, prior_n;
    double draft_us;                  /* cost of drafting one more token, per cycle */
    int32_t n_points;                 /* verify cost table: rows (increasing) -> us */
    double cost_rows[SPEC_KPOLICY_MAXPTS];
    double cost_us[SPEC_KPOLICY_MAXPTS];
    double tried[SPEC_KPOLICY_MAXK];  /* rounds that reached draft position j */
    double kept[SPEC_KPOLICY_MAXK];   /* ... and kept its draft */
} spec_kpolicy;

/* Sets every field and zeroes the counters. EINVAL unless 0 <= kmin <= kmax < 64,
 * 0 < prior_p <= 1, prior_n > 0, draft_us >= 0, 1 <= n_points <= 32 with positive,
 * strictly increasing rows and finite non-negative costs. All pointers are host. */
int spec_kpolicy_init(spec_kpolicy* p, int32_t kmin, int32_t kmax, double prior_p, double prior_n, double draft_us,
                      const double* cost_rows, const double* cost_us, int32_t n_points);
double spec_kpolicy_accept_prob(const spec_kpolicy* p, int32_t j);
double spec_kpolicy_verify_cost(const spec_kpolicy* p, double rows);
double spec_kpolicy_expected_tokens(const spec_kpolicy* p, int32_t k);
/* The chosen k (>= kmin), or -1 for a null policy or B < 1. */
int32_t spec_kpolicy_choose(const spec_kpolicy* p, int32_t B, int32_t row_cap);
void spec_kpolicy_update(spec_kpolicy* p, int32_t k, int32_t accepted);
/* update for every sequence with accept_len[s] >= 0 (host arrays k[B], accept_len[B];
 * flagged sequences, -1, are skipped). */
int spec_kpolicy_update_batch(spec_kpolicy* p, const int32_t* k, const int32_t* accept_len, int32_t B);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
