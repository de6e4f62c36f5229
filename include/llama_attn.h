/*
 * llama_attn.h — C ABI of a gfx950 (MI355X) library for the attention step of
 * the Llama 3.1 dense decoder: rotary position embeddings on queries and keys,
 * then grouped-query causal self-attention under the cross-document mask, for
 * prefill (many tokens) and for decode over a KV cache.
 *
 * What the calls compute comes from these web pages:
 *   [P1] "Llama 3.1 Architecture: Dense Scaling to 405B and 128K Context",
 *        section "Context Expansion: From 8K to 128K via RoPE Frequency
 *        Scaling", subsection "1. High Base Frequency" (the theta_k equation),
 *        and the "Architectural Deep Dive" flowchart (128 query heads on 8 KV
 *        heads, 16:1);
 *   [P2] "How Meta's Llama 3.1 405B Architecture Actually Works", the GQA
 *        paragraph (query heads grouped onto a shared key/value head, which
 *        shrinks the KV cache during decoding);
 *   [P4] "The Llama 3 Herd of Models", Chapter Roadmap entry "A Deliberately
 *        Standard Dense Transformer" (GQA with 8 KV heads, RoPE base 500,000,
 *        cross-document attention mask).
 *
 * Conventions shared by every call
 *   - Every tensor pointer is a DEVICE pointer on the current HIP device; the
 *     caller allocates and frees all memory (including the decode workspace).
 *     The library allocates nothing and keeps no pointer after returning.
 *   - Strides are in ELEMENTS. The innermost (head_dim) stride is always 1.
 *     Base pointers must be 16-byte aligned and every stride a multiple of
 *     16 bytes' worth of elements (8 for bf16, 4 for fp32).
 *   - All work is enqueued on `stream` (0 = the null stream) and is
 *     asynchronous: no call synchronises.
 *   - A bf16 gqa_prefill, gqa_prefill_rope or gqa_prefill_chunk with at least
 *     16 work items (sequence x KV head x query tile) per compute unit runs
 *     on a persistent grid: one workgroup per compute unit, taking its items
 *     from work-queue counters the library keeps in device memory, one set
 *     per stream for the first 64 streams of a device (any other stream, and
 *     a stream under graph capture, gets one workgroup per item). Calls on one
 *     stream run in order and leave the counters at zero; calls on different
 *     streams use different counters. The environment variable
 *     LLAMA_ATTN_PERSISTENT=0 turns the persistent grid off; a positive
 *     number n sets it to n workgroups wherever the items outnumber them.
 *   - All argument checks are made on the host before anything is enqueued;
 *     on any error nothing is launched. Device-resident CONTENTS (document
 *     offsets, sequence lengths, positions) are the caller's contract and are
 *     not read on the host.
 *   - Head mapping: query head h reads KV head h / (Hq / Hkv) (contiguous
 *     groups) [P2, P4].
 *   - RoPE rotates channel pair k by the angle position * theta_k,
 *     theta_k = rope_base^(-2k/D), k = 0..D/2-1 [P1]. Every call that takes
 *     rope_base also takes rope_pairing: 0 pairs adjacent channels (2k, 2k+1)
 *     (RoFormer's layout, which [P1] cites), 1 pairs channel k with k + D/2
 *     (the half-split layout; the pages do not fix the layout). Any other
 *     value is INVALID_ARG.
 *   - Supported: D in {64, 128}; Hq / Hkv in {1, 2, 4, 8, 16}.
 */
#ifndef LLAMA_ATTN_H
#define LLAMA_ATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LA_OK = 0,
  LA_ERR_INVALID_ARG = 1,   /* null pointer, bad size, stride or alignment */
  LA_ERR_UNSUPPORTED = 2,   /* a shape or dtype this library has no kernel for */
  LA_ERR_LAUNCH = 3,        /* the HIP runtime refused the launch */
  LA_ERR_SCRATCH = 4        /* gqa_decode_noalloc: the working set exceeds its scratch */
} la_status;

typedef enum { LA_BF16 = 0, LA_FP32 = 1 } la_dtype;

/* Pieces of a key block's query range in gqa_attention_backward. */
#define LA_BWD_PIECES 4

/* Human-readable name of a status code (static storage; never NULL). */
const char* la_status_str(la_status s);

/* Library version as major*10000 + minor*100 + patch. */
int la_version(void);

/*
 * rope_qk — rotary position embedding of queries and keys [P1].
 *
 * q_in/q_out: [B, S, Hq, D] with strides q_in_strides / q_out_strides = (b, s, h);
 * k_in/k_out: [B, S, Hkv, D] with strides k_in_strides / k_out_strides.
 * Element type `dt` for inputs and outputs (bf16 results are rounded to
 * nearest even from an fp32 rotation; the angle position*theta_k is formed and
 * reduced modulo 2*pi in fp64). Values are not rotated.
 * positions: int32 [B, S] (row-major, position of token s of sequence b), or
 * NULL for position = s. k_in/k_out may be NULL together (queries only) and
 * so may q_in/q_out (keys only); at least one pair must be given.
 * In place is allowed (q_out == q_in, k_out == k_in); other overlap is not.
 * Errors: INVALID_ARG for B, S, H < 1, rope_base <= 0, bad strides or
 * alignment; UNSUPPORTED for D not in {64, 128} or an unknown dtype.
 */
la_status rope_qk(const void* q_in, void* q_out, const int64_t q_in_strides[3],
                  const int64_t q_out_strides[3],
                  const void* k_in, void* k_out, const int64_t k_in_strides[3],
                  const int64_t k_out_strides[3],
                  la_dtype dt, int B, int S, int Hq, int Hkv, int D,
                  const int32_t* positions, double rope_base, int rope_pairing, hipStream_t stream);

/*
 * gqa_prefill — grouped-query causal attention with the cross-document mask,
 * on queries and keys that are ALREADY ROTATED (see rope_qk) [P2, P4].
 *
 * q: [B, S, Hq, D], k and v: [B, S, Hkv, D], o: [B, S, Hq, D], all of type
 * `dt`, strides (b, s, h) in q_strides, k_strides, v_strides, o_strides; the
 * token strides of k and v are at least D (rows do not overlap).
 * cu_docs: int32 [B, n_docs + 1], row b non-decreasing from 0 to S: document
 *   d of sequence b is the token range [cu_docs[b][d], cu_docs[b][d+1])
 *   (empty documents are allowed and hold no token). NULL means one document
 *   per sequence (n_docs is then ignored).
 * Key j is visible to query i iff j <= i and both lie in the same document.
 * Scores are (q_i . k_j) * softmax_scale (softmax_scale <= 0 means 1/sqrt(D));
 * o_i is the softmax-weighted sum of the visible v_j.
 * lse: optional fp32 [B, Hq, S] (contiguous): natural-log log-sum-exp of each
 *   row's visible scores; NULL to skip.
 * Arithmetic: bf16 MFMA products with fp32 accumulation, fp32 softmax
 * statistics, probabilities rounded to bf16 before the PV product. For
 * dt = LA_FP32 the operands are rounded to bf16 on load and o is fp32.
 * Errors: INVALID_ARG for null q/k/v/o, B, S, Hq, Hkv < 1, n_docs < 1 with
 * cu_docs given, Hq % Hkv != 0, bad strides or alignment; UNSUPPORTED for D or
 * group size outside the supported set.
 */
la_status gqa_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                      la_dtype dt, int B, int S, int Hq, int Hkv, int D,
                      const int64_t q_strides[3], const int64_t k_strides[3],
                      const int64_t v_strides[3], const int64_t o_strides[3],
                      const int32_t* cu_docs, int n_docs, float softmax_scale,
                      hipStream_t stream);

/*
 * gqa_prefill_rope — gqa_prefill on queries that are NOT rotated: the kernel
 * applies the rotary embedding of rope_qk to each query tile in registers
 * before its products [P1, P2, P4]; keys must arrive rotated (rope_qk with
 * q_in = q_out = NULL). Saves writing and re-reading the rotated queries.
 *
 * Arguments as gqa_prefill, plus positions (int32 [B, S] or NULL for
 * position = s) and rope_base, as rope_qk takes them. Rotation: the angle
 * position * theta_k is formed and reduced modulo one turn in fp64, its sine
 * and cosine are taken in fp32, the pair is rotated in fp32 and rounded to
 * bf16; a rotated query element may differ by one bf16 ulp from rope_qk's
 * (which rotates in fp64) in rare cases.
 * Errors: those of gqa_prefill; INVALID_ARG for rope_base <= 0 or not finite.
 */
la_status gqa_prefill_rope(const void* q, const void* k, const void* v, void* o, float* lse,
                           la_dtype dt, int B, int S, int Hq, int Hkv, int D,
                           const int64_t q_strides[3], const int64_t k_strides[3],
                           const int64_t v_strides[3], const int64_t o_strides[3],
                           const int32_t* cu_docs, int n_docs, float softmax_scale,
                           const int32_t* positions, double rope_base, int rope_pairing,
                           hipStream_t stream);

/*
 * gqa_prefill_chunk — prefill of a block of new tokens after a cached prefix
 * (chunked prefill): the Sq queries of each sequence are its LAST Sq tokens,
 * at positions S - Sq .. S - 1, and attend to the keys of all S tokens (the
 * cached prefix and the block itself) under the same causal and document
 * rules as gqa_prefill [P2, P4]. The result equals rows S - Sq .. S - 1 of
 * gqa_prefill over the whole sequence.
 *
 * q: [B, Sq, Hq, D]; k and v: [B, S, Hkv, D] (keys rotated, e.g. by rope_qk,
 *   each at its own position); o: [B, Sq, Hq, D]; strides as in gqa_prefill.
 * cu_docs: as in gqa_prefill, over the S tokens (row b non-decreasing from 0
 *   to S); NULL means one document per sequence.
 * lse: optional fp32 [B, Hq, Sq] (contiguous), NULL to skip.
 * rope_base: 0 means the queries arrive rotated; > 0 means they are rotated
 *   in the kernel as in gqa_prefill_rope, at positions (int32 [B, Sq], or NULL
 *   for position S - Sq + i of query row i).
 * Requirements: 1 <= Sq <= S. Arithmetic as gqa_prefill (and
 *   gqa_prefill_rope for the rotation).
 * Errors: those of gqa_prefill; INVALID_ARG for Sq < 1 or Sq > S, and for
 * rope_base < 0 or not finite.
 */
la_status gqa_prefill_chunk(const void* q, const void* k, const void* v, void* o, float* lse,
                            la_dtype dt, int B, int Sq, int S, int Hq, int Hkv, int D,
                            const int64_t q_strides[3], const int64_t k_strides[3],
                            const int64_t v_strides[3], const int64_t o_strides[3],
                            const int32_t* cu_docs, int n_docs, float softmax_scale,
                            const int32_t* positions, double rope_base, int rope_pairing,
                            hipStream_t stream);

/*
 * gqa_prefill_split — gqa_prefill_chunk with long key ranges split across
 * workgroups, for load balance when a few query tiles see far more keys than
 * the others (a block deep in a long document) [P2, P4]. Same result as
 * gqa_prefill_chunk up to rounding (the softmax is merged from pieces).
 *
 * Arguments as gqa_prefill_chunk (Sq = S gives a whole-sequence prefill),
 * plus: the key range of each query tile (256/g tokens) is cut into pieces of
 * split_tiles tiles of 64 keys, one workgroup per piece; a tile with one
 * piece writes o and lse directly, the others write per-piece partials to the
 * caller's workspace, which a second kernel (same stream) merges by their
 * log-sum-exp weights into o and lse.
 * o_part: fp32 [max_splits, B, Sq, Hq, D], lse_part: fp32 [max_splits, B, Hq,
 *   Sq] (contiguous, caller-owned, 16-byte aligned; contents are scratch).
 * Requirements: split_tiles >= 1; max_splits >= ceil(ceil(S / 64) /
 *   split_tiles) and <= 65535.
 * Errors: those of gqa_prefill_chunk; INVALID_ARG for split_tiles < 1, a null
 * or misaligned workspace, max_splits out of range.
 */
la_status gqa_prefill_split(const void* q, const void* k, const void* v, void* o, float* lse,
                            la_dtype dt, int B, int Sq, int S, int Hq, int Hkv, int D,
                            const int64_t q_strides[3], const int64_t k_strides[3],
                            const int64_t v_strides[3], const int64_t o_strides[3],
                            const int32_t* cu_docs, int n_docs, float softmax_scale,
                            const int32_t* positions, double rope_base, int rope_pairing,
                            int split_tiles,
                            int max_splits, float* o_part, float* lse_part, hipStream_t stream);

/*
 * gqa_prefill_ring_step — one step of context-parallel attention, as each
 * device of a ring runs it (here on one GPU): the Sq query rows at positions
 * q_off .. q_off + Sq - 1 against the Skv keys and values of one shard of the
 * same sequence, at positions k_off .. k_off + Skv - 1, with the causal and
 * document rules on those positions ([P1] "4D Parallelism": context
 * parallelism over the 128K sequence; [P2, P4] for the attention itself).
 * The shard's result for each row and head (softmax over the shard's visible
 * keys, and its log-sum-exp; o = 0 and lse = -inf where it has none) is
 * written (first != 0) or merged by log-sum-exp weight into the fp32
 * accumulators, so that after the steps over all shards they hold the
 * attention over all keys; gqa_prefill_ring_finalize turns them into o. A
 * merging step (first == 0) whose keys all lie after the block's queries
 * (k_off >= q_off + Sq: no row sees any key) leaves the accumulators as they
 * are and launches nothing (after the argument checks).
 *
 * q: [B, Sq, Hq, D] (rows of the query shard); k, v: [B, Skv, Hkv, D] (rows
 *   of the key shard, keys rotated at their positions); strides as in
 *   gqa_prefill. cu_docs: as in gqa_prefill, over the whole sequence's
 *   positions (it must cover every position of both shards).
 * o_acc: fp32 [B, Sq, Hq, D], lse_acc: fp32 [B, Hq, Sq] (contiguous,
 *   caller-owned); their contents are read only when first == 0.
 * rope_base: 0 means the queries arrive rotated; > 0 rotates them in the
 *   kernel at positions (int32 [B, Sq], or NULL for q_off + i).
 * Errors: those of gqa_prefill; INVALID_ARG for q_off, k_off < 0, Sq or
 * Skv < 1, position overflow, null or misaligned accumulators.
 */
la_status gqa_prefill_ring_step(const void* q, const void* k, const void* v, float* o_acc,
                                float* lse_acc, la_dtype dt, int B, int Sq, int q_off, int Skv,
                                int k_off, int Hq, int Hkv, int D, const int64_t q_strides[3],
                                const int64_t k_strides[3], const int64_t v_strides[3],
                                const int32_t* cu_docs, int n_docs, float softmax_scale,
                                const int32_t* positions, double rope_base, int rope_pairing,
                                int first,
                                hipStream_t stream);

/*
 * gqa_prefill_ring_step_final — the last step of a query shard's ring: as
 * gqa_prefill_ring_step, but instead of updating the accumulators it writes
 * the rows' final o (type dt, [B, Sq, Hq, D], strides o_strides) and
 * optional lse (fp32 [B, Hq, Sq]), the values gqa_prefill_ring_step followed
 * by gqa_prefill_ring_finalize would give, bit for bit ([P1] "4D
 * Parallelism": context parallelism; the merge is the log-sum-exp rule of the
 * ring steps). With first != 0 (a ring of one step) it is the shard's plain
 * prefill and the accumulators are not touched (they may be NULL); otherwise
 * they are read and left unspecified. A row that saw no key gets o = 0 and
 * lse = -inf. Keys that all lie after the block's queries make it the
 * finalize alone.
 * Errors: those of gqa_prefill_ring_step, and those of gqa_prefill for o and
 * its strides.
 */
la_status gqa_prefill_ring_step_final(const void* q, const void* k, const void* v, float* o_acc,
                                      float* lse_acc, void* o, const int64_t o_strides[3], float* lse,
                                      la_dtype dt, int B, int Sq, int q_off, int Skv, int k_off, int Hq,
                                      int Hkv, int D, const int64_t q_strides[3],
                                      const int64_t k_strides[3], const int64_t v_strides[3],
                                      const int32_t* cu_docs, int n_docs, float softmax_scale,
                                      const int32_t* positions, double rope_base, int rope_pairing,
                                      int first, hipStream_t stream);

/*
 * gqa_prefill_ring_finalize — o (type dt, [B, Sq, Hq, D], strides o_strides)
 * and optional lse (fp32 [B, Hq, Sq]) from the ring accumulators; a row that
 * saw no key gets o = 0 and lse = -inf.
 * Errors: INVALID_ARG for null or misaligned pointers, sizes < 1, bad strides;
 * UNSUPPORTED for D not in {64, 128} or an unknown dtype.
 */
la_status gqa_prefill_ring_finalize(const float* o_acc, const float* lse_acc, void* o,
                                    const int64_t o_strides[3], float* lse, la_dtype dt, int B,
                                    int Sq, int Hq, int D, hipStream_t stream);

/*
 * gqa_decode — split-KV attention of one new token per sequence over its KV
 * cache; writes per-split partial results for gqa_decode_combine [P2].
 *
 * q: bf16 [B, Hq, D], strides q_strides = (b, h), already rotated at position
 *   seq_lens[b] - 1.
 * k_cache, v_cache: bf16 [B, Hkv, Lmax, D] with strides cache_strides =
 *   (b, h, l) shared by both, D <= l-stride <= 2^24; slots 0..seq_lens[b]-1 hold the rotated keys and
 *   the values of every token of sequence b, the new token included.
 * seq_lens: int32 [B] on the device, 1 <= seq_lens[b] <= Lmax.
 * Split s of sequence b covers cache slots [s*kv_chunk, min((s+1)*kv_chunk,
 *   seq_lens[b])), s < n_b = ceil(seq_lens[b] / kv_chunk); every slot of the
 *   cache window is visible.
 * o_part: fp32 [B, Hq, max_splits, D], lse_part: fp32 [B, Hq, max_splits]
 *   (contiguous, caller-owned workspace of B*Hq*max_splits*(D+1)*4 bytes).
 *   For each (b, h) the splits s < n_b are covered by runs of consecutive
 *   splits; a run starting at split s stores at slot s the softmax-normalised
 *   output and natural-log log-sum-exp over all keys of the run, and its other
 *   slots get lse = -inf (their o is left unwritten). Slots s >= n_b are not
 *   written. Merging the slots s < n_b by their log-sum-exp weights (as
 *   gqa_decode_combine does) gives the attention output; the grouping into
 *   runs depends on the device and may change between calls.
 * Requirements: kv_chunk a positive multiple of 64; max_splits >=
 *   ceil(Lmax / kv_chunk); B <= 1024; dt of q and caches is bf16 only.
 * Errors: INVALID_ARG for null pointers, sizes < 1, kv_chunk not a multiple
 * of 64, max_splits too small, sizes whose index arithmetic would overflow,
 * bad strides or alignment; UNSUPPORTED for D or group size outside the
 * supported set, or B > 1024.
 */
la_status gqa_decode(const void* q, const int64_t q_strides[2],
                     const void* k_cache, const void* v_cache, const int64_t cache_strides[3],
                     const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int Lmax,
                     int kv_chunk, int max_splits, float softmax_scale,
                     float* o_part, float* lse_part, hipStream_t stream);

/*
 * gqa_decode_paged — gqa_decode over a paged KV cache (the serving layout:
 * fixed-size pages from a shared pool, a block table per sequence) [P2].
 *
 * k_pages, v_pages: bf16 pools of pages, page p holding page_size slots of
 *   every KV head, with strides page_strides = (page, h, slot) shared by both
 *   (D <= slot stride <= 2^24).
 * block_table: int32 [B, bt_stride] on the device: key j of sequence b (slot
 *   j of its logical cache) is slot j % page_size of page
 *   block_table[b][j / page_size]; entries for j < seq_lens[b] must name
 *   pages of the pool (caller's contract, not checked).
 * page_size: a power of two >= 16 (a 16-key tile never crosses a page);
 *   bt_stride >= ceil(Lmax / page_size).
 * Everything else (q, seq_lens, splits, o_part/lse_part workspace, the merge
 * by gqa_decode_combine) as gqa_decode; the results equal gqa_decode's on the
 * same logical cache bit for bit.
 * Errors: those of gqa_decode; INVALID_ARG for a null table or pool, a
 * page_size that is not a power of two >= 16, bt_stride too small.
 */
la_status gqa_decode_paged(const void* q, const int64_t q_strides[2], const void* k_pages,
                           const void* v_pages, const int64_t page_strides[3], int page_size,
                           const int32_t* block_table, int bt_stride, const int32_t* seq_lens,
                           int B, int Hq, int Hkv, int D, int Lmax, int kv_chunk, int max_splits,
                           float softmax_scale, float* o_part, float* lse_part,
                           hipStream_t stream);

/*
 * gqa_decode_combine — merge the split partials of gqa_decode by their
 * log-sum-exp weights: with M = max_s lse_s and w_s = exp(lse_s - M),
 * o = sum_s w_s o_s / sum_s w_s and lse = M + ln(sum_s w_s), over the slots
 * s < ceil(seq_lens[b] / kv_chunk) (min max_splits); slots with lse = -inf
 * carry no weight and their o is not read.
 * o: [B, Hq, D] of type dt (bf16 or fp32) with strides o_strides = (b, h);
 * lse: optional fp32 [B, Hq] (contiguous), NULL to skip.
 * Errors: as gqa_decode for the shared arguments; UNSUPPORTED for D not in
 * {64, 128}.
 */
la_status gqa_decode_combine(const float* o_part, const float* lse_part,
                             const int32_t* seq_lens, int B, int Hq, int D,
                             int kv_chunk, int max_splits,
                             void* o, const int64_t o_strides[2], float* lse,
                             la_dtype dt, hipStream_t stream);

/*
 * rope_qk_backward — the transpose of rope_qk: rotates each channel pair by
 * minus the angle that rope_qk uses (same positions, rope_base, pairing), so
 * that gradients with respect to rotated queries and keys become gradients
 * with respect to the unrotated ones (the rotation is orthogonal) [P1].
 * Arguments, layouts and errors as rope_qk, with dq/dk in place of q/k.
 */
la_status rope_qk_backward(const void* dq_in, void* dq_out, const int64_t dq_in_strides[3],
                           const int64_t dq_out_strides[3],
                           const void* dk_in, void* dk_out, const int64_t dk_in_strides[3],
                           const int64_t dk_out_strides[3],
                           la_dtype dt, int B, int S, int Hq, int Hkv, int D,
                           const int32_t* positions, double rope_base, int rope_pairing,
                           hipStream_t stream);

/*
 * gqa_attention_backward — gradients of gqa_prefill (the training step's
 * backward pass) under the same mask and head mapping [P2, P4]: for a loss L
 * with dL/do = dout,
 *   dv_j = sum_i P_ij dout_i,  dS_ij = P_ij (dout_i . v_j - dout_i . o_i),
 *   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
 * P_ij being the forward's softmax weights (exp(scale q_i . k_j - lse_i) on
 * visible pairs) and the sums over i for a KV head running over its Hq/Hkv
 * query heads. q, k are the ROTATED queries and keys and dq, dk the gradients
 * with respect to them (rope_qk_backward maps them to the unrotated inputs).
 *
 * q, o, dout, dq: [B, S, Hq, D]; k, v, dk, dv: [B, S, Hkv, D]; bf16 only,
 * strides (b, s, h) per tensor. The token stride of q and dout is at least
 * Hq times their head stride, which is at least D (each token's heads lie in
 * its row). o and lse are the forward's outputs for these q, k, v (lse fp32
 * [B, Hq, S] contiguous, natural log). delta: caller-owned fp32 workspace
 * [B, Hq, S] (contiguous), overwritten with -(dout_i . o_i). cu_docs, n_docs,
 * softmax_scale as gqa_prefill. dq, dk, dv are written, not accumulated.
 * dkv_workspace: optional caller-owned fp32 buffer of
 * LA_BWD_PIECES * B * S * Hkv * 2 * D elements (16-byte aligned; contents
 * need no initialisation). With it, keys whose visible queries span more
 * than 48 blocks of 64 (token, head) columns have their query range cut into
 * LA_BWD_PIECES pieces run by separate workgroups; each piece writes its
 * fp32 partial dk, dv there and a final pass sums the pieces in a fixed
 * order (the result does not depend on scheduling). NULL: no cut (one
 * workgroup per 128 keys, which leaves the long ranges of causal attention
 * on a few workgroups).
 * Arithmetic: bf16 MFMA products with fp32 accumulation; P and dS rounded to
 * bf16 before the products that use them.
 * Errors: UNSUPPORTED for dt != LA_BF16 or D / group size outside the
 * supported set; INVALID_ARG for null pointers, sizes < 1, Hq % Hkv != 0,
 * bad strides or alignment, or sizes whose offsets overflow the kernels'
 * 32-bit block offsets.
 */
la_status gqa_attention_backward(const void* q, const void* k, const void* v, const void* o,
                                 const void* dout, const float* lse, float* delta,
                                 void* dq, void* dk, void* dv, la_dtype dt,
                                 int B, int S, int Hq, int Hkv, int D,
                                 const int64_t q_strides[3], const int64_t k_strides[3],
                                 const int64_t v_strides[3], const int64_t o_strides[3],
                                 const int64_t dout_strides[3], const int64_t dq_strides[3],
                                 const int64_t dk_strides[3], const int64_t dv_strides[3],
                                 const int32_t* cu_docs, int n_docs, float softmax_scale,
                                 float* dkv_workspace, hipStream_t stream);

/*
 * gqa_decode_noalloc — gqa_decode followed by gqa_decode_combine, for callers
 * that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the split partials live in a scratch
 * array the library holds in device memory (32 MiB per device, from the
 * library's load until the process ends), so the caller passes only inputs
 * and outputs and the call performs no allocation.
 *
 * Arguments as gqa_decode (q, caches, strides, seq_lens, sizes, kv_chunk,
 * softmax_scale) and gqa_decode_combine (o [B, Hq, D] of type dt with strides
 * o_strides (b, h); lse fp32 [B, Hq] or NULL). The partials are kept one per
 * run of consecutive splits that one wave of the persistent decode grid
 * takes: (waves + B * Hkv) slots of (Hq / Hkv) * (D + 1) fp32 values, plus
 * 8 bytes per wave (waves = 4 per compute unit). Results equal those of
 * gqa_decode + gqa_decode_combine with the same kv_chunk.
 * Every call on a device shares that device's scratch: calls that overlap on
 * one device (different streams, or host threads without ordering) race and
 * must not be issued; calls in one stream are ordered and safe. Nothing in the
 * scratch needs clearing between calls (every value a call reads is written
 * earlier in the same call).
 * Errors: as gqa_decode and gqa_decode_combine; LA_ERR_SCRATCH (nothing
 * launched) when the slots above exceed the scratch; LA_ERR_LAUNCH if the
 * scratch's device address cannot be obtained.
 */
la_status gqa_decode_noalloc(const void* q, const int64_t q_strides[2], const void* k_cache,
                             const void* v_cache, const int64_t cache_strides[3],
                             const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int Lmax,
                             int kv_chunk, float softmax_scale, void* o, const int64_t o_strides[2],
                             float* lse, la_dtype dt, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LLAMA_ATTN_H */
