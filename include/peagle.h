/*
 * peagle.h -- C ABI of the P-EAGLE parallel-draft step for AMD MI355X (gfx950).
 *
 * One parallel-draft round takes the batch the target model just verified and
 * proposes K draft tokens per sequence with a single drafter pass:
 *
 *   pe_prepare_draft_batch  expand the verified batch into the draft layout and
 *                           (pe_prepare_draft_batch_compact: without rejected rows)
 *                           place the hidden states (target rows moved to their
 *                           new rows, the learned shared hidden state broadcast
 *                           into the MASK rows);
 *   pe_draft_forward        fc(emb ++ h) -> decoder layer(s) over the paged KV
 *                           cache -> LM head -> argmax, for all K drafts at once;
 *   pe_accept               greedy accepted length against target tokens.
 *   pe_draft_autoregressive the K-pass autoregressive baseline on the same kernels.
 *   pe_next_verified_batch  next round's verified batch from this round's results.
 *
 * Sources (page title, section):
 *   [PF] "P-EAGLE: Faster LLM Inference with Parallel Speculative Decoding in
 *        vLLM" -- how it works (Input_i equation); vLLM implementation details
 *        (hidden-state placement listing).
 *   [PP] "P-EAGLE: Parallel Speculative Decoding in vLLM" -- Step 2: Parallel
 *        Drafting; vLLM Implementation Details: Fused Triton Kernel, Hidden
 *        State Management, KV Cache and CUDA Graphs; Acceptance Length (AL).
 *
 * Conventions shared by every entry point
 *   - Every pointer argument except the `pe_model_desc`, `pe_weights`,
 *     `pe_layer_weights` structs and the host arrays of cache pointers is a
 *     DEVICE pointer on the current HIP device, owned by the caller and
 *     borrowed for the duration of the (asynchronous) work on `stream`.
 *     The library never allocates or frees device memory; scratch space comes
 *     from the caller's workspace.
 *   - All work is enqueued on `stream`; the calls return before it finishes.
 *   - Tensors are dense and row-major.  Floating-point tensors use the model
 *     dtype (`PE_F32`: IEEE float32, `PE_BF16`: bfloat16 bit patterns) except
 *     where stated.  Every tensor base pointer must be 16-byte aligned.
 *   - Paged KV cache of a layer: [num_blocks, n_kv, block_size, head_dim] in the
 *     model dtype; logical position p of sequence i lives at slot
 *     block_table[i*max_blocks + p/block_size]*block_size + p%block_size.
 *   - Errors: calls return a pe_status.  Misuse detectable on the host (null
 *     pointer, non-positive sizes, unsupported shape, misaligned pointer, too
 *     small workspace) returns PE_EINVAL / PE_EUNSUPPORTED / PE_EWORKSPACE
 *     before anything is enqueued.  A failed launch returns PE_EHIP.  Values
 *     held in device memory (token ids < vocab, 0 <= accepted <= L-1, block
 *     tables covering every position a row occupies) are the caller's contract
 *     and are not checked.
 */
#ifndef PEAGLE_H
#define PEAGLE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PE_OK = 0,
  PE_EINVAL = -1,       /* bad argument (null pointer, size out of range, misaligned) */
  PE_EUNSUPPORTED = -2, /* shape or dtype the library has no kernel for */
  PE_EWORKSPACE = -3,   /* workspace smaller than pe_workspace_bytes() */
  PE_EHIP = -4          /* a HIP launch or runtime call failed */
} pe_status;

typedef enum { PE_F32 = 0, PE_BF16 = 1 } pe_dtype;

/* Drafter shape and constants (host memory, copied by pe_model_create).
 * n_layers == 0 declares an expansion-only model: only h_shared is needed and
 * only pe_prepare_draft_batch may be called with it. */
typedef struct {
  int32_t hidden;        /* H; H % 8 == 0 */
  int32_t vocab;         /* V */
  int32_t n_layers;      /* decoder layers, >= 0 */
  int32_t n_q;           /* query heads */
  int32_t n_kv;          /* kv heads, n_q % n_kv == 0 (q head h reads kv head h/(n_q/n_kv)) */
  int32_t head_dim;      /* d in {16, 32, 64, 128} */
  int32_t inter;         /* SwiGLU intermediate size I, I % 8 == 0 */
  int32_t block_size;    /* KV page size in tokens; must be 16 */
  float rms_eps;         /* RMSNorm epsilon */
  float rope_theta;      /* rotary base; rotate-half pairs (j, j+d/2), angle p*theta^(-2j/d) */
  int32_t mask_token_id; /* id written into MASK rows; emb(mask) = embed[mask_token_id] */
  pe_dtype dtype;        /* storage/compute dtype of weights, hidden states and cache */
} pe_model_desc;

/* One pre-norm decoder layer (device pointers, row-major [out, in]). */
typedef struct {
  const void *ln1;    /* [H]            RMSNorm gain before attention */
  const void *wq;     /* [n_q*d, H] */
  const void *wk;     /* [n_kv*d, H] */
  const void *wv;     /* [n_kv*d, H] */
  const void *wo;     /* [H, n_q*d] */
  const void *ln2;    /* [H]            RMSNorm gain before the MLP */
  const void *w_gate; /* [I, H] */
  const void *w_up;   /* [I, H] */
  const void *w_down; /* [H, I] */
} pe_layer_weights;

/* Drafter weights (device pointers; `layers` is a HOST array of n_layers). */
typedef struct {
  const void *embed;    /* [V, H] token embeddings; row mask_token_id is emb(mask) */
  const void *w_fc;     /* [H, 2H] fc over concat(emb(id), h) ([PF] Input_i) */
  const void *ln_f;     /* [H] final RMSNorm gain */
  const void *w_lm;     /* [V, H] LM head */
  const void *h_shared; /* [H] learned shared hidden state for MASK rows ([PF], [PP] Hidden State Management) */
  const pe_layer_weights *layers;
} pe_weights;

/* Opaque drafter handle.  Set-up is pe_model_create followed, optionally, by
 * pe_model_pack_weights; those two are the only calls that modify the handle.
 * After set-up it is read-only: every other call takes it as const, and
 * concurrent calls from several host threads on several streams may share it
 * (each with its own workspace and outputs). */
typedef struct pe_model pe_model;

/* Validate the description and weight pointers and build a model handle
 * (host memory only; the compute-unit count of the current HIP device is
 * recorded for launch shapes).  Returns PE_EINVAL / PE_EUNSUPPORTED on bad
 * input. */
pe_status pe_model_create(const pe_model_desc *desc, const pe_weights *weights, pe_model **out);
void pe_model_destroy(pe_model *model);

/* Bytes of device memory for the packed copies of the weights: the projection
 * weights (fc and every layer's q/k/v, o, gate, up, down) in fragment order,
 * the LM head (vocab rounded up to 256 rows x hidden), and, when hidden,
 * n_q*head_dim and inter are multiples of 64, the projections once more in
 * tile order (outputs rounded up to whole tiles); 0 when the model has nothing to
 * pack (fp32 weights, no layers, or hidden / n_q*head_dim / inter not
 * multiples of 32 or head_dim not a multiple of 16). */
size_t pe_packed_weights_bytes(const pe_model *model);

/* Optional part of set-up, for speed.  Copies the projection weights into `packed` in the
 * fragment order of the bf16 matrix-core tiles (each 16-output x 32-input
 * fragment one contiguous KiB, the q/k/v rows grouped in rotary pairs), read
 * with few draft rows (at most 16 rows per pass, e.g. one sequence at K <= 8),
 * and the LM head tile-major (256-row groups, each 32-deep slice of a group one
 * contiguous 16 KiB block), read when more than 16 rows are sampled, and the
 * projections tile-major in the same layout, their rows in the order the
 * 128 x 256 (q/k/v: 128 x 128) tiles load them, read by passes over more than
 * 256 draft rows (whose activations are then also kept tile-major); attaches
 * the buffer to the model.  From then on those products stream the copies
 * instead of the row-major weights (same products, same results up to the
 * summation order of split partial sums).  `packed`: device buffer of at least
 * pe_packed_weights_bytes() bytes, 256-byte aligned, owned by the caller, not
 * modified and kept alive while the model is used; it snapshots the weights as
 * they are when the copy runs on `stream` (later changes to the row-major
 * weights are not seen).  Forward calls on other streams must be ordered after
 * that work; do not call it while a pass using the model is in flight.
 * Memory cost: the copies add to the caller's row-major weights, which stay
 * in use (the LM head over at most 16 sampled rows, the embedding, the norms);
 * for a GPT-OSS-20B-shaped drafter (hidden 2880, vocab 201088) that is
 * 219 MB of projections in fragment order, 226 MB in tile order and 1.16 GB
 * for the LM head, so the drafter's weight footprint grows from 1.38 GB to
 * about 2.99 GB.
 * Returns PE_OK (nothing to do when 0 bytes are needed), PE_EINVAL (null or
 * misaligned buffer), PE_EWORKSPACE (too small), PE_EHIP. */
pe_status pe_model_pack_weights(pe_model *model, void *packed, size_t packed_bytes, hipStream_t stream);

/* Bytes of workspace pe_draft_forward needs for a batch of `num_seqs`
 * sequences, depth K and `num_rows` draft rows (0 on invalid input). */
size_t pe_workspace_bytes(const pe_model *model, int32_t num_seqs, int32_t K, int32_t num_rows);

/* Expand the verified batch into the draft batch.  [PP] Fused Triton Kernel:
 * copy ids and positions, insert the bonus token, fill the K-1 parallel-drafting
 * slots with the MASK id and emit the rejected/masked masks and the hidden-state
 * map; [PP] KV Cache and CUDA Graphs: rejected rows get slot -1; [PF] vLLM
 * implementation details / [PP] Hidden State Management: target hidden rows are
 * moved to their mapped rows and h_shared is broadcast into the MASK rows.
 *
 * Inputs (c = num_seqs, T = total_target_rows = sum of query_lens):
 *   query_lens[c]    L_i >= 1 verified rows of sequence i (rows are sequence-major)
 *   target_ids[T]    token ids of the verified rows
 *   target_pos[T]    positions of the verified rows (consecutive within a sequence)
 *   num_accepted[c]  a_i, drafts accepted by the target, 0 <= a_i <= L_i-1
 *   bonus_ids[c]     b_i, the token the target produced after the accepted ones
 *   target_hidden[T,H]  target hidden state of every verified row
 *   block_table[c,max_blocks]  physical page of each logical page
 * Outputs (N = T + c*(K-1) draft rows; sequence i owns rows cu_draft[i]..cu_draft[i+1]-1):
 *   draft_ids[N], draft_pos[N]   row r < a_i: token of verified row r+1 at the
 *                                position of verified row r; row a_i: b_i (the
 *                                first prediction row); rows a_i+1..a_i+K-1: MASK
 *                                id at the next K-1 positions; then the L_i-1-a_i
 *                                rejected verified rows (shifted ids, own positions)
 *   slot_mapping[N]  cache slot of the row's position, -1 on rejected rows
 *   is_rejected[N], is_masked[N]  0/1 bytes
 *   hidden_map[T]    draft row that receives target row t
 *   cu_draft[c+1]    first draft row of each sequence, cu_draft[c] = N
 *   kv_lens[c]       cached positions after the pass: target_pos[first + a_i] + K
 *   sample_idx[c*K]  the K rows whose logits give the drafts (first prediction row, MASK rows)
 *   draft_hidden[N,H]  placed hidden states
 */
pe_status pe_prepare_draft_batch(const pe_model *model, int32_t num_seqs, int32_t K,
                                 int32_t total_target_rows, const int32_t *query_lens,
                                 const int32_t *target_ids, const int32_t *target_pos,
                                 const int32_t *num_accepted, const int32_t *bonus_ids,
                                 const void *target_hidden, const int32_t *block_table,
                                 int32_t max_blocks, int32_t *draft_ids, int32_t *draft_pos,
                                 int64_t *slot_mapping, uint8_t *is_rejected, uint8_t *is_masked,
                                 int32_t *hidden_map, int32_t *cu_draft, int32_t *kv_lens,
                                 int32_t *sample_idx, void *draft_hidden, hipStream_t stream);

/* Compacted draft layout (the fixed layout keeps rejected rows as inert
 * slot -1 rows, "P-EAGLE: Parallel Speculative Decoding in vLLM", KV Cache and
 * CUDA Graphs; this one drops them).  Same arguments and buffer sizes as
 * pe_prepare_draft_batch (N = T + c(K-1) rows), but sequence i owns only its
 * a_i + K live rows -- the accepted rows, the bonus row and the K-1 MASK rows
 * -- at cu_draft[i] = sum_{j<i} (a_j + K).  cu_draft[c] holds the number of
 * live rows; the rows from there to N are inert padding (slot -1, flagged
 * rejected, zero hidden state) that pe_draft_forward skips tile by tile.
 * hidden_map[t] is -1 for target rows past the accepted prefix (no draft row
 * inherits them).  Tokens and logits equal those of the fixed layout. */
pe_status pe_prepare_draft_batch_compact(const pe_model *model, int32_t num_seqs, int32_t K,
                                 int32_t total_target_rows, const int32_t *query_lens,
                                 const int32_t *target_ids, const int32_t *target_pos,
                                 const int32_t *num_accepted, const int32_t *bonus_ids,
                                 const void *target_hidden, const int32_t *block_table,
                                 int32_t max_blocks, int32_t *draft_ids, int32_t *draft_pos,
                                 int64_t *slot_mapping, uint8_t *is_rejected, uint8_t *is_masked,
                                 int32_t *hidden_map, int32_t *cu_draft, int32_t *kv_lens,
                                 int32_t *sample_idx, void *draft_hidden, hipStream_t stream);

/* One drafter pass over every draft row, producing K tokens per sequence.
 * [PF] how it works / [PP] Step 2: Parallel Drafting: all positions go through
 * the layer(s) and the LM head together and t_1..t_K come out of one pass.
 *
 * Per row r: x = W_fc [embed[draft_ids[r]] ; draft_hidden[r]]; per layer:
 * RMSNorm, q/k/v projections, rotate-half RoPE at draft_pos[r], (k, v) written
 * to the layer's cache at slot_mapping[r] unless it is -1, grouped-query
 * attention over positions 0..draft_pos[r] of the row's sequence (after all
 * writes of the layer), output projection + residual, RMSNorm, SwiGLU MLP +
 * residual; then RMSNorm and the LM head on the rows sample_idx[], greedy
 * argmax (lowest id on ties).  Rejected rows are not computed.
 *
 *   metadata arrays: as produced by pe_prepare_draft_batch for the same batch
 *   k_cache, v_cache: HOST arrays [n_layers] of device caches (read and written)
 *   workspace: device scratch of at least pe_workspace_bytes(model, c, K, N)
 *   draft_tokens[c*K]   int32 output, sequence-major
 *   logits_or_null      optional float32 [c*K, V] logits of the sampled rows
 *   top2_gap_or_null    optional float32 [c*K]: best minus second-best logit
 */
pe_status pe_draft_forward(const pe_model *model, int32_t num_seqs, int32_t K, int32_t num_rows,
                           const int32_t *draft_ids, const int32_t *draft_pos,
                           const int64_t *slot_mapping, const uint8_t *is_rejected,
                           const int32_t *cu_draft, const int32_t *kv_lens,
                           const int32_t *sample_idx, const void *draft_hidden,
                           const int32_t *block_table, int32_t max_blocks,
                           void *const *k_cache, void *const *v_cache, void *workspace,
                           size_t workspace_bytes, int32_t *draft_tokens, float *logits_or_null,
                           float *top2_gap_or_null, hipStream_t stream);

/* Allocation-free variant of pe_draft_forward, for callers that cannot
 * allocate device memory or carry a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments
 * (minus the workspace), kernels and results as pe_draft_forward.  Its scratch
 * is a static device array of PE_STATIC_SCRATCH_BYTES inside the library, one
 * per GPU it runs on, held until the process ends; the call itself never
 * allocates or frees memory.
 *   - Returns PE_EWORKSPACE before anything is enqueued when the batch needs
 *     more scratch than that (pe_workspace_bytes(model, c, K, N) >
 *     PE_STATIC_SCRATCH_BYTES; 32 MiB covers, e.g., one sequence of a
 *     GPT-OSS-20B-shaped drafter at K <= 8, or 16 sequences of a
 *     Qwen3-Coder-30B-shaped one at K = 3), PE_EHIP when the array's device
 *     address cannot be obtained; otherwise as pe_draft_forward.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents (the pass writes every scratch region it reads first).
 *     Calls that overlap in time on one GPU -- on different streams, or from
 *     host threads without ordering between them -- race on the array and
 *     corrupt each other's results: serialize them.
 *   - Its launches are not recorded by the kernel timing (pe_timing_*). */
#define PE_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
pe_status pe_draft_forward_noalloc(const pe_model *model, int32_t num_seqs, int32_t K, int32_t num_rows,
                                   const int32_t *draft_ids, const int32_t *draft_pos,
                                   const int64_t *slot_mapping, const uint8_t *is_rejected,
                                   const int32_t *cu_draft, const int32_t *kv_lens,
                                   const int32_t *sample_idx, const void *draft_hidden,
                                   const int32_t *block_table, int32_t max_blocks,
                                   void *const *k_cache, void *const *v_cache, int32_t *draft_tokens,
                                   float *logits_or_null, float *top2_gap_or_null, hipStream_t stream);

/* Greedy acceptance ([PP] Acceptance Length (AL)): num_accepted[i] = length of
 * the longest prefix on which draft_tokens[i*K..] equals target_tokens[i*(K+1)..],
 * bonus_ids[i] = target_tokens[i*(K+1) + num_accepted[i]].
 *   draft_tokens[c*K], target_tokens[c*(K+1)] int32 in; num_accepted[c], bonus_ids[c] int32 out. */
pe_status pe_accept(int32_t num_seqs, int32_t K, const int32_t *draft_tokens,
                    const int32_t *target_tokens, int32_t *num_accepted, int32_t *bonus_ids,
                    hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Autoregressive baseline on the same kernels ("P-EAGLE: Parallel Speculative
 * Decoding in vLLM", Solving the Autoregressive Drafting Bottleneck: EAGLE-style
 * drafters need one forward pass per draft token, so drafting latency grows
 * with K; P-EAGLE replaces the K passes by one).
 *
 * Pass 1 is the parallel-draft pass with K = 1 over the verified batch (the
 * bonus row, no MASK rows) and yields token 0.  Pass k = 1..K-1 runs one row
 * per sequence: token k-1 at position base_i + k (base_i = position of the
 * bonus row), with the drafter's own final residual (pre final RMSNorm) of the
 * row that produced token k-1 as hidden input, rounded to the model dtype; its
 * (k, v) are appended to the cache at that position and the row yields token k.
 *
 *   inputs: the verified batch exactly as for pe_prepare_draft_batch; the
 *           block table must cover positions up to base_i + K - 1
 *   k_cache, v_cache: HOST arrays [n_layers] of device caches (read and written)
 *   workspace: device scratch of at least pe_autoregressive_workspace_bytes(
 *              model, c, K, T) bytes, 256-byte aligned
 *   draft_tokens[c*K]  int32 output, sequence-major
 *   logits_or_null     optional float32 [K, c, V], step-major: row (k, i) holds
 *                      the logits that gave token k of sequence i
 *   fed_hidden_or_null optional [K-1, c, H] model dtype, 16-byte aligned:
 *                      receives the hidden input of pass k = 1..K-1 (row
 *                      (k-1, i): sequence i's rounded final residual fed back);
 *                      when given, the passes read their hidden rows from it
 * Returns PE_EWORKSPACE for a short workspace; otherwise as pe_draft_forward.
 * Launches K forward passes plus small row builders on the stream; nothing is
 * synchronized on the host.
 * ------------------------------------------------------------------------- */
size_t pe_autoregressive_workspace_bytes(const pe_model *model, int32_t num_seqs, int32_t K,
                                         int32_t total_target_rows);
pe_status pe_draft_autoregressive(const pe_model *model, int32_t num_seqs, int32_t K,
                                  int32_t total_target_rows, const int32_t *query_lens,
                                  const int32_t *target_ids, const int32_t *target_pos,
                                  const int32_t *num_accepted, const int32_t *bonus_ids,
                                  const void *target_hidden, const int32_t *block_table,
                                  int32_t max_blocks, void *const *k_cache, void *const *v_cache,
                                  void *workspace, size_t workspace_bytes, int32_t *draft_tokens,
                                  float *logits_or_null, void *fed_hidden_or_null, hipStream_t stream);

/* Next round's verified batch, on the device ("P-EAGLE: Faster LLM Inference
 * with Parallel Speculative Decoding in vLLM", 怎么做的: each round drafts K
 * tokens that the target model then verifies).  The target verified, for
 * sequence i, the K + 1 rows [bonus_ids[i], draft_tokens[i*K .. i*K+K-1]] at
 * positions base_i + 1 .. base_i + K + 1, where base_i = kv_lens[i] - K is the
 * position of this round's bonus row (kv_lens as produced by
 * pe_prepare_draft_batch for this round), and accepted num_accepted_next[i]
 * drafts with new bonus bonus_next[i] (pe_accept's outputs).
 *   outputs: query_lens_out[c] = K + 1; target_ids_out / target_pos_out
 *   [c*(K+1)]; num_accepted_out[c], bonus_ids_out[c] copies of the inputs.
 * The target hidden states of those rows come from the verifier.  Inputs and
 * outputs may not alias. */
pe_status pe_next_verified_batch(int32_t num_seqs, int32_t K, const int32_t *kv_lens,
                                 const int32_t *bonus_ids, const int32_t *draft_tokens,
                                 const int32_t *num_accepted_next, const int32_t *bonus_next,
                                 int32_t *query_lens_out, int32_t *target_ids_out,
                                 int32_t *target_pos_out, int32_t *num_accepted_out,
                                 int32_t *bonus_ids_out, hipStream_t stream);

/* Check, on the device, the preconditions of pe_prepare_draft_batch that live
 * in device memory (the host checks the rest): a debug aid for callers, which
 * pe_prepare_draft_batch itself does not run.  [PP] Fused Triton Kernel lists
 * the fields of the verified batch; the expansion assumes them well formed.
 * Each violated condition ORs its bit into *error_bits (a device int32 the
 * caller zeroes beforehand; the call never clears it, so checks accumulate):
 *   PE_CHECK_QUERY_LEN    some L_i < 1, or the L_i do not sum to T
 *   PE_CHECK_ACCEPTED     some a_i outside 0..L_i-1
 *   PE_CHECK_TOKEN_ID     a target id or bonus id outside 0..V-1
 *   PE_CHECK_POSITION     a negative position, or positions not consecutive
 *                         within a sequence
 *   PE_CHECK_BLOCK_TABLE  a page the pass reads or writes (positions up to
 *                         target_pos[first + a_i] + K - 1) past max_blocks or
 *                         mapped to a negative physical page
 * The check reads only in-bounds locations of the given arrays: every value is
 * range-checked before it is used as an index.  Whether a physical page lies
 * inside the caller's cache cannot be checked (its size is not passed). */
enum {
  PE_CHECK_QUERY_LEN = 1,
  PE_CHECK_ACCEPTED = 2,
  PE_CHECK_TOKEN_ID = 4,
  PE_CHECK_POSITION = 8,
  PE_CHECK_BLOCK_TABLE = 16
};
pe_status pe_check_verified_batch(const pe_model *model, int32_t num_seqs, int32_t K,
                                  int32_t total_target_rows, const int32_t *query_lens,
                                  const int32_t *target_ids, const int32_t *target_pos,
                                  const int32_t *num_accepted, const int32_t *bonus_ids,
                                  const int32_t *block_table, int32_t max_blocks,
                                  int32_t *error_bits, hipStream_t stream);

/* Static description of a status code. */
const char *pe_status_string(pe_status status);

/* Kernel timing for measurement harnesses (process-wide, not part of any
 * model).  While enabled for a kernel class, every launch of that class, from
 * any model, thread or stream, records a pair of HIP events on the stream it
 * is launched on; enabling (or re-enabling) discards earlier records.
 * pe_timing_read synchronizes on the recorded events and returns the summed
 * elapsed milliseconds and the number of launches since enable, and, when
 * per_launch_ms is given, the first `capacity` launch times in launch order.
 * Thread-safe; while a class is enabled its launches are serialized on the
 * host.  Do not enable timing while a stream is being captured into a graph. */
typedef enum { PE_KERNEL_LM_HEAD = 0, PE_KERNEL_PREPARE = 1, PE_KERNEL_ATTENTION = 2 } pe_kernel_class;
pe_status pe_timing_enable(pe_kernel_class kernel, int32_t enable);
pe_status pe_timing_read(pe_kernel_class kernel, double *total_ms, int64_t *launches, float *per_launch_ms,
                         int64_t capacity);

#ifdef __cplusplus
}
#endif

#endif /* PEAGLE_H */
