/*
 * sdm.h -- C ABI of the block-wise decoding forward (AR / block diffusion /
 * self-speculation) for one AMD Instinct MI355X (gfx950).
 *
 * The method: one decoder serves three decoding modes, which differ only in
 * the attention mask of the block and in how tokens are chosen from the
 * logits (Nemotron-Labs-Diffusion pages: ai-feeds "inference: three modes";
 * fintech-frontier-insights "three generation modes"; hotpaper abstract).
 *   - AR: one token per forward (sdm_decode_ar).
 *   - Block diffusion: a block of MASK placeholders is denoised in parallel
 *     over several forwards; each step unmasks the masked positions whose
 *     confidence clears a threshold (sdm_diffuse_step), then the finished
 *     block is committed through a causal forward (sdm_verify_block +
 *     sdm_commit_kv).
 *   - Self-speculation: a bidirectional forward drafts a block
 *     (sdm_draft_block), one causal forward verifies it (sdm_verify_block),
 *     and the longest prefix matching the AR argmax plus one AR token is kept
 *     (sdm_commit_kv).  At temperature 0 the output equals greedy AR
 *     (fintech-frontier-insights, self-speculation bullet).
 *
 * Conventions for every call
 *   - d_ pointers are device pointers, h_ pointers host pointers.  The caller
 *     owns every buffer (weights, KV pool, workspace, inputs, outputs) and
 *     keeps them alive until sdm_free_model.  The library owns only the
 *     model handle and host-side bookkeeping.
 *   - Calls are asynchronous on the HIP stream given to sdm_init_model;
 *     outputs are valid once that stream has been synchronised.
 *   - Every call validates its arguments and the sequence state before it
 *     enqueues anything: a call that returns an error has changed nothing.
 *     The message of the last error on the calling thread is returned by
 *     sdm_last_error().
 *   - A handle must not be used from two threads at once.
 *
 * Numerics.  bf16 models keep the weights and k/v after RoPE (hence the KV
 * cache) in bf16 (round to nearest, ties to even), and hand the normalised
 * activations, q, the attention output and the SwiGLU product between
 * kernels as two-term bf16 values (hi = bf16(x), lo = bf16(x - hi)); every
 * contraction accumulates in fp32; the residual stream and logits are fp32.
 * f32 models keep all of it in fp32.  The MASK id never wins an argmax and is
 * left out of the softmax.
 */
#ifndef SDM_H
#define SDM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sdm_model sdm_model; /* opaque, library-owned host object */

typedef enum {
  SDM_OK = 0,
  SDM_ERR_ARG = -1,        /* null pointer, size or id out of range          */
  SDM_ERR_STATE = -2,      /* call not allowed in the sequence's state        */
  SDM_ERR_CAPACITY = -3,   /* KV pool / context / workspace / seq slots full  */
  SDM_ERR_DEVICE = -4,     /* a HIP call failed; sticky for the handle        */
  SDM_ERR_UNSUPPORTED = -5 /* shape or dtype the library does not implement  */
} sdm_status;

typedef enum { SDM_F32 = 0, SDM_BF16 = 1 } sdm_dtype;

/* Storage of the decoder's QKV, O, gate/up and down matrices (bf16 models).
 *   SDM_WEIGHTS_BF16: bf16 (sdm_pack_matrix).
 *   SDM_WEIGHTS_INT4: weight-only 4-bit ("w4a16", the DGX Spark row of
 *     fintech-frontier-insights' hardware table; the format is this library's
 *     reading): two's-complement codes in [-8, 7] and one bf16 scale per
 *     output row and group of 128 input columns, weight = scale * code
 *     (sdm_pack_matrix_int4).  Activations stay as for bf16 weights; the
 *     embedding and the LM head stay bf16.  Needs d_model and ffn_dim
 *     multiples of 128. */
typedef enum { SDM_WEIGHTS_BF16 = 0, SDM_WEIGHTS_INT4 = 1 } sdm_weight_format;

typedef enum { SDM_CAUSAL = 0, SDM_BIDIR = 1 } sdm_attn_mode;

/* Model and capacity description.
 *   dtype bf16 requires head_dim 128, d_model and q/kv widths multiples of 32,
 *   ffn_dim a multiple of 16 and vocab a multiple of 32; f32 requires an even
 *   head_dim.  n_q_heads must be a multiple of n_kv_heads.  mask_id is the
 *   reserved MASK token (vocab - 1 in every shipped shape).  page_tokens must
 *   be 64.  max_rows bounds the rows of one forward (n_seq * block, or a
 *   prefill chunk); max_context (<= 65536) bounds a sequence's length (prompt + output
 *   + one block).  weight_format is an sdm_weight_format. */
typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab, mask_id;
  float rope_base, rms_eps;
  int32_t dtype;
  int32_t page_tokens, max_seqs, max_block, max_context, max_rows;
  int32_t weight_format;
} sdm_config;

/* Device weights in the library's layout (see sdm_pack_matrix).  Gains are
 * [d_model] vectors in the model dtype; matrices are packed.  The per-layer
 * members are host arrays of n_layers device pointers; the arrays are copied
 * by sdm_init_model.
 *   embed     [vocab, d_model] row-major, NOT packed (rows are gathered)
 *   lm_head   packed SDM_PACK_PLAIN of [vocab, d_model]
 *   w_qkv     packed SDM_PACK_QKV of [(Hq + 2 Hkv) * hd, d_model] (q rows, k rows, v rows)
 *   w_o       packed SDM_PACK_PLAIN of [d_model, Hq * hd]
 *   w_gate_up packed SDM_PACK_GATE_UP of gate [ffn, d_model] and up [ffn, d_model]
 *   w_down    packed SDM_PACK_PLAIN of [d_model, ffn]
 * With SDM_WEIGHTS_INT4, w_qkv, w_o, w_gate_up and w_down are packed by
 * sdm_pack_matrix_int4 with the same kinds.                                     */
typedef struct {
  const void *embed, *final_norm, *lm_head;
  const void *const *attn_norm, *const *w_qkv, *const *w_o;
  const void *const *ffn_norm, *const *w_gate_up, *const *w_down;
} sdm_weights;

typedef enum { SDM_PACK_PLAIN = 0, SDM_PACK_QKV = 1, SDM_PACK_GATE_UP = 2 } sdm_pack_kind;

/* Bytes of device workspace a model with this config needs (0 on a bad config). */
size_t sdm_workspace_bytes(const sdm_config* cfg);
/* Bytes of one KV page (all layers' K and V of page_tokens positions). */
size_t sdm_kv_page_bytes(const sdm_config* cfg);
/* Bytes of a packed [rows, cols] matrix of the config's dtype. */
size_t sdm_packed_bytes(const sdm_config* cfg, int64_t rows, int64_t cols);

/* Rearrange a row-major [rows, cols] matrix (out-major: row = output feature)
 * into the layout the GEMM kernels stream.  For SDM_PACK_GATE_UP, d_src is the
 * gate matrix and d_src2 the up matrix, each [rows, cols], and the result holds
 * 2*rows rows.  A pure permutation: no arithmetic.  Enqueued on hip_stream. */
sdm_status sdm_pack_matrix(const sdm_config* cfg, int32_t kind, const void* d_src, const void* d_src2,
                           void* d_dst, int64_t rows, int64_t cols, void* hip_stream);

/* Bytes of a packed 4-bit [rows, cols] matrix (codes, then scales); 0 if the
 * config is bad, rows % 32 != 0 or cols % 128 != 0.  For SDM_PACK_GATE_UP pass
 * rows = 2 * ffn_dim, as for sdm_packed_bytes. */
size_t sdm_packed_bytes_int4(const sdm_config* cfg, int64_t rows, int64_t cols);

/* Rearrange a 4-bit [rows, cols] matrix (out-major) into the layout the 4-bit
 * GEMM streams.  d_codes is uint8 [rows, cols / 2]: byte j of a row holds
 * column 2j in its low nibble and column 2j + 1 in its high nibble, each a
 * two's-complement code in [-8, 7].  d_scales is bf16 [rows, cols / 128].  For
 * SDM_PACK_GATE_UP, d_codes / d_scales hold the gate matrix and d_codes2 /
 * d_scales2 the up matrix, each [rows, cols].  A pure permutation (the same
 * row order as sdm_pack_matrix); d_dst holds sdm_packed_bytes_int4 bytes.
 * Needs a bf16 config, cols % 128 == 0 and rows % 32 == 0 (% 16 for gate/up);
 * device pointers 4-byte aligned.  Enqueued on hip_stream. */
sdm_status sdm_pack_matrix_int4(const sdm_config* cfg, int32_t kind, const void* d_codes, const void* d_scales,
                                const void* d_codes2, const void* d_scales2, void* d_dst, int64_t rows, int64_t cols,
                                void* hip_stream);

/* Create a model.  kv_pool holds n_pages pages of sdm_kv_page_bytes; the
 * workspace holds ws_bytes >= sdm_workspace_bytes.  Uploads the RoPE table
 * (angles p * base^(-2t/hd) in fp64, cos/sin stored fp32) into the workspace. */
sdm_status sdm_init_model(const sdm_config* cfg, const sdm_weights* w, void* kv_pool, int64_t n_pages,
                          void* workspace, size_t ws_bytes, void* hip_stream, sdm_model** out);

/* Causal forward over the prompt d_tokens[n] of an empty sequence, in chunks of
 * at most max_rows rows; commits all n positions.  d_next_token[0] = argmax of
 * the last row (the first generated token).  d_logits (nullable) receives the
 * last row's logits [vocab] fp32. */
sdm_status sdm_prefill(sdm_model* m, int32_t seq, const int32_t* d_tokens, int32_t n, int32_t* d_next_token,
                       float* d_logits);

/* One denoising step for n_seq sequences in lockstep (ids in h_seq_ids).
 * d_block [n_seq][B] holds each sequence's block (MASK where still masked) and
 * is updated in place.  A bidirectional forward over the blocks at positions
 * n..n+B-1; the row at a masked position predicts that position.  Per
 * sequence, over its masked set Mk: U = {i in Mk : conf_i > tau} plus the most
 * confident i in Mk (lowest i on ties); force_all != 0 makes U = Mk.  Positions
 * in U take their argmax token; d_n_masked[s] = |Mk \ U|.  conf is the max
 * softmax probability over non-MASK ids.  d_conf (nullable) [n_seq][B] gets
 * every row's conf; d_logits (nullable) [n_seq*B][vocab].  K/V of the block
 * are written to the uncommitted slots and are not committed. */
sdm_status sdm_diffuse_step(sdm_model* m, int32_t n_seq, const int32_t* h_seq_ids, int32_t* d_block, int32_t B,
                            float tau, int32_t force_all, int32_t* d_n_masked, float* d_conf, float* d_logits);

/* A denoising step that may also rewrite positions already written (the
 * pages: in diffusion mode the model can go back and modify content it has
 * generated -- fintech-frontier-insights "three generation modes", diffusion
 * bullet, and the aimodeling text; the rule is this library's reading).  As
 * sdm_diffuse_step, and from the same forward every position i of a block
 * that does not hold MASK, whose argmax tok_i differs from its token and whose
 * conf_i > tau_revise, takes tok_i.  Every decision is made on the block as it
 * was before the step.  d_n_revised (nullable) [n_seq] receives the number of
 * rewritten positions.  conf <= 1, so tau_revise >= 1 gives exactly
 * sdm_diffuse_step.  NaN tau or tau_revise: SDM_ERR_ARG. */
sdm_status sdm_diffuse_step_revise(sdm_model* m, int32_t n_seq, const int32_t* h_seq_ids, int32_t* d_block,
                                   int32_t B, float tau, float tau_revise, int32_t force_all, int32_t* d_n_masked,
                                   int32_t* d_n_revised, float* d_conf, float* d_logits);

/* Self-spec draft: a bidirectional forward over [anchor, MASK x (B-1)] at
 * positions n..n+B-1.  d_block_out[B] = anchor then the argmax of rows 1..B-1. */
sdm_status sdm_draft_block(sdm_model* m, int32_t seq, const int32_t* d_anchor, int32_t B, int32_t* d_block_out,
                           float* d_logits);

/* Causal forward over d_block [n_seq][B] (position j at n+j) for each sequence.
 * d_ar_argmax [n_seq][B]: row j's argmax (the AR prediction of position n+j+1).
 * d_accept_len [n_seq]: L = k+1, k the largest k <= B-1 with block[j] ==
 * argmax[j-1] for all 1 <= j <= k (the classic verify rule, gsyq.cn explainer
 * section 2.3).  The block's causal K/V become committable (sdm_commit_kv). */
sdm_status sdm_verify_block(sdm_model* m, int32_t n_seq, const int32_t* h_seq_ids, const int32_t* d_block, int32_t B,
                            int32_t* d_ar_argmax, int32_t* d_accept_len, float* d_logits);

/* Quadratic self-speculation (a variant the pages name with a higher
 * tokens-per-forward figure than linear self-speculation: ai-feeds item 3;
 * fintech-frontier-insights, release summary and TPF table; they give no
 * algorithm, so the rows below are this library's reading).  One forward of
 * B + B^2 rows on sequence seq (committed length n):
 *   - the block d_block [B] = [g, d_1..d_{B-1}] at positions n..n+B-1,
 *     causal: exactly sdm_verify_block's rows, outputs and committable K/V
 *     (d_ar_argmax [B], d_accept_len [1]);
 *   - for every k in 0..B-1 a candidate [MASK x B] at positions
 *     n+k+1..n+k+B that sees keys 0..n+k (the committed prefix and block rows
 *     0..k) and, bidirectionally, its own rows.  Its K/V stay in the
 *     workspace and are never committed.
 * d_next_blocks [B][B] (device, int32): row k = [argmax of block row k (the
 * token after an accept length of k + 1), argmax of candidate k's rows
 * 1..B-1] -- the next call's block when the accept length is k + 1, with no
 * draft forward in between.  d_logits (nullable) [B + B^2][vocab] fp32: the
 * block's rows then candidate k's rows at B + k*B.  Commit with
 * sdm_commit_kv(seq, L) as after sdm_verify_block.
 * Requires 2 <= B <= 63, max_block >= B, max_rows >= B * (B + 1) and
 * n + 2B <= max_context (SDM_ERR_ARG / SDM_ERR_CAPACITY otherwise).  d_block
 * must not overlap d_next_blocks (SDM_ERR_ARG).  Calls on one model share the
 * candidates' workspace, as every call shares the model's workspace. */
sdm_status sdm_verify_block_quadratic(sdm_model* m, int32_t seq, const int32_t* d_block, int32_t B,
                                      int32_t* d_ar_argmax, int32_t* d_accept_len, int32_t* d_next_blocks,
                                      float* d_logits);

/* Commit the first n_accept (1..B of the last verify) positions of the last
 * causal block forward of seq.  Requires a preceding sdm_verify_block (or
 * sdm_verify_block_quadratic, or sampled verify) on seq. */
sdm_status sdm_commit_kv(sdm_model* m, int32_t seq, int32_t n_accept);

/* Sampling at temperature > 0 (one sequence per call).  The pages state the
 * self-speculation identity only at temperature 0 and leave higher
 * temperatures open (fintech-frontier-insights, self-speculation bullet); these
 * calls are this library's reading: the standard lossless rejection-sampling
 * verify, under which self-speculation emits tokens distributed as AR sampling
 * at the same temperature.
 *   Random numbers: Philox4x64-10 (Salmon et al., "Parallel random numbers: as
 *   easy as 1, 2, 3") under key (seed, 0) and counter (vocab id / 4, position,
 *   sequence id, purpose: 1 draft, 2 accept, 3 residual, 4 sample); a 64-bit
 *   output x is the uniform u = ((x >> 40) + 1/2) * 2^-24.  A token's position
 *   is the absolute position it will occupy.
 *   A row is sampled from softmax(l / T) over non-MASK ids by the Gumbel-max
 *   trick: argmax of l_v / T - ln(-ln u_v), lowest id on ties.
 * temperature must be finite and > 0 (else SDM_ERR_ARG); the other arguments
 * and state rules are those of the greedy calls. */
/* As sdm_prefill; the first generated token (position n) is sampled. */
sdm_status sdm_prefill_sample(sdm_model* m, int32_t seq, const int32_t* d_tokens, int32_t n, float temperature,
                              uint64_t seed, int32_t* d_next_token, float* d_logits);
/* As sdm_decode_ar; the next token (position len + 1) is sampled. */
sdm_status sdm_decode_ar_sample(sdm_model* m, int32_t seq, const int32_t* d_token, float temperature, uint64_t seed,
                                int32_t* d_next_token, float* d_logits);
/* As sdm_draft_block; rows 1..B-1 are sampled (purpose draft, positions n + j)
 * instead of argmax.  d_draft_logits [B][vocab] fp32 receives the draft's
 * logits and d_draft_stats [2][B] fp32 ln q(d_j) and the row's
 * ln sum exp(l / T); both are inputs of sdm_verify_block_sample.  B >= 2. */
sdm_status sdm_draft_block_sample(sdm_model* m, int32_t seq, const int32_t* d_anchor, int32_t B, float temperature,
                                  uint64_t seed, int32_t* d_block_out, float* d_draft_logits, float* d_draft_stats);
/* Causal forward over the drafted block; draft j (1..B-1) is accepted while
 * ln u_j < ln p_j(d_j) - ln q_j(d_j) (p_j from verify row j - 1, u_j purpose
 * accept at position n + j).  d_accept_len[0] = L = accepted + 1;
 * d_next_token[0] = the token after the accepted drafts: at the first
 * rejection j a Gumbel-max draw from max(0, p_j - q_j) (purpose residual,
 * position n + j), else a draw from the last row (purpose sample, position
 * n + B).  Commit with sdm_commit_kv(seq, L) as after sdm_verify_block.
 * B >= 2, the same temperature and seed as the draft. */
sdm_status sdm_verify_block_sample(sdm_model* m, int32_t seq, const int32_t* d_block, int32_t B, float temperature,
                                   uint64_t seed, const float* d_draft_logits, const float* d_draft_stats,
                                   int32_t* d_accept_len, int32_t* d_next_token, float* d_logits);

/* AR: causal forward over d_token[0] at position n, commit it, d_next_token[0]
 * = argmax. */
sdm_status sdm_decode_ar(sdm_model* m, int32_t seq, const int32_t* d_token, int32_t* d_next_token, float* d_logits);

/* Per-row selection of the last forward: token, conf and top-2 margin, each
 * [rows] (nullable).  Device-to-device copies on the model's stream.  After a
 * sampling call (sdm_*_sample) tok holds the sampled tokens of the rows that
 * were sampled, and conf and margin are those of the last greedy forward. */
sdm_status sdm_row_stats(sdm_model* m, int32_t* d_tok, float* d_conf, float* d_margin);

/* Release a sequence's pages and reset it to empty. */
sdm_status sdm_seq_reset(sdm_model* m, int32_t seq);
/* Committed length of a sequence (host-side value). */
sdm_status sdm_seq_length(const sdm_model* m, int32_t seq, int32_t* out);
/* Number of free KV pages. */
int64_t sdm_free_pages(const sdm_model* m);
/* Reorder the free-page list with a seeded shuffle (layout independence tests). */
sdm_status sdm_shuffle_free_pages(sdm_model* m, uint64_t seed);

sdm_status sdm_free_model(sdm_model* m);
const char* sdm_last_error(void);

/* ---- kernel timing (measurement) -------------------------------------------
 * While a timing window is open, the runtime records a hipEvent pair on the
 * model's stream around every launch of one kernel class (or around whole
 * forwards), up to `capacity` launches.  sdm_timing_stop synchronises the
 * stream, returns the number of timed launches and their summed / shortest /
 * longest duration in milliseconds, and closes the window. */
typedef enum {
  SDM_K_QKV = 0, SDM_K_ATTN = 1, SDM_K_ATTN_COMBINE = 2, SDM_K_O = 3, SDM_K_GATE_UP = 4, SDM_K_DOWN = 5,
  SDM_K_LM_HEAD = 6, SDM_K_NORM = 7, SDM_K_FINISH = 8, SDM_K_FORWARD = 9
} sdm_kernel_class;
sdm_status sdm_timing_start(sdm_model* m, int32_t kernel_class, int32_t capacity);
sdm_status sdm_timing_stop(sdm_model* m, int64_t* launches, double* total_ms, double* min_ms, double* max_ms);

/* ---- standalone block attention (the op the decoder's layers run) --------
 * q:  d_q [T, Hq, hd] bf16 row-major (already rotated).
 * kv: d_k, d_v [n_prefix + T, Hkv, hd] bf16 row-major are first scattered into
 *     pages of d_pool (sdm_attn_pack_kv) through the page table d_pages.
 * out: d_out [T, Hq, hd] bf16, softmax(q.k / sqrt(hd)) over the visible keys
 *     applied to v; key j visible to block row i iff j < n_prefix or
 *     (j < n_prefix + T and (mode == SDM_BIDIR or j <= n_prefix + i)).
 * hd must be 128, Hq a multiple of Hkv, 1 <= T <= 4096, n_prefix + T <= 65536.  Every slot of the
 * pages that hold keys [0, n_prefix + T) must contain finite values (zero the
 * pool once): keys past the end of the last 32-key tile are read and given
 * probability 0. */
size_t sdm_attn_pool_bytes(int32_t n_kv_heads, int32_t head_dim, int32_t n_pages);
size_t sdm_attn_workspace_bytes(int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t T,
                                int32_t max_keys);
sdm_status sdm_attn_pack_kv(int32_t n_kv_heads, int32_t head_dim, const void* d_k, const void* d_v, int32_t n_keys,
                            const int32_t* d_pages, void* d_pool, void* hip_stream);
sdm_status sdm_attention(int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, const void* d_q,
                         const void* d_pool, const int32_t* d_pages, int32_t n_prefix, int32_t T, int32_t mode,
                         void* d_out, void* d_workspace, size_t ws_bytes, void* hip_stream);

/* ---- allocation-free attention ---------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation as sdm_attention, with the same arguments except the workspace.
 * Its per-split partials live in a device array of the library,
 * sdm_attention_scratch_max_bytes() bytes (16 MiB) on every device the library
 * runs on, held from the moment the library's code is loaded on that device
 * until the process ends.  The call allocates nothing (no hipMalloc, no
 * library allocation); the scratch address is looked up once per device, on
 * the first call made with that device current.
 * Limits and errors: as sdm_attention, plus SDM_ERR_CAPACITY (nothing
 * enqueued) when the partials, sdm_attn_workspace_bytes(n_q_heads, n_kv_heads,
 * head_dim, T, n_prefix + T), exceed the scratch (32 q / 8 KV heads, T = 32:
 * up to 7936 keys).  The stream must belong to the current device.  Every
 * call on a device shares that device's scratch and every partial is written
 * before it is read, so nothing needs clearing between calls; calls that
 * overlap on one device (concurrent streams, or host threads) race on the
 * scratch and must be serialised by the caller. */
size_t sdm_attention_scratch_max_bytes(void);
sdm_status sdm_attention_noalloc(int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, const void* d_q,
                                 const void* d_pool, const int32_t* d_pages, int32_t n_prefix, int32_t T,
                                 int32_t mode, void* d_out, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* SDM_H */
