/*
 * spec.h -- C ABI of libspec, the MI355X (gfx950) hot path of layer-parallel
 * ("fuzzy") speculative decoding.
 *
 * Method: "EasySpec: Layer-Parallel Speculative Decoding for Efficient
 * Multi-GPU Utilization" (abstract; rebuttal replies on Table 4, Figure 1(b),
 * the fuzzy KV cache and bonus calibration).  A small draft model proposes
 * k tokens; inside the draft, the attention modules of each layer-parallel set
 * read the same incoming hidden state (the inter-layer dependency is broken)
 * while the MLPs still run in order; the base model verifies the k tokens in
 * one forward pass; the acceptance decisions come back; and the draft KV cache
 * is then calibrated by one precise forward pass.  On one GPU a set of N
 * layers becomes one grouped launch over the N layers' weights and KV caches.
 *
 * Conventions shared by every call
 *  - All tensors are caller-owned.  "dev" pointers are device memory of the
 *    current HIP device; "host" pointers are ordinary host memory.  The library
 *    never allocates device memory and never synchronises the host: compute
 *    calls enqueue kernels on `stream` (a hipStream_t; NULL = default stream)
 *    and return.
 *  - Arguments are validated on the host before anything is launched; on an
 *    error nothing is launched and the outputs are untouched.  Errors are the
 *    negative spec_status codes; spec_last_error() gives a thread-local detail
 *    message.  SPEC_ERR_HIP reports a failed launch (outputs then undefined).
 *  - Token ids outside [0, vocab) are clamped on the device; positions at or
 *    beyond the KV capacity are treated as invalid rows (no KV write).
 *  - Floating point: weights and KV are float32 (SPEC_F32) or bfloat16
 *    (SPEC_BF16; K/V rounded to nearest, ties to even, when written).
 *    Activations, norms, RoPE, softmax and accumulation are float32 on both
 *    paths.  A bf16 weight product over two or more activation rows runs on
 *    the bf16 matrix cores with each float32 activation split into two bf16
 *    pieces hi + lo (together within 2^-16 of its value); over one row it
 *    runs as float32 FMAs.  Attention keeps q and the softmax probabilities
 *    at float32 precision against the bf16 K/V (three bf16 pieces on the
 *    matrix cores).
 *  - Random numbers: Philox4x64-10 (Salmon et al., SC'11), key = (seed, b),
 *    counter = (v >> 2, position of the token being decided, 0, purpose),
 *    word v & 3, u = ((word >> 41) + 0.5) * 2^-23.  Purposes: 0 draft
 *    sampling, 1 accept test (v = 0), 2 residual / bonus sampling.  Sampling is
 *    Gumbel-max: argmax_v (s_v - log(-log u_v)); ties go to the lowest index.
 */
#ifndef SPEC_H
#define SPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPEC_OK = 0,
    SPEC_ERR_INVALID_ARG = -1,    /* NULL pointer, negative size, bad flag      */
    SPEC_ERR_SHAPE = -2,          /* model or call shape unsupported            */
    SPEC_ERR_VOCAB_MISMATCH = -3, /* draft and base vocabularies differ         */
    SPEC_ERR_PLAN = -4,           /* plan is not a contiguous cover of layers   */
    SPEC_ERR_CAPACITY = -5,       /* max_pos + rows would exceed KV capacity    */
    SPEC_ERR_WORKSPACE = -6,      /* workspace NULL or smaller than required    */
    SPEC_ERR_HIP = -7,            /* a HIP launch failed                        */
    SPEC_ERR_UNSUPPORTED = -8     /* valid but not implemented (e.g. head_dim)  */
} spec_status;

enum { SPEC_F32 = 0, SPEC_BF16 = 1 };

/* Flags of spec_draft_group_step.  The rebuttal (reply on Table 4 / the MLP
 * question) states that only attention is layer-parallel and the MLPs run in
 * order: SPEC_MLP_SEQUENTIAL, the default, computes for a set with incoming
 * state h0:  h = h0; for each layer i of the set, in order:
 *            h = h + a_i;  h = h + MLP_i(RMSNorm(h)),
 * where a_i is layer i's attention output on h0.  SPEC_MLP_PARALLEL also
 * feeds every MLP from h0:  h = h0 + sum_i (a_i + MLP_i(RMSNorm(h0 + a_i))). */
enum { SPEC_MLP_SEQUENTIAL = 0, SPEC_MLP_PARALLEL = 1 };

/* Decoder shape.  head_dim must be 16, 32, 64 or 128; d_model, d_ffn and
 * n_q_heads*head_dim must be multiples of 8; n_q_heads a multiple of
 * n_kv_heads with at most 16 q heads per kv head (else
 * SPEC_ERR_UNSUPPORTED).  rope_theta: base of the rotate-half RoPE (pairs (j, j+hd/2),
 * angle pos * theta^(-2j/hd)); rms_eps: RMSNorm epsilon. */
typedef struct {
    int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, d_ffn, vocab;
    int32_t has_qkv_bias;  /* 0 or 1 */
    int32_t dtype;         /* SPEC_F32 or SPEC_BF16: weights and KV cache */
    float rms_eps, rope_theta;
} spec_model_desc;

/* Device weight arenas, layer-major, row-major.  D = (hq + 2*hkv) * hd.
 *   embed      [V][d]        dtype       attn_norm [L][d]   float32
 *   wqkv       [L][D][d]     dtype       rows: q heads, k heads, v heads
 *   bqkv       [L][D]        float32 or NULL (required iff has_qkv_bias)
 *   wo         [L][d][hq*hd] dtype       ffn_norm  [L][d]   float32
 *   w_gate_up  [L][2*ffn][d] dtype       rows: gate rows, then up rows
 *   w_down     [L][d][ffn]   dtype       final_norm [d]     float32
 *   lm_head    [V][d]        dtype
 * The library keeps the pointers; the caller keeps the memory alive for the
 * model's lifetime. */
typedef struct {
    const void *embed;
    const float *attn_norm;
    const void *wqkv;
    const float *bqkv;
    const void *wo;
    const float *ffn_norm;
    const void *w_gate_up;
    const void *w_down;
    const float *final_norm;
    const void *lm_head;
} spec_weights;

/* KV cache of one model: k and v each [L][batch][hkv][capacity][hd] of the
 * model dtype (dev).  Position p of sequence b of layer l holds the post-RoPE
 * key / the value of the token at absolute position p. */
typedef struct {
    void *k, *v;
    int32_t capacity, batch;
} spec_kv;

typedef struct spec_model spec_model;

/* Host object describing a model; allocates no device memory. */
spec_status spec_model_create(const spec_model_desc *desc, const spec_weights *w,
                              spec_model **out);
void spec_model_destroy(spec_model *m);

/* Draft and base must share the tokenizer (rebuttal: token ids must be
 * identical across the two models).  Returns SPEC_ERR_VOCAB_MISMATCH if not. */
spec_status spec_check_pair(const spec_model *draft, const spec_model *base);

/* Default layer-parallel plan (rebuttal reply on Table 4 and on Figure 1(b)):
 * layers 0 and L-1 are never parallelised; an intermediate layer l belongs to
 * set floor(l / N), so sets are {1..N-1}, {N..2N-1}, ... and the set before
 * the last layer may be smaller (N = 4, L = 32 ends with {28, 29, 30}).
 * Writes CSR offsets (host, n_stages + 1 entries, capacity max_offsets). */
spec_status spec_default_group_plan(int n_layers, int group_size, int32_t *offsets_out,
                                    int max_offsets, int *n_stages_out);

/* Bytes of workspace a compute call on `m` needs for `batch` sequences of at
 * most `max_m` new tokens each and plans whose largest set has `max_group`
 * layers.  Returns 0 for invalid arguments. */
size_t spec_workspace_bytes(const spec_model *m, int batch, int max_m, int max_group);

/* One layer-parallel ("fuzzy") draft step (EasySpec abstract: layers of the
 * draft run simultaneously as fuzzy speculation; rebuttal: the attentions of a
 * set take the same input and produce a set of fuzzy KV entries that live for
 * one speculation phase only).
 *   plan_offsets (host) [n_stages+1]: CSR cover of 0..L-1 by contiguous sets.
 *   tokens (dev) token of sequence b at tokens[b * tokens_stride];
 *   positions (dev) [batch]: its absolute position; writes draft K/V there.
 *   max_pos (host): an upper bound of max_b positions[b].
 *   inv_temperature: 1/T as float32; 0 => greedy argmax.
 *   logits_out (dev, nullable): float32 logits of sequence b at
 *     logits_out + b * logits_stride (vocab entries).
 *   token_out (dev): sampled token of sequence b (for position positions[b]+1,
 *     purpose 0) at token_out[b * token_out_stride].
 * Errors: SPEC_ERR_PLAN, SPEC_ERR_CAPACITY (max_pos >= capacity),
 * SPEC_ERR_WORKSPACE, SPEC_ERR_INVALID_ARG. */
spec_status spec_draft_group_step(const spec_model *draft, const spec_kv *kv,
                                  const int32_t *plan_offsets, int n_stages, int flags,
                                  int batch, const int32_t *tokens, int tokens_stride,
                                  const int32_t *positions, int max_pos,
                                  float inv_temperature, uint64_t seed,
                                  float *logits_out, int64_t logits_stride,
                                  int32_t *token_out, int token_out_stride,
                                  void *workspace, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the draft
 * step of spec_draft_group_step, same arguments and results, with the
 * workspace taken from a scratch array of SPEC_SCRATCH_BYTES that the library
 * holds in every GPU's memory from the first such call on that GPU until the
 * process ends.  The call allocates nothing and launches the same kernels.
 * Errors as for spec_draft_group_step; SPEC_ERR_WORKSPACE (nothing launched)
 * if spec_workspace_bytes(draft, batch, 1, largest set of the plan) exceeds
 * SPEC_SCRATCH_BYTES; SPEC_ERR_HIP if the scratch array's address cannot be
 * obtained.  Every call on one GPU uses that GPU's one array, which keeps
 * the last call's contents (the step needs no initial contents): calls that
 * overlap on one GPU (several streams or host threads) race. */
#define SPEC_SCRATCH_BYTES ((size_t)32 << 20)
spec_status spec_draft_group_step_noalloc(const spec_model *draft, const spec_kv *kv,
                                          const int32_t *plan_offsets, int n_stages, int flags,
                                          int batch, const int32_t *tokens, int tokens_stride,
                                          const int32_t *positions, int max_pos,
                                          float inv_temperature, uint64_t seed,
                                          float *logits_out, int64_t logits_stride,
                                          int32_t *token_out, int token_out_stride, void *stream);

/* Cosine-similarity diagnostic of the fuzzy inputs (review thread, the
 * discussion of Table 3: the similarity of the hidden states a layer-parallel
 * set feeds its attentions to the ones a sequential pass would feed, measured
 * as a cosine because each attention normalises its input first).  Runs the
 * layer-parallel step of spec_draft_group_step with sequential MLPs (and, like
 * it, writes the fuzzy K/V at `positions`) and, for every layer l of set
 * [l0, l0+n), writes
 *   cos_out[b * cos_stride + l] = cos(h0, h_l),
 * h0 = the set's input state (what all its attentions read), h_l = the state
 * after the members l0 .. l-1 have added their attention and MLP outputs
 * (what layer l's attention would read if the set ran in order; h_l0 = h0).
 * No head, no sampling.  cos_stride >= n_layers; other arguments as for
 * spec_draft_group_step.  Errors as for spec_draft_group_step. */
spec_status spec_draft_attention_cosine(const spec_model *draft, const spec_kv *kv,
                                        const int32_t *plan_offsets, int n_stages, int batch,
                                        const int32_t *tokens, int tokens_stride,
                                        const int32_t *positions, int max_pos, float *cos_out,
                                        int cos_stride, void *workspace, size_t ws_bytes, void *stream);

/* Bonus calibration / KV correction (EasySpec abstract: after each
 * drafting-and-verification iteration the draft KV cache is calibrated in a
 * single forward pass; rebuttal: calibrated entries replace the fuzzy ones).
 * One precise (sequential) draft forward over n_tokens[b] <= max_m tokens of
 * each sequence at positions start_pos[b] .. start_pos[b]+n_tokens[b]-1,
 * overwriting the draft KV there; the last position of each sequence gives
 * the draft distribution of the next token, which is sampled (purpose 0, for
 * position start_pos[b]+n_tokens[b]).  Also the draft's prompt prefill.
 *   tokens (dev): sequence b's tokens at tokens + b * tokens_stride
 *   (tokens_stride >= max_m); start_pos, n_tokens (dev) [batch]; n_tokens
 *   may be NULL (= max_m for all).  max_pos (host) bounds
 *   start_pos[b] + n_tokens[b] - 1.
 *   last_logits_out (dev, nullable): float32 logits of sequence b at
 *     last_logits_out + b * logits_stride (logits_stride >= vocab);
 *   token_out (dev) at token_out[b * token_out_stride]. */
spec_status spec_calibrate_kv(const spec_model *draft, const spec_kv *kv, int batch,
                              const int32_t *tokens, int tokens_stride, const int32_t *start_pos,
                              const int32_t *n_tokens, int max_m, int max_pos,
                              float inv_temperature, uint64_t seed,
                              float *last_logits_out, int64_t logits_stride,
                              int32_t *token_out, int token_out_stride,
                              void *workspace, size_t ws_bytes, void *stream);

/* Verification forward of the base model (EasySpec abstract: the draft token
 * sequence is verified by the original base model): the m tokens of each
 * sequence, [x_t, d_1 .. d_k] with m = k+1, at positions start_pos[b] ..
 * start_pos[b]+m-1, in one forward pass; writes the base K/V there.  Also the
 * base's prompt prefill (logits_out = NULL).
 *   tokens (dev) [batch][m]; start_pos (dev) [batch]; max_pos (host) bounds
 *   start_pos[b] + m - 1.  logits_out (dev, nullable) [batch][m][vocab]. */
spec_status spec_verify_forward(const spec_model *base, const spec_kv *kv, int batch,
                                const int32_t *tokens, const int32_t *start_pos, int m,
                                int max_pos, float *logits_out,
                                void *workspace, size_t ws_bytes, void *stream);

/* Accept / resample (speculative sampling of Leviathan et al. and Chen et al.,
 * cited by the pages; lossless per the abstract and the rebuttal reply on the
 * 7% drop).  For sequence b with pending position t = round_pos[b] and draft
 * d_j (position t+j):
 *   T > 0: p_j = softmax(p_logits[b][j-1] * inv_T), q_j likewise from
 *     q_logits.  For j = 1..k accept iff u_j * q_j(d_j) < p_j(d_j), u_j the
 *     purpose-1 uniform of position t+j.  At the first rejection y is drawn
 *     from max(0, p_j - q_j) (from p_j if that is identically zero) with the
 *     purpose-2 stream of position t+j; if all are accepted y ~ p_{k+1}.
 *   T = 0 (inv_temperature == 0): accept iff d_j == argmax p_j; y = argmax of
 *     the first mismatching row, else of row k+1.
 *   k = 0 is a plain sampling step from p_1 (vanilla decoding).
 *   p_logits (dev) [batch][k+1][vocab]; q_logits (dev) [batch][k][vocab]
 *   (unused when greedy, may be NULL then or when k = 0);
 *   draft_tokens (dev): d_j of sequence b at draft_tokens[b * draft_stride + j - 1]
 *   (draft_stride >= k; pass the verify tokens + 1 with stride k + 1 to reuse
 *   [x_t, d_1 .. d_k]); round_pos (dev) [batch].
 *   Outputs (dev): n_accepted_out [batch]; next_token_out[b * next_token_stride];
 *   commit_out (nullable) [batch][k+1] receives d_1..d_a, y.
 *   Workspace: spec_accept_workspace_bytes(batch, k, vocab). */
size_t spec_accept_workspace_bytes(int batch, int k, int vocab);
spec_status spec_accept_resample(int batch, int k, int vocab,
                                 const float *p_logits, const float *q_logits,
                                 const int32_t *draft_tokens, int draft_stride,
                                 const int32_t *round_pos, float inv_temperature, uint64_t seed,
                                 int32_t *n_accepted_out, int32_t *next_token_out,
                                 int next_token_stride, int32_t *commit_out,
                                 void *workspace, size_t ws_bytes, void *stream);

/* Measurement hook (not part of the method).  While enabled, every
 * weight-streaming product launch (the GEMV / matrix-core kernels that read
 * the weights) and every grouped-attention launch is bracketed by two HIP
 * events recorded on the caller's stream and attributed to its kernel
 * instance, e.g. "k_gemm_mfma<1, 2, 4>", together with the bytes the launch
 * must read (every weight row once plus the activation rows; for attention
 * the K/V rows up to the call's max_pos, a bound) and, for the products, the
 * flops 2 * rows * K * activation rows.  spec_profile_collect synchronises
 * the recorded events, folds them into per-instance totals and returns the
 * number of instances; spec_profile_entry reads one (any output pointer may
 * be NULL).  Enabling adds two event records per launch, so time the method
 * with it off. */
spec_status spec_profile_enable(int on);
void spec_profile_reset(void);
int spec_profile_collect(void);
spec_status spec_profile_entry(int i, char *name, int name_cap, int64_t *launches, double *total_ms,
                               double *total_bytes, double *total_flops);

const char *spec_status_string(spec_status s);
const char *spec_last_error(void);
/* Library version string ("<major>.<minor>.<patch> gfx950"). */
const char *spec_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPEC_H */
