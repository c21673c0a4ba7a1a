// Internal launch interface between the C-ABI host code and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spec {

// Activation row m of a call -> (sequence b, position, valid).  Rows are
// sequence-major: m = b * mseq + i, position = start_pos[b] + i, valid iff
// i < n_tok[b] (n_tok NULL: all) and 0 <= position < capacity.
struct RowMap {
    const int32_t *start_pos;
    const int32_t *n_tok;
    int mseq;
    int capacity;
};

enum GemvEpi : int {
    EPI_STORE = 0,      // out[m * out_ld + sel * out_sel_stride + row_in_sel] = y
    EPI_QKV_ROPE = 1,   // RoPE on q/k pairs; q -> q_out, k/v -> KV cache
    EPI_SILU_MUL = 2,   // act[m * act_ld + unit] = round(silu(gate) * up)
    EPI_RESID_ADD = 3,  // out[m * out_ld + row] += y
    EPI_LOGITS = 4,     // EPI_STORE (if out) + Gumbel / greedy arg-max partials
};

struct GemvParams {
    // weights: rows of length K, row-major; a unit is the row pair
    // (blk * pair_block + j, blk * pair_block + j + pair_block / 2) with
    // blk = u / (pair_block / 2), j = u % (pair_block / 2).
    const void *W;
    int K;
    int n_units;
    int pair_block;
    int rows_per_sel;     // activation set index sel = row / rows_per_sel
    // activations X: set sel, row m, element k at X[sel * x_sel_stride + m * K + k]
    const void *X;
    int64_t x_sel_stride;
    int m0, M;            // this launch covers rows m0 .. m0 + M - 1
    const float *bias;    // [rows] or NULL
    int epi;
    float *out;
    int64_t out_ld, out_sel_stride;
    void *act;
    int64_t act_ld;
    // QKV epilogue
    float *q_out;
    int64_t q_sel_stride;  // elements between group layers in q_out
    void *kc, *vc;         // KV arenas [L][B][hkv][cap][hd]
    int layer0, batch, hq, hkv, hd;
    float rope_theta;
    RowMap rows;
    // LOGITS epilogue: sampling row m is sequence m0 + m; the decided
    // position is samp_pos[b] + (samp_ntok ? samp_ntok[b] : samp_nconst).
    float inv_temp;
    uint64_t seed;
    const int32_t *samp_pos;
    const int32_t *samp_ntok;
    int samp_nconst;
    float *part_val;       // [M][gridDim.x]
    int32_t *part_idx;
};

// dtype: 0 float32, 1 bfloat16 (weights, activations X and act share it).
// VALU GEMV: units are row pairs, M <= gemv_max_rows() per launch.
hipError_t launch_gemv(int dtype, const GemvParams &p, int grid, hipStream_t s);
int gemv_max_rows();
int gemv_grid(int n_units);
// MFMA skinny GEMM (bf16): units are pairs of 16-row blocks (n_units = rows /
// 32), M <= 32 per launch, K a multiple of 64, pair_block a multiple of 32.
hipError_t launch_gemm_mfma(const GemvParams &p, int grid, int ks, hipStream_t s);
bool gemm_mfma_supported(const GemvParams &p);
int gemm_mfma_max_rows();
int gemm_mfma_grid(int n_units);
int gemm_mfma_splits(int n_units, int K);

// h[m] (+)= add[m]; normalise (src0 ? src0[m] + add[m] : h[m]) with each of
// n_gains gains and write xn[g][m][:] (rounded to the activation dtype).
// h0copy (nullable) receives h[m] before the add.  If gather_mseq > 0, output
// row m reads input row m * gather_mseq + (gather_ntok ? gather_ntok[m] :
// gather_mseq) - 1 and h is not written.
struct NormParams {
    float *h;
    const float *add;
    const float *src0;
    float *h0copy;
    const float *gains;
    int n_gains;
    int64_t gain_stride;
    void *xn;
    int64_t xn_sel_stride;
    int M, d;
    float eps;
    int gather_mseq;
    const int32_t *gather_ntok;
};
hipError_t launch_norm(int dtype, const NormParams &p, hipStream_t s);

// h[m][:] = E[clamp(tokens[...])] for m = b * mseq + i; token of row m is
// tokens[b * tok_ld + i * tok_step].
hipError_t launch_embed(int dtype, const void *E, int vocab, int d, const int32_t *tokens,
                        int64_t tok_ld, int tok_step, int B, int mseq, float *h, hipStream_t s);

// Grouped causal attention over n_group consecutive layers.
struct AttnParams {
    const float *q;        // [g][Mtot][hq][hd]
    int64_t q_sel_stride;
    const void *kc, *vc;   // arenas
    int layer0, n_group, batch, hq, hkv, hd, capacity;
    RowMap rows;
    int max_pos;           // host bound of positions in this call
    int splits;
    void *o;               // [g][Mtot][hq*hd] activation dtype
    int64_t o_sel_stride;
    float *part_acc;       // [splits][g][Mtot][hq][hd]
    float *part_ml;        // [splits][g][Mtot][hq][2]
    int Mtot;
};
hipError_t launch_attention(int dtype, const AttnParams &p, hipStream_t s);
int attention_splits(int n_group, int batch, int hq, int hkv, int mseq, int max_pos);
int attention_split_max();

// Arg-max reduction of lm-head partials -> tokens.
hipError_t launch_sample_reduce(const float *part_val, const int32_t *part_idx, int n_parts, int M,
                                int32_t *token_out, int token_stride, hipStream_t s);

// Accept / resample.
struct AcceptParams {
    int batch, k, vocab, nchunk;
    const float *p_logits, *q_logits;
    const int32_t *drafts, *round_pos;
    int draft_stride;
    float inv_temp;
    uint64_t seed;
    float *stats;          // [B][2k+1][nchunk][2] (max, sumexp)
    int32_t *stats_idx;    // [B][2k+1][nchunk]
    float *cand_val;       // [B][nchunk][2]
    int32_t *cand_idx;     // [B][nchunk][2]
    int32_t *decision;     // [B][2]
    int32_t *n_acc_out, *next_out;
    int next_stride;
    int32_t *commit_out;
};
hipError_t launch_accept(const AcceptParams &p, hipStream_t s);
int accept_chunks(int vocab);

}  // namespace spec
