// Internal launch interface between the C-ABI host code and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace spec {

constexpr int kMaxSel = 8;   // largest layer-parallel set whose MLP inputs get their own RMS

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
    EPI_SILU_MUL = 2,   // act[m * act_ld + unit] = silu(gate) * up (float32)
    EPI_RESID_ADD = 3,  // h[m][row] += y (+ add2[m][row]); row-norm partials of h
    EPI_LOGITS = 4,     // store (if out) + per-block Gumbel / greedy arg-max partials
    EPI_ATTN_OUT = 5,   // sequential MLPs: sel 0 -> h += y (+ partials), sel > 0 -> abuf
                        // parallel MLPs: every sel -> abuf, partials of h0 + y; sel 0
                        // also copies h to h0
};

// How a product reads its activations.
enum XMode : int {
    X_PLAIN = 0,   // X[sel * x_sel_stride + m * K + k] (float32)
    X_NORM = 1,    // gain_sel[k] * (xh[hrow][k] + xadd[sel][hrow][k]) / rms(hrow)
};

struct GemvParams {
    // weights: rows of length K, row-major.  VALU GEMV: a unit is the row pair
    // (blk * pair_block + j, ... + pair_block / 2), blk = u / (pair_block / 2),
    // j = u % (pair_block / 2).  MFMA: the same with 16-row blocks.
    const void *W;
    int K;
    int n_units;
    int pair_block;
    int rows_per_sel;     // activation set index sel = row / rows_per_sel
    int m0, M;            // this launch covers rows m0 .. m0 + M - 1
    int Mtot;             // rows of the whole call
    // activations
    int xmode;
    const void *X;        // X_PLAIN
    int64_t x_sel_stride;
    const float *xh;      // X_NORM: residual rows [Mtot][K]
    const float *xadd;    // X_NORM, nullable: [sel][Mtot][K]
    int64_t xadd_sel_stride;
    const float *xgain;   // X_NORM: gain of set member sel at xgain + sel * xgain_stride
    int64_t xgain_stride;
    const float *xss;     // X_NORM: sum-of-squares partials of residual row hrow at
    int xnparts;          //   xss[hrow * xnparts + 0 .. xnparts-1] (summed in order)
    int64_t xss_sel_stride;   // X_NORM: member sel's partials start at xss + sel * xss_sel_stride
                              //   (0: every member normalises with the same partials)
    int kseg;             // > 1: K is kseg equal segments (the set members' matrices side by side):
    int64_t w_seg_stride; //   segment s of weight row r at W + s * w_seg_stride + r * (K / kseg),
    int64_t x_seg_stride; //   of activation row m at X + s * x_seg_stride + m * (K / kseg)
    int act_packed;       // SILU_MUL: 0 -> float32 act rows; PR -> packed bf16
                          //   operand rows (hi at row m, lo at row m + PR / 2)
    // RESID_ADD / sequential ATTN_OUT, nx != NULL: also write the next
    // RMSNorm's operand for a skinny matrix-core consumer, the new residual
    // value times nx_gain[col] as packed bf16 rows [nx_packed][d] (hi at row
    // m, lo at row m + nx_packed / 2); the consumer scales its outputs by the
    // row's 1 / rms (x_inv)
    uint16_t *nx;
    int nx_packed;
    const float *nx_gain;
    // skinny matrix-core consumer: X holds gain * h rows; every output of row m
    // is multiplied by 1 / rms(h_m) formed from the xss partials (m * xnparts
    // + 0 .. xnparts - 1, at most gemm_mfma_inv_max(M) of them in all)
    int x_inv;
    int xgather_mseq;     // > 0: activation row m reads residual row
    const int32_t *xgather_ntok;   //   m * mseq + ntok[m] - 1 (last valid row)
    const float *bias;    // [rows] or NULL
    int epi;
    float *out;
    int64_t out_ld, out_sel_stride;
    void *act;
    int64_t act_ld;
    int64_t act_sel_stride;   // SILU_MUL: member sel's rows start at act + sel * act_sel_stride
    // RESID_ADD / ATTN_OUT
    float *h;             // [Mtot][d]
    float *h0;            // [Mtot][d] (parallel MLPs)
    const float *add2;    // RESID_ADD: nullable extra addends [n_add2][Mtot][d] (n_add2 0 or 1: one)
    int n_add2;
    int64_t add2_sel_stride;
    int par_mlp;          // ATTN_OUT: parallel-MLP reading
    // row-norm partials of the updated residual: ss[sel * ss_sel_stride +
    // m * gridDim.x + block]; consumers sum a row's partials in block order
    float *ss;
    int64_t ss_sel_stride;
    int n_norm_sel;       // 0: no partials; else number of sels with partials
    int d;
    float eps;
    // QKV epilogue
    float *q_out;
    int64_t q_sel_stride;  // elements between group layers in q_out
    void *kc, *vc;         // KV arenas [L][B][hkv][cap][hd]
    int layer0, batch, hq, hkv, hd;
    const float2 *rope_cs; // [Mtot][hd/2] (cos, sin) of each row's position
    RowMap rows;
    // LOGITS epilogue: sampling row m is sequence m0 + m; the decided
    // position is samp_pos[b] + (samp_ntok ? samp_ntok[b] : samp_nconst).
    float inv_temp;
    uint64_t seed;
    const int32_t *samp_pos;
    const int32_t *samp_ntok;
    int samp_nconst;
    float *part_val;       // [Mtot][gridDim.x]
    int32_t *part_idx;
};

// dtype: 0 float32, 1 bfloat16: the weights and the KV cache.  Activation
// buffers (normalised rows, attention outputs, SiLU products) are float32 on
// both paths.
// VALU GEMV: units are row pairs, M <= gemv_max_rows() per launch; ks waves
// (1, 2 or 4) split each unit's K.
hipError_t launch_gemv(int dtype, const GemvParams &p, int grid, int ks, hipStream_t s);
int gemv_max_rows();
int gemv_splits(const GemvParams &p, int elem_bytes);
int gemv_grid(const GemvParams &p, int ks);
// Operand mode of the GEMV instance a launch uses (0 plain rows, 1 normalised
// rows staged in LDS, 2 normalised per step): the last template argument.
int gemv_operand_mode(int dtype, const GemvParams &p);
// MFMA skinny GEMM (bf16) over all M <= 16 rows of a call in one launch (m0
// = 0), K a multiple of 32.  X is the packed operand: gemm_mfma_packed_rows(M)
// bf16 rows per set member, hi(x_m) in row m and lo(x_m) in row m + PR / 2
// (see split2_bf16; PR = 16 for M <= 8, else 32).  Units of unit_rows =
// gemm_mfma_unit_rows(epi, rows, rows_per_sel) weight rows: pairs of 16-row
// blocks for the paired epilogues (QKV RoPE, SiLU; pair_block a multiple of
// 32), single 16-row blocks otherwise; n_units = rows / unit_rows.  ks waves per workgroup (4 or 8), each over its own part of K.
// Residual writers run one unit per workgroup and leave rows_per_sel /
// unit_rows partials per row and set member.
hipError_t launch_gemm_mfma(const GemvParams &p, int grid, int ks, int unit_rows, hipStream_t s);
int gemm_mfma_unit_rows(int epi, int rows, int rows_per_sel);
// Tiled matrix-core GEMM (bf16) for more than 16 rows: every row of
// the call in one launch (p.m0 = 0, p.M = rows), K a multiple of 64, no
// LOGITS epilogue, a set member's rows a whole number of 64-row tiles (32
// units for the paired epilogues).  n_units as for the VALU GEMV (row pairs).
// part: float32 scratch of part_bytes (at most gemm_tiled_part_bytes() is
// used) for the K slices of small products; NULL: no K split.  Residual
// writers leave gemm_tiled_parts(p) partials per row and set member.
hipError_t launch_gemm_tiled(const GemvParams &p, float *part, size_t part_bytes, hipStream_t s);
bool gemm_tiled_supported(const GemvParams &p);
int gemm_tiled_min_rows();
int gemm_tiled_parts(const GemvParams &p);
size_t gemm_tiled_part_bytes();
std::string gemm_tiled_name(const GemvParams &p, size_t part_bytes);   // kernel instance, for measurement
// X_NORM operands written once as float32 rows xn[sel][m][K] for rows
// m0 .. m0 + M - 1 (the matrix-core products then read them plainly).
// packed > 0: the packed operand of the skinny matrix-core kernel instead
// (bf16 rows [sel][packed][K], hi of row m at m, lo at m + packed / 2).
hipError_t launch_norm_rows(int dtype, const GemvParams &p, int n_sel, void *xn, int packed, hipStream_t s);
bool gemm_mfma_supported(const GemvParams &p);
int gemm_mfma_max_rows();
int gemm_mfma_packed_rows(int M);
int gemm_mfma_inv_max(int M);   // largest M x xnparts an x_inv product of M rows takes
int gemm_mfma_grid(const GemvParams &p);
int gemm_mfma_splits(const GemvParams &p);

// out[r * out_stride] = cos(x[r], y[r] - a[r]) for rows of d floats (a nullable).
hipError_t launch_cosine(const float *x, const float *y, const float *a, int rows, int d, float *out,
                         int64_t out_stride, hipStream_t s);

// Embedding of every row (h = E[token]), its sum of squares (one partial),
// and the RoPE (cos, sin) of its position.
struct EmbedParams {
    const void *E;
    int vocab, d;
    const int32_t *tokens;
    int64_t tok_ld;
    int tok_step;
    RowMap rows;
    float *h;
    float *ss;             // [Mtot]
    float2 *rope_cs;       // [Mtot][hd/2]
    int hd;
    float rope_theta;
};
hipError_t launch_embed(int dtype, const EmbedParams &p, int Mtot, hipStream_t s);

// Grouped causal attention over n_group consecutive layers.  With several
// key splits a second small kernel merges the split partials.
struct AttnParams {
    const float *q;        // [g][Mtot][hq][hd]
    int64_t q_sel_stride;
    const void *kc, *vc;   // arenas
    int layer0, n_group, batch, hq, hkv, hd, capacity;
    RowMap rows;
    int max_pos;           // host bound of positions in this call
    int splits;
    void *o;               // [g][Mtot][hq*hd] float32, or o_packed > 0: packed
                           // bf16 operand rows [g][o_packed][hq*hd] (hi at row
                           // m, lo at row m + o_packed / 2)
    int o_packed;
    int64_t o_sel_stride;
    float *part_acc;       // [splits][g][Mtot][hq][hd]
    float *part_ml;        // [splits][g][Mtot][hq][2]
    int Mtot;
};
hipError_t launch_attention(int dtype, const AttnParams &p, hipStream_t s);
int attention_splits(int dtype, int hd, int n_group, int batch, int hq, int hkv, int mseq, int max_pos);
int attention_split_max();
int attention_max_group();   // largest n_q_heads / n_kv_heads

// Arg-max reduction of the lm-head sampling partials -> tokens.
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
