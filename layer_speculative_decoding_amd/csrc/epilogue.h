// Operand loading and epilogues shared by the weight-streaming products (VALU
// GEMV and MFMA skinny GEMM).
//
//  * X_NORM operands: RMSNorm is folded into the consumer.  Activation row m
//    is gain[k] * h[k] * inv_rms (float32); whoever last wrote h (the embedding,
//    or a residual-add epilogue below) left per-block partial sums of squares,
//    and every consuming block sums a row's partials in block order, so no
//    separate normalisation launch and no cross-block synchronisation exist.
//  * Epilogues add the bias and apply the fused consumer: QKV RoPE + KV
//    append and the SiLU gate take a pair of output rows; store, residual
//    add, attention-output routing and logits + arg-max take one row.
//  * Residual writers emit those per-block partial sums of squares.
#pragma once
#include "spec_device.h"
#include "spec_kernels.h"

namespace spec {

__device__ __forceinline__ void row_of(const RowMap &rm, int gm, int &b, int &pos, bool &valid) {
    b = gm / rm.mseq;
    const int i = gm - b * rm.mseq;
    const int nt = rm.n_tok ? rm.n_tok[b] : rm.mseq;
    pos = rm.start_pos[b] + i;
    valid = i < nt && pos >= 0 && pos < rm.capacity;
}

// residual row read by activation row gm (last valid row of a sequence when
// gathering)
__device__ __forceinline__ int x_row(const GemvParams &p, int gm) {
    if (p.xgather_mseq <= 0) return gm;
    int nt = p.xgather_ntok ? p.xgather_ntok[gm] : p.xgather_mseq;
    nt = nt < 1 ? 1 : (nt > p.xgather_mseq ? p.xgather_mseq : nt);
    return gm * p.xgather_mseq + nt - 1;
}

// 1/rms of residual row hrow from its p.xnparts sum-of-squares partials.
// Lane i adds partials i, i + 64, ... in that order,
// then a fixed xor tree: every caller forms the same bits.  Whole wave.
__device__ __forceinline__ float row_inv_rms(const GemvParams &p, int hrow, int sel = 0) {
    const int lane = threadIdx.x & 63;
    const float *src = p.xss + (int64_t)sel * p.xss_sel_stride + (int64_t)hrow * p.xnparts;
    const int n = p.xnparts;
    // every load of up to 2048 partials in flight at once (one round trip;
    // out-of-range slots add zero, so the order of the sum is unchanged)
    constexpr int NB = 32;
    float s = 0.f;
    for (int i0 = 0; i0 < n; i0 += NB * 64) {
        float v[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int i = i0 + lane + 64 * j;
            v[j] = i < n ? src[i] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) s += v[j];
    }
    s = wave_sum(s);
    return 1.0f / sqrtf(s / (float)p.K + p.eps);
}

// 8 normalised activations of residual row hrow at k .. k+7, as float
__device__ __forceinline__ void x_norm8(const GemvParams &p, int sel, int hrow, int k, float inv, float *o) {
    const float *h = p.xh + (int64_t)hrow * p.K + k;
    const float *g = p.xgain + (int64_t)sel * p.xgain_stride + k;
    float4 h0 = *reinterpret_cast<const float4 *>(h), h1 = *reinterpret_cast<const float4 *>(h + 4);
    if (p.xadd) {
        const float *a = p.xadd + (int64_t)sel * p.xadd_sel_stride + (int64_t)hrow * p.K + k;
        const float4 a0 = *reinterpret_cast<const float4 *>(a), a1 = *reinterpret_cast<const float4 *>(a + 4);
        h0.x += a0.x; h0.y += a0.y; h0.z += a0.z; h0.w += a0.w;
        h1.x += a1.x; h1.y += a1.y; h1.z += a1.z; h1.w += a1.w;
    }
    const float4 g0 = *reinterpret_cast<const float4 *>(g), g1 = *reinterpret_cast<const float4 *>(g + 4);
    o[0] = h0.x * inv * g0.x; o[1] = h0.y * inv * g0.y; o[2] = h0.z * inv * g0.z; o[3] = h0.w * inv * g0.w;
    o[4] = h1.x * inv * g1.x; o[5] = h1.y * inv * g1.y; o[6] = h1.z * inv * g1.z; o[7] = h1.w * inv * g1.w;
}

__device__ __forceinline__ void x_norm4(const GemvParams &p, int sel, int hrow, int k, float inv, float *o) {
    const float *h = p.xh + (int64_t)hrow * p.K + k;
    const float *g = p.xgain + (int64_t)sel * p.xgain_stride + k;
    float4 h0 = *reinterpret_cast<const float4 *>(h);
    if (p.xadd) {
        const float4 a0 = *reinterpret_cast<const float4 *>(p.xadd + (int64_t)sel * p.xadd_sel_stride +
                                                            (int64_t)hrow * p.K + k);
        h0.x += a0.x; h0.y += a0.y; h0.z += a0.z; h0.w += a0.w;
    }
    const float4 g0 = *reinterpret_cast<const float4 *>(g);
    o[0] = h0.x * inv * g0.x; o[1] = h0.y * inv * g0.y; o[2] = h0.z * inv * g0.z; o[3] = h0.w * inv * g0.w;
}

// add v to acc[sel] without a dynamically indexed register array
__device__ __forceinline__ void add_sel(float (&acc)[kMaxSel], int sel, float v) {
#pragma unroll
    for (int s = 0; s < kMaxSel; ++s) acc[s] += (s == sel) ? v : 0.f;
}

// Epilogues whose output rows come in pairs: EPI_QKV_ROPE (the rotate-half
// partners j, j + hd/2 of a q or k head; v rows pass through) and
// EPI_SILU_MUL (gate row r0, up row r1).  u: the unit (pair) index, which is
// the activation column of the SiLU product.
template <typename T, int EPI>
__device__ __forceinline__ void epi_pair(const GemvParams &p, int u, int r0, int r1, int sel, int m, float y0,
                                         float y1) {
    using S = Store<T>;
    const int gm = p.m0 + m;
    if (p.bias) { y0 += p.bias[r0]; y1 += p.bias[r1]; }
    if constexpr (EPI == EPI_QKV_ROPE) {
        const int rl = r0 - sel * p.rows_per_sel;
        const int hd = p.hd;
        const int head = rl / hd;
        const int j = rl - head * hd;  // < hd / 2
        int b, pos; bool valid;
        row_of(p.rows, gm, b, pos, valid);
        const bool is_v = head >= p.hq + p.hkv;
        if (!is_v) {
            // rotate (x_j, x_{j+hd/2}) by the row's angle pos * theta^(-2j/hd)
            const float2 cs = p.rope_cs[(int64_t)gm * (hd / 2) + j];
            const float a = y0 * cs.x - y1 * cs.y;
            const float c = y1 * cs.x + y0 * cs.y;
            y0 = a;
            y1 = c;
        }
        if (head < p.hq) {
            float *q = p.q_out + (int64_t)sel * p.q_sel_stride + ((int64_t)gm * p.hq + head) * hd;
            q[j] = y0;
            q[j + hd / 2] = y1;
        } else if (valid) {
            const int kvh = head - p.hq - (is_v ? p.hkv : 0);
            T *c = reinterpret_cast<T *>(is_v ? p.vc : p.kc) +
                   ((((int64_t)(p.layer0 + sel) * p.batch + b) * p.hkv + kvh) * p.rows.capacity + pos) * hd;
            c[j] = S::from_f32(y0);
            c[j + hd / 2] = S::from_f32(y1);
        }
    } else if constexpr (EPI == EPI_SILU_MUL) {
        // column = gate row within its set member's [gate; up] block
        const int64_t col = r0 - (int64_t)sel * p.rows_per_sel + (int64_t)sel * p.act_sel_stride;
        const float a = silu(y0) * y1;
        if (p.act_packed) {
            // packed operand rows of the down product's matrix-core kernel
            uint16_t hi, lo;
            split2_one(a, hi, lo);
            uint16_t *a16 = reinterpret_cast<uint16_t *>(p.act);
            a16[(int64_t)gm * p.act_ld + col] = hi;
            a16[(int64_t)(gm + p.act_packed / 2) * p.act_ld + col] = lo;
        } else {
            reinterpret_cast<float *>(p.act)[(int64_t)gm * p.act_ld + col] = a;
        }
        (void)u;
    }
}

// Gumbel noise of vocab row v of the draft stream (kept out of line: the
// matrix-core epilogue calls it for several rows per lane).
__device__ __noinline__ float gumbel_one(uint64_t seed, uint32_t b, uint32_t pos, uint32_t v) {
    const Philox4 w = philox4x64_10(v >> 2, pos, 0, kDraft, seed, b);
    return pick_word(w, v & 3);
}

// The next RMSNorm's operand (gain-scaled, packed hi / lo) of residual
// value v at (row gm, column col).
__device__ __forceinline__ void store_nx(const GemvParams &p, int gm, int col, float v) {
    uint16_t hi, lo;
    split2_one(v * p.nx_gain[col], hi, lo);
    p.nx[(int64_t)gm * p.d + col] = hi;
    p.nx[(int64_t)(gm + p.nx_packed / 2) * p.d + col] = lo;
}

// Epilogues of single output rows.  ssv: this row's contribution to the
// sum of squares of the residual row the epilogue wrote (set member `sel`
// for parallel-MLP attention outputs, else member 0); best_v / best_i: the
// running arg-max of the sampling scores.
template <typename T, int EPI>
__device__ __forceinline__ void epi_row(const GemvParams &p, int r, int sel, int m, float y, float &ssv,
                                        float &best_v, int &best_i) {
    const int gm = p.m0 + m;
    if (p.bias) y += p.bias[r];
    const int rl = r - sel * p.rows_per_sel;
    if constexpr (EPI == EPI_STORE) {
        p.out[(int64_t)gm * p.out_ld + (int64_t)sel * p.out_sel_stride + rl] = y;
    } else if constexpr (EPI == EPI_RESID_ADD) {
        float *h = p.h + (int64_t)gm * p.d;
        float v = h[rl] + y;
        if (p.add2) {
            const int na = p.n_add2 > 1 ? p.n_add2 : 1;
            for (int j = 0; j < na; ++j) v += p.add2[j * p.add2_sel_stride + (int64_t)gm * p.d + rl];
        }
        h[rl] = v;
        ssv = fmaf(v, v, ssv);
        if (p.nx) store_nx(p, gm, rl, v);
    } else if constexpr (EPI == EPI_ATTN_OUT) {
        const int64_t row = (int64_t)gm * p.d;
        if (!p.par_mlp) {
            if (sel == 0) {
                float *h = p.h + row;
                const float v = h[rl] + y;
                h[rl] = v;
                ssv = fmaf(v, v, ssv);
                if (p.nx) store_nx(p, gm, rl, v);
            } else {
                p.out[(int64_t)sel * p.out_sel_stride + row + rl] = y;
            }
        } else {
            const float hv = p.h[row + rl];
            if (sel == 0) p.h0[row + rl] = hv;
            p.out[(int64_t)sel * p.out_sel_stride + row + rl] = y;
            const float s0 = hv + y;
            ssv = fmaf(s0, s0, ssv);
        }
    } else if constexpr (EPI == EPI_LOGITS) {
        if (p.out) p.out[(int64_t)gm * p.out_ld + rl] = y;
        float sc = y;
        if (p.inv_temp != 0.0f) {
            const int pos = p.samp_pos[gm] + (p.samp_ntok ? p.samp_ntok[gm] : p.samp_nconst);
            sc = y * p.inv_temp + gumbel_one(p.seed, (uint32_t)gm, (uint32_t)pos, (uint32_t)rl);
        }
        argmax_merge(best_v, best_i, sc, rl);
    }
}

// EPI_LOGITS for two adjacent rows r0, r0 + 1 (one Philox block serves both)
template <typename T>
__device__ __forceinline__ void epi_logits2(const GemvParams &p, int r0, int r1, int m, float y0, float y1,
                                            float &best_v, int &best_i) {
    const int gm = p.m0 + m;
    if (p.bias) { y0 += p.bias[r0]; y1 += p.bias[r1]; }
    if (p.out) {
        p.out[(int64_t)gm * p.out_ld + r0] = y0;
        p.out[(int64_t)gm * p.out_ld + r1] = y1;
    }
    float s0 = y0, s1 = y1;
    if (p.inv_temp != 0.0f) {
        const int pos = p.samp_pos[gm] + (p.samp_ntok ? p.samp_ntok[gm] : p.samp_nconst);
        float g0, g1;
        gumbel_pair(p.seed, (uint32_t)gm, (uint32_t)pos, kDraft, (uint32_t)r0, (uint32_t)r1, g0, g1);
        s0 = y0 * p.inv_temp + g0;
        s1 = y1 * p.inv_temp + g1;
    }
    argmax_merge(best_v, best_i, s0, r0);
    argmax_merge(best_v, best_i, s1, r1);
}

constexpr bool epi_is_pair(int epi) { return epi == EPI_QKV_ROPE || epi == EPI_SILU_MUL; }
constexpr bool epi_has_ss(int epi) { return epi == EPI_RESID_ADD || epi == EPI_ATTN_OUT; }

}  // namespace spec
