// Operand loading and epilogues shared by the weight-streaming products (VALU
// GEMV and MFMA skinny GEMM).
//
//  * X_NORM operands: RMSNorm is folded into the consumer.  Activation row m
//    is round(gain[k] * h[k] * inv_rms); whoever last wrote h (the embedding,
//    or a residual-add epilogue below) left per-block partial sums of squares,
//    and every consuming block sums a row's partials in block order, so no
//    separate normalisation launch and no cross-block synchronisation exist.
//  * Epilogues get the two output rows r0, r1 of a unit for activation row m,
//    add the bias and apply the fused consumer: store, QKV RoPE + KV append,
//    SiLU gate, residual add, attention-output routing, logits + arg-max.
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

// 1/rms of this launch's activation rows into inv_s[0 .. M-1]: wave w sums the
// partials of rows w, w + nw, ... (lane-strided, then a fixed tree); every
// block computes bit-identical values.  Call with the whole block.
__device__ __forceinline__ void block_inv_rms(const GemvParams &p, float *inv_s) {
    if (p.xmode != X_NORM) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    for (int m = wave; m < p.M; m += nw) {
        const float *src = p.xss + (int64_t)x_row(p, p.m0 + m) * p.xnparts;
        float s = 0.f;
        for (int i = lane; i < p.xnparts; i += 64) s += src[i];
        s = wave_sum(s);
        if (lane == 0) inv_s[m] = 1.0f / sqrtf(s / (float)p.K + p.eps);
    }
    __syncthreads();
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

// kLogits: instance that carries the logits / sampling case (the Philox and
// Gumbel code is kept out of the register budget of the other instances)
template <typename T, bool kLogits>
__device__ __forceinline__ void epilogue(const GemvParams &p, int u, int r0, int r1, int sel, int m,
                                         float y0, float y1, float &best_v, int &best_i,
                                         float (&ss)[kMaxSel]) {
    using S = Store<T>;
    const int gm = p.m0 + m;
    if (p.bias) { y0 += p.bias[r0]; y1 += p.bias[r1]; }
    switch (p.epi) {
    case EPI_STORE: {
        const int64_t base = (int64_t)gm * p.out_ld + (int64_t)sel * p.out_sel_stride - (int64_t)sel * p.rows_per_sel;
        p.out[base + r0] = y0;
        p.out[base + r1] = y1;
        break;
    }
    case EPI_QKV_ROPE: {
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
        break;
    }
    case EPI_SILU_MUL: {
        T *a = reinterpret_cast<T *>(p.act) + (int64_t)gm * p.act_ld + u;
        *a = S::from_f32(silu(y0) * y1);
        break;
    }
    case EPI_RESID_ADD: {
        float *h = p.h + (int64_t)gm * p.d;
        float v0 = h[r0] + y0, v1 = h[r1] + y1;
        if (p.add2) {
            const float *a = p.add2 + (int64_t)gm * p.d;
            v0 += a[r0];
            v1 += a[r1];
        }
        h[r0] = v0;
        h[r1] = v1;
        add_sel(ss, 0, v0 * v0 + v1 * v1);
        break;
    }
    case EPI_ATTN_OUT: {
        const int rl0 = r0 - sel * p.rows_per_sel, rl1 = r1 - sel * p.rows_per_sel;
        const int64_t row = (int64_t)gm * p.d;
        if (!p.par_mlp) {
            if (sel == 0) {
                float *h = p.h + row;
                const float v0 = h[rl0] + y0, v1 = h[rl1] + y1;
                h[rl0] = v0;
                h[rl1] = v1;
                add_sel(ss, 0, v0 * v0 + v1 * v1);
            } else {
                float *a = p.out + (int64_t)sel * p.out_sel_stride + row;
                a[rl0] = y0;
                a[rl1] = y1;
            }
        } else {
            const float *h = p.h + row;
            const float h0 = h[rl0], h1 = h[rl1];
            if (sel == 0) {
                p.h0[row + rl0] = h0;
                p.h0[row + rl1] = h1;
            }
            float *a = p.out + (int64_t)sel * p.out_sel_stride + row;
            a[rl0] = y0;
            a[rl1] = y1;
            const float s0 = h0 + y0, s1 = h1 + y1;
            add_sel(ss, sel, s0 * s0 + s1 * s1);
        }
        break;
    }
    case EPI_LOGITS: {
        if constexpr (!kLogits) break;
        if (p.out) {
            float *o = p.out + (int64_t)gm * p.out_ld;
            o[r0] = y0;
            o[r1] = y1;
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
        break;
    }
    default:
        break;
    }
}

}  // namespace spec
