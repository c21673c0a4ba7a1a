// Epilogues shared by the weight-streaming products (VALU GEMV and MFMA
// skinny GEMM): given the two output rows r0, r1 of a unit for activation row
// m, apply bias and the fused consumer (store, QKV RoPE + KV append, SiLU
// gate, residual add, logits + sampling arg-max).
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

// Rotate the pair (x0, x1) = (x_j, x_{j+hd/2}) by pos * theta^(-2j/hd).  The
// angle is formed and reduced modulo 2*pi in double precision so that large
// positions keep full float32 accuracy.
__device__ __forceinline__ void rope_pair(float &x0, float &x1, int pos, int j, int hd, float theta) {
    const double inv_freq = pow((double)theta, -2.0 * (double)j / (double)hd);
    double ang = (double)pos * inv_freq;
    const double two_pi = 6.283185307179586476925286766559;
    ang -= two_pi * rint(ang / two_pi);
    float sn, cs;
    sincosf((float)ang, &sn, &cs);
    const float a = x0 * cs - x1 * sn;
    const float c = x1 * cs + x0 * sn;
    x0 = a;
    x1 = c;
}

template <typename T>
__device__ __forceinline__ void epilogue(const GemvParams &p, int u, int r0, int r1, int sel, int m,
                                         float y0, float y1, float &best_v, int &best_i) {
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
        if (head < p.hq) {
            rope_pair(y0, y1, valid ? pos : 0, j, hd, p.rope_theta);
            float *q = p.q_out + (int64_t)sel * p.q_sel_stride + ((int64_t)gm * p.hq + head) * hd;
            q[j] = y0;
            q[j + hd / 2] = y1;
        } else if (valid) {
            const bool is_k = head < p.hq + p.hkv;
            const int kvh = head - p.hq - (is_k ? 0 : p.hkv);
            if (is_k) rope_pair(y0, y1, pos, j, hd, p.rope_theta);
            T *c = reinterpret_cast<T *>(is_k ? p.kc : p.vc) +
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
        float *o = p.out + (int64_t)gm * p.out_ld;
        o[r0] += y0;
        o[r1] += y1;
        break;
    }
    case EPI_LOGITS: {
        if (p.out) {
            float *o = p.out + (int64_t)gm * p.out_ld;
            o[r0] = y0;
            o[r1] = y1;
        }
        float s0 = y0, s1 = y1;
        if (p.inv_temp != 0.0f) {
            const int pos = p.samp_pos[gm] + (p.samp_ntok ? p.samp_ntok[gm] : p.samp_nconst);
            float g[4];
            gumbel4(p.seed, (uint32_t)gm, (uint32_t)pos, kDraft, (uint32_t)(r0 >> 2), g);
            s0 = y0 * p.inv_temp + g[r0 & 3];
            s1 = y1 * p.inv_temp + g[r1 & 3];
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
