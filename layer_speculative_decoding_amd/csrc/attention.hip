// Grouped causal GQA attention over the KV caches of n_group consecutive
// layers in one launch (the attentions of a layer-parallel set, or one layer).
//
// A workgroup owns (query block, layer of the group, kv head, sequence, key
// split).  Its query vectors are the rows of the block times the q heads that
// share the kv head (GQA), so every K/V tile staged in LDS is used by all of
// them.  Softmax is online (running max / sum per query vector); with several
// key splits the partial (max, sum, unnormalised output) are merged by
// k_attn_merge in split order.
#include "spec_device.h"
#include "spec_kernels.h"

namespace spec {

namespace {

constexpr int kQV = 64;        // query vectors per workgroup
constexpr int kTK = 32;        // keys per LDS tile
constexpr int kSplitMax = 64;

template <typename T, int HD>
__global__ __launch_bounds__(256) void k_attn(AttnParams p) {
    using S = Store<T>;
    constexpr int E = S::kPer16;
    constexpr int NR = (kQV * HD + 255) / 256;
    __shared__ float q_s[kQV][HD];
    __shared__ float k_s[kTK][HD + 1];
    __shared__ float v_s[kTK][HD];
    __shared__ float s_s[kQV][kTK + 1];
    __shared__ float m_s[kQV], l_s[kQV], c_s[kQV];
    __shared__ int pos_s[kQV];

    const int tid = threadIdx.x;
    const int G = p.hq / p.hkv;
    const int QB = (kQV / G) > 0 ? kQV / G : 1;
    const int gi = blockIdx.y / p.hkv;
    const int kvh = blockIdx.y - gi * p.hkv;
    const int b = blockIdx.z / p.splits;
    const int sp = blockIdx.z - b * p.splits;
    const int mseq = p.rows.mseq;
    const int i0 = blockIdx.x * QB;
    const int nrows = min(QB, mseq - i0);
    const int QV = nrows * G;
    const int ntok = p.rows.n_tok ? p.rows.n_tok[b] : mseq;
    const int pos0 = p.rows.start_pos[b];
    const float scale = 1.0f / sqrtf((float)HD);

    for (int qv = tid; qv < kQV; qv += 256) {
        int pos = -1;
        if (qv < QV) {
            const int i = i0 + qv / G;
            if (i < ntok) {
                pos = pos0 + i;
                if (pos < 0 || pos >= p.capacity) pos = -1;
            }
        }
        pos_s[qv] = pos;
        m_s[qv] = -INFINITY;
        l_s[qv] = 0.f;
    }
    for (int idx = tid; idx < QV * HD; idx += 256) {
        const int qv = idx / HD, d = idx - (idx / HD) * HD;
        const int rr = qv / G, g = qv - rr * G;
        const int row = b * mseq + i0 + rr;
        q_s[qv][d] = p.q[(int64_t)gi * p.q_sel_stride + ((int64_t)row * p.hq + kvh * G + g) * HD + d];
    }
    // keys 0 .. kmax serve this block (rows hold consecutive positions)
    const int last_row = min(i0 + nrows, ntok) - 1;
    int kmax = last_row >= 0 ? pos0 + last_row : -1;
    if (kmax >= p.capacity) kmax = p.capacity - 1;
    const int total = kmax + 1;
    int per = (total + p.splits - 1) / p.splits;
    per = ((per + kTK - 1) / kTK) * kTK;
    const int ks = sp * per;
    const int ke = min(total, ks + per);

    const int64_t cache_off = ((((int64_t)(p.layer0 + gi) * p.batch + b) * p.hkv + kvh) * p.capacity) * HD;
    const T *Kc = reinterpret_cast<const T *>(p.kc) + cache_off;
    const T *Vc = reinterpret_cast<const T *>(p.vc) + cache_off;

    float acc[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = 0.f;
    __syncthreads();

    for (int t0 = ks; t0 < ke; t0 += kTK) {
        for (int idx = tid * E; idx < kTK * HD; idx += 256 * E) {
            const int s = idx / HD, d = idx - (idx / HD) * HD;
            float fk[E], fv[E];
            if (t0 + s < ke) {
                S::unpack(ld16(Kc + (int64_t)(t0 + s) * HD + d), fk);
                S::unpack(ld16(Vc + (int64_t)(t0 + s) * HD + d), fv);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) { fk[e] = 0.f; fv[e] = 0.f; }
            }
#pragma unroll
            for (int e = 0; e < E; ++e) { k_s[s][d + e] = fk[e]; v_s[s][d + e] = fv[e]; }
        }
        __syncthreads();
        for (int idx = tid; idx < QV * kTK; idx += 256) {
            const int qv = idx / kTK, s = idx - (idx / kTK) * kTK;
            const int key = t0 + s;
            float dot = 0.f;
#pragma unroll 16
            for (int d = 0; d < HD; ++d) dot = fmaf(q_s[qv][d], k_s[s][d], dot);
            s_s[qv][s] = (key < ke && key <= pos_s[qv]) ? dot * scale : -INFINITY;
        }
        __syncthreads();
        for (int qv = tid; qv < QV; qv += 256) {
            float mx = -INFINITY;
            for (int s = 0; s < kTK; ++s) mx = fmaxf(mx, s_s[qv][s]);
            const float m_old = m_s[qv];
            const float m_new = fmaxf(m_old, mx);
            if (m_new == -INFINITY) {
                for (int s = 0; s < kTK; ++s) s_s[qv][s] = 0.f;
                c_s[qv] = 1.f;
            } else {
                const float c = expf(m_old - m_new);
                float sum = 0.f;
                for (int s = 0; s < kTK; ++s) {
                    const float e = expf(s_s[qv][s] - m_new);
                    s_s[qv][s] = e;
                    sum += e;
                }
                l_s[qv] = l_s[qv] * c + sum;
                m_s[qv] = m_new;
                c_s[qv] = c;
            }
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int idx = tid + 256 * r;
            if (idx < QV * HD) {
                const int qv = idx / HD, d = idx - (idx / HD) * HD;
                float a = acc[r] * c_s[qv];
#pragma unroll 8
                for (int s = 0; s < kTK; ++s) a = fmaf(s_s[qv][s], v_s[s][d], a);
                acc[r] = a;
            }
        }
        __syncthreads();
    }

    T *obase = reinterpret_cast<T *>(p.o) + (int64_t)gi * p.o_sel_stride;
    if (p.splits == 1) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int idx = tid + 256 * r;
            if (idx < QV * HD) {
                const int qv = idx / HD, d = idx - (idx / HD) * HD;
                const int rr = qv / G, g = qv - rr * G;
                const int row = b * mseq + i0 + rr;
                const float l = l_s[qv];
                const float val = (pos_s[qv] >= 0 && l > 0.f) ? acc[r] / l : 0.f;
                obase[(int64_t)row * p.hq * HD + (kvh * G + g) * HD + d] = S::from_f32(val);
            }
        }
        return;
    }
    // several key splits: publish (max, sum, unnormalised output)
    const int64_t stride_sp = (int64_t)p.n_group * p.Mtot * p.hq;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int idx = tid + 256 * r;
        if (idx < QV * HD) {
            const int qv = idx / HD, d = idx - (idx / HD) * HD;
            const int rr = qv / G, g = qv - rr * G;
            const int row = b * mseq + i0 + rr;
            const int64_t pr = (int64_t)sp * stride_sp + ((int64_t)gi * p.Mtot + row) * p.hq + kvh * G + g;
            p.part_acc[pr * HD + d] = acc[r];
            if (d == 0) {
                p.part_ml[pr * 2 + 0] = m_s[qv];
                p.part_ml[pr * 2 + 1] = l_s[qv];
            }
        }
    }
}

// Merge the key splits of one (layer, row, q head) per wave: out = sum_s w_s
// acc_s / sum_s w_s l_s with w_s = exp(m_s - max_s m_s), in split order.
template <typename T>
__global__ __launch_bounds__(256) void k_attn_merge(AttnParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t n_items = (int64_t)p.n_group * p.Mtot * p.hq;
    if (item >= n_items) return;
    const int HD = p.hd;
    const int64_t stride_sp = n_items;
    float mx = -INFINITY;
    for (int s2 = 0; s2 < p.splits; ++s2) mx = fmaxf(mx, p.part_ml[(item + s2 * stride_sp) * 2]);
    const int gi = (int)(item / ((int64_t)p.Mtot * p.hq));
    const int64_t rh = item - (int64_t)gi * p.Mtot * p.hq;       // row * hq + head
    T *o = reinterpret_cast<T *>(p.o) + (int64_t)gi * p.o_sel_stride + rh * HD;
    for (int d = lane; d < HD; d += 64) {
        float num = 0.f, den = 0.f;
        if (mx != -INFINITY) {
            for (int s2 = 0; s2 < p.splits; ++s2) {
                const int64_t pr = item + s2 * stride_sp;
                const float mm = p.part_ml[pr * 2];
                const float w = mm == -INFINITY ? 0.f : expf(mm - mx);
                num = fmaf(w, p.part_acc[pr * HD + d], num);
                den = fmaf(w, p.part_ml[pr * 2 + 1], den);
            }
        }
        o[d] = Store<T>::from_f32(den > 0.f ? num / den : 0.f);
    }
}

template <typename T, int HD>
hipError_t launch_hd(const AttnParams &p, hipStream_t s) {
    const int G = p.hq / p.hkv;
    const int QB = (kQV / G) > 0 ? kQV / G : 1;
    dim3 grid((p.rows.mseq + QB - 1) / QB, p.n_group * p.hkv, p.batch * p.splits);
    hipLaunchKernelGGL((k_attn<T, HD>), grid, dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    const int64_t items = (int64_t)p.n_group * p.Mtot * p.hq;
    hipLaunchKernelGGL(k_attn_merge<T>, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const AttnParams &p, hipStream_t s) {
    switch (p.hd) {
    case 16: return launch_hd<T, 16>(p, s);
    case 32: return launch_hd<T, 32>(p, s);
    case 64: return launch_hd<T, 64>(p, s);
    case 128: return launch_hd<T, 128>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int attention_split_max() { return kSplitMax; }

// Key splits so that decode-shaped calls (one query block per sequence) fill
// the GPU; prompt-length calls already have many query blocks.
int attention_splits(int n_group, int batch, int hq, int hkv, int mseq, int max_pos) {
    const int G = hq / hkv;
    const int QB = (kQV / G) > 0 ? kQV / G : 1;
    const int nqb = (mseq + QB - 1) / QB;
    if (nqb > 1 || batch * mseq > 64) return 1;
    const int base = n_group * hkv * batch;
    const int tiles = (max_pos + 1 + kTK - 1) / kTK;
    int sp = (1024 + base - 1) / base;
    if (sp > tiles) sp = tiles;
    if (sp > kSplitMax) sp = kSplitMax;
    return sp < 1 ? 1 : sp;
}

hipError_t launch_attention(int dtype, const AttnParams &p, hipStream_t s) {
    return dtype ? launch_t<uint16_t>(p, s) : launch_t<float>(p, s);
}

}  // namespace spec
