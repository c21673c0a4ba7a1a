// Grouped causal GQA attention over the KV caches of n_group consecutive
// layers in one launch (the attentions of a layer-parallel set, or one layer).
//
// A workgroup owns (query block, layer of the group, kv head, sequence, key
// split).  Its query vectors are the rows of the block times the q heads that
// share the kv head (GQA), so every K/V tile staged in LDS serves all of them.
// Per 64-key tile:
//   QK   lane = key, the four waves split the query vectors; the key's row is
//        read from LDS in 16-byte pieces and every query element is a
//        wave-uniform (broadcast) LDS read, so one K read feeds many FMAs;
//   softmax  wave = query vector, lane = key: running max / sum with wave
//        reductions (online softmax, float32);
//   PV   lane = head dimension, four keys per step.
// The next tile's K/V is prefetched into registers while the current one is
// processed.  With several key splits the partial (max, sum, unnormalised
// output) are merged by k_attn_merge in split order.
#include "spec_device.h"
#include "spec_kernels.h"

namespace spec {

namespace {

constexpr int kQV = 64;        // query vectors per workgroup
constexpr int kTK = 64;        // keys per tile
constexpr int kSplitMax = 64;

template <typename T, int HD>
__global__ __launch_bounds__(256) void k_attn(AttnParams p) {
    using S = Store<T>;
    constexpr int E = S::kPer16;                 // elements per 16-byte piece
    constexpr int KROW = HD + 16 / sizeof(T);    // LDS row stride (elements), padded by 16 bytes
    constexpr int NPF = (kTK * HD / E + 255) / 256;   // 16-byte pieces of one tile per thread
    constexpr int QVW = kQV / 4;                 // query vectors per wave in QK
    constexpr int DPT = 256 / HD;                // threads per head dimension in PV
    constexpr int NQP = kQV / DPT;               // query vectors per thread in PV (max)
    __shared__ __align__(16) float q_s[kQV][HD];
    __shared__ __align__(16) T k_s[kTK][KROW];
    __shared__ __align__(16) T v_s[kTK][KROW];
    __shared__ __align__(16) float p_s[kQV][kTK];
    __shared__ float m_s[kQV], l_s[kQV], c_s[kQV];
    __shared__ int pos_s[kQV];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

    // prefetch of one tile: piece f (16 bytes) of thread tid covers key
    // (tid + 256 f) / (HD / E), elements ((tid + 256 f) % (HD / E)) * E
    uint4 kpf[NPF], vpf[NPF];
    auto fetch = [&](int t0) {
#pragma unroll
        for (int f = 0; f < NPF; ++f) {
            const int idx = tid + 256 * f;
            const int key = idx / (HD / E), e0 = (idx % (HD / E)) * E;
            kpf[f] = make_uint4(0, 0, 0, 0);
            vpf[f] = make_uint4(0, 0, 0, 0);
            if (key < kTK && t0 + key < ke) {
                kpf[f] = ld16(Kc + (int64_t)(t0 + key) * HD + e0);
                vpf[f] = ld16(Vc + (int64_t)(t0 + key) * HD + e0);
            }
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int f = 0; f < NPF; ++f) {
            const int idx = tid + 256 * f;
            const int key = idx / (HD / E), e0 = (idx % (HD / E)) * E;
            if (key < kTK) {
                *reinterpret_cast<uint4 *>(&k_s[key][e0]) = kpf[f];
                *reinterpret_cast<uint4 *>(&v_s[key][e0]) = vpf[f];
            }
        }
    };
    if (ks < ke) fetch(ks);

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
    for (int idx = tid; idx < QV * (HD / 4); idx += 256) {
        const int qv = idx / (HD / 4), d4 = (idx % (HD / 4)) * 4;
        const int rr = qv / G, g = qv - rr * G;
        const int row = b * mseq + i0 + rr;
        *reinterpret_cast<float4 *>(&q_s[qv][d4]) = *reinterpret_cast<const float4 *>(
            p.q + (int64_t)gi * p.q_sel_stride + ((int64_t)row * p.hq + kvh * G + g) * HD + d4);
    }

    // PV ownership: thread -> head dimension pd, query vectors qg + DPT * j
    const int pd = tid % HD;
    const int qg = tid / HD;
    float acc[NQP];
#pragma unroll
    for (int j = 0; j < NQP; ++j) acc[j] = 0.f;

    for (int t0 = ks; t0 < ke; t0 += kTK) {
        __syncthreads();   // previous tile consumed; q_s, pos_s, m_s ready
        stash();
        if (t0 + kTK < ke) fetch(t0 + kTK);
        __syncthreads();
        // ---- QK: lane = key, wave handles query vectors wave, wave+4, ...
        float sc[QVW];
#pragma unroll
        for (int j = 0; j < QVW; ++j) sc[j] = 0.f;
        for (int e0 = 0; e0 < HD; e0 += E) {
            float kf[E];
            S::unpack(*reinterpret_cast<const uint4 *>(&k_s[lane][e0]), kf);
#pragma unroll
            for (int j = 0; j < QVW; ++j) {
                const int qv = wave + 4 * j;
                if (qv < QV) {
#pragma unroll
                    for (int e = 0; e < E; e += 4) {
                        const float4 qq = *reinterpret_cast<const float4 *>(&q_s[qv][e0 + e]);
                        sc[j] = fmaf(qq.x, kf[e], sc[j]);
                        sc[j] = fmaf(qq.y, kf[e + 1], sc[j]);
                        sc[j] = fmaf(qq.z, kf[e + 2], sc[j]);
                        sc[j] = fmaf(qq.w, kf[e + 3], sc[j]);
                    }
                }
            }
        }
        const int key = t0 + lane;
#pragma unroll
        for (int j = 0; j < QVW; ++j) {
            const int qv = wave + 4 * j;
            if (qv < QV) {
                // ---- online softmax of this query vector over the tile
                const float s = (key < ke && key <= pos_s[qv]) ? sc[j] * scale : -INFINITY;
                const float mx = wave_max(s);
                const float m_old = m_s[qv];
                const float m_new = fmaxf(m_old, mx);
                float pv = 0.f, c = 1.f;
                if (m_new != -INFINITY) {
                    pv = expf(s - m_new);
                    c = expf(m_old - m_new);
                }
                const float sum = wave_sum(pv);
                p_s[qv][lane] = pv;
                if (lane == 0) {
                    l_s[qv] = l_s[qv] * c + sum;
                    m_s[qv] = m_new;
                    c_s[qv] = c;
                }
            }
        }
        __syncthreads();
        // ---- PV: lane = head dimension, four keys per step
#pragma unroll
        for (int j = 0; j < NQP; ++j) {
            const int qv = qg + DPT * j;
            if (qv < QV) acc[j] *= c_s[qv];
        }
        const int nk = min(kTK, ke - t0);
        for (int kk = 0; kk < nk; kk += 4) {
            float vv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) vv[u] = S::to_f32(v_s[kk + u][pd]);
#pragma unroll
            for (int j = 0; j < NQP; ++j) {
                const int qv = qg + DPT * j;
                if (qv < QV) {
                    const float4 pp = *reinterpret_cast<const float4 *>(&p_s[qv][kk]);
                    float a = acc[j];
                    a = fmaf(pp.x, vv[0], a);
                    a = fmaf(pp.y, vv[1], a);
                    a = fmaf(pp.z, vv[2], a);
                    a = fmaf(pp.w, vv[3], a);
                    acc[j] = a;
                }
            }
        }
    }
    __syncthreads();

    T *obase = reinterpret_cast<T *>(p.o) + (int64_t)gi * p.o_sel_stride;
    const int64_t stride_sp = (int64_t)p.n_group * p.Mtot * p.hq;
#pragma unroll
    for (int j = 0; j < NQP; ++j) {
        const int qv = qg + DPT * j;
        if (qv >= QV) continue;
        const int rr = qv / G, g = qv - rr * G;
        const int row = b * mseq + i0 + rr;
        if (p.splits == 1) {
            const float l = l_s[qv];
            const float val = (pos_s[qv] >= 0 && l > 0.f) ? acc[j] / l : 0.f;
            obase[(int64_t)row * p.hq * HD + (kvh * G + g) * HD + pd] = S::from_f32(val);
        } else {
            // several key splits: publish (max, sum, unnormalised output)
            const int64_t pr = (int64_t)sp * stride_sp + ((int64_t)gi * p.Mtot + row) * p.hq + kvh * G + g;
            p.part_acc[pr * HD + pd] = acc[j];
            if (pd == 0) {
                p.part_ml[pr * 2 + 0] = m_s[qv];
                p.part_ml[pr * 2 + 1] = l_s[qv];
            }
        }
    }
}

// Merge the key splits of one (layer, row, q head) per wave: out = sum_s w_s
// acc_s / sum_s w_s l_s with w_s = exp(m_s - max_s m_s).  Lane s reads split
// s's (m, l); the weights' sum uses a fixed reduction tree and the outputs
// accumulate in split order.
template <typename T>
__global__ __launch_bounds__(256) void k_attn_merge(AttnParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t n_items = (int64_t)p.n_group * p.Mtot * p.hq;
    if (item >= n_items) return;
    const int HD = p.hd;
    const int64_t stride_sp = n_items;
    float m = -INFINITY, l = 0.f;
    if (lane < p.splits) {
        m = p.part_ml[(item + lane * stride_sp) * 2];
        l = p.part_ml[(item + lane * stride_sp) * 2 + 1];
    }
    const float mx = wave_max(m);
    const float w = (lane < p.splits && m != -INFINITY) ? expf(m - mx) : 0.f;
    const float den = wave_sum(w * l);
    const int gi = (int)(item / ((int64_t)p.Mtot * p.hq));
    const int64_t rh = item - (int64_t)gi * p.Mtot * p.hq;       // row * hq + head
    T *o = reinterpret_cast<T *>(p.o) + (int64_t)gi * p.o_sel_stride + rh * HD;
    for (int d = lane; d < HD; d += 64) {
        float num = 0.f;
        int s2 = 0;
        for (; s2 + 4 <= p.splits; s2 += 4) {
            float a[4], ww[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                a[u] = p.part_acc[(item + (s2 + u) * stride_sp) * HD + d];
                ww[u] = __shfl(w, s2 + u, 64);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) num = fmaf(ww[u], a[u], num);
        }
        for (; s2 < p.splits; ++s2) num = fmaf(__shfl(w, s2, 64), p.part_acc[(item + s2 * stride_sp) * HD + d], num);
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
    int sp = (512 + base - 1) / base;
    if (sp > tiles) sp = tiles;
    if (sp > kSplitMax) sp = kSplitMax;
    return sp < 1 ? 1 : sp;
}

hipError_t launch_attention(int dtype, const AttnParams &p, hipStream_t s) {
    return dtype ? launch_t<uint16_t>(p, s) : launch_t<float>(p, s);
}

}  // namespace spec
