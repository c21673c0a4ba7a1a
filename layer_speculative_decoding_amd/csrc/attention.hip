// Grouped causal GQA attention over the KV caches of n_group consecutive
// layers in one launch (the attentions of a layer-parallel set, or one layer).
//
// A workgroup owns (query block, layer of the group, kv head, sequence, key
// split).  Its query vectors are the rows of the block times the q heads that
// share the kv head (GQA): 16 of them (NQB = 1), zero-padded, held in registers as
// the B operand of float32 matrix-core products (v_mfma_f32_16x16x4_f32).
// The four waves take interleaved 16-key blocks of the split's key range and
// run independently, reading K and V straight from HBM (no LDS staging):
//   QK   S[key][qv] = sum_d K[key][d] q[qv][d]; lane (c, g) = (l % 16, l / 16)
//        supplies K[key c][dims of group g] and q[qv c][the same dims], so
//        each lane's K slice is contiguous in memory.  With a bfloat16 cache
//        and head_dim a multiple of 32 the slices are eight dims, exactly the
//        operand of v_mfma_f32_16x16x32_bf16: K goes in as loaded and q as
//        two bfloat16 pieces (hi + lo, within 2^-16 of the float32 value: the
//        products' operand precision), two products per 32 dims instead of
//        eight float32 ones, which matters where the matrix cores bound the
//        kernel (long contexts, many rows);
//   softmax  online (running max and sum per query vector) in float32, the
//        scores in log2 units (1/sqrt(hd) * log2(e)) so that v_exp_f32 (2^x)
//        forms the weights; the scores of query vector c sit in lane group
//        column c;
//   PV   O[qv][dim] += P[qv][key] V[key][dim]: the probabilities are used in
//        place as the A operand, lane (c, g) supplies V[key 4g + r][dims
//        (HD / 16) c ...], so each lane reads HD / 16 contiguous elements.
//        On the bfloat16 path a wave takes 32-key chunks (two blocks): lane
//        (c, g) then holds P of keys 4g..4g+3 and 16+4g..16+4g+3, which is an
//        A operand of v_mfma_f32_16x16x32_bf16 as it stands (the order of the
//        summed keys inside one instruction is free as long as B matches);
//        the chunk's V rows go to a per-wave LDS stage and each lane reads
//        back the same eight keys of one dim (V is key-major in the cache, the
//        instruction wants eight keys per lane), P in two bfloat16 pieces.
// K and V enter exactly (bfloat16 in the cache); each piece times them is
// exact in float32, so the result equals the float32 dot products of the
// pieces' sums (within 2^-16 of q and P) up to summation order.  The
// waves' (max, sum, output) are merged in wave order through LDS; with several
// key splits the workgroup publishes them and k_attn_merge combines the splits
// in split order.
#include <cstdlib>

#include "spec_device.h"
#include "spec_kernels.h"

namespace spec {

namespace {

constexpr int kKB = 16;        // keys per block (one MFMA row block)
constexpr int kSplitMax = 64;
constexpr int kWaves = 4;
constexpr int kSpan = kKB * kWaves;   // keys per round of the four waves
constexpr int kMaxQV = 16;     // query vectors per workgroup (and q heads per kv head) at most

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8 as_bf16x8u(const uint4 &v) {
    bf16x8 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

// N consecutive elements of the cache type, widened to float.
template <int N>
__device__ __forceinline__ void load_span(const uint16_t *p, float *o) {
    if constexpr (N % 8 == 0) {
#pragma unroll
        for (int i = 0; i < N / 8; ++i) Store<uint16_t>::unpack(ld16(p + 8 * i), o + 8 * i);
    } else if constexpr (N == 4) {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
    } else if constexpr (N == 2) {
        const uint32_t v = *reinterpret_cast<const uint32_t *>(p);
        o[0] = bf16_lo(v); o[1] = bf16_hi(v);
    } else {
        static_assert(N == 1, "span");
        o[0] = bf16_to_f32(p[0]);
    }
}
template <int N>
__device__ __forceinline__ void load_span(const float *p, float *o) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) Store<float>::unpack(ld16(p + 4 * i), o + 4 * i);
    } else if constexpr (N == 2) {
        const float2 v = *reinterpret_cast<const float2 *>(p);
        o[0] = v.x; o[1] = v.y;
    } else {
        static_assert(N == 1, "span");
        o[0] = p[0];
    }
}

template <typename T, int N>
__device__ __forceinline__ void store_span(T *p, const float *v) {
#pragma unroll
    for (int i = 0; i < N; ++i) p[i] = Store<T>::from_f32(v[i]);
}

// N output elements of (layer gi, row, q head) from dim d0: float32 rows, or
// the packed operand of the O product's matrix-core kernel (bf16 hi pieces
// at row `row`, lo pieces at row + o_packed / 2)
template <int N>
__device__ __forceinline__ void store_out(const AttnParams &p, int gi, int row, int head, int d0, const float *v) {
    if (p.o_packed) {
        uint16_t *o = reinterpret_cast<uint16_t *>(p.o) + (int64_t)gi * p.o_sel_stride;
        uint16_t *hp = o + ((int64_t)row * p.hq + head) * p.hd + d0;
        uint16_t *lp = o + ((int64_t)(row + p.o_packed / 2) * p.hq + head) * p.hd + d0;
#pragma unroll
        for (int i = 0; i < N; ++i) split2_one(v[i], hp[i], lp[i]);
    } else {
        float *o = reinterpret_cast<float *>(p.o) + (int64_t)gi * p.o_sel_stride;
        store_span<float, N>(o + ((int64_t)row * p.hq + head) * p.hd + d0, v);
    }
}

// N consecutive cache elements kept as loaded (bf16 pairs stay packed until
// used, which halves the registers a K or V slice needs).
template <typename T, int N> struct Raw;
template <int N> struct Raw<uint16_t, N> {
    static constexpr int W = N >= 2 ? N / 2 : 1;
    uint32_t w[W];
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < W; ++i) w[i] = 0u;
    }
    __device__ __forceinline__ void load(const uint16_t *p) {
        if constexpr (N % 8 == 0) {
#pragma unroll
            for (int i = 0; i < N / 8; ++i) {
                const uint4 v = ld16(p + 8 * i);
                w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
            }
        } else if constexpr (N == 4) {
            const uint2 v = *reinterpret_cast<const uint2 *>(p);
            w[0] = v.x; w[1] = v.y;
        } else if constexpr (N == 2) {
            w[0] = *reinterpret_cast<const uint32_t *>(p);
        } else {
            static_assert(N == 1, "span");
            w[0] = p[0];
        }
    }
    __device__ __forceinline__ float operator[](int e) const {
        if constexpr (N == 1) return bf16_lo(w[0]);
        else return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
    }
};
template <int N> struct Raw<float, N> {
    float v[N];
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = 0.f;
    }
    __device__ __forceinline__ void load(const float *p) { load_span<N>(p, v); }
    __device__ __forceinline__ float operator[](int e) const { return v[e]; }
};

// The workgroup's query vector qv -> (row of the call, q head); -1 if padding.
struct QvMap {
    int G, QV, row0, head0;
    __device__ __forceinline__ bool valid(int qv) const { return qv < QV; }
    __device__ __forceinline__ int row(int qv) const { return row0 + qv / G; }
    __device__ __forceinline__ int head(int qv) const { return head0 + qv % G; }
};

template <typename T, int HD, int NQB>
__global__ __launch_bounds__(256) void k_attn(AttnParams p) {
    constexpr int DK = HD / 4 < 8 ? HD / 4 : 8;   // dims per lane per QK piece
    constexpr int NP = HD / (4 * DK);             // QK pieces per key
    constexpr int NT = HD / 4;                    // QK products per block (NP * DK)
    constexpr int DV = HD / 16;                   // dims per lane per key in PV
    constexpr int QVB = 16 * NQB;
    constexpr int NREG = NQB * DV * 4;            // output values per lane
    // bfloat16 caches with 8 dims per lane and piece run both products on the
    // bfloat16 matrix cores (two pieces per float32 operand): QK with the K slices as loaded,
    // PV over 32-key chunks whose V rows are staged per wave in LDS and read
    // back key-contiguous per lane, the layout of the B operand
    constexpr bool kBf = sizeof(T) == 2 && DK == 8;
    constexpr int CK = 32;                        // keys per chunk (two 16-key blocks)
    constexpr int VLD = HD + 8;                   // staged V row stride (elements)
    constexpr int NVL = kBf ? CK * HD / (8 * kWave) : 1;   // 16-byte V loads per lane and chunk
    __shared__ float m_s[kWaves][QVB], l_s[kWaves][QVB];
    __shared__ __align__(16) float o_s[kWaves - 1][NREG][64];
    __shared__ __align__(16) uint16_t vst[kBf ? kWaves * CK * VLD : 8];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, g = lane >> 4;
    const int G = p.hq / p.hkv;
    const int QB = QVB / G;                       // rows per workgroup
    // Workgroups are dispatched to the eight XCDs round robin by linear id,
    // and each XCD has its own L2.  The query blocks of one (layer, kv head,
    // sequence, split) read the same K / V, so the linear ids are renumbered
    // to put them eight apart (same XCD, close in time); a tail of fewer
    // than eight such groups keeps the plain order.
    int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
    {
        const int nqb = gridDim.x, ny = gridDim.y;
        const int lin = bx + nqb * (by + ny * bz);
        const int span = 8 * nqb;
        const int full = (nqb * ny * (int)gridDim.z) / span * span;
        if (nqb > 1 && lin < full) {
            const int off = lin % span;
            const int grp = (lin / span) * 8 + (off & 7);
            bx = off >> 3;
            by = grp % ny;
            bz = grp / ny;
        }
    }
    const int gi = by / p.hkv;
    const int kvh = by - gi * p.hkv;
    const int b = bz / p.splits;
    const int sp = bz - b * p.splits;
    const int mseq = p.rows.mseq;
    const int i0 = bx * QB;
    const int nrows = min(QB, mseq - i0);
    const int ntok = p.rows.n_tok ? p.rows.n_tok[b] : mseq;
    const int pos0 = p.rows.start_pos[b];
    // scores in log2 units (1/sqrt(hd) * log2(e)); exp2 forms the weights
    const float scale = 1.4426950408889634f / sqrtf((float)HD);
    const QvMap qm{G, nrows * G, b * mseq + i0, kvh * G};

    // keys 0 .. kmax serve this block (rows hold consecutive positions)
    const int last_row = min(i0 + nrows, ntok) - 1;
    int kmax = last_row >= 0 ? pos0 + last_row : -1;
    if (kmax >= p.capacity) kmax = p.capacity - 1;
    const int total = kmax + 1;
    // split ranges are whole rounds of the four waves (16-key blocks, or
    // 32-key chunks on the bfloat16 path)
    constexpr int SPAN = kBf ? CK * kWaves : kSpan;
    int per = (total + p.splits - 1) / p.splits;
    per = ((per + SPAN - 1) / SPAN) * SPAN;
    const int ks = sp * per;
    const int ke = min(total, ks + per);

    const int64_t cache_off = ((((int64_t)(p.layer0 + gi) * p.batch + b) * p.hkv + kvh) * p.capacity) * HD;
    const T *Kc = reinterpret_cast<const T *>(p.kc) + cache_off;
    const T *Vc = reinterpret_cast<const T *>(p.vc) + cache_off;

    // K / V slices of one key block: A operand of QK (K[key kb + c][dims of
    // lane group g]) and B operand of PV (V[key kb + 4 g + r][dims DV c ...])
    Raw<T, DK> kr[NP];
    Raw<T, DV> vr[4];
    auto load_kv = [&](int kb) {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            kr[i].zero();
            if (kb + c < ke) kr[i].load(Kc + (int64_t)(kb + c) * HD + DK * g + 4 * DK * i);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            vr[r].zero();
            if (kb + 4 * g + r < ke) vr[r].load(Vc + (int64_t)(kb + 4 * g + r) * HD + DV * c);
        }
    };
    // bfloat16 path: K of the chunk's two blocks and its V rows (16-byte
    // pieces, row-major, zero past the split's end)
    Raw<T, DK> kn[kBf ? 2 : 1][NP];
    uint4 vn[NVL];
    auto load_chunk = [&](int kb) {
#pragma unroll
        for (int hb = 0; hb < (kBf ? 2 : 1); ++hb)
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                kn[hb][i].zero();
                if (kb + 16 * hb + c < ke) kn[hb][i].load(Kc + (int64_t)(kb + 16 * hb + c) * HD + DK * g + 4 * DK * i);
            }
#pragma unroll
        for (int v = 0; v < NVL; ++v) {
            const int e = (v * kWave + lane) * 8, key = e / HD, dim = e - key * HD;
            vn[v] = kb + key < ke ? ld16(Vc + (int64_t)(kb + key) * HD + dim) : make_uint4(0, 0, 0, 0);
        }
    };
    // the first block is requested before the query vectors, the next one
    // before the current one is consumed
    if constexpr (kBf) {
        if (ks + CK * wave < ke) load_chunk(ks + CK * wave);
    } else {
        if (ks + kKB * wave < ke) load_kv(ks + kKB * wave);
    }

    // B operand of QK: q[qv = 16 nb + c][dim (4 DK) i + DK g + e] at t = DK i + e
    float qreg[NQB][NT];
    int qpos[NQB];
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) {
        const int qv = 16 * nb + c;
        int pos = -1;
        if (qm.valid(qv)) {
            const float *qp = p.q + (int64_t)gi * p.q_sel_stride + ((int64_t)qm.row(qv) * p.hq + qm.head(qv)) * HD;
#pragma unroll
            for (int i = 0; i < NP; ++i) load_span<DK>(qp + 4 * DK * i + DK * g, &qreg[nb][DK * i]);
            const int irow = i0 + qv / G;
            if (irow < ntok) {
                pos = pos0 + irow;
                if (pos < 0 || pos >= p.capacity) pos = -1;
            }
        } else {
#pragma unroll
            for (int t = 0; t < NT; ++t) qreg[nb][t] = 0.f;
        }
        qpos[nb] = pos;
    }

    // q as three bfloat16 pieces (B operand of QK on the bfloat16 path)
    uint4 qh[kBf ? NQB : 1][kBf ? NP : 1], ql[kBf ? NQB : 1][kBf ? NP : 1];
    if constexpr (kBf) {
#pragma unroll
        for (int nb = 0; nb < NQB; ++nb)
#pragma unroll
            for (int i = 0; i < NP; ++i) split2_bf16_hw(&qreg[nb][DK * i], qh[nb][i], ql[nb][i]);
    }

    float m_run[NQB], l_run[NQB];
    f32x4 acc[NQB][DV];
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) {
        m_run[nb] = -INFINITY;
        l_run[nb] = 0.f;
#pragma unroll
        for (int j = 0; j < DV; ++j) acc[nb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    if constexpr (kBf) {
        uint16_t *vt = vst + wave * CK * VLD;
        for (int kb = ks + CK * wave; kb < ke; kb += CK * kWaves) {
            // stage this chunk's V rows, then request the next chunk
#pragma unroll
            for (int v = 0; v < NVL; ++v) {
                const int e = (v * kWave + lane) * 8, key = e / HD, dim = e - key * HD;
                *reinterpret_cast<uint4 *>(&vt[key * VLD + dim]) = vn[v];
            }
            Raw<T, DK> kc2[2][NP];
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int i = 0; i < NP; ++i) kc2[hb][i] = kn[hb][i];
            if (kb + CK * kWaves < ke) load_chunk(kb + CK * kWaves);
            // the wave's own LDS writes precede its reads below (in-order LDS)
            asm volatile("" ::: "memory");
#pragma unroll
            for (int nb = 0; nb < NQB; ++nb) {
                // QK of both blocks: lane holds S[key kb + 16 hb + 4 g + r][qv 16 nb + c]
                float pr[8];
                float mx = -INFINITY;
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < NP; ++i) {
                        bf16x8 kv;
                        __builtin_memcpy(&kv, kc2[hb][i].w, 16);
                        // the small piece first
                        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, as_bf16x8u(ql[nb][i]), sc, 0, 0, 0);
                        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, as_bf16x8u(qh[nb][i]), sc, 0, 0, 0);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = kb + 16 * hb + 4 * g + r;
                        pr[4 * hb + r] = (key < ke && key <= qpos[nb]) ? sc[r] * scale : -INFINITY;
                        mx = fmaxf(mx, pr[4 * hb + r]);
                    }
                }
                mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
                mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
                const float m_new = fmaxf(m_run[nb], mx);
                const bool none = m_new == -INFINITY;
                float sum = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    pr[j] = none ? 0.f : __builtin_amdgcn_exp2f(pr[j] - m_new);
                    sum += pr[j];
                }
                sum += __shfl_xor(sum, 16, kWave);
                sum += __shfl_xor(sum, 32, kWave);
                const float corr = none ? 1.f : __builtin_amdgcn_exp2f(m_run[nb] - m_new);
                l_run[nb] = l_run[nb] * corr + sum;
                m_run[nb] = m_new;
                f32x4 cr;
#pragma unroll
                for (int r = 0; r < 4; ++r) cr[r] = __shfl(corr, 4 * g + r, kWave);
#pragma unroll
                for (int j = 0; j < DV; ++j) acc[nb][j] *= cr;
                // PV: A = P[qv c][keys of lane group g: 4g..4g+3, 16+4g..16+4g+3]
                // (as the QK output holds them), B = V[the same keys][dim DV c + j]
                uint4 ph4, pl4;
                split2_bf16_hw(pr, ph4, pl4);
                const bf16x8 ph = as_bf16x8u(ph4), pl = as_bf16x8u(pl4);
#pragma unroll
                for (int j = 0; j < DV; ++j) {
                    uint16_t vv[8];
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const int key = (t < 4 ? 0 : 16) + 4 * g + (t & 3);
                        vv[t] = vt[key * VLD + DV * c + j];
                    }
                    bf16x8 vb;
                    __builtin_memcpy(&vb, vv, 16);
                    acc[nb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, acc[nb][j], 0, 0, 0);
                    acc[nb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vb, acc[nb][j], 0, 0, 0);
                }
            }
            // this chunk's reads precede the next chunk's staging writes
            asm volatile("" ::: "memory");
        }
    } else {
        for (int kb = ks + kKB * wave; kb < ke; kb += kSpan) {
            Raw<T, DK> kcur[NP];
            Raw<T, DV> vcur[4];
    #pragma unroll
            for (int i = 0; i < NP; ++i) kcur[i] = kr[i];
    #pragma unroll
            for (int r = 0; r < 4; ++r) vcur[r] = vr[r];
            if (kb + kSpan < ke) load_kv(kb + kSpan);
    #pragma unroll
            for (int nb = 0; nb < NQB; ++nb) {
                f32x4 sc = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
                for (int i = 0; i < NP; ++i)
    #pragma unroll
                    for (int e = 0; e < DK; ++e)
                        sc = __builtin_amdgcn_mfma_f32_16x16x4f32(kcur[i][e], qreg[nb][DK * i + e], sc, 0, 0, 0);
                // lane holds S[key kb + 4 g + r][qv 16 nb + c]
                float pr[4];
                float mx = -INFINITY;
    #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = kb + 4 * g + r;
                    pr[r] = (key < ke && key <= qpos[nb]) ? sc[r] * scale : -INFINITY;
                    mx = fmaxf(mx, pr[r]);
                }
                mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
                mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
                const float m_new = fmaxf(m_run[nb], mx);
                const bool none = m_new == -INFINITY;
                float sum = 0.f;
    #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pr[r] = none ? 0.f : __builtin_amdgcn_exp2f(pr[r] - m_new);
                    sum += pr[r];
                }
                sum += __shfl_xor(sum, 16, kWave);
                sum += __shfl_xor(sum, 32, kWave);
                const float corr = none ? 1.f : __builtin_amdgcn_exp2f(m_run[nb] - m_new);
                l_run[nb] = l_run[nb] * corr + sum;
                m_run[nb] = m_new;
                // rescale of the outputs of query vectors 16 nb + 4 g + r (held by lane 4 g + r)
                f32x4 cr;
    #pragma unroll
                for (int r = 0; r < 4; ++r) cr[r] = __shfl(corr, 4 * g + r, kWave);
    #pragma unroll
                for (int j = 0; j < DV; ++j) acc[nb][j] *= cr;
    #pragma unroll
                for (int r = 0; r < 4; ++r)
    #pragma unroll
                    for (int j = 0; j < DV; ++j)
                        acc[nb][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(pr[r], vcur[r][j], acc[nb][j], 0, 0, 0);
            }
        }

    }

    // merge the four waves in wave order
    if (g == 0) {
#pragma unroll
        for (int nb = 0; nb < NQB; ++nb) {
            m_s[wave][16 * nb + c] = m_run[nb];
            l_s[wave][16 * nb + c] = l_run[nb];
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int nb = 0; nb < NQB; ++nb)
#pragma unroll
            for (int j = 0; j < DV; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) o_s[wave - 1][(nb * DV + j) * 4 + r][lane] = acc[nb][j][r];
    }
    __syncthreads();
    if (wave != 0) return;

    const int64_t stride_sp = (int64_t)p.n_group * p.Mtot * p.hq;
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int qv = 16 * nb + 4 * g + r;    // this lane's output rows
            float mw[kWaves], M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                mw[w] = m_s[w][qv];
                M = fmaxf(M, mw[w]);
            }
            float wt[kWaves], L = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                wt[w] = mw[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
                L = fmaf(wt[w], l_s[w][qv], L);
            }
            float ov[DV];
#pragma unroll
            for (int j = 0; j < DV; ++j) {
                float o = wt[0] * acc[nb][j][r];
#pragma unroll
                for (int w = 1; w < kWaves; ++w) o = fmaf(wt[w], o_s[w - 1][(nb * DV + j) * 4 + r][lane], o);
                ov[j] = o;
            }
            if (!qm.valid(qv)) continue;
            const int row = qm.row(qv), head = qm.head(qv);
            if (p.splits == 1) {
                const bool ok = L > 0.f;   // rows without a valid position have no keys
#pragma unroll
                for (int j = 0; j < DV; ++j) ov[j] = ok ? ov[j] / L : 0.f;
                store_out<DV>(p, gi, row, head, DV * c, ov);
            } else {
                // several key splits: publish (max, sum, unnormalised output)
                const int64_t pr = (int64_t)sp * stride_sp + ((int64_t)gi * p.Mtot + row) * p.hq + head;
                store_span<float, DV>(p.part_acc + pr * HD + DV * c, ov);
                if (c == 0) {
                    p.part_ml[pr * 2 + 0] = M;
                    p.part_ml[pr * 2 + 1] = L;
                }
            }
        }
    }
}

// Merge the key splits of one (layer, row, q head) per wave (a separate
// launch: merging in the last split's workgroup behind an agent-scope fence
// and a counter measured 3 us slower per call, the fence writing the XCD's
// L2 back): out = sum_s w_s
// acc_s / sum_s w_s l_s with w_s = 2^(m_s - max_s m_s) (scores in log2 units).  Lane s reads split
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
    const float w = (lane < p.splits && m != -INFINITY) ? __builtin_amdgcn_exp2f(m - mx) : 0.f;
    const float den = wave_sum(w * l);
    const int gi = (int)(item / ((int64_t)p.Mtot * p.hq));
    const int64_t rh = item - (int64_t)gi * p.Mtot * p.hq;       // row * hq + head
    const int row = (int)(rh / p.hq), head = (int)(rh - (int64_t)row * p.hq);
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
        const float v = den > 0.f ? num / den : 0.f;
        store_out<1>(p, gi, row, head, d, &v);
    }
}

// ---------------------------------------------------------------- prompt
// Causal attention of many consecutive rows (prompt prefills, long
// calibrations) over a bfloat16 cache, flash style: a workgroup owns QR
// consecutive rows of one sequence and all G q heads of one kv head (layer gi
// of the group).  Its 16-vector blocks are (head, 16 consecutive rows); wave w
// takes blocks w and w + 4.  Key tiles of 64 go once through LDS per
// workgroup and serve every block: K key-major (the A operand of QK, 16
// contiguous bytes per lane), V transposed to dim-major (the B operand of PV,
// a lane's eight keys in two 8-byte runs; PREF: the next tile is requested into
// registers during this tile's products).  q and the probabilities enter the
// bfloat16 matrix instructions as hi + lo pieces (split2_bf16: within 2^-16 of
// the float32 value), the products accumulate in float32, the softmax is online
// in float32 as in the decode kernel.  The key loop reads the K operand once
// per (key block, dim step) for both of a wave's blocks and the V operand once
// per (key chunk, dim block), and runs both blocks' products without branches
// (a wave's unused block, for G that does not divide 8, computes on zeros).
template <int HD, bool PREF>
__global__ __launch_bounds__(256, 2) void k_attn_prompt(AttnParams p, int QR) {
    constexpr int KT = 64;                 // keys per LDS tile
    constexpr int NQB = 2;                 // 16-vector blocks per wave
    constexpr int NS = HD / 32;            // 32-dim steps of QK
    constexpr int NJ = HD / 16;            // 16-dim blocks of PV
    constexpr int KLD = HD + 16;           // K row stride in LDS (elements: 160 or 288 bytes, where the
                                           // fragment reads are free of bank conflicts)
    constexpr int VLD = KT + 4;            // transposed V row stride (elements)
    __shared__ __align__(16) uint16_t ks[KT * KLD];
    __shared__ __align__(16) uint16_t vt[HD * VLD];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lg = lane >> 4;
    const int G = p.hq / p.hkv;
    const int NBK = G * (QR / 16);         // 16-vector blocks of the workgroup (<= 8)
    // Same-K/V workgroups eight apart in linear id (one XCD), heaviest query
    // tiles (latest rows) first.
    int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
    {
        const int nqb = gridDim.x, ny = gridDim.y;
        const int lin = bx + nqb * (by + ny * bz);
        const int span = 8 * nqb;
        const int full = (nqb * ny * (int)gridDim.z) / span * span;
        if (nqb > 1 && lin < full) {
            const int off = lin % span;
            const int grp = (lin / span) * 8 + (off & 7);
            bx = off >> 3;
            by = grp % ny;
            bz = grp / ny;
        }
        bx = nqb - 1 - bx;
    }
    const int gi = by / p.hkv, kvh = by - gi * p.hkv, b = bz;
    const int mseq = p.rows.mseq;
    const int i0 = bx * QR;
    const int ntok = p.rows.n_tok ? p.rows.n_tok[b] : mseq;
    const int pos0 = p.rows.start_pos[b];
    // scores in log2 units: q carries 1/sqrt(hd) * log2(e), exp2 forms the weights
    const float qscale = 1.4426950408889634f / sqrtf((float)HD);
    const int last = min(min(i0 + QR, ntok), mseq) - 1;
    int kend = last >= 0 ? pos0 + last + 1 : 0;
    if (kend > p.capacity) kend = p.capacity;
    const int64_t cache_off = ((((int64_t)(p.layer0 + gi) * p.batch + b) * p.hkv + kvh) * p.capacity) * HD;
    const uint16_t *Kc = reinterpret_cast<const uint16_t *>(p.kc) + cache_off;
    const uint16_t *Vc = reinterpret_cast<const uint16_t *>(p.vc) + cache_off;

    // this wave's blocks: head, first row, q operand pieces of row li, position
    bool bok[NQB];
    int head[NQB], rb0[NQB], qpos[NQB], qfull[NQB];
    uint4 qh[NQB][NS], ql[NQB][NS];
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) {
        const int blk = wave + 4 * nb;
        bok[nb] = blk < NBK;
        head[nb] = kvh * G + (bok[nb] ? blk % G : 0);
        rb0[nb] = i0 + 16 * (bok[nb] ? blk / G : 0);
        const int row = rb0[nb] + li;
        int pos = -1;
        if (bok[nb] && row < mseq && row < ntok) {
            pos = pos0 + row;
            if (pos < 0 || pos >= p.capacity) pos = -1;
        }
        qpos[nb] = pos;
        const bool rok = bok[nb] && row < mseq;
        const float *qp = p.q + (int64_t)gi * p.q_sel_stride + (((int64_t)b * mseq + row) * p.hq + head[nb]) * HD;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            float x[8];
            if (rok) {
                load_span<8>(qp + 32 * st + 8 * lg, x);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = 0.f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] *= qscale;
            split2_bf16_hw(x, qh[nb][st], ql[nb][st]);
        }
        // no row of the block masks a key below its first row's position
        // (and every row is a valid one): tiles ending there skip the mask
        const int nval = min(ntok, mseq) - rb0[nb];
        qfull[nb] = bok[nb] && nval >= 16 && pos0 + rb0[nb] + 15 < p.capacity ? pos0 + rb0[nb] : -1;
    }

    float m_run[NQB], l_run[NQB];
    f32x4 acc[NQB][NJ];
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) {
        m_run[nb] = -INFINITY;
        l_run[nb] = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[nb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // K / V of a tile: 16-byte pieces per thread, requested one tile ahead
    // (global -> registers during the previous tile's products)
    constexpr int NKL = KT * HD / 8 / 256;          // K pieces per thread
    constexpr int NVL = (KT / 2) * (HD / 8) / 256;  // V key-pair pieces per thread
    static_assert(NKL * 256 * 8 == KT * HD && NVL * 256 * 16 == KT * HD, "tile split");
    // (keys past kend read row kend - 1, a written row: the mask gives them
    // weight 0 and 0 times a finite V is 0)
    uint4 kreg[NKL], vreg[NVL][2];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int i = 0; i < NKL; ++i) {
            const int e = tid + 256 * i, key = e / (HD / 8), c8 = e - key * (HD / 8);
            kreg[i] = ld16(Kc + (int64_t)min(k0 + key, kend - 1) * HD + 8 * c8);
        }
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
            const int e = tid + 256 * i, kp = e / (HD / 8), c8 = e - kp * (HD / 8), key = 2 * kp;
            vreg[i][0] = ld16(Vc + (int64_t)min(k0 + key, kend - 1) * HD + 8 * c8);
            vreg[i][1] = ld16(Vc + (int64_t)min(k0 + key + 1, kend - 1) * HD + 8 * c8);
        }
    };
    if constexpr (PREF) {
        if (kend > 0) fetch(0);
    }

    for (int kt0 = 0; kt0 < kend; kt0 += KT) {
        if constexpr (!PREF) fetch(kt0);
        __syncthreads();   // the previous tile is consumed
        // K tile key-major; V tile transposed: two keys' 8 dims -> 8 (key pair) words
#pragma unroll
        for (int i = 0; i < NKL; ++i) {
            const int e = tid + 256 * i, key = e / (HD / 8), c8 = e - key * (HD / 8);
            *reinterpret_cast<uint4 *>(&ks[key * KLD + 8 * c8]) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
            const int e = tid + 256 * i, kp = e / (HD / 8), c8 = e - kp * (HD / 8), key = 2 * kp;
            const uint4 v0 = vreg[i][0], v1 = vreg[i][1];
            const uint32_t a[4] = {v0.x, v0.y, v0.z, v0.w}, c[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                *reinterpret_cast<uint32_t *>(&vt[(8 * c8 + 2 * w) * VLD + key]) = (a[w] & 0xFFFFu) | (c[w] << 16);
                *reinterpret_cast<uint32_t *>(&vt[(8 * c8 + 2 * w + 1) * VLD + key]) =
                    (a[w] >> 16) | (c[w] & 0xFFFF0000u);
            }
        }
        __syncthreads();
        if constexpr (PREF) {
            if (kt0 + KT < kend) fetch(kt0 + KT);
        }

        // QK: lane (li, lg), register r of key block kb holds S[key 16 kb + 4 lg + r][row li]
        f32x4 sc[NQB][4];
#pragma unroll
        for (int nb = 0; nb < NQB; ++nb)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) sc[nb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                const uint4 kv = *reinterpret_cast<const uint4 *>(&ks[(16 * kb + li) * KLD + 32 * st + 8 * lg]);
#pragma unroll
                for (int nb = 0; nb < NQB; ++nb) {
                    sc[nb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8u(kv), as_bf16x8u(ql[nb][st]),
                                                                         sc[nb][kb], 0, 0, 0);
                    sc[nb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8u(kv), as_bf16x8u(qh[nb][st]),
                                                                         sc[nb][kb], 0, 0, 0);
                }
            }

        // online softmax; the probabilities of chunk c (keys 32 c + 4 lg + r
        // and 32 c + 16 + 4 lg + r) become the A operand of PV as they sit
        uint4 ph[NQB][2], pl[NQB][2];
#pragma unroll
        for (int nb = 0; nb < NQB; ++nb) {
            float pr[16];
            float mx = -INFINITY;
            if (kt0 + KT - 1 <= qfull[nb] && kt0 + KT <= kend) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pr[4 * kb + r] = sc[nb][kb][r];
                        mx = fmaxf(mx, pr[4 * kb + r]);
                    }
            } else {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = kt0 + 16 * kb + 4 * lg + r;
                        const float v = (key < kend && key <= qpos[nb]) ? sc[nb][kb][r] : -INFINITY;
                        pr[4 * kb + r] = v;
                        mx = fmaxf(mx, v);
                    }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
            mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
            const float m_new = fmaxf(m_run[nb], mx);
            const bool none = m_new == -INFINITY;
            const float msub = none ? 0.f : m_new;   // exp2(-inf - 0) = 0
            float sum = 0.f;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                pr[t] = __builtin_amdgcn_exp2f(pr[t] - msub);
                sum += pr[t];
            }
            sum += __shfl_xor(sum, 16, kWave);
            sum += __shfl_xor(sum, 32, kWave);
            const float corr = none ? 1.f : __builtin_amdgcn_exp2f(m_run[nb] - m_new);
            l_run[nb] = l_run[nb] * corr + sum;
            m_run[nb] = m_new;
            f32x4 cr;
#pragma unroll
            for (int r = 0; r < 4; ++r) cr[r] = __shfl(corr, 4 * lg + r, kWave);
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[nb][j] *= cr;
#pragma unroll
            for (int c = 0; c < 2; ++c) split2_bf16_hw(&pr[8 * c], ph[nb][c], pl[nb][c]);
        }

        // PV: B = V[the same eight keys][dim 16 j + li]
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const uint16_t *vr = &vt[(16 * j + li) * VLD + 32 * c + 4 * lg];
                const uint2 v0 = *reinterpret_cast<const uint2 *>(vr);
                const uint2 v1 = *reinterpret_cast<const uint2 *>(vr + 16);
                const uint4 vb = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
                for (int nb = 0; nb < NQB; ++nb) {
                    acc[nb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8u(pl[nb][c]), as_bf16x8u(vb),
                                                                         acc[nb][j], 0, 0, 0);
                    acc[nb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8u(ph[nb][c]), as_bf16x8u(vb),
                                                                         acc[nb][j], 0, 0, 0);
                }
            }
    }

    // lane (li, lg), register r of dim block j holds O[row 4 lg + r][dim 16 j + li]
#pragma unroll
    for (int nb = 0; nb < NQB; ++nb) {
        if (!bok[nb]) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rr = 4 * lg + r;
            const float L = __shfl(l_run[nb], rr, kWave);
            const int row = rb0[nb] + rr;
            if (row >= mseq) continue;
            const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const float v = L > 0.f ? acc[nb][j][r] * inv : 0.f;
                store_out<1>(p, gi, b * mseq + row, head[nb], 16 * j + li, &v);
            }
        }
    }
}

// Rows per workgroup of the prompt kernel: blocks of 16 rows per q head, at
// most 8 blocks (two per wave).
int prompt_rows(int G) { return 16 * (8 / G >= 1 ? 8 / G : 1); }

// Calls of at least this many rows per sequence (and no key splits) use the
// prompt kernel on bfloat16 caches with head_dim 64 or 128 and at most 8 q
// heads per kv head (SPEC_ATTN_PROMPT=0: the decode kernel throughout).
constexpr int kPromptMinRows = 32;
bool prompt_kernel_enabled() {
    static const bool on = [] {
        const char *e = getenv("SPEC_ATTN_PROMPT");
        return !(e && e[0] == '0');
    }();
    return on;
}

// 16 query vectors per workgroup: measured against 32 (two blocks), the
// smaller register footprint and the doubled workgroup count win at every
// decode shape (8B verify, 6 rows, context 560: 12.9 vs 15.5 us; 8B verify,
// 9 rows, context 2100: 21.8 vs 33.6 us; 70B verify, 4 x 7 rows, context
// 8200: 128 vs 138 us).
int qv_blocks(int G, int mseq) { (void)G; (void)mseq; return 1; }

template <typename T, int HD, int NQB>
hipError_t launch_hd(const AttnParams &p, hipStream_t s) {
    const int G = p.hq / p.hkv;
    const int QB = 16 * NQB / G;
    dim3 grid((p.rows.mseq + QB - 1) / QB, p.n_group * p.hkv, p.batch * p.splits);
    hipLaunchKernelGGL((k_attn<T, HD, NQB>), grid, dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    const int64_t items = (int64_t)p.n_group * p.Mtot * p.hq;
    hipLaunchKernelGGL(k_attn_merge<T>, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <typename T, int HD>
hipError_t launch_nqb(const AttnParams &p, hipStream_t s) {
    return launch_hd<T, HD, 1>(p, s);
}

template <typename T>
hipError_t launch_t(const AttnParams &p, hipStream_t s) {
    if (p.hkv < 1 || p.hq % p.hkv || p.hq / p.hkv > kMaxQV || p.splits < 1 || p.splits > kSplitMax)
        return hipErrorInvalidValue;
    if constexpr (sizeof(T) == 2) {
        const int G = p.hq / p.hkv;
        if (p.splits == 1 && p.rows.mseq >= kPromptMinRows && G <= 8 && (p.hd == 64 || p.hd == 128) &&
            prompt_kernel_enabled()) {
            const int QR = prompt_rows(G);
            dim3 grid((p.rows.mseq + QR - 1) / QR, p.n_group * p.hkv, p.batch);
            // head_dim 128 fetches each tile after the barrier: requesting it a
            // tile ahead needs 32 more VGPRs and spills (8B layer, 2047 rows:
            // 172 vs 137 us); head_dim 64 has the room (1B layer: 74 us)
            if (p.hd == 64) hipLaunchKernelGGL((k_attn_prompt<64, true>), grid, dim3(256), 0, s, p, QR);
            else hipLaunchKernelGGL((k_attn_prompt<128, false>), grid, dim3(256), 0, s, p, QR);
            return hipGetLastError();
        }
    }
    switch (p.hd) {
    case 16: return launch_nqb<T, 16>(p, s);
    case 32: return launch_nqb<T, 32>(p, s);
    case 64: return launch_nqb<T, 64>(p, s);
    case 128: return launch_nqb<T, 128>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int attention_split_max() { return kSplitMax; }

// Key splits so that the workgroups of a call fill the GPU: about
// kTargetWG workgroups, each split at least one round of the four waves.
// Calls with more than 64 rows (prompt prefills) have many query blocks and
// never split (the split partials are sized for 64 rows).
int attention_splits(int dtype, int hd, int n_group, int batch, int hq, int hkv, int mseq, int max_pos) {
    constexpr int kTargetWG = 512;
    // keys per round of a workgroup: 32-key chunks per wave on the bfloat16
    // path (bf16 cache, head_dim a multiple of 32), 16-key blocks otherwise
    const int span = (dtype != 0 && hd % 32 == 0) ? 2 * kSpan : kSpan;
    if ((long)batch * mseq > 64) return 1;
    const int G = hq / hkv;
    const int QB = 16 * qv_blocks(G, mseq) / G;
    const int nqb = (mseq + QB - 1) / QB;
    const long base = (long)nqb * n_group * hkv * batch;
    const int rounds = (max_pos + 1 + span - 1) / span;
    long sp = (kTargetWG + base - 1) / base;
    if (sp > rounds) sp = rounds;
    if (sp > kSplitMax) sp = kSplitMax;
    return sp < 1 ? 1 : (int)sp;
}

int attention_max_group() { return kMaxQV; }


hipError_t launch_attention(int dtype, const AttnParams &p, hipStream_t s) {
    return dtype ? launch_t<uint16_t>(p, s) : launch_t<float>(p, s);
}

}  // namespace spec
