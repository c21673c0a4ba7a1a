// Skinny bf16 GEMM on the matrix cores for 2..32 activation rows (the k+1
// verification rows, the calibration rows), with the same fused epilogues as
// the VALU GEMV.
//
// Y[m][n] = sum_k X[m][k] W[n][k] with v_mfma_f32_16x16x32_bf16: the
// activations are the A operand (16 rows, zero padded), a 16-row block of W
// is the B operand, so every lane loads 16 contiguous bytes of a weight row
// per MFMA and each weight byte is read from HBM exactly once.  At these row
// counts the product is bandwidth bound (a few flops per weight byte); the
// matrix cores remove the VALU bottleneck that a per-row FMA loop hits once
// there are more than a handful of activation rows.
//
// A workgroup owns a unit = a pair of 16-row blocks (r0 .. r0+15 and the
// partner block r1 = r0 + pair_block/2, so RoPE pairs and (gate, up) pairs
// meet in one workgroup) and splits K over KS wave pairs; the KS partial
// tiles are summed in a fixed order through LDS.
#include "epilogue.h"
#include "spec_device.h"
#include "spec_kernels.h"

namespace spec {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxKS = 4;        // K splits (wave pairs) per workgroup
constexpr int kMaxGridM = 256 * 8;

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &v) {
    bf16x8 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

__device__ __forceinline__ uint4 pack_bf16x8(const float *f) {
    uint4 r;
    r.x = (uint32_t)f32_to_bf16(f[0]) | ((uint32_t)f32_to_bf16(f[1]) << 16);
    r.y = (uint32_t)f32_to_bf16(f[2]) | ((uint32_t)f32_to_bf16(f[3]) << 16);
    r.z = (uint32_t)f32_to_bf16(f[4]) | ((uint32_t)f32_to_bf16(f[5]) << 16);
    r.w = (uint32_t)f32_to_bf16(f[6]) | ((uint32_t)f32_to_bf16(f[7]) << 16);
    return r;
}

// A-operand pieces (16 consecutive k of one activation row) for one 64-wide
// chunk: plain bf16 rows, or RMSNorm-ed residual rows rounded to bf16.
__device__ __forceinline__ void x_tile(const GemvParams &p, const uint16_t *xrow, int sel, int hrow, float inv,
                                       int k, uint4 &x0, uint4 &x1) {
    if (p.xmode == X_PLAIN) {
        x0 = ld16(xrow + k);
        x1 = ld16(xrow + k + 8);
    } else {
        float f[8];
        x_norm8(p, sel, hrow, k, inv, f);
        x0 = pack_bf16x8(f);
        x_norm8(p, sel, hrow, k + 8, inv, f);
        x1 = pack_bf16x8(f);
    }
}

// MT: number of 16-row activation tiles (1: M <= 16, 2: M <= 32)
// kSingle: a unit is one 16-row block (rows r0 .. r0+15, epilogue pairs
// (r0 + j, r0 + 8 + j)) and all 2 KS waves split K; otherwise a unit is a
// pair of 16-row blocks and KS wave pairs split K.
template <int MT, bool kLogits, bool kSingle>
__global__ __launch_bounds__(512) void k_gemm_mfma(GemvParams p, int KS) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;     // 0 .. 2*KS-1
    const int blk = kSingle ? 0 : (wave & 1);      // which block of the pair
    const int part = kSingle ? wave : (wave >> 1); // K split index
    const int nparts_k = kSingle ? 2 * KS : KS;
    const int K = p.K;
    const int nchunk = K >> 6;             // 64-element chunks
    const int per = (nchunk + nparts_k - 1) / nparts_k;
    const int c0 = part * per;
    const int c1 = min(nchunk, c0 + per);
    const int half = p.pair_block >> 1;
    const int bph = half >> 4;             // 16-row blocks per half
    const int li = lane & 15;              // row within the block / activation row
    const int lg = lane >> 4;              // lane group: k offset 16 * lg within a chunk

    __shared__ f32x4 red[2 * kMaxKS][MT][64];
    __shared__ float tile[2][MT * 16][17];
    float best_v = -INFINITY;
    int best_i = 0x7FFFFFFF;
    float ss[kMaxSel];
#pragma unroll
    for (int s = 0; s < kMaxSel; ++s) ss[s] = 0.f;
    __shared__ float inv_s[MT * 16];
    block_inv_rms(p, inv_s);

    for (int u = blockIdx.x; u < p.n_units; u += gridDim.x) {
        int r0, r1;
        if (kSingle) {
            r0 = u * 16;
            r1 = r0 + 8;
        } else {
            const int bb = u / bph;
            const int jb = u - bb * bph;
            r0 = bb * p.pair_block + jb * 16;
            r1 = r0 + half;
        }
        const int rb = blk ? r1 : r0;
        const int sel = r0 / p.rows_per_sel;
        const uint16_t *w = reinterpret_cast<const uint16_t *>(p.W) + (int64_t)(rb + li) * K + 16 * lg;
        const uint16_t *x = reinterpret_cast<const uint16_t *>(p.X) + (int64_t)sel * p.x_sel_stride +
                            (int64_t)p.m0 * K + 16 * lg;
        f32x4 acc[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        bool xok[MT];
        int hrow[MT];
        float inv[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            xok[t] = (t * 16 + li) < p.M;
            hrow[t] = 0;
            inv[t] = 0.f;
            if (xok[t] && p.xmode == X_NORM) {
                hrow[t] = x_row(p, p.m0 + t * 16 + li);
                inv[t] = inv_s[t * 16 + li];
            }
        }
        const int kl = 16 * lg;   // this lane group's offset inside a chunk

        int c = c0;
        for (; c + 3 < c1; c += 4) {
            uint4 wv[4][2];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                wv[q][0] = ld16_stream(w + (c + q) * 64);
                wv[q][1] = ld16_stream(w + (c + q) * 64 + 8);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    uint4 x0 = make_uint4(0, 0, 0, 0), x1 = make_uint4(0, 0, 0, 0);
                    if (xok[t])
                        x_tile(p, x - kl + (int64_t)(t * 16 + li) * K, sel, hrow[t], inv[t], (c + q) * 64 + kl, x0, x1);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(x0), as_bf16x8(wv[q][0]), acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(x1), as_bf16x8(wv[q][1]), acc[t], 0, 0, 0);
                }
            }
        }
        for (; c < c1; ++c) {
            const uint4 w0 = ld16_stream(w + c * 64), w1 = ld16_stream(w + c * 64 + 8);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                uint4 x0 = make_uint4(0, 0, 0, 0), x1 = make_uint4(0, 0, 0, 0);
                if (xok[t])
                    x_tile(p, x - kl + (int64_t)(t * 16 + li) * K, sel, hrow[t], inv[t], c * 64 + kl, x0, x1);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(x0), as_bf16x8(w0), acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(x1), as_bf16x8(w1), acc[t], 0, 0, 0);
            }
        }
        // fixed-order sum of the K splits; C layout: lane l, register r holds
        // C[4 * (l / 16) + r][l % 16]
#pragma unroll
        for (int t = 0; t < MT; ++t) red[wave][t][lane] = acc[t];
        __syncthreads();
        if (part == 0) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                f32x4 s = red[blk][t][lane];
                for (int q = 1; q < nparts_k; ++q) {
                    const f32x4 o = red[kSingle ? q : 2 * q + blk][t][lane];
                    s[0] += o[0]; s[1] += o[1]; s[2] += o[2]; s[3] += o[3];
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) tile[blk][t * 16 + 4 * lg + r][li] = s[r];
            }
        }
        __syncthreads();
        constexpr int EPR = kSingle ? 8 : 16;   // epilogue elements per activation row
        for (int e = threadIdx.x; e < p.M * EPR; e += blockDim.x) {
            const int m = e / EPR, j = e % EPR;
            const float y0 = tile[0][m][j];
            const float y1 = kSingle ? tile[0][m][j + 8] : tile[1][m][j];
            epilogue<uint16_t, kLogits>(p, r0 + j, r0 + j, r1 + j, sel, m, y0, y1, best_v, best_i, ss);
        }
        __syncthreads();
    }

    // block partials: thread e < EPR M always handled activation row e / EPR
    // (the launch guarantees blockDim >= 16 M)
    constexpr int EPR = kSingle ? 8 : 16;
    const bool norm = p.n_norm_sel > 0;
    const bool logits = p.epi == EPI_LOGITS;
    if (!norm && !logits) return;
    __shared__ float sbv[MT * 16][16];
    __shared__ int sbi[MT * 16][16];
    __shared__ float sss[kMaxSel][MT * 16][16];
    const int e = threadIdx.x;
    if (e < p.M * EPR) {
        sbv[e / EPR][e % EPR] = best_v;
        sbi[e / EPR][e % EPR] = best_i;
#pragma unroll
        for (int s = 0; s < kMaxSel; ++s) sss[s][e / EPR][e % EPR] = ss[s];
    }
    __syncthreads();
    if (e < p.M) {
        if (logits) {
            float v = sbv[e][0];
            int i = sbi[e][0];
            for (int j = 1; j < EPR; ++j) argmax_merge(v, i, sbv[e][j], sbi[e][j]);
            p.part_val[(int64_t)(p.m0 + e) * gridDim.x + blockIdx.x] = v;
            p.part_idx[(int64_t)(p.m0 + e) * gridDim.x + blockIdx.x] = i;
        }
        for (int s = 0; s < p.n_norm_sel; ++s) {
            float t = sss[s][e][0];
            for (int j = 1; j < EPR; ++j) t += sss[s][e][j];
            p.ss[(int64_t)s * p.ss_sel_stride + (int64_t)(p.m0 + e) * gridDim.x + blockIdx.x] = t;
        }
    }
}

}  // namespace

int gemm_mfma_max_rows() { return 32; }

int gemm_mfma_grid(int n_units) { return n_units < kMaxGridM ? (n_units < 1 ? 1 : n_units) : kMaxGridM; }

// K splits so that a launch has about 8K waves in flight, at least two
// 64-element chunks per wave.
int gemm_mfma_splits(int n_units, int K, bool single) {
    const int per_ks = single ? 2 : 1;     // K parts per unit and KS step
    int ks = 1;
    while (ks < kMaxKS && (int64_t)n_units * 2 * ks < 8192 && (K >> 6) >= 4 * ks * per_ks) ks *= 2;
    return ks;
}

bool gemm_mfma_supported(const GemvParams &p) {
    return (p.K % 64) == 0 && (p.pair_block == 2 || (p.pair_block % 32) == 0) && p.M >= 1 && p.M <= 32;
}

template <int MT, bool kSingle>
void launch_mt(const GemvParams &p, dim3 g, dim3 b, int ks, hipStream_t s) {
    if (p.epi == EPI_LOGITS) hipLaunchKernelGGL((k_gemm_mfma<MT, true, kSingle>), g, b, 0, s, p, ks);
    else hipLaunchKernelGGL((k_gemm_mfma<MT, false, kSingle>), g, b, 0, s, p, ks);
}

// single: units are single 16-row blocks (adjacent-row products)
hipError_t launch_gemm_mfma(const GemvParams &p, int grid, int ks, bool single, hipStream_t s) {
    while (128 * ks < 16 * p.M) ks *= 2;   // one epilogue element per thread
    dim3 g(grid), b(128 * ks);
    if (p.M <= 16) {
        if (single) launch_mt<1, true>(p, g, b, ks, s);
        else launch_mt<1, false>(p, g, b, ks, s);
    } else {
        if (single) launch_mt<2, true>(p, g, b, ks, s);
        else launch_mt<2, false>(p, g, b, ks, s);
    }
    return hipGetLastError();
}

}  // namespace spec
