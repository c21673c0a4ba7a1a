// Tiled bf16 GEMM on the matrix cores for prompt-length activation counts
// (the base's and the draft's prompt prefills: M = rows of the prompt), with
// the decoder's fused epilogues.  Y[m][n] = sum_k X[m][k] W[n][k].
//
// At M >= 64 the products are compute-bound (the weights are reused by every
// activation row), so the kernel is organised around the matrix cores:
//  * a workgroup (4 waves, 2 x 2) owns a 128-row activation tile and a
//    2 x NH-row weight tile; the weight tile is two halves, rows n0 .. n0+NH
//    and n0+off .. n0+off+NH, so the paired epilogues (RoPE partners at half
//    a head apart, gate / up rows d_ffn apart) find both rows of a pair in
//    the same lane's accumulators; unpaired products use off = NH;
//  * K advances in 64-element steps: the next step's tiles are loaded into
//    registers (16 bytes per lane, 128 contiguous bytes per row) while the
//    matrix cores consume the current step from LDS (rows padded by 16 bytes);
//  * each wave computes 64 activation rows x NH weight rows (NH / 2 of each
//    half) with v_mfma_f32_16x16x32_bf16;
//  * workgroups that share a weight tile are launched next to each other
//    (activation tiles on blockIdx.x), so the weights come from the caches
//    after the first read.
#include "epilogue.h"
#include "spec_device.h"
#include "spec_kernels.h"

namespace spec {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128;          // activation rows per workgroup
constexpr int kBK = 64;           // K elements per step
constexpr int kLDK = kBK + 8;     // LDS row stride in elements (16 bytes of padding)

__device__ __forceinline__ bf16x8 as_bf8(const uint4 &v) {
    bf16x8 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

__device__ __forceinline__ float sum16(float v) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// grid: (activation tiles, weight tiles).  off: row distance of the second
// weight half; parts: sum-of-squares partials per row and set member (two
// per weight tile, one per wave column).
template <int EPI, int NH>
__global__ __launch_bounds__(256) void k_gemm_tile(GemvParams p, int off, int tiles_per_pair, int parts) {
    constexpr bool kPair = epi_is_pair(EPI);
    constexpr int BN = 2 * NH;
    constexpr int CB = NH / 32;                 // 16-row column blocks per half per wave
    constexpr int NLB = BN * kBK / 8 / 256;     // 16-byte weight loads per thread per step
    __shared__ __align__(16) uint16_t As[kBM * kLDK];
    __shared__ __align__(16) uint16_t Bs[BN * kLDK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int li = lane & 15, lg = lane >> 4;
    const int K = p.K;
    const int m0 = blockIdx.x * kBM;
    int n0, u0 = 0;   // first weight row; first pair unit (paired epilogues)
    if (kPair) {
        const int bb = blockIdx.y / tiles_per_pair, t = blockIdx.y - bb * tiles_per_pair;
        n0 = bb * p.pair_block + t * NH;
        u0 = bb * (p.pair_block / 2) + t * NH;
    } else {
        n0 = blockIdx.y * BN;
    }
    const int sel = n0 / p.rows_per_sel;
    const uint16_t *W = reinterpret_cast<const uint16_t *>(p.W);
    const uint16_t *X = reinterpret_cast<const uint16_t *>(p.X) + (int64_t)sel * p.x_sel_stride;

    // loader: thread t moves 16 bytes of rows t / 8 + 32 i, elements 8 (t % 8)
    const int lr = tid >> 3, lc = 8 * (tid & 7);
    uint4 ra[4], rb[NLB];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + lr + 32 * i;
            ra[i] = m < p.M ? ld16(X + (int64_t)(p.m0 + m) * K + k0 + lc) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NLB; ++i) {
            const int r = lr + 32 * i;
            const int n = r < NH ? n0 + r : n0 + off + (r - NH);
            rb[i] = ld16(W + (int64_t)n * K + k0 + lc);
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4 *>(&As[(lr + 32 * i) * kLDK + lc]) = ra[i];
#pragma unroll
        for (int i = 0; i < NLB; ++i) *reinterpret_cast<uint4 *>(&Bs[(lr + 32 * i) * kLDK + lc]) = rb[i];
    };

    f32x4 acc[4][2][CB];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int c = 0; c < CB; ++c) acc[a][h][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    load(0);
    for (int k0 = 0; k0 < K; k0 += kBK) {
        __syncthreads();          // previous step consumed
        stash();
        __syncthreads();
        if (k0 + kBK < K) load(k0 + kBK);
#pragma unroll
        for (int s = 0; s < kBK / 32; ++s) {
            uint4 av[4], bv[2][CB];
#pragma unroll
            for (int a = 0; a < 4; ++a)
                av[a] = *reinterpret_cast<const uint4 *>(&As[(64 * wm + 16 * a + li) * kLDK + 32 * s + 8 * lg]);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int c = 0; c < CB; ++c)
                    bv[h][c] = *reinterpret_cast<const uint4 *>(
                        &Bs[(h * NH + (NH / 2) * wn + 16 * c + li) * kLDK + 32 * s + 8 * lg]);
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int c = 0; c < CB; ++c)
                        acc[a][h][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(av[a]), as_bf8(bv[h][c]),
                                                                                acc[a][h][c], 0, 0, 0);
        }
    }

    // epilogue: lane (li, lg), register r of tile (a, h, c) holds activation
    // row 64 wm + 16 a + 4 lg + r and weight row (half h) (NH / 2) wn + 16 c + li
    float best_v = -INFINITY;
    int best_i = 0;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        float ssv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + 64 * wm + 16 * a + 4 * lg + r;
            if (m >= p.M) continue;
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                const int j = (NH / 2) * wn + 16 * c + li;
                const int r0 = n0 + j;
                if constexpr (kPair) {
                    epi_pair<uint16_t, EPI>(p, u0 + j, r0, r0 + off, sel, m, acc[a][0][c][r], acc[a][1][c][r]);
                } else {
                    epi_row<uint16_t, EPI>(p, r0, sel, m, acc[a][0][c][r], ssv[r], best_v, best_i);
                    epi_row<uint16_t, EPI>(p, r0 + off, sel, m, acc[a][1][c][r], ssv[r], best_v, best_i);
                }
            }
        }
        if constexpr (epi_has_ss(EPI)) {
            if (p.n_norm_sel > 0 && (EPI == EPI_RESID_ADD || p.par_mlp || sel == 0)) {
                const int si = (EPI == EPI_ATTN_OUT && p.par_mlp) ? sel : 0;
                const int part = ((n0 - sel * p.rows_per_sel) / BN) * 2 + wn;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float s = sum16(ssv[r]);
                    const int m = m0 + 64 * wm + 16 * a + 4 * lg + r;
                    if (li == 0 && m < p.M)
                        p.ss[(int64_t)si * p.ss_sel_stride + (int64_t)(p.m0 + m) * parts + part] = s;
                }
            }
        }
    }
}

template <int EPI, int NH>
void launch_en(const GemvParams &p, dim3 g, int off, int tpp, int parts, hipStream_t s) {
    hipLaunchKernelGGL((k_gemm_tile<EPI, NH>), g, dim3(256), 0, s, p, off, tpp, parts);
}

template <int NH>
hipError_t launch_nh(const GemvParams &p, dim3 g, int off, int tpp, int parts, hipStream_t s) {
    switch (p.epi) {
    case EPI_STORE: launch_en<EPI_STORE, NH>(p, g, off, tpp, parts, s); break;
    case EPI_QKV_ROPE: launch_en<EPI_QKV_ROPE, NH>(p, g, off, tpp, parts, s); break;
    case EPI_SILU_MUL: launch_en<EPI_SILU_MUL, NH>(p, g, off, tpp, parts, s); break;
    case EPI_RESID_ADD: launch_en<EPI_RESID_ADD, NH>(p, g, off, tpp, parts, s); break;
    case EPI_ATTN_OUT: launch_en<EPI_ATTN_OUT, NH>(p, g, off, tpp, parts, s); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Weight-half width of a launch: 64, or 32 for RoPE pairs of 64-dim heads.
int tile_nh(const GemvParams &p) {
    if (epi_is_pair(p.epi)) {
        const int half = p.pair_block / 2;
        return half % 64 == 0 ? 64 : (half % 32 == 0 ? 32 : 0);
    }
    return 64;
}

}  // namespace

int gemm_tiled_min_rows() { return 64; }

bool gemm_tiled_supported(const GemvParams &p) {
    if (p.K % kBK != 0 || p.epi == EPI_LOGITS || p.M < 1) return false;
    const int nh = tile_nh(p);
    if (nh == 0) return false;
    if (epi_is_pair(p.epi)) return p.rows_per_sel % p.pair_block == 0;
    return p.rows_per_sel % (2 * nh) == 0;
}

// Sum-of-squares partials per row and set member a residual writer leaves.
int gemm_tiled_parts(const GemvParams &p) { return p.rows_per_sel / tile_nh(p); }

// p.n_units: row pairs (rows / 2) as for the other products; p.M rows from
// p.m0 (the kernel reads X rows m0 .. m0 + M - 1 and the epilogue writes them).
hipError_t launch_gemm_tiled(const GemvParams &p, hipStream_t s) {
    if (!gemm_tiled_supported(p)) return hipErrorInvalidValue;
    const int nh = tile_nh(p);
    const int rows = p.n_units * 2;
    int ntiles, off, tpp = 0;
    if (epi_is_pair(p.epi)) {
        const int half = p.pair_block / 2;
        tpp = half / nh;
        ntiles = (rows / p.pair_block) * tpp;
        off = half;
    } else {
        ntiles = rows / (2 * nh);
        off = nh;
    }
    dim3 g((p.M + kBM - 1) / kBM, ntiles);
    const int parts = p.rows_per_sel / nh;
    if (nh == 64) return launch_nh<64>(p, g, off, tpp, parts, s);
    return launch_nh<32>(p, g, off, tpp, parts, s);
}

}  // namespace spec
