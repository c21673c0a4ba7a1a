// Skinny bf16 GEMM on the matrix cores for 2..16 activation rows (the k+1
// verification rows, the calibration rows, several sequences' draft rows),
// with the same fused epilogues as the VALU GEMV.
//
// Y[m][n] = sum_k X[m][k] W[n][k] with v_mfma_f32_16x16x32_bf16: the
// activations are the A operand, a 16-row block of W the B operand.  The
// float32 activation rows arrive as bf16 pieces packed into the operand's
// rows by their producer (the normalisation pass, the attention output, the
// SiLU epilogue): with M <= 8 rows, row m holds hi(x_m) and row m + 8 holds
// lo(x_m) in one 16-row tile; with M <= 16, tile 0 holds the hi rows and
// tile 1 the lo rows.  hi + lo is within 2^-16 of x, each piece times a bf16
// weight is exact in float32, so the two halves of the result add up to the
// float32 product at that precision; up to 8 rows this costs no matrix
// instruction more than bf16 activations would.  At these row counts the product is bound by HBM
// bandwidth (a few flops per weight byte), so the kernel is organised around
// the weight stream:
//
//  * A workgroup owns one unit: a 16-row block of W, or for paired epilogues
//    (RoPE partners, gate/up) the two blocks r0 and r0 + pair_block/2.  KS
//    waves per block split K into contiguous ranges of 256-element tiles.
//  * Weights are read with whole-row coalescing: each 16-byte-per-lane load
//    instruction covers two rows x 512 contiguous bytes.  The MFMA operand
//    layout needs 16 rows x 64 bytes per instruction instead, which halves the
//    bytes per memory request, so each wave stages its tile through a private
//    LDS buffer (padded rows keep the operand reads conflict-free) and loads
//    the next tile while the matrix cores consume the current one.
//  * The partial tiles are summed in wave order through LDS by the first
//    wave, which then holds both blocks of a pair in the same lane layout
//    and runs the epilogue straight from registers.
#include "epilogue.h"
#include "spec_device.h"
#include "spec_kernels.h"

namespace spec {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTK = 256;          // K elements per staged tile
constexpr int kLD = kTK + 8;      // LDS row stride in elements (16 bytes of padding)
constexpr int kMaxKS = 8;         // waves per 16-row block
constexpr int kLogitGrid = 2048;  // workgroups of a sampling product (= arg-max partials per row)

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &v) {
    bf16x8 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

// sum over the 16 lanes of a lane group (fixed xor tree)
__device__ __forceinline__ float group16_sum(float v) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ void group16_argmax(float &v, int &i) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
        const float v2 = __shfl_xor(v, o, kWave);
        const int i2 = __shfl_xor(i, o, kWave);
        argmax_merge(v, i, v2, i2);
    }
}

// MT: 16-row operand tiles (1: M <= 8, 2: M <= 16).  A unit has NB
// 16-row blocks (2 for the paired epilogues, else 1); the workgroup runs KS
// waves per block, wave w streaming block w / KS over K part w % KS.
template <int MT, int EPI, int KS, bool SEG = false>
__global__ __launch_bounds__(64 * KS * (epi_is_pair(EPI) ? 2 : 1)) void k_gemm_mfma(GemvParams p, int ups) {
    constexpr bool kPair = epi_is_pair(EPI);
    constexpr int NB = kPair ? 2 : 1;       // 16-row blocks per unit
    constexpr int NW = NB * KS;             // waves per workgroup
    constexpr int NL = 8;                   // 16-byte loads per lane per tile
    constexpr int TILE = 16 * kLD;          // elements of one wave's LDS tile
    __shared__ __align__(16) uint16_t smem[NW * TILE];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int blk = wave / KS, part = wave - blk * KS;
    const int li = lane & 15, lg = lane >> 4;
    uint16_t *tile = smem + (size_t)wave * TILE;
    const int K = p.K;
    const int ntile = (K + kTK - 1) / kTK;
    const int per = (ntile + KS - 1) / KS;
    const int t0 = part * per, t1 = min(ntile, t0 + per);
    const int half = p.pair_block >> 1;
    const int bph = half >> 4;              // 16-row blocks per half (paired)
    const int lrow = lane >> 5, lcol = 8 * (lane & 31);   // load lane -> (row of a pair, element)

    float best_v[MT][4];
    int best_i[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) { best_v[t][r] = -INFINITY; best_i[t][r] = 0x7FFFFFFF; }

    // first weight rows of unit u's two blocks
    auto unit_blocks = [&](int u, int &r0b, int &r1b) {
        if (kPair) {
            const int bb = u / bph, jb = u - bb * bph;
            r0b = bb * p.pair_block + jb * 16;
            r1b = r0b + half;
        } else {
            r0b = u * 16;
            r1b = r0b;
        }
    };
    // The weight tile in flight lives outside the unit loop, and a workgroup
    // that takes several units (sampling products) requests its next unit's
    // first tile before the current unit's reduction.  In this form the
    // paired products compile to about 124 VGPRs, so two 8-wave workgroups
    // share a CU (measured: 8B gate/up at 6 rows 47.1 -> 43.2 us against the
    // loop-local form at 136 VGPRs, one workgroup per CU).
    uint4 wv[NL];
    bool have_first = false;   // wv already holds this unit's first tile
    // K in segments (set members' matrices side by side; Ks a multiple of the
    // tile): where tile tt starts within a row of a segmented layout
    // (SEG instances: the down projection over a set's members)
    constexpr bool kSegOk = SEG;
    const int Ks = (kSegOk && p.kseg > 1) ? K / p.kseg : K;
    auto tile_off = [&](int tt, int64_t seg_stride) -> int64_t {
        if constexpr (!kSegOk) {
            return tt * kTK;
        } else {
            if (p.kseg <= 1) return tt * kTK;
            const int k = tt * kTK, sg = k / Ks;
            return sg * seg_stride + (k - sg * Ks);
        }
    };
    for (int u = blockIdx.x; u < p.n_units; u += gridDim.x) {
        int r0b, r1b;
        unit_blocks(u, r0b, r1b);
        const int sel = r0b / p.rows_per_sel;
        const int rb = blk ? r1b : r0b;         // this wave's block
        const uint16_t *W = reinterpret_cast<const uint16_t *>(p.W) + (int64_t)rb * Ks;
        const uint16_t *xb = reinterpret_cast<const uint16_t *>(p.X) + (int64_t)sel * p.x_sel_stride;
        bool xok[MT];
        const uint16_t *xr[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            // operand row t * 16 + li carries a piece of call row (t * 16 + li) % (8 * MT)
            xok[t] = (t * 16 + li) % (8 * MT) < p.M;
            xr[t] = xb + (int64_t)(t * 16 + li) * Ks + 8 * lg;
        }
        f32x4 acc[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

        auto load_from = [&](const uint16_t *Wr, int tt) {
            const bool in = tt * kTK + lcol < K;
            const uint16_t *wt0 = Wr + tile_off(tt, p.w_seg_stride) + lcol;
#pragma unroll
            for (int i = 0; i < NL; ++i)
                wv[i] = in ? ld16_stream(wt0 + (int64_t)(2 * i + lrow) * Ks) : make_uint4(0, 0, 0, 0);
        };
        auto load = [&](int tt) { load_from(W, tt); };
        if (t0 < t1 && !have_first) load(t0);
        have_first = false;
        for (int tt = t0; tt < t1; ++tt) {
#pragma unroll
            for (int i = 0; i < NL; ++i) *reinterpret_cast<uint4 *>(&tile[(2 * i + lrow) * kLD + lcol]) = wv[i];
            // the tile's activation operands are requested before the next
            // tile's weights, so the matrix cores wait only for them
            const int nsteps = min(kTK, K - tt * kTK) >> 5;     // 32-element MFMA steps in this tile
            uint4 xv[kTK / 32][MT];
            const int64_t xo = tile_off(tt, p.x_seg_stride);
#pragma unroll
            for (int s2 = 0; s2 < kTK / 32; ++s2)
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    xv[s2][t] = (xok[t] && s2 < nsteps) ? ld16(xr[t] + xo + 32 * s2) : make_uint4(0, 0, 0, 0);
            if (tt + 1 < t1) load(tt + 1);
#pragma unroll
            for (int s2 = 0; s2 < kTK / 32; ++s2) {
                if (s2 < nsteps) {
                    const uint4 wt = *reinterpret_cast<const uint4 *>(&tile[li * kLD + 32 * s2 + 8 * lg]);
#pragma unroll
                    for (int t = 0; t < MT; ++t)
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xv[s2][t]), as_bf16x8(wt), acc[t],
                                                                          0, 0, 0);
                }
            }
        }
        if (u + (int)gridDim.x < p.n_units && t0 < t1) {
            int n0, n1;
            unit_blocks(u + gridDim.x, n0, n1);
            load_from(reinterpret_cast<const uint16_t *>(p.W) + (int64_t)(blk ? n1 : n0) * Ks, t0);
            have_first = true;
        }
        // fixed-order sum of the K parts of each block by wave 0; C layout:
        // lane l, register r holds C[4 * (l / 16) + r][l % 16] = (activation
        // row, weight row of the block)
        f32x4 res[NB][MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) res[0][t] = acc[t];
        if (NW > 1) {
            __syncthreads();   // every wave is done with its tile
            f32x4 *red = reinterpret_cast<f32x4 *>(tile);
#pragma unroll
            for (int t = 0; t < MT; ++t) red[t * 64 + lane] = acc[t];
            __syncthreads();
            if (wave == 0) {
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    for (int q = (j == 0 ? 1 : 0); q < KS; ++q) {
                        const f32x4 *o = reinterpret_cast<const f32x4 *>(smem + (size_t)(j * KS + q) * TILE);
#pragma unroll
                        for (int t = 0; t < MT; ++t) {
                            if (j == 0) res[0][t] += o[t * 64 + lane];
                            else if (q == 0) res[j][t] = o[t * 64 + lane];
                            else res[j][t] += o[t * 64 + lane];
                        }
                    }
                }
            }
            __syncthreads();
        }
        if (wave != 0) continue;
        // hi and lo halves of each output: rows m and m + 8 of one tile sit in
        // lane groups g and g + 2 (lanes l and l ^ 32); with two tiles they
        // sit in the same lane and register of tiles 0 and 1
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            if constexpr (MT == 1) {
#pragma unroll
                for (int r = 0; r < 4; ++r) res[j][0][r] += __shfl_xor(res[j][0][r], 32, kWave);
            } else {
                res[j][0] += res[j][1];
            }
        }
#pragma unroll
        for (int t = 0; t < 1; ++t) {
            float ssv[4] = {0.f, 0.f, 0.f, 0.f};
            // one activation row at a time (keeps the epilogue's registers
            // out of the streaming loop's budget)
#pragma unroll 1
            for (int r = 0; r < 4; ++r) {
                const int m = t * 16 + 4 * lg + r;
                if (m >= p.M) continue;
                if constexpr (kPair) {
                    epi_pair<uint16_t, EPI>(p, r0b + li, r0b + li, r1b + li, sel, m, res[0][t][r], res[NB - 1][t][r]);
                } else {
                    epi_row<uint16_t, EPI>(p, r0b + li, sel, m, res[0][t][r], ssv[r], best_v[t][r], best_i[t][r]);
                }
            }
            if constexpr (epi_has_ss(EPI)) {
                // one unit per workgroup: partial index = unit within its set member
                if (p.n_norm_sel > 0 && (EPI == EPI_RESID_ADD || p.par_mlp || sel == 0)) {
                    const int si = (EPI == EPI_ATTN_OUT && p.par_mlp) ? sel : 0;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float s = group16_sum(ssv[r]);
                        const int m = t * 16 + 4 * lg + r;
                        if (li == 0 && m < p.M)
                            p.ss[(int64_t)si * p.ss_sel_stride + (int64_t)(p.m0 + m) * ups + (u - sel * ups)] = s;
                    }
                }
            }
        }
    }
    if constexpr (EPI == EPI_LOGITS) {
        if (wave != 0) return;
#pragma unroll
        for (int t = 0; t < 1; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = best_v[t][r];
                int i = best_i[t][r];
                group16_argmax(v, i);
                const int m = t * 16 + 4 * lg + r;
                if (li == 0 && m < p.M) {
                    p.part_val[(int64_t)(p.m0 + m) * gridDim.x + blockIdx.x] = v;
                    p.part_idx[(int64_t)(p.m0 + m) * gridDim.x + blockIdx.x] = i;
                }
            }
    }
}

template <int MT, int EPI>
void launch_epi(const GemvParams &p, dim3 g, int ks, int ups, hipStream_t s) {
    if constexpr (epi_is_pair(EPI)) {
        hipLaunchKernelGGL((k_gemm_mfma<MT, EPI, 4>), g, dim3(512), 0, s, p, ups);
    } else {
        if constexpr (EPI == EPI_RESID_ADD) {
            if (p.kseg > 1) {
                if (ks == 4) hipLaunchKernelGGL((k_gemm_mfma<MT, EPI, 4, true>), g, dim3(256), 0, s, p, ups);
                else hipLaunchKernelGGL((k_gemm_mfma<MT, EPI, 8, true>), g, dim3(512), 0, s, p, ups);
                return;
            }
        }
        if (ks == 4) hipLaunchKernelGGL((k_gemm_mfma<MT, EPI, 4>), g, dim3(256), 0, s, p, ups);
        else hipLaunchKernelGGL((k_gemm_mfma<MT, EPI, 8>), g, dim3(512), 0, s, p, ups);
    }
}

template <int MT>
hipError_t launch_mt(const GemvParams &p, dim3 g, int ks, int ups, hipStream_t s) {
    switch (p.epi) {
    case EPI_STORE: launch_epi<MT, EPI_STORE>(p, g, ks, ups, s); break;
    case EPI_QKV_ROPE: launch_epi<MT, EPI_QKV_ROPE>(p, g, ks, ups, s); break;
    case EPI_SILU_MUL: launch_epi<MT, EPI_SILU_MUL>(p, g, ks, ups, s); break;
    case EPI_RESID_ADD: launch_epi<MT, EPI_RESID_ADD>(p, g, ks, ups, s); break;
    case EPI_LOGITS: launch_epi<MT, EPI_LOGITS>(p, g, ks, ups, s); break;
    case EPI_ATTN_OUT: launch_epi<MT, EPI_ATTN_OUT>(p, g, ks, ups, s); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

int gemm_mfma_max_rows() { return 16; }

// One unit per workgroup, except sampling products, which keep a fixed grid
// (their arg-max partials are per workgroup).
// One unit per workgroup (measured against one or two persistent workgroups
// per CU that take several units each with the next unit's first tile
// requested early: 8B gate/up at 6 rows 43.2 vs 45.0-45.4 us), except
// sampling products, which keep a fixed grid (their arg-max partials are per
// workgroup).
int gemm_mfma_grid(const GemvParams &p) {
    const int n = p.n_units < 1 ? 1 : p.n_units;
    return p.epi == EPI_LOGITS && n > kLogitGrid ? kLogitGrid : n;
}

// Waves per block (4 or 8): 8 when the launch would otherwise have fewer than
// about 3K waves and every wave keeps at least one tile.  Paired units keep 4
// (8, in 1024-thread workgroups, measured slower: 8B QKV 16.2 -> 18.6 us,
// gate/up 43.2 -> 51.5 us at 6 rows).
int gemm_mfma_splits(const GemvParams &p) {
    if (epi_is_pair(p.epi)) return 4;
    const int ntile = (p.K + kTK - 1) / kTK;
    int ks = 4;
    while (ks < kMaxKS && (int64_t)p.n_units * ks < 3072 && ks * 2 <= ntile) ks *= 2;
    return ks;
}

bool gemm_mfma_supported(const GemvParams &p) {
    if (p.K % 32 != 0 || p.M < 1 || p.M > 16 || p.rows_per_sel % 16 != 0) return false;
    if (p.kseg > 1 && (p.K % p.kseg != 0 || (p.K / p.kseg) % kTK != 0)) return false;
    if (epi_is_pair(p.epi)) return p.pair_block % 32 == 0;
    return true;
}

int gemm_mfma_packed_rows(int M) { return M <= 8 ? 16 : 32; }

hipError_t launch_gemm_mfma(const GemvParams &p, int grid, int ks, hipStream_t s) {
    if ((ks != 4 && ks != 8) || (epi_is_pair(p.epi) && ks != 4)) return hipErrorInvalidValue;
    // partial index of a residual writer: the unit within its set member
    const int ups = p.rows_per_sel / 16;
    if (epi_has_ss(p.epi) && p.n_norm_sel > 0 && grid != p.n_units) return hipErrorInvalidValue;
    // every row of the call in one launch, operand packed as gemm_mfma_packed_rows says
    if (p.m0 != 0 || p.M > 16) return hipErrorInvalidValue;
    if (p.M <= 8) return launch_mt<1>(p, dim3(grid), ks, ups, s);
    return launch_mt<2>(p, dim3(grid), ks, ups, s);
}

}  // namespace spec
