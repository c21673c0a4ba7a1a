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
// sum-of-squares partials an x_inv product reads (M x xnparts): 2048 with one
// operand tile (its LDS beside two paired workgroups per CU), 4096 with two
constexpr int inv_max(int MT) { return MT == 1 ? 2048 : 4096; }

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &v) {
    bf16x8 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

// 1 / rms of rows m = first, first + step, ... < M from their n sum-of-squares
// partials ssl[m * n + 0 .. n - 1] into ssl[off + m]: lane-strided sums,
// then a fixed xor tree (every workgroup forms the same bits).  Out of line:
// inlined, its temporaries raise the register budget of the whole kernel.
__device__ __noinline__ void rows_inv_rms(float *ssl, int off, int M, int n, int K, float eps, int first, int step,
                                         int lane) {
    for (int m = first; m < M; m += step) {
        float sm = 0.f;
        for (int k = lane; k < n; k += 64) sm += ssl[m * n + k];
        sm = wave_sum(sm);
        if (lane == 0) ssl[off + m] = 1.0f / sqrtf(sm / (float)K + eps);
    }
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

// MT: 16-row operand tiles (1: M <= 8, 2: M <= 16).  A unit is NBU 16-row
// blocks of W: the two blocks of a pair for the paired epilogues, one block
// otherwise.  Each of the workgroup's KS waves streams every block of the
// unit over its own contiguous part of K, in tiles of 8 KB of weights (NBU
// blocks x kTK / NBU elements), so one activation fragment feeds NBU matrix
// instructions: the activation reads per weight byte fall by NBU, which
// matters once the operand carries two pieces per row.  One weight tile per
// wave is in flight while the previous one is consumed (two, at about 190
// VGPRs, measured slower: 8B down at 6 rows 29.0 -> 30.5 us, O 14.6 -> 15.5,
// lm head 175 -> 196).
template <int MT, int EPI, int KS, bool SEG = false>
__global__ __launch_bounds__(64 * KS) void k_gemm_mfma(GemvParams p, int ups) {
    constexpr bool kPair = epi_is_pair(EPI);
    constexpr int NBU = kPair ? 2 : 1;      // 16-row blocks per unit
    constexpr int TKL = kTK / NBU;          // K elements per tile
    // LDS row stride: 544 bytes for the 256-element tiles, where a wave's
    // fragment reads meet every bank once (at 528 bytes: twice); the paired
    // tiles keep 272 bytes (two-way conflicts), since 288 would put two
    // eight-wave workgroups and their partial-sum area past the CU's 160 KB
    constexpr int LDK = TKL + (kPair ? 8 : 16);
    constexpr int RPL = 512 / TKL;          // weight rows per 16-byte-per-lane load
    constexpr int NL = 8;                   // loads per lane per tile
    constexpr int BL = NL / NBU;            // of them per block
    constexpr int NS = TKL / 32;            // matrix steps per tile
    constexpr int TILE = 16 * NBU * LDK;    // elements of one wave's LDS tile
    static_assert(NBU * MT * 64 * 16 <= TILE * 2, "reduction area");
    __shared__ __align__(16) uint16_t smem[KS * TILE];
    // x_inv: the rows' sum-of-squares partials, requested before the weight
    // stream (NPL per lane over the workgroup) and summed by wave 0 after it
    constexpr int INV = inv_max(MT);
    constexpr int NPL = INV / (64 * KS);
    __shared__ float ssl[INV + 16];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    uint16_t *tile = smem + (size_t)wave * TILE;
    const int K = p.K;
    const int ntile = (K + TKL - 1) / TKL;
    const int per = (ntile + KS - 1) / KS;
    const int t0 = wave * per, t1 = min(ntile, t0 + per);
    const int half = p.pair_block >> 1;
    const int bph = half >> 4;              // 16-row blocks per half (paired)
    const int lrow = lane / (TKL / 8), lcol = 8 * (lane % (TKL / 8));   // load lane -> (row, element)

    float best_v[4];
    int best_i[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) { best_v[r] = -INFINITY; best_i[r] = 0x7FFFFFFF; }

    // first weight row of each block of unit u
    auto unit_blocks = [&](int u, int (&rb)[NBU]) {
        if constexpr (kPair) {
            const int bb = u / bph, jb = u - bb * bph;
            rb[0] = bb * p.pair_block + jb * 16;
            rb[1] = rb[0] + half;
        } else {
#pragma unroll
            for (int j = 0; j < NBU; ++j) rb[j] = (u * NBU + j) * 16;
        }
    };
    // The weight tile in flight lives outside the unit loop, and a workgroup
    // that takes several units (sampling products) requests its next unit's
    // first tile before the current unit's reduction.
    uint4 wv[NL];
    bool have_first = false;   // wv already holds this unit's first tile
    // K in segments (set members' matrices side by side; Ks a multiple of the
    // tile): where tile tt starts within a row of a segmented layout
    // (SEG instances: the down projection over a set's members)
    constexpr bool kSegOk = SEG;
    const int Ks = (kSegOk && p.kseg > 1) ? K / p.kseg : K;
    auto tile_off = [&](int tt, int64_t seg_stride) -> int64_t {
        if constexpr (!kSegOk) {
            return (int64_t)tt * TKL;
        } else {
            if (p.kseg <= 1) return (int64_t)tt * TKL;
            const int k = tt * TKL, sg = k / Ks;
            return sg * seg_stride + (k - sg * Ks);
        }
    };
    const uint16_t *W0 = reinterpret_cast<const uint16_t *>(p.W);
    auto load_from = [&](uint4 (&w)[NL], const int (&rb)[NBU], int tt) {
        const bool in = tt * TKL + lcol < K;
        const int64_t off = tile_off(tt, p.w_seg_stride) + lcol;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int j = i / BL, r = RPL * (i % BL) + lrow;
            w[i] = in ? ld16_stream(W0 + (int64_t)(rb[j] + r) * Ks + off) : make_uint4(0, 0, 0, 0);
        }
    };
    // (straight from global memory into LDS: no registers held across the
    // weight stream; slots past the rows' partials receive partial 0, unread)
    const int nss = p.x_inv ? p.M * p.xnparts : 0;
    if (nss > 0) {
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
            const int i = threadIdx.x + j * 64 * KS;
            __builtin_amdgcn_global_load_lds(p.xss + (i < nss ? i : 0), &ssl[wave * 64 + j * 64 * KS], 4, 0, 0);
        }
    }
    for (int u = blockIdx.x; u < p.n_units; u += gridDim.x) {
        int rb[NBU];
        unit_blocks(u, rb);
        const int sel = rb[0] / p.rows_per_sel;
        const uint16_t *xb = reinterpret_cast<const uint16_t *>(p.X) + (int64_t)sel * p.x_sel_stride;
        bool xok[MT];
        const uint16_t *xr[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            // operand row t * 16 + li carries a piece of call row (t * 16 + li) % (8 * MT)
            xok[t] = (t * 16 + li) % (8 * MT) < p.M;
            xr[t] = xb + (int64_t)(t * 16 + li) * Ks + 8 * lg;
        }
        f32x4 acc[NBU][MT];
#pragma unroll
        for (int j = 0; j < NBU; ++j)
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};

        if (t0 < t1 && !have_first) load_from(wv, rb, t0);
        have_first = false;
        {
            for (int tt = t0; tt < t1; ++tt) {
#pragma unroll
                for (int i = 0; i < NL; ++i) {
                    const int j = i / BL, r = RPL * (i % BL) + lrow;
                    *reinterpret_cast<uint4 *>(&tile[(16 * j + r) * LDK + lcol]) = wv[i];
                }
                // the tile's activation operands are requested before the
                // next weight tile, so the matrix cores wait only for them
                const int nsteps = min(TKL, K - tt * TKL) >> 5;     // 32-element steps in this tile
                uint4 xv[NS][MT];
                const int64_t xo = tile_off(tt, p.x_seg_stride);
#pragma unroll
                for (int s2 = 0; s2 < NS; ++s2)
#pragma unroll
                    for (int t = 0; t < MT; ++t)
                        xv[s2][t] = (xok[t] && s2 < nsteps) ? ld16(xr[t] + xo + 32 * s2) : make_uint4(0, 0, 0, 0);
                if (tt + 1 < t1) load_from(wv, rb, tt + 1);
#pragma unroll
                for (int s2 = 0; s2 < NS; ++s2) {
                    if (s2 < nsteps) {
#pragma unroll
                        for (int j = 0; j < NBU; ++j) {
                            const uint4 wt =
                                *reinterpret_cast<const uint4 *>(&tile[(16 * j + li) * LDK + 32 * s2 + 8 * lg]);
#pragma unroll
                            for (int t = 0; t < MT; ++t)
                                acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    as_bf16x8(xv[s2][t]), as_bf16x8(wt), acc[j][t], 0, 0, 0);
                        }
                    }
                }
            }
        }
        // (only sampling products take several units per workgroup)
        if constexpr (EPI == EPI_LOGITS) {
            if (u + (int)gridDim.x < p.n_units && t0 < t1) {
                int nb[NBU];
                unit_blocks(u + gridDim.x, nb);
                load_from(wv, nb, t0);
                have_first = true;
            }
        }
        // fixed-order sum of the K parts by wave 0; C layout: lane l,
        // register r holds C[4 * (l / 16) + r][l % 16] = (activation row,
        // weight row of the block)
        if (nss > 0) __builtin_amdgcn_s_waitcnt(0);   // this wave's copies into LDS have landed
        if (KS > 1) {
            __syncthreads();   // every wave is done with its tile
            f32x4 *red = reinterpret_cast<f32x4 *>(tile);
#pragma unroll
            for (int j = 0; j < NBU; ++j)
#pragma unroll
                for (int t = 0; t < MT; ++t) red[(j * MT + t) * 64 + lane] = acc[j][t];
            __syncthreads();
            if (wave == 0) {
                for (int q = 1; q < KS; ++q) {
                    const f32x4 *o = reinterpret_cast<const f32x4 *>(smem + (size_t)q * TILE);
#pragma unroll
                    for (int j = 0; j < NBU; ++j)
#pragma unroll
                        for (int t = 0; t < MT; ++t) acc[j][t] += o[(j * MT + t) * 64 + lane];
                }
            } else if (nss > 0) {
                // meanwhile the other waves form 1 / rms of the rows
                rows_inv_rms(ssl, INV, p.M, p.xnparts, p.K, p.eps, wave - 1, KS - 1, lane);
            }
            __syncthreads();
        }
        if (wave != 0) continue;
        // hi and lo halves of each output: rows m and m + 8 of one tile sit in
        // lane groups g and g + 2 (lanes l and l ^ 32); with two tiles they
        // sit in the same lane and register of tiles 0 and 1
        f32x4 res[NBU];
#pragma unroll
        for (int j = 0; j < NBU; ++j) {
            if constexpr (MT == 1) {
                res[j] = acc[j][0];
#pragma unroll
                for (int r = 0; r < 4; ++r) res[j][r] += __shfl_xor(res[j][r], 32, kWave);
            } else {
                res[j] = acc[j][0] + acc[j][MT - 1];
            }
        }
        float ssv[4] = {0.f, 0.f, 0.f, 0.f};
        // one activation row at a time (keeps the epilogue's registers out of
        // the streaming loop's budget)
#pragma unroll 1
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * lg + r;
            if (m >= p.M) continue;
            const float sc = nss > 0 ? ssl[INV + m] : 1.f;
            if constexpr (kPair) {
                epi_pair<uint16_t, EPI>(p, rb[0] + li, rb[0] + li, rb[1] + li, sel, m, res[0][r] * sc,
                                        res[1][r] * sc);
            } else {
#pragma unroll
                for (int j = 0; j < NBU; ++j)
                    epi_row<uint16_t, EPI>(p, rb[j] + li, sel, m, res[j][r] * sc, ssv[r], best_v[r], best_i[r]);
            }
        }
        if constexpr (epi_has_ss(EPI)) {
            // one unit per workgroup: partial index = unit within its set member
            if (p.n_norm_sel > 0 && (EPI == EPI_RESID_ADD || p.par_mlp || sel == 0)) {
                const int si = (EPI == EPI_ATTN_OUT && p.par_mlp) ? sel : 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float s = group16_sum(ssv[r]);
                    const int m = 4 * lg + r;
                    if (li == 0 && m < p.M)
                        p.ss[(int64_t)si * p.ss_sel_stride + (int64_t)(p.m0 + m) * ups + (u - sel * ups)] = s;
                }
            }
        }
    }
    if constexpr (EPI == EPI_LOGITS) {
        if (wave != 0) return;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v = best_v[r];
            int i = best_i[r];
            group16_argmax(v, i);
            const int m = 4 * lg + r;
            if (li == 0 && m < p.M) {
                p.part_val[(int64_t)(p.m0 + m) * gridDim.x + blockIdx.x] = v;
                p.part_idx[(int64_t)(p.m0 + m) * gridDim.x + blockIdx.x] = i;
            }
        }
    }
}

template <int MT, int EPI, int KS>
void launch_ks(const GemvParams &p, dim3 g, int ups, hipStream_t s) {
    if constexpr (EPI == EPI_RESID_ADD) {
        if (p.kseg > 1) {
            hipLaunchKernelGGL((k_gemm_mfma<MT, EPI, KS, true>), g, dim3(64 * KS), 0, s, p, ups);
            return;
        }
    }
    hipLaunchKernelGGL((k_gemm_mfma<MT, EPI, KS>), g, dim3(64 * KS), 0, s, p, ups);
}

template <int MT, int EPI>
void launch_epi(const GemvParams &p, dim3 g, int ks, int ups, hipStream_t s) {
    if (ks == 4) launch_ks<MT, EPI, 4>(p, g, ups, s);
    else launch_ks<MT, EPI, 8>(p, g, ups, s);
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

int env_int(const char *name, int dflt) {
    const char *e = getenv(name);
    return e ? atoi(e) : dflt;
}

}  // namespace

int gemm_mfma_max_rows() { return 16; }

// Weight rows of a unit: the two 16-row blocks of a pair for the paired
// epilogues, one block otherwise (two consecutive blocks per unit, measured:
// 8B verify 4.12 vs 3.87 ms, since the unpaired products then have half the
// workgroups).
int gemm_mfma_unit_rows(int epi, int rows, int rows_per_sel) {
    (void)rows; (void)rows_per_sel;
    return epi_is_pair(epi) ? 32 : 16;
}

// One unit per workgroup (measured against one or two persistent workgroups
// per CU that take several units each with the next unit's first tile
// requested early: 8B gate/up at 6 rows 43.2 vs 45.0-45.4 us), except
// sampling products, which keep a fixed grid (their arg-max partials are per
// workgroup).
int gemm_mfma_grid(const GemvParams &p) {
    const int n = p.n_units < 1 ? 1 : p.n_units;
    return p.epi == EPI_LOGITS && n > kLogitGrid ? kLogitGrid : n;
}

// Waves per workgroup (4 or 8), each streaming its own part of K: paired
// units take 8 (SPEC_MFMA_PAIR_KS overrides); other products 8 when the
// launch would otherwise have fewer than about 3K waves and every wave keeps
// at least one tile.
int gemm_mfma_splits(const GemvParams &p) {
    if (epi_is_pair(p.epi)) {
        static const int pk = env_int("SPEC_MFMA_PAIR_KS", 8) == 4 ? 4 : 8;
        return pk;
    }
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

int gemm_mfma_inv_max(int M) { return inv_max(M <= 8 ? 1 : 2); }

// p.n_units counts units of unit_rows weight rows (gemm_mfma_unit_rows).
hipError_t launch_gemm_mfma(const GemvParams &p, int grid, int ks, int unit_rows, hipStream_t s) {
    if (ks != 4 && ks != 8) return hipErrorInvalidValue;
    if (epi_is_pair(p.epi) ? unit_rows != 32 : (unit_rows != 16 && unit_rows != 32)) return hipErrorInvalidValue;
    const int ur = unit_rows;
    if (ur != gemm_mfma_unit_rows(p.epi, 0, 0) || p.rows_per_sel % ur != 0) return hipErrorInvalidValue;
    // partial index of a residual writer: the unit within its set member
    const int ups = p.rows_per_sel / ur;
    if (epi_has_ss(p.epi) && p.n_norm_sel > 0 && grid != p.n_units) return hipErrorInvalidValue;
    // every row of the call in one launch, operand packed as gemm_mfma_packed_rows says
    if (p.m0 != 0 || p.M > 16) return hipErrorInvalidValue;
    if (p.M <= 8) return launch_mt<1>(p, dim3(grid), ks, ups, s);
    return launch_mt<2>(p, dim3(grid), ks, ups, s);
}

}  // namespace spec
