// Tiled bf16 GEMM on the matrix cores for prompt-length activation counts
// (the base's and the draft's prompt prefills: M = rows of the prompt), with
// the decoder's fused epilogues.  Y[m][n] = sum_k X[m][k] W[n][k].
//
// At M >= 64 the products are compute-bound (every weight row is reused by
// all activation rows), so the kernel is organised around the matrix cores:
//  * a workgroup of 2 x 2 waves owns 128 activation rows and BN = 128 (or 64)
//    weight rows; a wave computes 64 x BN / 2 outputs with
//    v_mfma_f32_16x16x32_bf16, so each operand fragment read from LDS feeds
//    several matrix instructions;
//  * the weight tile is NH = BN / 2 units of two rows each: for the paired
//    epilogues a unit is the (RoPE partner, or gate / up) row pair, so both
//    rows of a pair end up in the same lane's accumulators; for the other
//    products a unit's rows are simply n0 + i and n0 + NH + i;
//  * K advances in 64-element steps through one LDS stage (rows padded by 16
//    bytes, so the fragment reads of a wave spread over all banks); each
//    lane moves 16 bytes per row (128 contiguous bytes per row per 8 lanes),
//    the weights two steps ahead of the matrix instructions (HBM latency),
//    the activations one step ahead (they stay in L2);
//  * the 64-row weight tile is chosen when 128-row tiles would leave CUs
//    without a workgroup.
#include "epilogue.h"
#include "spec_device.h"
#include "spec_kernels.h"

namespace spec {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 64;           // K elements per step
constexpr int kLDK = kBK + 8;     // LDS row stride in elements (16 bytes of padding)
constexpr int kXcds = 8;

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

struct TileArgs {
    int gm, gn;        // activation tiles, weight tiles
    int parts;         // sum-of-squares partials per row and set member
    int remap;         // number tiles XCD by XCD
};

// 4 waves (2 x 2), each 64 activation rows x 16 WNB weight rows; K steps of
// 64 through one LDS stage, with the global loads of step k + DIST issued
// before step k's matrix instructions (DIST register sets in flight).
template <int EPI, int WNB, int DIST>
__global__ __launch_bounds__(256, 2) void k_gemm_tile(GemvParams p, TileArgs ta) {
    constexpr bool kPair = epi_is_pair(EPI);
    constexpr int WMB = 4, NWM = 2, NWN = 2;
    constexpr int BM = 16 * WMB * NWM, BN = 16 * WNB * NWN, NH = BN / 2;
    constexpr int HB = WNB / 2;                 // 16-unit blocks per wave per member
    constexpr int RPP = 32;                     // rows per load pass (8 lanes x 16 bytes per row)
    constexpr int LA = BM / RPP, LB = BN / RPP; // load passes per step
    static_assert(WNB % 2 == 0 && BN % RPP == 0, "tile shape");
    __shared__ __align__(16) uint16_t lds[(BM + BN) * kLDK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % NWM, wn = wave / NWM;
    const int li = lane & 15, lg = lane >> 4;
    const int K = p.K;

    const int L = blockIdx.x, T = ta.gm * ta.gn;
    const int Q = (ta.remap && T % kXcds == 0) ? (L % kXcds) * (T / kXcds) + L / kXcds : L;
    const int mt = Q % ta.gm, nt = Q / ta.gm;
    const int m0 = mt * BM;
    const int u0 = nt * NH;                    // first unit (pairs)
    const int n0 = nt * BN;                    // first row (unpaired)
    int sel;
    if (kPair) sel = (((u0 / (p.pair_block / 2)) * p.pair_block) / p.rows_per_sel);
    else sel = n0 / p.rows_per_sel;
    // operands as a uniform base plus 32-bit per-lane byte offsets
    const char *Xb = reinterpret_cast<const char *>(reinterpret_cast<const uint16_t *>(p.X) +
                                                    (int64_t)sel * p.x_sel_stride + (int64_t)p.m0 * K);
    const char *Wb = reinterpret_cast<const char *>(p.W);

    // loader: thread t moves 16 bytes of tile rows t / 8 + 32 i, elements 8 (t % 8)
    const int lr = tid >> 3, lc = 8 * (tid & 7);
    uint32_t oa[LA], ob[LB];
    bool va[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int m = m0 + lr + RPP * i;
        va[i] = m < p.M;
        oa[i] = (uint32_t)(((va[i] ? m : 0) * K + lc) * 2);
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int r = lr + RPP * i;          // tile row: member r / NH, unit r % NH
        int w;
        if (kPair) {
            const int hb = p.pair_block / 2, u = u0 + r % NH;
            w = (u / hb) * p.pair_block + u % hb + (r / NH) * hb;
        } else {
            w = n0 + r;
        }
        ob[i] = (uint32_t)w * (uint32_t)K * 2u + (uint32_t)lc * 2u;
    }
    // weights DIST steps ahead (HBM latency), activations one step ahead
    // (they are re-read from L2 by every weight tile)
    uint4 ra[LA], rb[DIST][LB];
    auto load_w = [&](int k0, uint4 (&xb)[LB]) {
#pragma unroll
        for (int i = 0; i < LB; ++i) xb[i] = ld16(Wb + (uint64_t)(ob[i] + (uint32_t)k0 * 2u));
    };
    auto load_x = [&](int k0) {
#pragma unroll
        for (int i = 0; i < LA; ++i)
            ra[i] = va[i] ? ld16(Xb + (uint64_t)(oa[i] + (uint32_t)k0 * 2u)) : make_uint4(0, 0, 0, 0);
    };
    auto stash = [&](const uint4 (&xa)[LA], const uint4 (&xb)[LB]) {
#pragma unroll
        for (int i = 0; i < LA; ++i) *reinterpret_cast<uint4 *>(&lds[(lr + RPP * i) * kLDK + lc]) = xa[i];
#pragma unroll
        for (int i = 0; i < LB; ++i) *reinterpret_cast<uint4 *>(&lds[(BM + lr + RPP * i) * kLDK + lc]) = xb[i];
    };

    f32x4 acc[WMB][WNB];
#pragma unroll
    for (int a = 0; a < WMB; ++a)
#pragma unroll
        for (int c = 0; c < WNB; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    // LDS rows of this lane's fragments: activation block a, weight block c
    // (member c / HB, unit block c % HB of this wave column)
    const int arow = (16 * WMB * wm + li) * kLDK + 8 * lg;
    const int brow = (BM + (NH / NWN) * wn + li) * kLDK + 8 * lg;
    auto compute = [&]() {
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            uint4 av[WMB], bv[WNB];
#pragma unroll
            for (int a = 0; a < WMB; ++a)
                av[a] = *reinterpret_cast<const uint4 *>(&lds[arow + 16 * a * kLDK + 32 * ks]);
#pragma unroll
            for (int c = 0; c < WNB; ++c)
                bv[c] = *reinterpret_cast<const uint4 *>(
                    &lds[brow + ((c / HB) * NH + 16 * (c % HB)) * kLDK + 32 * ks]);
#pragma unroll
            for (int a = 0; a < WMB; ++a)
#pragma unroll
                for (int c = 0; c < WNB; ++c)
                    acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(av[a]), as_bf8(bv[c]), acc[a][c],
                                                                        0, 0, 0);
        }
    };

    const int nk = K / kBK;
    load_x(0);
#pragma unroll
    for (int d = 0; d < DIST; ++d)
        if (d < nk) load_w(d * kBK, rb[d]);
    for (int kt = 0; kt < nk; kt += DIST) {
#pragma unroll
        for (int d = 0; d < DIST; ++d) {
            const int k = kt + d;
            if (k < nk) {
                __syncthreads();      // previous step's fragments read
                stash(ra, rb[d]);
                __syncthreads();
                if (k + DIST < nk) load_w((k + DIST) * kBK, rb[d]);
                if (k + 1 < nk) load_x((k + 1) * kBK);
                compute();
            }
        }
    }

    // epilogue: lane (li, lg), register r of block (a, c) holds activation
    // row 16 WMB wm + 16 a + 4 lg + r and unit (NH / NWN) wn + 16 (c % HB) + li
    // of member c / HB
    float best_v = -INFINITY;
    int best_i = 0;
#pragma unroll
    for (int a = 0; a < WMB; ++a) {
        float ssv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + 16 * WMB * wm + 16 * a + 4 * lg + r;
            if (m >= p.M) continue;
#pragma unroll
            for (int c = 0; c < HB; ++c) {
                const int j = (NH / NWN) * wn + 16 * c + li;
                if constexpr (kPair) {
                    const int hb = p.pair_block / 2, u = u0 + j;
                    const int r0 = (u / hb) * p.pair_block + u % hb;
                    epi_pair<uint16_t, EPI>(p, u, r0, r0 + hb, sel, m, acc[a][c][r], acc[a][c + HB][r]);
                } else {
                    epi_row<uint16_t, EPI>(p, n0 + j, sel, m, acc[a][c][r], ssv[r], best_v, best_i);
                    epi_row<uint16_t, EPI>(p, n0 + NH + j, sel, m, acc[a][c + HB][r], ssv[r], best_v, best_i);
                }
            }
        }
        if constexpr (epi_has_ss(EPI)) {
            if (p.n_norm_sel > 0 && (EPI == EPI_RESID_ADD || p.par_mlp || sel == 0)) {
                const int si = (EPI == EPI_ATTN_OUT && p.par_mlp) ? sel : 0;
                const int part = ((n0 - sel * p.rows_per_sel) / BN) * NWN + wn;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float s = sum16(ssv[r]);
                    const int m = m0 + 16 * WMB * wm + 16 * a + 4 * lg + r;
                    if (li == 0 && m < p.M)
                        p.ss[(int64_t)si * p.ss_sel_stride + (int64_t)(p.m0 + m) * ta.parts + part] = s;
                }
            }
        }
    }
}

template <int WNB, int DIST, int EPI>
void launch_one(const GemvParams &p, const TileArgs &ta, hipStream_t s) {
    hipLaunchKernelGGL((k_gemm_tile<EPI, WNB, DIST>), dim3(ta.gm * ta.gn), dim3(256), 0, s, p, ta);
}

template <int WNB, int DIST>
hipError_t launch_shape(const GemvParams &p, int remap, hipStream_t s) {
    constexpr int BM = 128, BN = 32 * WNB;
    TileArgs ta;
    ta.gm = (p.M + BM - 1) / BM;
    ta.gn = (p.n_units * 2) / BN;
    ta.parts = (p.rows_per_sel / BN) * 2;
    ta.remap = remap;
    switch (p.epi) {
    case EPI_STORE: launch_one<WNB, DIST, EPI_STORE>(p, ta, s); break;
    case EPI_QKV_ROPE: launch_one<WNB, DIST, EPI_QKV_ROPE>(p, ta, s); break;
    case EPI_SILU_MUL: launch_one<WNB, DIST, EPI_SILU_MUL>(p, ta, s); break;
    case EPI_RESID_ADD: launch_one<WNB, DIST, EPI_RESID_ADD>(p, ta, s); break;
    case EPI_ATTN_OUT: launch_one<WNB, DIST, EPI_ATTN_OUT>(p, ta, s); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Weight rows per tile the product's layout allows.
bool fits(const GemvParams &p, int bn) {
    if (epi_is_pair(p.epi)) return (p.rows_per_sel / 2) % (bn / 2) == 0 && p.rows_per_sel % p.pair_block == 0;
    return p.rows_per_sel % bn == 0;
}

// Launch choice (overridable for measurement: SPEC_TILE = "<bn> <dist> <remap>").
struct Pick {
    int bn, dist, remap;
};
Pick pick(const GemvParams &p) {
    static const Pick forced = [] {
        Pick f{0, 0, 0};
        if (const char *e = getenv("SPEC_TILE")) sscanf(e, "%d %d %d", &f.bn, &f.dist, &f.remap);
        return f;
    }();
    const int rows = p.n_units * 2;
    if (forced.bn && fits(p, forced.bn)) return forced;
    const int gm = (p.M + 127) / 128;
    if (fits(p, 128) && (int64_t)gm * (rows / 128) >= 256) return {128, 2, 0};
    if (fits(p, 64)) return {64, 2, 0};
    return {0, 0, 0};
}

}  // namespace

int gemm_tiled_min_rows() { return 64; }

bool gemm_tiled_supported(const GemvParams &p) {
    if (p.K % kBK != 0 || p.epi == EPI_LOGITS || p.M < 1) return false;
    return pick(p).bn != 0;
}

// Sum-of-squares partials per row and set member a residual writer leaves
// (two per weight tile: one per wave column).
int gemm_tiled_parts(const GemvParams &p) { return (p.rows_per_sel / pick(p).bn) * 2; }

std::string gemm_tiled_name(const GemvParams &p) {
    const Pick k = pick(p);
    return "k_gemm_tile<" + std::to_string(p.epi) + ", " + std::to_string(k.bn / 32) + ", " +
           std::to_string(k.dist) + ">";
}

// p.n_units: row pairs (rows / 2) as for the other products; p.M rows from
// p.m0 (the kernel reads X rows m0 .. m0 + M - 1 and the epilogue writes them).
hipError_t launch_gemm_tiled(const GemvParams &p, hipStream_t s) {
    if (!gemm_tiled_supported(p)) return hipErrorInvalidValue;
    const Pick k = pick(p);
    if (k.bn == 128) return k.dist == 2 ? launch_shape<4, 2>(p, k.remap, s) : launch_shape<4, 1>(p, k.remap, s);
    return k.dist == 2 ? launch_shape<2, 2>(p, k.remap, s) : launch_shape<2, 1>(p, k.remap, s);
}

}  // namespace spec
