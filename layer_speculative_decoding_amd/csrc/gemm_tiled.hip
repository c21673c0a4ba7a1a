// Tiled bf16 GEMM on the matrix cores for more than 16 activation rows (the
// base's and the draft's prompt prefills, M = rows of the prompt, and the
// verify / calibration rows of several sequences), with the decoder's fused
// epilogues.  Y[m][n] = sum_k X[m][k] W[n][k].
//
// At prompt lengths the products are compute-bound (every weight row is
// reused by all activation rows), so the kernel is organised around the
// matrix cores:
//  * a workgroup of 2 x 2 waves owns 128 activation rows and BN = 128 (or 64)
//    weight rows; a wave computes 64 x BN / 2 outputs with
//    v_mfma_f32_16x16x32_bf16, so each operand fragment read from LDS feeds
//    several matrix instructions;
//  * the weight tile is NH = BN / 2 units of two rows each: for the paired
//    epilogues a unit is the (RoPE partner, or gate / up) row pair, so both
//    rows of a pair end up in the same lane's accumulators; for the other
//    products a unit's rows are simply n0 + i and n0 + NH + i;
//  * the float32 activations enter the matrix cores as two bfloat16 pieces
//    hi + lo (split when the step's rows are written to LDS), so every
//    fragment pair takes two matrix instructions and the products carry the
//    activations to within 2^-16 of their magnitude; a tile with fewer call
//    rows than its 128 (verify rows of a few sequences) stashes and
//    multiplies only the 16-row blocks that hold rows;
//  * K advances in 64-element steps through one LDS stage (rows padded by 32
//    bytes, so the fragment reads of a wave spread over all banks); each
//    lane moves 16 bytes of weights per row (128 contiguous bytes per row per
//    8 lanes) and 32 bytes of activations, the weights two (128-row tiles) or
//    three (64-row) steps ahead of the matrix instructions (HBM latency), the
//    activations one step ahead (they stay in L2);
//  * workgroups take tiles in an XCD-aware grouped order (tile_of), so the
//    tiles resident on one XCD at a time share a few activation and weight
//    tiles in that XCD's L2;
//  * the 64-row weight tile is chosen when 128-row tiles would leave CUs
//    without a workgroup, and when even those are too few, K is split: each
//    K slice stores its float32 accumulators, and a second kernel adds the
//    slices in slice order and applies the epilogue.
#include "epilogue.h"
#include "spec_device.h"
#include "spec_kernels.h"

#include <stdio.h>
#include <stdlib.h>

namespace spec {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 64;           // K elements per step
// LDS row stride in elements: 160 bytes.  A fragment read (16 rows x 16
// bytes at four K offsets) meets every bank once at a 160-byte stride and
// twice at 144 (hardware conflict counters on a one-wave probe: 4 cycles per
// ds_read_b128 against 8); the stash writes are conflict-free at both.
constexpr int kLDK = kBK + 16;
// activation rows per tile: 2 wave rows of WMB 16-row blocks (WMB = 4: 128
// rows for prompt-length calls, WMB = 1: 32 rows for calls of at most 32)
constexpr int kMaxSplit = 8;

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
    int grp;           // > 0: XCD-aware grouped tile order (activation tiles per group)
    int bm;            // activation rows per tile (32 WMB)
    int parts;         // sum-of-squares partials per row and set member
    int ks;            // K slices (1: no split)
    int kc;            // K steps per slice
    float *part;       // ks > 1: [ks][tile][WMB * WNB][256 lanes] float4
};

// Tile of workgroup b (0 <= b < T) when several activation tiles share each
// weight tile.  The dispatcher deals workgroups to the eight XCDs in turn
// (b % 8), and each XCD has its own L2; so XCD x gets the contiguous run x of
// the logical order, and that order walks groups of ta.grp activation tiles
// across all weight tiles, activation tile fastest.  The workgroups one XCD
// holds at a time then share about grp activation tiles and (resident / grp)
// weight tiles, where the plain order (activation tile fastest over all of
// them) gave every XCD a different activation tile for every workgroup of a
// 256-tile-high product.  A bijection of [0, T): the result is the plain
// index nt * gm + mt.
__device__ __forceinline__ int tile_of(const TileArgs &ta, int b) {
    if (ta.grp <= 0 || ta.gm < 2) return b;
    const int T = ta.gm * ta.gn;
    const int xcd = b & 7, i = b >> 3;
    const int per = T >> 3, extra = T & 7;
    const int L = xcd * per + min(xcd, extra) + i;
    const int G = min(ta.gm, ta.grp);
    const int group = L / (G * ta.gn);
    const int first = group * G;
    const int gsz = min(G, ta.gm - first);
    const int w = L - first * ta.gn;
    return (w / gsz) * ta.gm + first + w % gsz;
}

// Where tile t sits: first activation row, first weight row (unpaired), first
// unit (paired), set member.
struct TilePos {
    int m0, n0, u0, sel;
};
template <int EPI, int BN>
__device__ __forceinline__ TilePos tile_pos(const GemvParams &p, const TileArgs &ta, int t) {
    TilePos q;
    const int mt = t % ta.gm, nt = t / ta.gm;
    q.m0 = mt * ta.bm;
    q.u0 = nt * (BN / 2);
    q.n0 = nt * BN;
    if (epi_is_pair(EPI)) q.sel = ((q.u0 / (p.pair_block / 2)) * p.pair_block) / p.rows_per_sel;
    else q.sel = q.n0 / p.rows_per_sel;
    return q;
}

// The fused epilogue of one tile.  Lane (li, lg) of wave (wm, wn), register r
// of block (a, c) holds activation row 64 wm + 16 a + 4 lg + r and unit
// (NH / 2) wn + 16 (c % HB) + li of member c / HB.
template <int EPI, int WNB, int WMB>
__device__ __forceinline__ void tile_epilogue(const GemvParams &p, const TileArgs &ta, const TilePos &q,
                                              const f32x4 (&acc)[WMB][WNB]) {
    constexpr bool kPair = epi_is_pair(EPI);
    constexpr int BN = 32 * WNB, NH = BN / 2, HB = WNB / 2;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int li = lane & 15, lg = lane >> 4;
    float best_v = -INFINITY;
    int best_i = 0;
#pragma unroll
    for (int a = 0; a < WMB; ++a) {
        float ssv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = q.m0 + 16 * WMB * wm + 16 * a + 4 * lg + r;
            if (m >= p.M) continue;
#pragma unroll
            for (int c = 0; c < HB; ++c) {
                const int j = (NH / 2) * wn + 16 * c + li;
                if constexpr (kPair) {
                    const int hb = p.pair_block / 2, u = q.u0 + j;
                    const int r0 = (u / hb) * p.pair_block + u % hb;
                    epi_pair<uint16_t, EPI>(p, u, r0, r0 + hb, q.sel, m, acc[a][c][r], acc[a][c + HB][r]);
                } else {
                    epi_row<uint16_t, EPI>(p, q.n0 + j, q.sel, m, acc[a][c][r], ssv[r], best_v, best_i);
                    epi_row<uint16_t, EPI>(p, q.n0 + NH + j, q.sel, m, acc[a][c + HB][r], ssv[r], best_v, best_i);
                }
            }
        }
        if constexpr (epi_has_ss(EPI)) {
            if (p.n_norm_sel > 0 && (EPI == EPI_RESID_ADD || p.par_mlp || q.sel == 0)) {
                const int si = (EPI == EPI_ATTN_OUT && p.par_mlp) ? q.sel : 0;
                const int part = ((q.n0 - q.sel * p.rows_per_sel) / BN) * 2 + wn;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float s = sum16(ssv[r]);
                    const int m = q.m0 + 16 * WMB * wm + 16 * a + 4 * lg + r;
                    if (li == 0 && m < p.M)
                        p.ss[(int64_t)si * p.ss_sel_stride + (int64_t)(p.m0 + m) * ta.parts + part] = s;
                }
            }
        }
    }
}

// 4 waves (2 x 2), each 64 activation rows x 16 WNB weight rows; K steps of
// 64 through one LDS stage, the weights of step k + DIST requested before
// step k's matrix instructions, the activations of step k + 1.  SPLIT: workgroup
// b covers tile b % T over K slice b / T and stores its accumulators.
template <int EPI, int WNB, bool SPLIT, int WMB>
__global__ __launch_bounds__(256, 2) void k_gemm_tile(GemvParams p, TileArgs ta) {
    constexpr int BM = 32 * WMB;
    constexpr bool kPair = epi_is_pair(EPI);
    constexpr int BN = 32 * WNB, NH = BN / 2;
    constexpr int HB = WNB / 2;                  // 16-unit blocks per wave per member
    constexpr int RPP = 32;                      // rows per load pass (8 lanes x 16 bytes per row)
    constexpr int LA = BM / RPP, LB = BN / RPP;  // load passes per step
    // weight steps in flight: three for 64-row tiles (their per-step bytes are
    // half, and three workgroups share a CU), two for 128-row tiles (whose
    // register budget has no room for a third); four with 32 activation rows
    // (few accumulators: the weight stream is all there is)
    constexpr int DIST = WMB == 1 ? 4 : (WNB == 2 ? 3 : 2);
    // activation hi pieces, lo pieces, weights
    __shared__ __align__(16) uint16_t lds[(2 * BM + BN) * kLDK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int li = lane & 15, lg = lane >> 4;
    const int K = p.K;
    const int T = ta.gm * ta.gn;
    const int t = tile_of(ta, SPLIT ? (int)blockIdx.x % T : (int)blockIdx.x);
    const int slice = SPLIT ? (int)blockIdx.x / T : 0;
    const TilePos q = tile_pos<EPI, BN>(p, ta, t);
    const int kbeg = slice * ta.kc;
    const int nk = SPLIT ? min(ta.kc, K / kBK - kbeg) : K / kBK;

    // operands as a uniform base plus 32-bit per-lane byte offsets
    const char *Xb = reinterpret_cast<const char *>(reinterpret_cast<const float *>(p.X) +
                                                    (int64_t)q.sel * p.x_sel_stride + (int64_t)p.m0 * K +
                                                    (int64_t)kbeg * kBK);
    const char *Wb = reinterpret_cast<const char *>(reinterpret_cast<const uint16_t *>(p.W) + (int64_t)kbeg * kBK);

    // loader: thread t moves 16 bytes of tile rows t / 8 + 32 i, elements 8 (t % 8)
    const int lr = tid >> 3, lc = 8 * (tid & 7);
    uint32_t oa[LA], ob[LB];
    bool va[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int m = q.m0 + lr + RPP * i;
        va[i] = m < p.M;
        oa[i] = ((uint32_t)(va[i] ? m : 0) * (uint32_t)K + (uint32_t)lc) * 4u;
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int r = lr + RPP * i;          // tile row: member r / NH, unit r % NH
        int w;
        if (kPair) {
            const int hb = p.pair_block / 2, u = q.u0 + r % NH;
            w = (u / hb) * p.pair_block + u % hb + (r / NH) * hb;
        } else {
            w = q.n0 + r;
        }
        ob[i] = (uint32_t)w * (uint32_t)K * 2u + (uint32_t)lc * 2u;
    }
    // weights DIST steps ahead (HBM latency), activations one step ahead
    // (they are re-read from L2 by every weight tile)
    uint4 ra[LA][2], rb[DIST][LB];
    auto load_w = [&](int k0, uint4 (&xb)[LB]) {
#pragma unroll
        for (int i = 0; i < LB; ++i) xb[i] = ld16(Wb + (uint64_t)(ob[i] + (uint32_t)k0 * 2u));
    };
    auto load_x = [&](int k0) {
#pragma unroll
        for (int i = 0; i < LA; ++i) {
            const char *x = Xb + (uint64_t)(oa[i] + (uint32_t)k0 * 4u);
            ra[i][0] = va[i] ? ld16(x) : make_uint4(0, 0, 0, 0);
            ra[i][1] = va[i] ? ld16(x + 16) : make_uint4(0, 0, 0, 0);
        }
    };
    // activation rows any wave reads (16-row blocks that hold call rows)
    const int mneed = min(BM, (p.M - q.m0 + 15) / 16 * 16);
    auto stash = [&](const uint4 (&xa)[LA][2], const uint4 (&xb)[LB]) {
#pragma unroll
        for (int i = 0; i < LA; ++i) {
            if (RPP * i >= mneed) continue;
            const float x[8] = {__uint_as_float(xa[i][0].x), __uint_as_float(xa[i][0].y), __uint_as_float(xa[i][0].z),
                                __uint_as_float(xa[i][0].w), __uint_as_float(xa[i][1].x), __uint_as_float(xa[i][1].y),
                                __uint_as_float(xa[i][1].z), __uint_as_float(xa[i][1].w)};
            uint4 hi, lo;
            split2_bf16_hw(x, hi, lo);
            *reinterpret_cast<uint4 *>(&lds[(lr + RPP * i) * kLDK + lc]) = hi;
            *reinterpret_cast<uint4 *>(&lds[(BM + lr + RPP * i) * kLDK + lc]) = lo;
        }
#pragma unroll
        for (int i = 0; i < LB; ++i) *reinterpret_cast<uint4 *>(&lds[(2 * BM + lr + RPP * i) * kLDK + lc]) = xb[i];
    };

    f32x4 acc[WMB][WNB];
#pragma unroll
    for (int a = 0; a < WMB; ++a)
#pragma unroll
        for (int c = 0; c < WNB; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};

    // LDS rows of this lane's fragments: activation block a, weight block c
    // (member c / HB, unit block c % HB of this wave column)
    const int arow = (16 * WMB * wm + li) * kLDK + 8 * lg;
    const int brow = (2 * BM + (NH / 2) * wn + li) * kLDK + 8 * lg;
    // 16-row activation blocks of this wave that hold call rows (a tile of a
    // few verify rows leaves most of them empty: their products are skipped)
    const int nva = __builtin_amdgcn_readfirstlane(min(WMB, max(0, (p.M - q.m0 - 16 * WMB * wm + 15) / 16)));
    auto compute = [&]() {
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            uint4 bv[WNB];
#pragma unroll
            for (int c = 0; c < WNB; ++c)
                bv[c] = *reinterpret_cast<const uint4 *>(
                    &lds[brow + ((c / HB) * NH + 16 * (c % HB)) * kLDK + 32 * ks]);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint4 av[WMB];
#pragma unroll
                for (int a = 0; a < WMB; ++a)
                    av[a] = *reinterpret_cast<const uint4 *>(&lds[arow + (h * BM + 16 * a) * kLDK + 32 * ks]);
#pragma unroll
                for (int a = 0; a < WMB; ++a)
#pragma unroll
                    for (int c = 0; c < WNB; ++c)
                        acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(av[a]), as_bf8(bv[c]),
                                                                            acc[a][c], 0, 0, 0);
            }
        }
    };
    // the same for the first nva blocks only
    auto compute_part = [&]() {
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            uint4 bv[WNB];
#pragma unroll
            for (int c = 0; c < WNB; ++c)
                bv[c] = *reinterpret_cast<const uint4 *>(
                    &lds[brow + ((c / HB) * NH + 16 * (c % HB)) * kLDK + 32 * ks]);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int a = 0; a < WMB; ++a) {
                    if (a < nva) {
                        const uint4 av = *reinterpret_cast<const uint4 *>(&lds[arow + (h * BM + 16 * a) * kLDK + 32 * ks]);
#pragma unroll
                        for (int c = 0; c < WNB; ++c)
                            acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(av), as_bf8(bv[c]),
                                                                                acc[a][c], 0, 0, 0);
                    }
                }
            }
        }
    };

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
                if (nva == WMB) compute();
                else if (nva > 0) compute_part();
            }
        }
    }

    if constexpr (SPLIT) {
        // 16-row activation blocks past the call's rows hold nothing; they
        // are neither stored here nor read back by the slice sum
        float4 *dst = reinterpret_cast<float4 *>(ta.part) + ((int64_t)slice * T + t) * (WMB * WNB) * 256 + tid;
#pragma unroll
        for (int a = 0; a < WMB; ++a)
            if (q.m0 + 16 * WMB * wm + 16 * a < p.M)
#pragma unroll
                for (int c = 0; c < WNB; ++c)
                    dst[(a * WNB + c) * 256] = make_float4(acc[a][c][0], acc[a][c][1], acc[a][c][2], acc[a][c][3]);
    } else {
        tile_epilogue<EPI, WNB, WMB>(p, ta, q, acc);
    }
}

// Sum of a split product's K slices (in slice order) and its epilogue; one
// workgroup per tile, lanes as in the product kernel.
template <int EPI, int WNB, int WMB>
__global__ __launch_bounds__(256) void k_gemm_tile_epi(GemvParams p, TileArgs ta) {
    constexpr int BN = 32 * WNB;
    const int T = ta.gm * ta.gn, t = blockIdx.x;
    const TilePos q = tile_pos<EPI, BN>(p, ta, t);
    const int wm = (threadIdx.x >> 6) & 1;
    const float4 *src = reinterpret_cast<const float4 *>(ta.part) + (int64_t)t * (WMB * WNB) * 256 + threadIdx.x;
    // the blocks of up to SG slices are requested together, then added in
    // slice order (the sum's order is fixed: slice 0, 1, 2, ...)
    constexpr int SG = WNB == 2 ? 4 : 2;
    const int64_t sstride = (int64_t)T * (WMB * WNB) * 256;
    f32x4 acc[WMB][WNB];
#pragma unroll
    for (int a = 0; a < WMB; ++a)
#pragma unroll
        for (int c = 0; c < WNB; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < ta.ks; k0 += SG) {
        float4 v[SG][WMB][WNB];
#pragma unroll
        for (int g = 0; g < SG; ++g)
#pragma unroll
            for (int a = 0; a < WMB; ++a)
#pragma unroll
                for (int c = 0; c < WNB; ++c)
                    v[g][a][c] = (k0 + g < ta.ks && q.m0 + 16 * WMB * wm + 16 * a < p.M)
                                     ? src[(k0 + g) * sstride + (a * WNB + c) * 256]
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int g = 0; g < SG; ++g)
#pragma unroll
            for (int a = 0; a < WMB; ++a)
#pragma unroll
                for (int c = 0; c < WNB; ++c)
                    if (k0 + g < ta.ks) acc[a][c] += f32x4{v[g][a][c].x, v[g][a][c].y, v[g][a][c].z, v[g][a][c].w};
    }
    tile_epilogue<EPI, WNB, WMB>(p, ta, q, acc);
}

template <int WNB, int EPI, int WMB>
void launch_wmb(const GemvParams &p, const TileArgs &ta, hipStream_t s) {
    const int T = ta.gm * ta.gn;
    if (ta.ks > 1) {
        hipLaunchKernelGGL((k_gemm_tile<EPI, WNB, true, WMB>), dim3(T * ta.ks), dim3(256), 0, s, p, ta);
        hipLaunchKernelGGL((k_gemm_tile_epi<EPI, WNB, WMB>), dim3(T), dim3(256), 0, s, p, ta);
    } else {
        hipLaunchKernelGGL((k_gemm_tile<EPI, WNB, false, WMB>), dim3(T), dim3(256), 0, s, p, ta);
    }
}

template <int WNB, int EPI>
void launch_one(const GemvParams &p, const TileArgs &ta, hipStream_t s) {
    if (ta.bm == 32) launch_wmb<WNB, EPI, 1>(p, ta, s);
    else launch_wmb<WNB, EPI, 4>(p, ta, s);
}

template <int WNB>
hipError_t launch_shape(const GemvParams &p, TileArgs ta, hipStream_t s) {
    switch (p.epi) {
    case EPI_STORE: launch_one<WNB, EPI_STORE>(p, ta, s); break;
    case EPI_QKV_ROPE: launch_one<WNB, EPI_QKV_ROPE>(p, ta, s); break;
    case EPI_SILU_MUL: launch_one<WNB, EPI_SILU_MUL>(p, ta, s); break;
    case EPI_RESID_ADD: launch_one<WNB, EPI_RESID_ADD>(p, ta, s); break;
    case EPI_ATTN_OUT: launch_one<WNB, EPI_ATTN_OUT>(p, ta, s); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Weight rows per tile the product's layout allows.
bool fits(const GemvParams &p, int bn) {
    if (epi_is_pair(p.epi)) return (p.rows_per_sel / 2) % (bn / 2) == 0 && p.rows_per_sel % p.pair_block == 0;
    return p.rows_per_sel % bn == 0;
}

// Launch choice: tile width bn and K slices.  SPEC_TILE="<bn> <slices>"
// overrides it (read at every call, for measurement and tests).
struct Pick {
    int bn, ks;
};
// Activation rows per tile: 32 for calls of at most 32 rows (SPEC_TILE_SMALL=0:
// always 128).
int tile_rows(int M) {
    static const bool small = [] {
        const char *e = getenv("SPEC_TILE_SMALL");
        return !(e && e[0] == '0');
    }();
    return (small && M <= 32) ? 32 : 128;
}
// Activation tiles per group of the XCD-aware tile order (SPEC_TILE_GROUP,
// read at every call like SPEC_TILE; 0: plain order).  Measured on the
// 70B-shaped prefill (four 8192-token prompts as one 32768-row call, 256
// activation tiles per product): 16.1 s in plain order, 12.0-12.3 s with
// groups of 2 or 4, 12.5 s with 1, 13.4 s with 8; the 2048- and 512-row
// prefills gain 0.5-2 %.
int tile_group() {
    const char *e = getenv("SPEC_TILE_GROUP");
    return e ? atoi(e) : 4;
}
Pick pick(const GemvParams &p, size_t part_bytes) {
    const int rows = p.n_units * 2, nk = p.K / kBK;
    const int bm = tile_rows(p.M);
    const int gm = (p.M + bm - 1) / bm;
    Pick k{0, 1};
    if (const char *e = getenv("SPEC_TILE")) {
        Pick f{0, 1};
        if (sscanf(e, "%d %d", &f.bn, &f.ks) >= 1 && (f.bn == 64 || f.bn == 128) && fits(p, f.bn)) k = f;
    }
    if (k.bn == 0) {
        if (fits(p, 128) && (int64_t)gm * (rows / 128) >= 256) return {128, 1};
        if (!fits(p, 64)) return {0, 1};
        k.bn = 64;
        // fewer than 384 tiles: slices so that at most 768 workgroups run
        // (three per CU resident at once: no tail round), each over >= 2 K
        // steps (more tiles run better unsplit: the slices' float32 partials
        // cost a write and a read each)
        const int64_t T = (int64_t)gm * (rows / 64);
        k.ks = T >= 384 ? 1 : (int)(768 / T);
    }
    k.ks = k.ks < 1 ? 1 : (k.ks > kMaxSplit ? kMaxSplit : k.ks);
    if (k.ks > nk / 2) k.ks = nk / 2 < 1 ? 1 : nk / 2;
    // the partial buffer bounds the slices
    const int64_t tile_bytes = (int64_t)gm * (rows / k.bn) * bm * k.bn * 4;
    while (k.ks > 1 && (size_t)(tile_bytes * k.ks) > part_bytes) --k.ks;
    return k;
}

TileArgs tile_args(const GemvParams &p, Pick k, float *part) {
    TileArgs ta;
    const int nk = p.K / kBK;
    ta.bm = tile_rows(p.M);
    ta.gm = (p.M + ta.bm - 1) / ta.bm;
    ta.grp = tile_group();
    ta.gn = (p.n_units * 2) / k.bn;
    ta.parts = (p.rows_per_sel / k.bn) * 2;
    ta.kc = (nk + k.ks - 1) / k.ks;
    ta.ks = (nk + ta.kc - 1) / ta.kc;      // every slice non-empty
    ta.part = part;
    return ta;
}

}  // namespace

// From 17 rows on (where the skinny matrix-core kernel would need a second
// 16-row activation tile) the tiled kernel is the faster of the two: measured
// at 28 rows on the 70B-shaped products, 176 vs 271 us (gate / up), 111 vs
// 148 us (down), 63 vs 82 us (QKV).
int gemm_tiled_min_rows() { return 17; }

bool gemm_tiled_supported(const GemvParams &p) {
    if (p.K % kBK != 0 || p.epi == EPI_LOGITS || p.M < 1) return false;
    return pick(p, 0).bn != 0;
}

// Sum-of-squares partials per row and set member a residual writer leaves
// (two per weight tile: one per wave column).
int gemm_tiled_parts(const GemvParams &p) { return (p.rows_per_sel / pick(p, 0).bn) * 2; }

std::string gemm_tiled_name(const GemvParams &p, size_t part_bytes) {
    const Pick k = pick(p, part_bytes);
    const TileArgs ta = tile_args(p, k, nullptr);
    return "k_gemm_tile<" + std::to_string(p.epi) + ", " + std::to_string(k.bn / 32) + ", " +
           std::to_string(ta.bm / 32) + (ta.ks > 1 ? ", split " + std::to_string(ta.ks) + ">" : ">");
}

size_t gemm_tiled_part_bytes() { return (size_t)64 << 20; }

// p.n_units: row pairs (rows / 2) as for the other products; p.M rows from
// p.m0 (the kernel reads X rows m0 .. m0 + M - 1 and the epilogue writes them).
hipError_t launch_gemm_tiled(const GemvParams &p, float *part, size_t part_bytes, hipStream_t s) {
    if (!gemm_tiled_supported(p)) return hipErrorInvalidValue;
    const Pick k = pick(p, part ? part_bytes : 0);
    const TileArgs ta = tile_args(p, k, part);
    if (k.bn == 128) return launch_shape<4>(p, ta, s);
    return launch_shape<2>(p, ta, s);
}

}  // namespace spec
