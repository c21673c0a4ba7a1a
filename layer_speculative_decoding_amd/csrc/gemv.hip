// Weight-streaming matrix-vector products for few activation rows (the draft
// step's one row per sequence, and the float32 path), with RMSNorm folded
// into the operand load and the decoder's consumers fused into the epilogue;
// plus the embedding kernel that starts every forward call.
//
// At decode batch sizes these products read every weight byte once and do a
// handful of flops per byte, so they are bound by HBM bandwidth: each wave
// streams two weight rows with 16-byte non-temporal loads (four loads in flight
// per row), multiplies them with up to MR activation rows held in L1/L2, and
// reduces across the wave.  A unit is a *pair* of rows so that the epilogue
// sees both halves of a RoPE pair (j, j + hd/2) or a (gate, up) pair.
#include <cstdlib>

#include "epilogue.h"
#include "spec_device.h"
#include "spec_kernels.h"

namespace spec {

namespace {

constexpr int kWaves = 4;          // waves per workgroup
constexpr int kMaxRows = 8;        // activation rows per launch
constexpr int kMaxGrid = 256 * 8;  // workgroups (8 per CU)
constexpr int kUnroll = 4;

// A workgroup's four waves take 4 / KS units at a time; the KS waves of a
// unit (a row pair) each stream a contiguous, step-aligned part of K, and
// their partial dot products meet in LDS and are summed in part order by the
// unit's first wave, which runs the epilogue.  Per chunk of kUnroll 16-byte
// steps the weights are requested first, then the activation operands, and
// every load of a chunk is in flight before the arithmetic starts.
//
// Normalised operands: every wave forms the rows' 1/rms from the residual
// writers' partials (summed in partial order, so all waves agree bit for
// bit).  When the normalised rows of all set members fit in kStageBytes of
// LDS, the workgroup writes them there once (float32) and the units read them
// from LDS; the first chunk of weights is requested before, so the staging
// overlaps the weight stream.  Otherwise each step normalises its own
// operands.  Activations are float32 on both paths (only weights and the KV
// cache are bfloat16 on the bfloat16 path), so the products are float32 dot
// products of the stored weights.
constexpr int kStageBytes = 32768;

// plain rows, normalised rows staged in LDS, normalised per step, plain rows
// with K in segments (the down projection over a set's members)
enum : int { XM_PLAIN = 0, XM_STAGED = 1, XM_DIRECT = 2, XM_SEG = 3 };

template <typename T, int MR, int EPI, int XM>
__global__ __launch_bounds__(256) void k_gemv(GemvParams p, int KS) {
    using S = Store<T>;
    constexpr bool kNorm = XM == XM_STAGED || XM == XM_DIRECT;
    constexpr bool staged = XM == XM_STAGED;
    constexpr int E = S::kPer16;
    constexpr bool kPair = epi_is_pair(EPI);
    // staged operand rows: dynamic LDS of exactly n_sel * MR * K floats (the
    // call's own size rather than a fixed 32 KB stage per workgroup)
    extern __shared__ __align__(16) float xs[];
    __shared__ float red[kWaves][kMaxRows][2];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int upb = kWaves / KS;                 // units per workgroup and round
    const int slot = wave / KS, part = wave - slot * KS;
    const int K = p.K;
    const int step = kWave * E;
    const int chunk = kUnroll * step;
    const int nsteps = (K + step - 1) / step;
    const int sper = (nsteps + KS - 1) / KS;
    const int kb = min(K, part * sper * step), ke = min(K, (part + 1) * sper * step);
    const int half = p.pair_block >> 1;
    const int n_sel = (p.n_units * 2) / p.rows_per_sel;
    float best_v = -INFINITY;
    int best_i = 0x7FFFFFFF;
    float ss[kMaxSel];
#pragma unroll
    for (int s = 0; s < kMaxSel; ++s) ss[s] = 0.f;
    float inv[MR];
    int hrow[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) { inv[m] = 0.f; hrow[m] = 0; }

    auto unit_rows = [&](int u, int &r0, int &r1, int &sel) {
        const int blk = u / half, j = u - blk * half;
        r0 = blk * p.pair_block + j;
        r1 = r0 + half;
        sel = r0 / p.rows_per_sel;
    };
    // K in segments (set members' matrices side by side): segment of k and
    // the offset of element k of row r
    constexpr bool kSegOk = XM == XM_SEG;
    const int Ks = (kSegOk && p.kseg > 1) ? K / p.kseg : K;
    auto seg_of = [&](int k) {
        int sg = 0;
#pragma unroll
        for (int i = 1; i < kMaxSel; ++i) sg += (i < p.kseg && k >= i * Ks) ? 1 : 0;
        return sg;
    };
    auto load_w = [&](const T *w0, const T *w1, int k0, uint4 (&wa)[kUnroll], uint4 (&wb)[kUnroll]) {
#pragma unroll
        for (int q = 0; q < kUnroll; ++q) {
            const int k = k0 + q * step + lane * E;
            wa[q] = make_uint4(0, 0, 0, 0);
            wb[q] = make_uint4(0, 0, 0, 0);
            if (k < ke) {
                int64_t off = k;
                if (kSegOk && p.kseg > 1) {
                    // w0 / w1 hold row * Ks; segment sg starts sg * w_seg_stride further
                    const int sg = seg_of(k);
                    off = sg * p.w_seg_stride + (k - sg * Ks);
                }
                wa[q] = ld16_stream(w0 + off);
                wb[q] = ld16_stream(w1 + off);
            }
        }
    };

    // first chunk of the wave's first unit, requested before the norm work
    // (the chunk loop finds it in wa / wb)
    uint4 wa[kUnroll], wb[kUnroll];
    bool have_pf = false;
    if (kNorm && blockIdx.x * upb + slot < p.n_units && kb < ke) {
        int r0, r1, sel;
        unit_rows(blockIdx.x * upb + slot, r0, r1, sel);
        load_w(reinterpret_cast<const T *>(p.W) + (int64_t)r0 * Ks, reinterpret_cast<const T *>(p.W) + (int64_t)r1 * Ks,
               kb, wa, wb);
        have_pf = true;
    }
    if constexpr (kNorm) {
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if (m < p.M) {
                hrow[m] = x_row(p, p.m0 + m);
                inv[m] = row_inv_rms(p, hrow[m]);
            }
        }
        if constexpr (staged) {
            for (int sel = 0; sel < n_sel; ++sel)
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    if (m >= p.M) continue;
                    // members with their own residual rows (parallel MLPs) have their own
                    // RMS (staged operands only: the host sends such products here)
                    const float iv = p.xss_sel_stride ? row_inv_rms(p, hrow[m], sel) : inv[m];
                    for (int k = threadIdx.x * E; k < K; k += 256 * E) {
                        float f[E];
                        if constexpr (E == 8) x_norm8(p, sel, hrow[m], k, iv, f);
                        else x_norm4(p, sel, hrow[m], k, iv, f);
#pragma unroll
                        for (int e = 0; e < E; ++e) xs[(sel * MR + m) * K + k + e] = f[e];
                    }
                }
            __syncthreads();
        }
    }

    for (int ub = blockIdx.x * upb; ub < p.n_units; ub += gridDim.x * upb) {
        const int u = ub + slot;
        const bool active = u < p.n_units;
        float y0 = 0.f, y1 = 0.f;
        int r0 = 0, r1 = 0, sel = 0;
        if (active) {
            unit_rows(u, r0, r1, sel);
            const T *w0 = reinterpret_cast<const T *>(p.W) + (int64_t)r0 * Ks;
            const T *w1 = reinterpret_cast<const T *>(p.W) + (int64_t)r1 * Ks;
            const float *xp = reinterpret_cast<const float *>(p.X) + (int64_t)sel * p.x_sel_stride + (int64_t)p.m0 * Ks;
            const float *xl = xs + (int64_t)sel * MR * K;

            float a0[MR], a1[MR];
#pragma unroll
            for (int m = 0; m < MR; ++m) { a0[m] = 0.f; a1[m] = 0.f; }
            for (int k0 = kb; k0 < ke; k0 += chunk) {
                if (!have_pf) load_w(w0, w1, k0, wa, wb);
                have_pf = false;
                // activation operands of the chunk (zero past the part's end)
                float xo[kUnroll][MR][E];
#pragma unroll
                for (int q = 0; q < kUnroll; ++q) {
                    const int k = k0 + q * step + lane * E;
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
#pragma unroll
                        for (int e = 0; e < E; ++e) xo[q][m][e] = 0.f;
                        if (m >= p.M || k >= ke) continue;
                        if constexpr (staged) {
#pragma unroll
                            for (int e = 0; e < E; e += 4)
                                Store<float>::unpack(*reinterpret_cast<const uint4 *>(xl + m * K + k + e), xo[q][m] + e);
                        } else if constexpr (!kNorm) {
                            int64_t off = (int64_t)m * Ks + k;
                            if (kSegOk && p.kseg > 1) {
                                const int sg = seg_of(k);
                                off = sg * p.x_seg_stride + (int64_t)m * Ks + (k - sg * Ks);
                            }
#pragma unroll
                            for (int e = 0; e < E; e += 4) Store<float>::unpack(ld16(xp + off + e), xo[q][m] + e);
                        } else {
                            if constexpr (E == 8) x_norm8(p, sel, hrow[m], k, inv[m], xo[q][m]);
                            else x_norm4(p, sel, hrow[m], k, inv[m], xo[q][m]);
                        }
                    }
                }
#pragma unroll
                for (int q = 0; q < kUnroll; ++q) {
                    float fa[E], fb[E];
                    S::unpack(wa[q], fa);
                    S::unpack(wb[q], fb);
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
                        if (m < p.M) {
#pragma unroll
                            for (int e = 0; e < E; ++e) {
                                a0[m] = fmaf(fa[e], xo[q][m][e], a0[m]);
                                a1[m] = fmaf(fb[e], xo[q][m][e], a1[m]);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                if (m < p.M) {
                    const float s0 = wave_sum(a0[m]);
                    const float s1 = wave_sum(a1[m]);
                    if (lane == m) { y0 = s0; y1 = s1; }
                }
            }
        }
        if (KS > 1) {
            if (lane < p.M) {
                red[wave][lane][0] = y0;
                red[wave][lane][1] = y1;
            }
            __syncthreads();
            if (part == 0 && lane < p.M) {
                for (int q = 1; q < KS; ++q) {
                    y0 += red[wave + q][lane][0];
                    y1 += red[wave + q][lane][1];
                }
            }
            __syncthreads();
        }
        if (active && part == 0 && lane < p.M) {
            if constexpr (kPair) {
                epi_pair<T, EPI>(p, u, r0, r1, sel, lane, y0, y1);
            } else if constexpr (EPI == EPI_LOGITS) {
                epi_logits2<T>(p, r0, r1, lane, y0, y1, best_v, best_i);
            } else {
                float t = 0.f;
                epi_row<T, EPI>(p, r0, sel, lane, y0, t, best_v, best_i);
                epi_row<T, EPI>(p, r1, sel, lane, y1, t, best_v, best_i);
                if constexpr (epi_has_ss(EPI)) add_sel(ss, (EPI == EPI_ATTN_OUT && p.par_mlp) ? sel : 0, t);
            }
        }
    }

    if constexpr (epi_has_ss(EPI) || EPI == EPI_LOGITS) {
        // block partials: lane m of every wave holds row m's contribution
        // (waves with part > 0 hold neutral values)
        __shared__ float sv[kWaves][kMaxRows];
        __shared__ int si[kWaves][kMaxRows];
        __shared__ float sss[kWaves][kMaxSel][kMaxRows];
        if (lane < p.M) {
            sv[wave][lane] = best_v;
            si[wave][lane] = best_i;
#pragma unroll
            for (int s = 0; s < kMaxSel; ++s) sss[wave][s][lane] = ss[s];
        }
        __syncthreads();
        if (threadIdx.x < p.M) {
            const int m = threadIdx.x;
            if constexpr (EPI == EPI_LOGITS) {
                float v = sv[0][m];
                int i = si[0][m];
                for (int w = 1; w < kWaves; ++w) argmax_merge(v, i, sv[w][m], si[w][m]);
                p.part_val[(int64_t)(p.m0 + m) * gridDim.x + blockIdx.x] = v;
                p.part_idx[(int64_t)(p.m0 + m) * gridDim.x + blockIdx.x] = i;
            } else {
                for (int s = 0; s < p.n_norm_sel; ++s) {
                    float t = sss[0][s][m];
                    for (int w = 1; w < kWaves; ++w) t += sss[w][s][m];
                    p.ss[(int64_t)s * p.ss_sel_stride + (int64_t)(p.m0 + m) * gridDim.x + blockIdx.x] = t;
                }
            }
        }
    }
}

// LDS bytes of the staged operand rows (every set member's MR rows of K floats)
int64_t gemv_stage_bytes(const GemvParams &p) {
    const int mr = p.M <= 1 ? 1 : (p.M <= 2 ? 2 : (p.M <= 4 ? 4 : 8));
    const int64_t n_sel = (int64_t)p.n_units * 2 / p.rows_per_sel;
    return n_sel * mr * p.K * 4;
}

// normalised (float32) operands go through LDS when every set member's rows fit
bool gemv_staged(const GemvParams &p) { return gemv_stage_bytes(p) <= kStageBytes; }

template <typename T, int EPI, int XM>
void launch_tex(const GemvParams &p, int grid, int ks, hipStream_t s) {
    dim3 g(grid), b(256);
    const size_t lds = XM == XM_STAGED ? (size_t)gemv_stage_bytes(p) : 0;
    if (p.M <= 1) hipLaunchKernelGGL((k_gemv<T, 1, EPI, XM>), g, b, lds, s, p, ks);
    else if (p.M <= 2) hipLaunchKernelGGL((k_gemv<T, 2, EPI, XM>), g, b, lds, s, p, ks);
    else if (p.M <= 4) hipLaunchKernelGGL((k_gemv<T, 4, EPI, XM>), g, b, lds, s, p, ks);
    else hipLaunchKernelGGL((k_gemv<T, 8, EPI, XM>), g, b, lds, s, p, ks);
}

template <typename T, int EPI>
void launch_ten(const GemvParams &p, int grid, int ks, bool norm, hipStream_t s) {
    if (!norm) launch_tex<T, EPI, XM_PLAIN>(p, grid, ks, s);
    else if (gemv_staged(p)) launch_tex<T, EPI, XM_STAGED>(p, grid, ks, s);
    else launch_tex<T, EPI, XM_DIRECT>(p, grid, ks, s);
}

// The decoder's products: QKV, gate/up and the head read normalised
// residual rows, the others plain activation rows.
template <typename T>
hipError_t launch_t(const GemvParams &p, int grid, int ks, hipStream_t s) {
    const bool nrm = p.xmode == X_NORM;
    switch (p.epi) {
    case EPI_STORE:
        launch_ten<T, EPI_STORE>(p, grid, ks, nrm, s);
        break;
    case EPI_QKV_ROPE:
        launch_ten<T, EPI_QKV_ROPE>(p, grid, ks, nrm, s);
        break;
    case EPI_SILU_MUL:
        launch_ten<T, EPI_SILU_MUL>(p, grid, ks, nrm, s);
        break;
    case EPI_RESID_ADD:
        if (nrm) return hipErrorInvalidValue;
        if (p.kseg > 1) launch_tex<T, EPI_RESID_ADD, XM_SEG>(p, grid, ks, s);
        else launch_tex<T, EPI_RESID_ADD, XM_PLAIN>(p, grid, ks, s);
        break;
    case EPI_LOGITS:
        launch_ten<T, EPI_LOGITS>(p, grid, ks, nrm, s);
        break;
    case EPI_ATTN_OUT:
        if (nrm) return hipErrorInvalidValue;
        launch_tex<T, EPI_ATTN_OUT, XM_PLAIN>(p, grid, ks, s);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------ norm
// Normalised float32 activations for the matrix-core products:
// xn[sel][m][k] = gain_sel[k] * (xh[hrow][k] + xadd[sel][hrow][k]) / rms(hrow),
// rms from the row's sum-of-squares partials (summed in block order by every
// wave, so all blocks agree bit for bit).  Grid (K / 2048, M, n_sel).  The
// row's values and gains are requested before the partials, so the two
// memory round trips overlap (same arithmetic as x_norm8).
template <typename T>
__global__ __launch_bounds__(256) void k_norm_rows(GemvParams p, void *xn, int packed) {
    const int m = blockIdx.y, sel = blockIdx.z;
    const int hrow = x_row(p, p.m0 + m);
    const int k = (blockIdx.x * 256 + threadIdx.x) * 8;
    const bool live = k < p.K;
    float4 h0 = make_float4(0.f, 0.f, 0.f, 0.f), h1 = h0, a0 = h0, a1 = h0, g0 = h0, g1 = h0;
    if (live) {
        const float *h = p.xh + (int64_t)hrow * p.K + k;
        const float *g = p.xgain + (int64_t)sel * p.xgain_stride + k;
        h0 = *reinterpret_cast<const float4 *>(h);
        h1 = *reinterpret_cast<const float4 *>(h + 4);
        g0 = *reinterpret_cast<const float4 *>(g);
        g1 = *reinterpret_cast<const float4 *>(g + 4);
        if (p.xadd) {
            const float *a = p.xadd + (int64_t)sel * p.xadd_sel_stride + (int64_t)hrow * p.K + k;
            a0 = *reinterpret_cast<const float4 *>(a);
            a1 = *reinterpret_cast<const float4 *>(a + 4);
        }
    }
    const float inv = row_inv_rms(p, hrow, sel);   // whole wave
    if (!live) return;
    if (p.xadd) {
        h0.x += a0.x; h0.y += a0.y; h0.z += a0.z; h0.w += a0.w;
        h1.x += a1.x; h1.y += a1.y; h1.z += a1.z; h1.w += a1.w;
    }
    const float f[8] = {h0.x * inv * g0.x, h0.y * inv * g0.y, h0.z * inv * g0.z, h0.w * inv * g0.w,
                        h1.x * inv * g1.x, h1.y * inv * g1.y, h1.z * inv * g1.z, h1.w * inv * g1.w};
    if (packed) {
        // packed operand rows of the skinny matrix-core kernel (m0 = 0)
        uint16_t hs[8], ls[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) split2_one(f[e], hs[e], ls[e]);
        uint4 hv, lv;
        __builtin_memcpy(&hv, hs, 16);
        __builtin_memcpy(&lv, ls, 16);
        uint16_t *o = reinterpret_cast<uint16_t *>(xn) + ((int64_t)sel * packed + m) * p.K + k;
        *reinterpret_cast<uint4 *>(o) = hv;
        *reinterpret_cast<uint4 *>(o + (int64_t)(packed / 2) * p.K) = lv;
        return;
    }
    float4 *o = reinterpret_cast<float4 *>(reinterpret_cast<float *>(xn) + ((int64_t)sel * p.Mtot + p.m0 + m) * p.K + k);
    o[0] = make_float4(f[0], f[1], f[2], f[3]);
    o[1] = make_float4(f[4], f[5], f[6], f[7]);
}

// ------------------------------------------------------------------ sampling
__global__ __launch_bounds__(256) void k_sample_reduce(const float *pv, const int32_t *pi, int n, int32_t *out,
                                                       int stride) {
    __shared__ float sv[kWaves];
    __shared__ int si[kWaves];
    const int m = blockIdx.x;
    float v = -INFINITY;
    int i = 0x7FFFFFFF;
    for (int j = threadIdx.x; j < n; j += blockDim.x) argmax_merge(v, i, pv[(int64_t)m * n + j], pi[(int64_t)m * n + j]);
    wave_argmax(v, i);
    if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = v; si[threadIdx.x >> 6] = i; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kWaves; ++w) argmax_merge(sv[0], si[0], sv[w], si[w]);
        out[(int64_t)m * stride] = si[0];
    }
}

// ------------------------------------------------------------------ embed
template <typename T>
__global__ __launch_bounds__(256) void k_embed(EmbedParams p) {
    __shared__ float red[kWaves];
    const int m = blockIdx.x;
    const int mseq = p.rows.mseq;
    const int b = m / mseq, i = m - b * mseq;
    int tok = p.tokens[(int64_t)b * p.tok_ld + (int64_t)i * p.tok_step];
    tok = tok < 0 ? 0 : (tok >= p.vocab ? p.vocab - 1 : tok);
    const T *e = reinterpret_cast<const T *>(p.E) + (int64_t)tok * p.d;
    float *o = p.h + (int64_t)m * p.d;
    float ss = 0.f;
    for (int j = threadIdx.x; j < p.d; j += 256) {
        const float v = Store<T>::to_f32(e[j]);
        o[j] = v;
        ss = fmaf(v, v, ss);
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    // RoPE table of this row's position: angle pos * theta^(-2j/hd) formed and
    // reduced modulo 2 pi in double precision, then sin / cos in float32
    int pos = p.rows.start_pos[b] + i;
    if (pos < 0 || pos >= p.rows.capacity) pos = 0;
    const int half = p.hd / 2;
    for (int j = threadIdx.x; j < half; j += 256) {
        const double inv_freq = pow((double)p.rope_theta, -2.0 * (double)j / (double)p.hd);
        double ang = (double)pos * inv_freq;
        const double two_pi = 6.283185307179586476925286766559;
        ang -= two_pi * rint(ang / two_pi);
        float sn, cs;
        sincosf((float)ang, &sn, &cs);
        p.rope_cs[(int64_t)m * half + j] = make_float2(cs, sn);
    }
    __syncthreads();
    if (threadIdx.x == 0) p.ss[m] = red[0] + red[1] + red[2] + red[3];
}

}  // namespace

int gemv_max_rows() { return kMaxRows; }

int env_splits(const char *name) {
    const char *e = getenv(name);
    const int n = e ? atoi(e) : 0;
    return (n == 1 || n == 2 || n == 4) ? n : 0;
}

// Workgroups per CU of the normalised-operand products other than the head
// (SPEC_GEMV_NORM_WG overrides, 1 .. 8).
int norm_wg_per_cu() {
    static const int v = [] {
        const char *e = getenv("SPEC_GEMV_NORM_WG");
        const int n = e ? atoi(e) : 4;
        return n < 1 ? 1 : (n > 8 ? 8 : n);
    }();
    return v;
}

// Waves per unit.  Normalised-operand products other than the head: one wave
// per unit over the whole of K (measured on the 1B draft step, one row: the
// QKV launches of one and two layers, 1536 / 3072 units, took 12.4 us on
// average with two or four waves per unit, which leaves a second round of
// units for half the workgroups, and 10.8 us with one; the draft step went
// from 741 to 727 us; the gate/up product already had one).  Plain-operand
// products split K in two while the launch has fewer than 4096 waves and each
// part keeps at least one 16-byte step per lane (four-way splits of the
// one-row down and O products: draft step 724-728 us, two-way 717-721 us);
// the head as long as both hold and the split is at most four.
// SPEC_GEMV_KS / SPEC_GEMV_KS_PLAIN (1, 2 or 4) fix the split of the
// normalised / plain-operand products.
int gemv_splits(const GemvParams &p, int elem_bytes) {
    const int step = kWave * 16 / elem_bytes;
    const bool norm = p.xmode == X_NORM && p.epi != EPI_LOGITS;
    static const int forced_norm = env_splits("SPEC_GEMV_KS");
    static const int forced_plain = env_splits("SPEC_GEMV_KS_PLAIN");
    if (norm) return forced_norm ? forced_norm : 1;
    if (p.xmode != X_NORM && forced_plain) return forced_plain;
    const int ks_max = p.xmode != X_NORM ? 2 : kWaves;
    int ks = 1;
    while (ks < ks_max && (int64_t)p.n_units * ks < 4096 && p.K >= 2 * ks * step) ks *= 2;
    return ks;
}

// Workgroups: every unit once, at most kMaxGrid; normalised-operand launches
// keep three or four workgroups per CU so that each stages its operand once
// for several units.
int gemv_grid(const GemvParams &p, int ks) {
    const int upb = kWaves / ks;
    int g = (p.n_units + upb - 1) / upb;
    // measured at one row (1B draft): four workgroups per CU for the QKV and
    // gate/up products (11.9 / 16.9 us against 12.3 / 17.5 with three; with
    // one wave per unit, draft step 727 us against 749 with three, 773 with
    // six and 772 with eight, whose second dispatch round the 116-VGPR
    // gate/up kernel cannot hold resident), three for the sampling head (84.6
    // us against 100.6 with four)
    const int cap = p.xmode != X_NORM ? kMaxGrid : (p.epi == EPI_LOGITS ? 3 * 256 : norm_wg_per_cu() * 256);
    return g < cap ? (g < 1 ? 1 : g) : cap;
}

int gemv_operand_mode(int dtype, const GemvParams &p) {
    (void)dtype;
    if (p.xmode != X_NORM) return p.kseg > 1 ? XM_SEG : XM_PLAIN;
    return gemv_staged(p) ? XM_STAGED : XM_DIRECT;
}

hipError_t launch_gemv(int dtype, const GemvParams &p, int grid, int ks, hipStream_t s) {
    if (ks != 1 && ks != 2 && ks != 4) return hipErrorInvalidValue;
    return dtype ? launch_t<uint16_t>(p, grid, ks, s) : launch_t<float>(p, grid, ks, s);
}

hipError_t launch_norm_rows(int dtype, const GemvParams &p, int n_sel, void *xn, int packed, hipStream_t s) {
    if (packed && (p.m0 != 0 || 2 * p.M > packed || p.K % 8)) return hipErrorInvalidValue;
    dim3 grid((p.K + 2047) / 2048, p.M, n_sel);
    if (dtype) hipLaunchKernelGGL(k_norm_rows<uint16_t>, grid, dim3(256), 0, s, p, xn, packed);
    else hipLaunchKernelGGL(k_norm_rows<float>, grid, dim3(256), 0, s, p, xn, packed);
    return hipGetLastError();
}

// cos(x[r], y[r] - a[r]) over d elements of row r (a nullable), fixed
// summation order: thread strides, then the waves in order.
__global__ __launch_bounds__(256) void k_cosine(const float *x, const float *y, const float *a, int d, float *out,
                                                int64_t out_stride) {
    __shared__ float part[kWaves][3];
    const int r = blockIdx.x;
    const float *xr = x + (int64_t)r * d, *yr = y + (int64_t)r * d;
    const float *ar = a ? a + (int64_t)r * d : nullptr;
    float xy = 0.f, xx = 0.f, yy = 0.f;
    for (int k = threadIdx.x; k < d; k += 256) {
        const float u = xr[k], v = ar ? yr[k] - ar[k] : yr[k];
        xy = fmaf(u, v, xy);
        xx = fmaf(u, u, xx);
        yy = fmaf(v, v, yy);
    }
    xy = wave_sum(xy);
    xx = wave_sum(xx);
    yy = wave_sum(yy);
    if ((threadIdx.x & 63) == 0) {
        part[threadIdx.x >> 6][0] = xy;
        part[threadIdx.x >> 6][1] = xx;
        part[threadIdx.x >> 6][2] = yy;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        xy = part[0][0];
        xx = part[0][1];
        yy = part[0][2];
        for (int w = 1; w < kWaves; ++w) {
            xy += part[w][0];
            xx += part[w][1];
            yy += part[w][2];
        }
        const float den = sqrtf(xx) * sqrtf(yy);
        out[(int64_t)r * out_stride] = den > 0.f ? xy / den : 0.f;
    }
}

hipError_t launch_cosine(const float *x, const float *y, const float *a, int rows, int d, float *out,
                         int64_t out_stride, hipStream_t s) {
    hipLaunchKernelGGL(k_cosine, dim3(rows), dim3(256), 0, s, x, y, a, d, out, out_stride);
    return hipGetLastError();
}

hipError_t launch_sample_reduce(const float *pv, const int32_t *pi, int n, int M, int32_t *out, int stride,
                                hipStream_t s) {
    hipLaunchKernelGGL(k_sample_reduce, dim3(M), dim3(256), 0, s, pv, pi, n, out, stride);
    return hipGetLastError();
}

hipError_t launch_embed(int dtype, const EmbedParams &p, int Mtot, hipStream_t s) {
    if (dtype) hipLaunchKernelGGL(k_embed<uint16_t>, dim3(Mtot), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(k_embed<float>, dim3(Mtot), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace spec
