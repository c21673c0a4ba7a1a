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
#include "epilogue.h"
#include "spec_device.h"
#include "spec_kernels.h"

namespace spec {

namespace {

constexpr int kWaves = 4;          // waves per workgroup
constexpr int kMaxRows = 8;        // activation rows per launch
constexpr int kMaxGrid = 256 * 8;  // workgroups (8 per CU)
constexpr int kUnroll = 4;

template <typename T, int E>
__device__ __forceinline__ void load_x(const GemvParams &p, const T *xplain, int sel, int m, int hrow, float inv,
                                       int k, float *fx) {
    if (p.xmode == X_PLAIN) {
        Store<T>::unpack(ld16(xplain + (int64_t)m * p.K + k), fx);
    } else {
        if constexpr (E == 8) x_norm8(p, sel, hrow, k, inv, fx);
        else x_norm4(p, sel, hrow, k, inv, fx);
#pragma unroll
        for (int e = 0; e < E; ++e) fx[e] = Store<T>::round(fx[e]);
    }
}

template <typename T, int MR, bool kLogits>
__global__ __launch_bounds__(256) void k_gemv(GemvParams p) {
    using S = Store<T>;
    constexpr int E = S::kPer16;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int K = p.K;
    const int step = kWave * E;
    const int half = p.pair_block >> 1;
    float best_v = -INFINITY;
    int best_i = 0x7FFFFFFF;
    float ss[kMaxSel];
#pragma unroll
    for (int s = 0; s < kMaxSel; ++s) ss[s] = 0.f;
    __shared__ float inv_s[kMaxRows];
    block_inv_rms(p, inv_s);

    for (int u = blockIdx.x * kWaves + wave; u < p.n_units; u += gridDim.x * kWaves) {
        const int blk = u / half;
        const int j = u - blk * half;
        const int r0 = blk * p.pair_block + j;
        const int r1 = r0 + half;
        const int sel = r0 / p.rows_per_sel;
        const T *w0 = reinterpret_cast<const T *>(p.W) + (int64_t)r0 * K;
        const T *w1 = reinterpret_cast<const T *>(p.W) + (int64_t)r1 * K;
        const T *xp = reinterpret_cast<const T *>(p.X) + (int64_t)sel * p.x_sel_stride + (int64_t)p.m0 * K;
        int hrow[MR];
        float inv[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            hrow[m] = 0;
            inv[m] = 0.f;
            if (p.xmode == X_NORM && m < p.M) {
                hrow[m] = x_row(p, p.m0 + m);
                inv[m] = inv_s[m];
            }
        }
        float a0[MR], a1[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) { a0[m] = 0.f; a1[m] = 0.f; }

        int k = lane * E;
        for (; k + (kUnroll - 1) * step < K; k += kUnroll * step) {
            uint4 wa[kUnroll], wb[kUnroll];
#pragma unroll
            for (int q = 0; q < kUnroll; ++q) {
                wa[q] = ld16_stream(w0 + k + q * step);
                wb[q] = ld16_stream(w1 + k + q * step);
            }
#pragma unroll
            for (int q = 0; q < kUnroll; ++q) {
                float fa[E], fb[E];
                S::unpack(wa[q], fa);
                S::unpack(wb[q], fb);
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    if (m < p.M) {
                        float fx[E];
                        load_x<T, E>(p, xp, sel, m, hrow[m], inv[m], k + q * step, fx);
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            a0[m] = fmaf(fa[e], fx[e], a0[m]);
                            a1[m] = fmaf(fb[e], fx[e], a1[m]);
                        }
                    }
                }
            }
        }
        for (; k < K; k += step) {
            float fa[E], fb[E];
            S::unpack(ld16_stream(w0 + k), fa);
            S::unpack(ld16_stream(w1 + k), fb);
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                if (m < p.M) {
                    float fx[E];
                    load_x<T, E>(p, xp, sel, m, hrow[m], inv[m], k, fx);
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        a0[m] = fmaf(fa[e], fx[e], a0[m]);
                        a1[m] = fmaf(fb[e], fx[e], a1[m]);
                    }
                }
            }
        }
        float y0 = 0.f, y1 = 0.f;
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if (m < p.M) {
                const float s0 = wave_sum(a0[m]);
                const float s1 = wave_sum(a1[m]);
                if (lane == m) { y0 = s0; y1 = s1; }
            }
        }
        if (lane < p.M) epilogue<T, kLogits>(p, u, r0, r1, sel, lane, y0, y1, best_v, best_i, ss);
    }

    const bool norm = p.n_norm_sel > 0;
    const bool logits = p.epi == EPI_LOGITS;
    if (!norm && !logits) return;
    // block partials: lane m of every wave holds row m's contribution
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
        if (logits) {
            float v = sv[0][m];
            int i = si[0][m];
            for (int w = 1; w < kWaves; ++w) argmax_merge(v, i, sv[w][m], si[w][m]);
            p.part_val[(int64_t)(p.m0 + m) * gridDim.x + blockIdx.x] = v;
            p.part_idx[(int64_t)(p.m0 + m) * gridDim.x + blockIdx.x] = i;
        }
        for (int s = 0; s < p.n_norm_sel; ++s) {
            float t = sss[0][s][m];
            for (int w = 1; w < kWaves; ++w) t += sss[w][s][m];
            p.ss[(int64_t)s * p.ss_sel_stride + (int64_t)(p.m0 + m) * gridDim.x + blockIdx.x] = t;
        }
    }
}

template <typename T, bool kLogits>
hipError_t launch_tl(const GemvParams &p, int grid, hipStream_t s) {
    dim3 g(grid), b(256);
    if (p.M <= 1) hipLaunchKernelGGL((k_gemv<T, 1, kLogits>), g, b, 0, s, p);
    else if (p.M <= 2) hipLaunchKernelGGL((k_gemv<T, 2, kLogits>), g, b, 0, s, p);
    else if (p.M <= 4) hipLaunchKernelGGL((k_gemv<T, 4, kLogits>), g, b, 0, s, p);
    else hipLaunchKernelGGL((k_gemv<T, 8, kLogits>), g, b, 0, s, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const GemvParams &p, int grid, hipStream_t s) {
    return p.epi == EPI_LOGITS ? launch_tl<T, true>(p, grid, s) : launch_tl<T, false>(p, grid, s);
}

// ------------------------------------------------------------------ norm
// Normalised activations for the matrix-core products:
// xn[sel][m][k] = round(gain_sel[k] * (xh[hrow][k] + xadd[sel][hrow][k]) / rms(hrow)),
// rms from the row's sum-of-squares partials (summed in block order by every
// wave, so all blocks agree bit for bit).  Grid (K / 2048, M, n_sel).
template <typename T>
__global__ __launch_bounds__(256) void k_norm_rows(GemvParams p, void *xn) {
    const int m = blockIdx.y, sel = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int hrow = x_row(p, p.m0 + m);
    const float *src = p.xss + (int64_t)hrow * p.xnparts;
    float s = 0.f;
    for (int i = lane; i < p.xnparts; i += 64) s += src[i];
    s = wave_sum(s);
    const float inv = 1.0f / sqrtf(s / (float)p.K + p.eps);
    const int k = (blockIdx.x * 256 + threadIdx.x) * 8;
    if (k >= p.K) return;
    float f[8];
    x_norm8(p, sel, hrow, k, inv, f);
    T *o = reinterpret_cast<T *>(xn) + ((int64_t)sel * p.Mtot + p.m0 + m) * p.K + k;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = Store<T>::from_f32(f[e]);
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

int gemv_grid(int n_units) {
    int g = (n_units + kWaves - 1) / kWaves;
    return g < kMaxGrid ? (g < 1 ? 1 : g) : kMaxGrid;
}

hipError_t launch_gemv(int dtype, const GemvParams &p, int grid, hipStream_t s) {
    return dtype ? launch_t<uint16_t>(p, grid, s) : launch_t<float>(p, grid, s);
}

hipError_t launch_norm_rows(int dtype, const GemvParams &p, int n_sel, void *xn, hipStream_t s) {
    dim3 grid((p.K + 2047) / 2048, p.M, n_sel);
    if (dtype) hipLaunchKernelGGL(k_norm_rows<uint16_t>, grid, dim3(256), 0, s, p, xn);
    else hipLaunchKernelGGL(k_norm_rows<float>, grid, dim3(256), 0, s, p, xn);
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
