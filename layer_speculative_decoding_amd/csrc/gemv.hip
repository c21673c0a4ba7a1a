// Weight-streaming matrix-vector products for few activation rows, with the
// epilogues of the decoder fused in (QKV + RoPE + KV append, SiLU-gate,
// residual add, logits + sampling partials), plus RMSNorm and embedding.
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

template <typename T, int MR>
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

    for (int u = blockIdx.x * kWaves + wave; u < p.n_units; u += gridDim.x * kWaves) {
        const int blk = u / half;
        const int j = u - blk * half;
        const int r0 = blk * p.pair_block + j;
        const int r1 = r0 + half;
        const int sel = r0 / p.rows_per_sel;
        const T *w0 = reinterpret_cast<const T *>(p.W) + (int64_t)r0 * K;
        const T *w1 = reinterpret_cast<const T *>(p.W) + (int64_t)r1 * K;
        const T *x = reinterpret_cast<const T *>(p.X) + (int64_t)sel * p.x_sel_stride + (int64_t)p.m0 * K;
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
                        S::unpack(ld16(x + (int64_t)m * K + k + q * step), fx);
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
                    S::unpack(ld16(x + (int64_t)m * K + k), fx);
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
        if (lane < p.M) epilogue<T>(p, u, r0, r1, sel, lane, y0, y1, best_v, best_i);
    }

    if (p.epi == EPI_LOGITS) {
        // per-workgroup arg-max of each sampling row; lane m holds row m
        __shared__ float sv[kWaves][kMaxRows];
        __shared__ int si[kWaves][kMaxRows];
        if (lane < p.M) { sv[wave][lane] = best_v; si[wave][lane] = best_i; }
        __syncthreads();
        if (threadIdx.x < p.M) {
            float v = sv[0][threadIdx.x];
            int i = si[0][threadIdx.x];
            for (int w = 1; w < kWaves; ++w) argmax_merge(v, i, sv[w][threadIdx.x], si[w][threadIdx.x]);
            p.part_val[(int64_t)(p.m0 + threadIdx.x) * gridDim.x + blockIdx.x] = v;
            p.part_idx[(int64_t)(p.m0 + threadIdx.x) * gridDim.x + blockIdx.x] = i;
        }
    }
}

template <typename T>
hipError_t launch_t(const GemvParams &p, int grid, hipStream_t s) {
    dim3 g(grid), b(256);
    if (p.M <= 1) hipLaunchKernelGGL((k_gemv<T, 1>), g, b, 0, s, p);
    else if (p.M <= 2) hipLaunchKernelGGL((k_gemv<T, 2>), g, b, 0, s, p);
    else if (p.M <= 4) hipLaunchKernelGGL((k_gemv<T, 4>), g, b, 0, s, p);
    else hipLaunchKernelGGL((k_gemv<T, 8>), g, b, 0, s, p);
    return hipGetLastError();
}

// ------------------------------------------------------------------ norm
template <typename T>
__global__ __launch_bounds__(256) void k_norm(NormParams p) {
    extern __shared__ float src[];
    __shared__ float red[kWaves];
    const int m = blockIdx.x;
    const int d = p.d;
    int in_row = m;
    if (p.gather_mseq > 0) {
        int nt = p.gather_ntok ? p.gather_ntok[m] : p.gather_mseq;
        nt = nt < 1 ? 1 : (nt > p.gather_mseq ? p.gather_mseq : nt);
        in_row = m * p.gather_mseq + nt - 1;
    }
    float *h = p.h + (int64_t)in_row * d;
    const float *add = p.add ? p.add + (int64_t)in_row * d : nullptr;
    const float *s0 = p.src0 ? p.src0 + (int64_t)in_row * d : nullptr;
    float ss = 0.f;
    for (int j = threadIdx.x; j < d; j += 256) {
        const float hv = h[j];
        float v = hv;
        if (add) {
            v = hv + add[j];
            if (p.gather_mseq == 0) h[j] = v;
        }
        if (p.h0copy) p.h0copy[(int64_t)in_row * d + j] = hv;
        const float sv = s0 ? s0[j] + add[j] : v;
        src[j] = sv;
        ss = fmaf(sv, sv, ss);
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = red[0] + red[1] + red[2] + red[3];
    const float inv = 1.0f / sqrtf(tot / (float)d + p.eps);
    for (int g = 0; g < p.n_gains; ++g) {
        const float *gain = p.gains + (int64_t)g * p.gain_stride;
        T *o = reinterpret_cast<T *>(p.xn) + (int64_t)g * p.xn_sel_stride + (int64_t)m * d;
        for (int j = threadIdx.x; j < d; j += 256) o[j] = Store<T>::from_f32(src[j] * inv * gain[j]);
    }
}

template <typename T>
__global__ __launch_bounds__(256) void k_embed(const T *E, int vocab, int d, const int32_t *tokens,
                                               int64_t tok_ld, int tok_step, int mseq, float *h) {
    const int m = blockIdx.x;
    const int b = m / mseq, i = m - b * mseq;
    int tok = tokens[(int64_t)b * tok_ld + (int64_t)i * tok_step];
    tok = tok < 0 ? 0 : (tok >= vocab ? vocab - 1 : tok);
    const T *e = E + (int64_t)tok * d;
    float *o = h + (int64_t)m * d;
    for (int j = threadIdx.x; j < d; j += 256) o[j] = Store<T>::to_f32(e[j]);
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

hipError_t launch_norm(int dtype, const NormParams &p, hipStream_t s) {
    const size_t lds = (size_t)p.d * sizeof(float);
    if (dtype) hipLaunchKernelGGL(k_norm<uint16_t>, dim3(p.M), dim3(256), lds, s, p);
    else hipLaunchKernelGGL(k_norm<float>, dim3(p.M), dim3(256), lds, s, p);
    return hipGetLastError();
}

hipError_t launch_embed(int dtype, const void *E, int vocab, int d, const int32_t *tokens,
                        int64_t tok_ld, int tok_step, int B, int mseq, float *h, hipStream_t s) {
    if (dtype)
        hipLaunchKernelGGL(k_embed<uint16_t>, dim3(B * mseq), dim3(256), 0, s,
                           reinterpret_cast<const uint16_t *>(E), vocab, d, tokens, tok_ld, tok_step, mseq, h);
    else
        hipLaunchKernelGGL(k_embed<float>, dim3(B * mseq), dim3(256), 0, s,
                           reinterpret_cast<const float *>(E), vocab, d, tokens, tok_ld, tok_step, mseq, h);
    return hipGetLastError();
}

}  // namespace spec
