// The fused speculative accept / resample over the vocabulary.
//
// Accept / resample follows the speculative sampling rule (Leviathan et al.;
// Chen et al.; the EasySpec pages cite both and require the base distribution
// to be preserved).  Three launches, all reductions in a fixed order:
//   k_acc_stats    per (vocab chunk, row, sequence): max, sum of exp and the
//                  first arg-max of the 2k+1 logit rows (scaled by 1/T)
//   k_acc_decide   per (chunk, sequence): merge the row statistics, run the
//                  accept chain for j = 1..k, then the chunk's Gumbel arg-max
//                  of the residual max(0, p_j - q_j) (and of p_j, the fallback)
//                  or of the bonus row p_{k+1}
//   k_acc_final    per sequence: merge the chunk candidates, write outputs
#include "spec_device.h"
#include "spec_kernels.h"

namespace spec {

namespace {

constexpr int kChunk = 8192;   // vocab entries per workgroup
constexpr int kThreads = 256;

__device__ __forceinline__ void block_argmax(float &v, int &i) {
    __shared__ float sv[4];
    __shared__ int si[4];
    wave_argmax(v, i);
    if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = v; si[threadIdx.x >> 6] = i; }
    __syncthreads();
    v = sv[0]; i = si[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) argmax_merge(v, i, sv[w], si[w]);
    __syncthreads();
}

__device__ __forceinline__ const float *acc_row(const AcceptParams &p, int b, int r) {
    // rows 0..k: base rows p_1..p_{k+1}; rows k+1..2k: draft rows q_1..q_k
    if (r <= p.k) return p.p_logits + ((int64_t)b * (p.k + 1) + r) * p.vocab;
    return p.q_logits + ((int64_t)b * p.k + (r - p.k - 1)) * p.vocab;
}

__global__ __launch_bounds__(256) void k_acc_stats(AcceptParams p) {
    const int c = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
    const float *z = acc_row(p, b, r);
    const int v0 = c * kChunk, v1 = min(p.vocab, v0 + kChunk);
    const float sc = p.inv_temp == 0.0f ? 1.0f : p.inv_temp;
    float mx = -INFINITY;
    int ix = 0x7FFFFFFF;
    for (int v = v0 + threadIdx.x; v < v1; v += kThreads) argmax_merge(mx, ix, z[v] * sc, v);
    block_argmax(mx, ix);
    float sum = 0.f;
    if (p.inv_temp != 0.0f)
        for (int v = v0 + threadIdx.x; v < v1; v += kThreads) sum += expf(z[v] * sc - mx);
    sum = wave_sum(sum);
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sum;
    __syncthreads();
    if (threadIdx.x == 0) {
        const int64_t o = ((int64_t)b * (2 * p.k + 1) + r) * p.nchunk + c;
        p.stats[o * 2 + 0] = mx;
        p.stats[o * 2 + 1] = red[0] + red[1] + red[2] + red[3];
        p.stats_idx[o] = ix;
    }
}

// Merge the chunk statistics of row r: log-sum-exp of z/T and first arg-max.
__device__ void row_merge(const AcceptParams &p, int b, int r, float &lse, int &amax) {
    const int64_t o = ((int64_t)b * (2 * p.k + 1) + r) * p.nchunk;
    float mx = -INFINITY;
    int ix = 0x7FFFFFFF;
    for (int c = 0; c < p.nchunk; ++c) argmax_merge(mx, ix, p.stats[(o + c) * 2], p.stats_idx[o + c]);
    float s = 0.f;
    for (int c = 0; c < p.nchunk; ++c) s += p.stats[(o + c) * 2 + 1] * expf(p.stats[(o + c) * 2] - mx);
    lse = mx + logf(s);
    amax = ix;
}

__global__ __launch_bounds__(256) void k_acc_decide(AcceptParams p) {
    const int c = blockIdx.x, b = blockIdx.y;
    const int k = p.k;
    __shared__ float lse_s[2 * 64 + 1];
    __shared__ int amax_s[2 * 64 + 1];
    __shared__ int dec_a, dec_mode;   // mode 0: bonus row k+1, 1: residual row a+1
    const int nrow = (p.inv_temp == 0.0f) ? k + 1 : 2 * k + 1;
    for (int r = threadIdx.x; r < nrow; r += blockDim.x) row_merge(p, b, r, lse_s[r], amax_s[r]);
    __syncthreads();
    if (threadIdx.x == 0) {
        const int t = p.round_pos[b];
        int a = k;
        for (int j = 1; j <= k; ++j) {
            int d = p.drafts[(int64_t)b * p.draft_stride + j - 1];
            d = d < 0 ? 0 : (d >= p.vocab ? p.vocab - 1 : d);
            bool ok;
            if (p.inv_temp == 0.0f) {
                ok = d == amax_s[j - 1];
            } else {
                const float pz = acc_row(p, b, j - 1)[d] * p.inv_temp;
                const float qz = acc_row(p, b, k + j)[d] * p.inv_temp;
                const float pd = expf(pz - lse_s[j - 1]);
                const float qd = expf(qz - lse_s[k + j]);
                const float u = accept_uniform(p.seed, (uint32_t)b, (uint32_t)(t + j));
                ok = u * qd < pd;
            }
            if (!ok) { a = j - 1; break; }
        }
        dec_a = a;
        dec_mode = (a < k && p.inv_temp != 0.0f) ? 1 : 0;
        if (c == 0) {
            p.decision[b * 2 + 0] = a;
            p.decision[b * 2 + 1] = dec_mode;
        }
    }
    __syncthreads();
    if (p.inv_temp == 0.0f) return;   // greedy: y is the arg-max of row a+1
    const int a = dec_a;
    const int t = p.round_pos[b];
    const uint32_t pos = (uint32_t)(t + a + 1);
    const float *zp = acc_row(p, b, a);
    const float lp = lse_s[a];
    const float *zq = dec_mode ? acc_row(p, b, k + 1 + a) : nullptr;
    const float lq = dec_mode ? lse_s[k + 1 + a] : 0.f;
    const int v0 = c * kChunk, v1 = min(p.vocab, v0 + kChunk);
    float bv = -INFINITY, fv = -INFINITY;   // residual / plain-p candidates
    int bi = 0x7FFFFFFF, fi = 0x7FFFFFFF;
    for (int v4 = v0 + threadIdx.x * 4; v4 < v1; v4 += kThreads * 4) {
        float g[4];
        gumbel4(p.seed, (uint32_t)b, pos, kTarget, (uint32_t)(v4 >> 2), g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int v = v4 + e;
            if (v >= v1) break;
            const float sp = zp[v] * p.inv_temp;
            argmax_merge(fv, fi, sp + g[e], v);
            if (dec_mode) {
                const float diff = expf(sp - lp) - expf(zq[v] * p.inv_temp - lq);
                if (diff > 0.f) argmax_merge(bv, bi, logf(diff) + g[e], v);
            }
        }
    }
    block_argmax(bv, bi);
    block_argmax(fv, fi);
    if (threadIdx.x == 0) {
        const int64_t o = ((int64_t)b * p.nchunk + c) * 2;
        p.cand_val[o + 0] = bv; p.cand_idx[o + 0] = bi;
        p.cand_val[o + 1] = fv; p.cand_idx[o + 1] = fi;
    }
}

__global__ __launch_bounds__(64) void k_acc_final(AcceptParams p) {
    const int b = blockIdx.x;
    if (threadIdx.x != 0) return;
    const int a = p.decision[b * 2 + 0];
    const int mode = p.decision[b * 2 + 1];
    int y;
    if (p.inv_temp == 0.0f) {
        float lse;
        row_merge(p, b, a, lse, y);
    } else {
        float rv = -INFINITY, fv = -INFINITY;
        int ri = 0x7FFFFFFF, fi = 0x7FFFFFFF;
        for (int c = 0; c < p.nchunk; ++c) {
            const int64_t o = ((int64_t)b * p.nchunk + c) * 2;
            argmax_merge(rv, ri, p.cand_val[o], p.cand_idx[o]);
            argmax_merge(fv, fi, p.cand_val[o + 1], p.cand_idx[o + 1]);
        }
        y = (mode == 1 && rv != -INFINITY) ? ri : fi;
    }
    p.n_acc_out[b] = a;
    p.next_out[(int64_t)b * p.next_stride] = y;
    if (p.commit_out) {
        int32_t *cm = p.commit_out + (int64_t)b * (p.k + 1);
        for (int j = 0; j < a; ++j) cm[j] = p.drafts[(int64_t)b * p.draft_stride + j];
        cm[a] = y;
    }
}

}  // namespace

int accept_chunks(int vocab) { return (vocab + kChunk - 1) / kChunk; }

hipError_t launch_accept(const AcceptParams &p, hipStream_t s) {
    const int rows = p.inv_temp == 0.0f ? p.k + 1 : 2 * p.k + 1;
    hipLaunchKernelGGL(k_acc_stats, dim3(p.nchunk, rows, p.batch), dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_acc_decide, dim3(p.nchunk, p.batch), dim3(kThreads), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_acc_final, dim3(p.batch), dim3(64), 0, s, p);
    return hipGetLastError();
}

}  // namespace spec
