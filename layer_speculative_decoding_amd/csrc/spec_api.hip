// libspec C ABI: argument validation, workspace layout and kernel dispatch.
// Every compute call validates on the host first and launches nothing on an
// error.  No call allocates device memory or synchronises the host.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/spec.h"
#include "spec_kernels.h"

using namespace spec;

struct spec_model {
    spec_model_desc d;
    spec_weights w;
    int D;      // (hq + 2 hkv) * hd
    int qd;     // hq * hd
    int xs;     // weight and KV element size (4 f32, 2 bf16); activations are float32
};

namespace {

thread_local char g_err[512] = "";

spec_status fail(spec_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

spec_status hip_fail(hipError_t e, const char *where) {
    return fail(SPEC_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

inline size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// ------------------------------------------------------------ measurement
// While enabled, each product and attention launch is bracketed by two HIP
// events on its stream and attributed to its kernel instance with the bytes
// the launch must read (weights + activation rows; the K/V rows attention
// reads) and, for the products, the multiply-add flops 2 * M * rows * K.
struct ProfPending {
    std::string name;
    double bytes, flops;
    hipEvent_t a, b;
};
struct ProfAgg {
    std::string name;
    int64_t launches;
    double ms, bytes, flops;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfPending> g_prof_pending;
std::vector<ProfAgg> g_prof_agg;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
    if (!g_prof_pool.empty()) {
        hipEvent_t e = g_prof_pool.back();
        g_prof_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    (void)hipEventCreate(&e);
    return e;
}

struct ProfScope {
    bool on;
    hipEvent_t a = nullptr;
    hipStream_t s;
    ProfScope(hipStream_t s_) : s(s_) {
        std::lock_guard<std::mutex> g(g_prof_mu);
        on = g_prof_on;
        if (on) {
            a = prof_event();
            (void)hipEventRecord(a, s);
        }
    }
    void done(const std::string &name, double bytes, double flops = 0.0) {
        if (!on) return;
        std::lock_guard<std::mutex> g(g_prof_mu);
        hipEvent_t b = prof_event();
        (void)hipEventRecord(b, s);
        g_prof_pending.push_back({name, bytes, flops, a, b});
    }
};

std::string gemv_name(int dtype, const GemvParams &p) {
    const int mr = p.M <= 1 ? 1 : (p.M <= 2 ? 2 : (p.M <= 4 ? 4 : 8));
    return std::string("k_gemv<") + (dtype ? "unsigned short" : "float") + ", " + std::to_string(mr) + ", " +
           std::to_string(p.epi) + ", " + std::to_string(gemv_operand_mode(dtype, p)) + ">";
}

constexpr bool epi_is_pair_host(int epi) { return epi == EPI_QKV_ROPE || epi == EPI_SILU_MUL; }

// the instance launch_gemm_mfma takes for product q (all template arguments,
// as the profiler prints them)
std::string mfma_name(const GemvParams &q, int ks, int unit_rows) {
    const bool pair = epi_is_pair_host(q.epi);
    const bool seg = !pair && q.epi == EPI_RESID_ADD && q.kseg > 1;
    (void)unit_rows;
    return std::string("k_gemm_mfma<") + (q.M <= 8 ? "1" : "2") + ", " + std::to_string(q.epi) + ", " +
           std::to_string(ks) + ", " + (seg ? "true" : "false") + ">";
}


// Workspace layout for R activation rows and sets of at most G layers.
struct Carve {
    size_t h, h0, abuf, xn, q, o, act, pacc, pml, pval, pidx, ss, rope, tpart, tpart_bytes, total;
    int64_t ss_sel_stride;   // floats per set member in ss
};

constexpr int kPartialsMax = 2048;   // largest grid of a partial-sum producer

Carve carve(const spec_model *m, int batch, int max_m, int G) {
    const size_t R = (size_t)batch * max_m;
    const size_t d = m->d.d_model, xs = m->xs;
    const size_t hq = m->d.n_q_heads, hd = m->d.head_dim;
    const size_t prow = R < 64 ? R : 64;
    const size_t nsel = G < kMaxSel ? G : kMaxSel;
    Carve c{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
    c.h = take(R * d * 4);
    c.h0 = take(R * d * 4);
    c.abuf = take((size_t)G * R * d * 4);
    // activation operands: float32 rows, or up to 32 packed bf16 rows
    const size_t arow = R * 4 > 64 ? R * 4 : 64;
    c.xn = take((size_t)G * d * arow);
    c.q = take((size_t)G * R * hq * hd * 4);
    c.o = take((size_t)G * hq * hd * arow);
    c.act = take((size_t)G * m->d.d_ffn * arow);   // one block per set member (parallel MLPs)
    c.pacc = take((size_t)attention_split_max() * G * prow * hq * hd * 4);
    c.pml = take((size_t)attention_split_max() * G * prow * hq * 2 * 4);
    c.pval = take((size_t)batch * kPartialsMax * 4);
    c.pidx = take((size_t)batch * kPartialsMax * 4);
    c.ss_sel_stride = (int64_t)R * kPartialsMax;
    c.ss = take(nsel * R * kPartialsMax * 4);
    c.rope = take(R * (hd / 2) * 8);
    // K-slice partials of the tiled products (calls of more than 16 rows)
    c.tpart_bytes = R >= (size_t)gemm_tiled_min_rows() ? gemm_tiled_part_bytes() : 0;
    c.tpart = take(c.tpart_bytes);
    c.total = off;
    return c;
}

template <typename P> P *at(void *ws, size_t off) { return reinterpret_cast<P *>(reinterpret_cast<char *>(ws) + off); }

const void *layer_ptr(const void *base, size_t layer, size_t elems_per_layer, int xs) {
    return reinterpret_cast<const char *>(base) + layer * elems_per_layer * xs;
}

// Everything a forward over R = batch * mseq rows needs, plus the number of
// sum-of-squares partials each set member's residual row currently has.
struct Fwd {
    const spec_model *m;
    const spec_kv *kv;
    int batch, mseq, max_pos;
    RowMap rows;
    void *ws;
    Carve c;
    hipStream_t s;
    int nparts[kMaxSel];
    // the last residual writer also wrote the next RMSNorm operand (gain
    // nx_gain) for a skinny matrix-core consumer (section fuse_next_norm)
    bool nx_ready = false;
    const float *nx_gain = nullptr;
};

// The X_NORM consumer that follows a stage's last residual write: the next
// stage's QKV (when that stage is a single layer) or the lm head; gain NULL
// when there is none to prepare.
struct NextNorm {
    const float *gain = nullptr;
    int rows = 0, pair_block = 0, epi = 0;
};

// Activation-row count from which bf16 products use the matrix-core kernel
// (SPEC_MFMA_MIN_ROWS overrides; the VALU GEMV serves fewer rows and float32).
int mfma_min_rows() {
    static int v = [] {
        const char *e = getenv("SPEC_MFMA_MIN_ROWS");
        return e ? atoi(e) : 2;
    }();
    return v;
}

// Activation-row count from which bf16 products use the tiled matrix-core
// GEMM (SPEC_TILED_MIN_ROWS overrides).
int tiled_min_rows() {
    static int v = [] {
        const char *e = getenv("SPEC_TILED_MIN_ROWS");
        return e ? atoi(e) : gemm_tiled_min_rows();
    }();
    return v;
}

// Which kernel serves a product over p.Mtot rows: the VALU GEMV (one row,
// the float32 path, shapes the matrix-core kernels do not take), the skinny
// matrix-core kernel (2..16 rows, one launch, packed bf16 hi/lo operand rows)
// or the tiled matrix-core GEMM (17 rows and more, float32 operand rows).
enum ProdPath { PP_VALU, PP_MFMA, PP_TILED };

// Weight rows per unit of the skinny matrix-core kernel for product p.
int mfma_unit_rows(const GemvParams &p) {
    return gemm_mfma_unit_rows(p.epi, p.n_units * 2, p.rows_per_sel);
}

GemvParams mfma_params(const GemvParams &p) {
    GemvParams q = p;
    q.n_units = p.n_units * 2 / mfma_unit_rows(p);
    q.m0 = 0;
    q.M = p.Mtot;
    return q;
}

ProdPath product_path(const spec_model *m, const GemvParams &p) {
    if (m->d.dtype != SPEC_BF16) return PP_VALU;
    const int Mtot = p.Mtot;
    GemvParams t = p;
    t.m0 = 0;
    t.M = Mtot;
    if (Mtot >= tiled_min_rows() && gemm_tiled_supported(t)) return PP_TILED;
    const int rows = p.n_units * 2;
    if (Mtot >= mfma_min_rows() && Mtot <= gemm_mfma_max_rows() && rows % (epi_is_pair_host(p.epi) ? 32 : 16) == 0 &&
        gemm_mfma_supported(mfma_params(p)))
        return PP_MFMA;
    return PP_VALU;
}

// Rows of the packed operand a producer writes for this product (0: float32
// rows).
int packed_rows(const spec_model *m, const GemvParams &consumer) {
    return product_path(m, consumer) == PP_MFMA ? gemm_mfma_packed_rows(consumer.Mtot) : 0;
}

// Weight-streaming product over the call's p.Mtot activation rows.  A plain
// (X_PLAIN) operand must already be in the form product_path gives (packed
// rows for the skinny matrix-core kernel, x_sel_stride in its elements).
// *parts_out: the sum-of-squares or sampling partials each output row now has.
hipError_t product(Fwd &f, GemvParams p, int *parts_out = nullptr) {
    const spec_model *m = f.m;
    const int Mtot = p.Mtot;
    p.ss = at<float>(f.ws, f.c.ss);
    p.ss_sel_stride = f.c.ss_sel_stride;
    p.part_val = at<float>(f.ws, f.c.pval);
    p.part_idx = at<int32_t>(f.ws, f.c.pidx);
    const int rows = p.n_units * 2;
    const double wbytes = (double)rows * p.K * m->xs;   // every weight row once
    const ProdPath path = product_path(m, p);
    if (path == PP_TILED) {
        GemvParams t = p;
        t.m0 = 0;
        t.M = Mtot;
        if (parts_out) *parts_out = gemm_tiled_parts(t);
        double xbytes = (double)Mtot * p.K * 4;
        if (p.xmode == X_NORM) {
            const int n_sel = rows / p.rows_per_sel;
            void *xn = at<char>(f.ws, f.c.xn);
            hipError_t e = launch_norm_rows(m->d.dtype, t, n_sel, xn, 0, f.s);
            if (e != hipSuccess) return e;
            t.xmode = X_PLAIN;
            t.X = xn;
            t.x_sel_stride = (int64_t)Mtot * p.K;
            xbytes *= n_sel;
        }
        ProfScope ps(f.s);
        float *part = f.c.tpart_bytes ? at<float>(f.ws, f.c.tpart) : nullptr;
        hipError_t e = launch_gemm_tiled(t, part, f.c.tpart_bytes, f.s);
        ps.done(gemm_tiled_name(t, f.c.tpart_bytes), wbytes + xbytes, 2.0 * Mtot * rows * (double)p.K);
        return e;
    }
    if (path == PP_MFMA) {
        GemvParams q = mfma_params(p);
        const int grid = gemm_mfma_grid(q);
        const int ks = gemm_mfma_splits(q);
        const int ur = mfma_unit_rows(p);
        if (parts_out) *parts_out = (p.epi == EPI_LOGITS) ? grid : p.rows_per_sel / ur;
        double xbytes = (double)Mtot * p.K * 4;
        if (p.xmode == X_NORM) {
            const int n_sel = rows / p.rows_per_sel;
            const int pr = gemm_mfma_packed_rows(Mtot);
            void *xn = at<char>(f.ws, f.c.xn);
            if (f.nx_ready && f.nx_gain == p.xgain && n_sel == 1 && !p.xadd && p.xgather_mseq == 0 &&
                (int64_t)Mtot * p.xnparts <= gemm_mfma_inv_max(Mtot)) {
                // the residual writer left gain * h as packed rows: the 1 / rms
                // scale moves to this product's epilogue
                q.x_inv = 1;
            } else {
                // normalise once into packed operand rows, then stream the weights
                hipError_t e = launch_norm_rows(m->d.dtype, q, n_sel, xn, pr, f.s);
                if (e != hipSuccess) return e;
            }
            f.nx_ready = false;
            q.xmode = X_PLAIN;
            q.X = xn;
            q.x_sel_stride = (int64_t)pr * p.K;
            xbytes *= n_sel;
        }
        ProfScope ps(f.s);
        hipError_t e = launch_gemm_mfma(q, grid, ks, ur, f.s);
        ps.done(mfma_name(q, ks, ur), wbytes + xbytes, 2.0 * Mtot * rows * (double)p.K);
        return e;
    }
    const int mr = gemv_max_rows();
    const int ks = gemv_splits(p, m->xs);
    const int grid = gemv_grid(p, ks);
    if (parts_out) *parts_out = grid;
    for (int m0 = 0; m0 < Mtot; m0 += mr) {
        p.m0 = m0;
        p.M = (Mtot - m0) < mr ? (Mtot - m0) : mr;
        ProfScope ps(f.s);
        hipError_t e = launch_gemv(m->d.dtype, p, grid, ks, f.s);
        ps.done(gemv_name(m->d.dtype, p), wbytes + (double)p.M * p.K * 4,
                2.0 * p.M * rows * (double)p.K);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Norm fusion switch (SPEC_NORM_FUSION=0: every skinny matrix-core consumer
// normalises its operand in its own pass).
bool norm_fusion() {
    static const bool on = [] {
        const char *e = getenv("SPEC_NORM_FUSION");
        return !(e && e[0] == '0');
    }();
    return on;
}

// Residual writer prod is followed by an X_NORM consumer of `rows` weight rows
// (one set member, gain `gain`, epilogue epi).  When both run on the skinny
// matrix-core kernel, prod also writes that consumer's operand (gain * h,
// packed) and the consumer scales by 1 / rms in its epilogue instead of a
// normalisation pass.
void fuse_next_norm(Fwd &f, GemvParams &prod, const float *gain, int rows, int pair_block, int epi) {
    f.nx_ready = false;
    if (!gain || !norm_fusion()) return;
    const spec_model *m = f.m;
    GemvParams c{};
    c.Mtot = prod.Mtot; c.K = m->d.d_model; c.n_units = rows / 2; c.pair_block = pair_block;
    c.rows_per_sel = rows; c.epi = epi; c.xmode = X_NORM;
    if (product_path(m, c) != PP_MFMA || product_path(m, prod) != PP_MFMA) return;
    const int parts = prod.rows_per_sel / mfma_unit_rows(prod);
    if ((int64_t)prod.Mtot * parts > gemm_mfma_inv_max(prod.Mtot)) return;
    prod.nx = at<uint16_t>(f.ws, f.c.xn);
    prod.nx_packed = gemm_mfma_packed_rows(prod.Mtot);
    prod.nx_gain = gain;
    f.nx_ready = true;
    f.nx_gain = gain;
}

NextNorm next_qkv(const spec_model *m, int l, int n) {
    NextNorm nn;
    if (n != 1) return nn;
    nn.gain = m->w.attn_norm + (size_t)l * m->d.d_model;
    nn.rows = m->D; nn.pair_block = m->d.head_dim; nn.epi = EPI_QKV_ROPE;
    return nn;
}

NextNorm head_norm(const spec_model *m, int epi) {
    NextNorm nn;
    nn.gain = m->w.final_norm;
    nn.rows = m->d.vocab; nn.pair_block = 2; nn.epi = epi;
    return nn;
}

// Embedding, the sum of squares of every row (one partial), RoPE table.
hipError_t run_embed(Fwd &f, const int32_t *tokens, int64_t tok_ld, int tok_step) {
    const spec_model *m = f.m;
    EmbedParams e{};
    e.E = m->w.embed; e.vocab = m->d.vocab; e.d = m->d.d_model;
    e.tokens = tokens; e.tok_ld = tok_ld; e.tok_step = tok_step; e.rows = f.rows;
    e.h = at<float>(f.ws, f.c.h); e.ss = at<float>(f.ws, f.c.ss);
    e.rope_cs = at<float2>(f.ws, f.c.rope); e.hd = m->d.head_dim; e.rope_theta = m->d.rope_theta;
    f.nparts[0] = 1;
    return launch_embed(m->d.dtype, e, f.batch * f.mseq, f.s);
}

// One stage: attention of the set [l0, l0 + n) on the stage input h0, then
// the set's MLPs.  A stage of one layer is the ordinary decoder layer.
// cos_out (nullable, sequential MLPs only): cos_out[b * cos_stride + l] for
// each layer l of the set = the cosine between the input its attention read
// (h0) and the running state a sequential layer would have read there.
hipError_t run_stage(Fwd &f, int l0, int n, int mlp_mode, const NextNorm &nn = NextNorm{}, float *cos_out = nullptr,
                     int64_t cos_stride = 0) {
    const spec_model *m = f.m;
    const spec_model_desc &d = m->d;
    const int R = f.batch * f.mseq;
    const int dm = d.d_model, D = m->D, qd = m->qd, xs = m->xs;
    const bool par = mlp_mode == SPEC_MLP_PARALLEL && n > 1;
    float *h = at<float>(f.ws, f.c.h);
    float *h0 = at<float>(f.ws, f.c.h0);
    float *abuf = at<float>(f.ws, f.c.abuf);
    float *ss = at<float>(f.ws, f.c.ss);
    float *q = at<float>(f.ws, f.c.q);
    void *o = at<char>(f.ws, f.c.o);
    void *act = at<char>(f.ws, f.c.act);
    hipError_t e;
    int grid = 0;
    if (cos_out) {
        // keep the stage input; the first member reads exactly it
        if ((e = hipMemcpyAsync(h0, h, (size_t)R * dm * 4, hipMemcpyDeviceToDevice, f.s)) != hipSuccess) return e;
        if ((e = launch_cosine(h0, h0, nullptr, R, dm, cos_out + l0, cos_stride, f.s)) != hipSuccess) return e;
    }

    // 1. grouped QKV over the N layers' concatenated rows: operand = one RMS
    //    of h0 with each layer's gain; epilogue = RoPE + KV append
    GemvParams gp{};
    gp.Mtot = R; gp.d = dm; gp.eps = d.rms_eps;
    gp.W = layer_ptr(m->w.wqkv, l0, (size_t)D * dm, xs);
    gp.K = dm; gp.n_units = n * D / 2; gp.pair_block = d.head_dim; gp.rows_per_sel = D;
    gp.xmode = X_NORM; gp.xh = h; gp.xgain = m->w.attn_norm + (size_t)l0 * dm; gp.xgain_stride = dm;
    gp.xss = ss; gp.xnparts = f.nparts[0];
    gp.bias = m->w.bqkv ? m->w.bqkv + (size_t)l0 * D : nullptr;
    gp.epi = EPI_QKV_ROPE;
    gp.q_out = q; gp.q_sel_stride = (int64_t)R * qd;
    gp.kc = f.kv->k; gp.vc = f.kv->v; gp.layer0 = l0; gp.batch = f.batch;
    gp.hq = d.n_q_heads; gp.hkv = d.n_kv_heads; gp.hd = d.head_dim;
    gp.rope_cs = at<float2>(f.ws, f.c.rope);
    gp.rows = f.rows;
    if ((e = product(f, gp)) != hipSuccess) return e;

    // the O product's operand format decides how the attention writes o
    GemvParams go{};
    go.Mtot = R; go.d = dm; go.eps = d.rms_eps;
    go.W = layer_ptr(m->w.wo, l0, (size_t)dm * qd, xs);
    go.K = qd; go.n_units = n * dm / 2; go.pair_block = 2; go.rows_per_sel = dm;
    go.xmode = X_PLAIN; go.epi = EPI_ATTN_OUT;
    const int o_packed = packed_rows(m, go);

    // 2. grouped attention
    AttnParams ap{};
    ap.q = q; ap.q_sel_stride = (int64_t)R * qd;
    ap.kc = f.kv->k; ap.vc = f.kv->v; ap.layer0 = l0; ap.n_group = n; ap.batch = f.batch;
    ap.hq = d.n_q_heads; ap.hkv = d.n_kv_heads; ap.hd = d.head_dim; ap.capacity = f.kv->capacity;
    ap.rows = f.rows; ap.max_pos = f.max_pos;
    ap.splits = attention_splits(d.dtype, d.head_dim, n, f.batch, d.n_q_heads, d.n_kv_heads, f.mseq, f.max_pos);
    ap.o = o; ap.o_packed = o_packed; ap.o_sel_stride = (int64_t)(o_packed ? o_packed : R) * qd;
    ap.part_acc = at<float>(f.ws, f.c.pacc); ap.part_ml = at<float>(f.ws, f.c.pml); ap.Mtot = R;
    {
        // K/V rows of every set member, every sequence, up to max_pos (a bound)
        ProfScope ps(f.s);
        e = launch_attention(d.dtype, ap, f.s);
        ps.done(ap.splits > 1 ? "k_attn (split)" : "k_attn",
                2.0 * n * f.batch * (f.max_pos + 1.0) * d.n_kv_heads * d.head_dim * xs);
        if (e != hipSuccess) return e;
    }

    // 3. grouped O projection: a_0 goes into the residual (sequential MLPs),
    //    the others wait in abuf; partial sums give the MLP inputs' RMS
    gp = go;
    gp.X = o; gp.x_sel_stride = ap.o_sel_stride;
    gp.h = h; gp.h0 = h0; gp.par_mlp = par ? 1 : 0;
    gp.out = abuf; gp.out_sel_stride = (int64_t)R * dm;
    gp.n_norm_sel = par ? n : 1;
    if (!par && !cos_out) fuse_next_norm(f, gp, m->w.ffn_norm + (size_t)l0 * dm, 2 * d.d_ffn, 2 * d.d_ffn, EPI_SILU_MUL);
    else f.nx_ready = false;
    if ((e = product(f, gp, &grid)) != hipSuccess) return e;
    for (int i = 0; i < gp.n_norm_sel; ++i) f.nparts[i] = grid;

    // 4. parallel reading: the set's MLPs as two launches, the N members'
    //    [gate; up] blocks concatenated in one product (member i normalises
    //    h0 + a_i with its own gain and RMS) and the N down projections as one
    //    product over K = N x ffn (the members' matrices side by side), adding
    //    sum_i (a_i + m_i) to h
    if (par) {
        GemvParams gd{};
        gd.Mtot = R; gd.d = dm; gd.eps = d.rms_eps;
        gd.W = layer_ptr(m->w.w_down, l0, (size_t)dm * d.d_ffn, xs);
        gd.K = n * d.d_ffn; gd.kseg = n; gd.w_seg_stride = (int64_t)dm * d.d_ffn;
        gd.n_units = dm / 2; gd.pair_block = 2; gd.rows_per_sel = dm;
        gd.xmode = X_PLAIN; gd.X = act; gd.epi = EPI_RESID_ADD;
        const int pk = packed_rows(m, gd);
        const int64_t arows = pk ? pk : R;           // act rows per member block
        gd.x_seg_stride = arows * d.d_ffn;
        gp = GemvParams{};
        gp.Mtot = R; gp.d = dm; gp.eps = d.rms_eps;
        gp.W = layer_ptr(m->w.w_gate_up, l0, (size_t)2 * d.d_ffn * dm, xs);
        gp.K = dm; gp.n_units = n * d.d_ffn; gp.pair_block = 2 * d.d_ffn; gp.rows_per_sel = 2 * d.d_ffn;
        gp.xmode = X_NORM; gp.xh = h0; gp.xadd = abuf; gp.xadd_sel_stride = (int64_t)R * dm;
        gp.xgain = m->w.ffn_norm + (size_t)l0 * dm; gp.xgain_stride = dm;
        gp.xss = ss; gp.xss_sel_stride = f.c.ss_sel_stride; gp.xnparts = f.nparts[0];
        gp.epi = EPI_SILU_MUL; gp.act = act; gp.act_ld = d.d_ffn; gp.act_sel_stride = arows * d.d_ffn;
        gp.act_packed = pk;
        // the float32 GEMV takes members with their own RMS only with staged
        // operands; the tiled kernel takes no K segments
        GemvParams tv = gp;
        tv.M = R < gemv_max_rows() ? R : gemv_max_rows();
        const ProdPath pu = product_path(m, gp), pd = product_path(m, gd);
        const bool ok = pu != PP_TILED && pd != PP_TILED &&
                        (pu != PP_VALU || gemv_operand_mode(d.dtype, tv) == 1);
        if (ok) {
            if ((e = product(f, gp)) != hipSuccess) return e;
            gd.h = h;
            gd.add2 = abuf; gd.n_add2 = n; gd.add2_sel_stride = (int64_t)R * dm;
            gd.n_norm_sel = 1;
            fuse_next_norm(f, gd, nn.gain, nn.rows, nn.pair_block, nn.epi);
            if ((e = product(f, gd, &grid)) != hipSuccess) return e;
            f.nparts[0] = grid;
            return hipSuccess;
        }
    }

    // 4. MLPs in set order (sequential reading; parallel reading where the
    //    concatenated products above do not apply)
    for (int i = 0; i < n; ++i) {
        const int l = l0 + i;
        const int si = par ? i : 0;
        gp = GemvParams{};
        gp.Mtot = R; gp.d = dm; gp.eps = d.rms_eps;
        gp.W = layer_ptr(m->w.w_gate_up, l, (size_t)2 * d.d_ffn * dm, xs);
        gp.K = dm; gp.n_units = d.d_ffn; gp.pair_block = 2 * d.d_ffn; gp.rows_per_sel = 2 * d.d_ffn;
        gp.xmode = X_NORM; gp.xgain = m->w.ffn_norm + (size_t)l * dm;
        gp.xss = ss + (size_t)si * f.c.ss_sel_stride; gp.xnparts = f.nparts[si];
        if (par) { gp.xh = h0; gp.xadd = abuf + (size_t)i * R * dm; }
        else gp.xh = h;
        // the down product's operand format decides how the SiLU writes act
        GemvParams gd{};
        gd.Mtot = R; gd.d = dm; gd.eps = d.rms_eps;
        gd.W = layer_ptr(m->w.w_down, l, (size_t)dm * d.d_ffn, xs);
        gd.K = d.d_ffn; gd.n_units = dm / 2; gd.pair_block = 2; gd.rows_per_sel = dm;
        gd.xmode = X_PLAIN; gd.X = act; gd.epi = EPI_RESID_ADD;
        gp.epi = EPI_SILU_MUL; gp.act = act; gp.act_ld = d.d_ffn; gp.act_packed = packed_rows(m, gd);
        if ((e = product(f, gp)) != hipSuccess) return e;

        gp = gd;
        gp.x_sel_stride = 0;
        gp.h = h;
        // sequential: h += m_i + a_{i+1} (the next member's attention output);
        // parallel: h += a_i + m_i
        gp.add2 = par ? abuf + (size_t)i * R * dm : (i + 1 < n ? abuf + (size_t)(i + 1) * R * dm : nullptr);
        gp.n_norm_sel = 1;
        if (cos_out || (par && i + 1 < n)) f.nx_ready = false;
        else if (i + 1 < n) fuse_next_norm(f, gp, m->w.ffn_norm + (size_t)(l + 1) * dm, 2 * d.d_ffn, 2 * d.d_ffn,
                                           EPI_SILU_MUL);
        else fuse_next_norm(f, gp, nn.gain, nn.rows, nn.pair_block, nn.epi);
        if ((e = product(f, gp, &grid)) != hipSuccess) return e;
        f.nparts[0] = grid;
        if (cos_out && i + 1 < n) {
            // h now also holds a_{i+1}: the state before it is h - a_{i+1}
            e = launch_cosine(h0, h, abuf + (size_t)(i + 1) * R * dm, R, dm, cos_out + l0 + i + 1, cos_stride, f.s);
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

// Final RMSNorm (folded into the operand; optionally of the last valid row of
// each sequence) + lm head; with token_out, per-block arg-max partials of the
// sampling scores are reduced by a small kernel.
hipError_t run_head(Fwd &f, bool last_only, const int32_t *ntok, float *logits, int64_t logits_ld,
                    float inv_temp, uint64_t seed, const int32_t *samp_pos, const int32_t *samp_ntok,
                    int samp_nconst, int32_t *token_out, int token_stride) {
    const spec_model *m = f.m;
    const int dm = m->d.d_model;
    const int R = f.batch * f.mseq;
    if (!token_out && !logits) return hipSuccess;
    GemvParams gp{};
    gp.Mtot = last_only ? f.batch : R; gp.d = dm; gp.eps = m->d.rms_eps;
    gp.W = m->w.lm_head; gp.K = dm; gp.n_units = m->d.vocab / 2; gp.pair_block = 2; gp.rows_per_sel = m->d.vocab;
    gp.xmode = X_NORM; gp.xh = at<float>(f.ws, f.c.h); gp.xgain = m->w.final_norm; gp.xgain_stride = 0;
    gp.xss = at<float>(f.ws, f.c.ss); gp.xnparts = f.nparts[0];
    gp.xgather_mseq = last_only ? f.mseq : 0; gp.xgather_ntok = ntok;
    gp.epi = token_out ? EPI_LOGITS : EPI_STORE;
    gp.out = logits; gp.out_ld = logits_ld; gp.out_sel_stride = 0;
    gp.inv_temp = inv_temp; gp.seed = seed; gp.samp_pos = samp_pos; gp.samp_ntok = samp_ntok;
    gp.samp_nconst = samp_nconst;
    int grid = 0;
    hipError_t e = product(f, gp, &grid);
    if (e != hipSuccess || !token_out) return e;
    return launch_sample_reduce(at<float>(f.ws, f.c.pval), at<int32_t>(f.ws, f.c.pidx), grid, gp.Mtot, token_out,
                                token_stride, f.s);
}

spec_status check_model(const spec_model *m, const spec_kv *kv, int batch) {
    if (!m) return fail(SPEC_ERR_INVALID_ARG, "model is NULL");
    if (!kv || !kv->k || !kv->v) return fail(SPEC_ERR_INVALID_ARG, "kv cache pointers are NULL");
    if (batch < 1 || batch > kv->batch) return fail(SPEC_ERR_SHAPE, "batch %d outside [1, kv batch %d]", batch, kv->batch);
    if (kv->capacity < 1) return fail(SPEC_ERR_SHAPE, "kv capacity %d < 1", kv->capacity);
    return SPEC_OK;
}

// Scratch array of the entry point that allocates nothing: one copy per GPU
// (the code object is loaded on each device), its device address looked up
// once per device with that device current.  Host code never passes the
// array's name itself to a kernel (on the host it only stands for the
// symbol), always the looked-up address.
static __device__ __align__(256) unsigned char scratch[SPEC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
std::vector<void *> g_scratch_ptr;   // by device ordinal

spec_status scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (dev >= (int)g_scratch_ptr.size()) g_scratch_ptr.resize(dev + 1, nullptr);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(SPEC_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SPEC_OK;
}

spec_status check_ws(const spec_model *m, int batch, int max_m, int G, void *ws, size_t ws_bytes) {
    const size_t need = spec_workspace_bytes(m, batch, max_m, G);
    if (!ws || ws_bytes < need)
        return fail(SPEC_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
    return SPEC_OK;
}

}  // namespace

extern "C" {

const char *spec_version(void) { return "0.1.0 gfx950"; }

spec_status spec_profile_enable(int on) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    g_prof_on = on != 0;
    return SPEC_OK;
}

void spec_profile_reset(void) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    for (auto &p : g_prof_pending) {
        g_prof_pool.push_back(p.a);
        g_prof_pool.push_back(p.b);
    }
    g_prof_pending.clear();
    g_prof_agg.clear();
}

int spec_profile_collect(void) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    for (auto &p : g_prof_pending) {
        float ms = 0.f;
        if (hipEventSynchronize(p.b) == hipSuccess) (void)hipEventElapsedTime(&ms, p.a, p.b);
        ProfAgg *agg = nullptr;
        for (auto &x : g_prof_agg)
            if (x.name == p.name) agg = &x;
        if (!agg) {
            g_prof_agg.push_back({p.name, 0, 0.0, 0.0, 0.0});
            agg = &g_prof_agg.back();
        }
        agg->launches += 1;
        agg->ms += ms;
        agg->bytes += p.bytes;
        agg->flops += p.flops;
        g_prof_pool.push_back(p.a);
        g_prof_pool.push_back(p.b);
    }
    g_prof_pending.clear();
    return (int)g_prof_agg.size();
}

spec_status spec_profile_entry(int i, char *name, int name_cap, int64_t *launches, double *total_ms,
                               double *total_bytes, double *total_flops) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    if (i < 0 || i >= (int)g_prof_agg.size() || !name || name_cap < 1)
        return fail(SPEC_ERR_INVALID_ARG, "profile entry %d out of range", i);
    const ProfAgg &a = g_prof_agg[i];
    snprintf(name, (size_t)name_cap, "%s", a.name.c_str());
    if (launches) *launches = a.launches;
    if (total_ms) *total_ms = a.ms;
    if (total_bytes) *total_bytes = a.bytes;
    if (total_flops) *total_flops = a.flops;
    return SPEC_OK;
}
const char *spec_last_error(void) { return g_err; }

const char *spec_status_string(spec_status s) {
    switch (s) {
    case SPEC_OK: return "ok";
    case SPEC_ERR_INVALID_ARG: return "invalid argument";
    case SPEC_ERR_SHAPE: return "unsupported shape";
    case SPEC_ERR_VOCAB_MISMATCH: return "draft and base vocabularies differ";
    case SPEC_ERR_PLAN: return "invalid layer plan";
    case SPEC_ERR_CAPACITY: return "KV capacity exceeded";
    case SPEC_ERR_WORKSPACE: return "workspace too small";
    case SPEC_ERR_HIP: return "HIP error";
    case SPEC_ERR_UNSUPPORTED: return "unsupported";
    }
    return "unknown status";
}

spec_status spec_model_create(const spec_model_desc *desc, const spec_weights *w, spec_model **out) {
    if (!desc || !w || !out) return fail(SPEC_ERR_INVALID_ARG, "NULL argument");
    const spec_model_desc &d = *desc;
    if (d.n_layers < 1 || d.d_model < 8 || d.n_q_heads < 1 || d.n_kv_heads < 1 || d.d_ffn < 8 || d.vocab < 2)
        return fail(SPEC_ERR_SHAPE, "non-positive model dimension");
    if (d.dtype != SPEC_F32 && d.dtype != SPEC_BF16) return fail(SPEC_ERR_INVALID_ARG, "dtype %d", d.dtype);
    if (d.head_dim != 16 && d.head_dim != 32 && d.head_dim != 64 && d.head_dim != 128)
        return fail(SPEC_ERR_UNSUPPORTED, "head_dim %d not in {16, 32, 64, 128}", d.head_dim);
    if (d.n_q_heads % d.n_kv_heads) return fail(SPEC_ERR_SHAPE, "n_q_heads %% n_kv_heads != 0");
    if (d.n_q_heads / d.n_kv_heads > attention_max_group())
        return fail(SPEC_ERR_UNSUPPORTED, "n_q_heads / n_kv_heads %d > %d", d.n_q_heads / d.n_kv_heads,
                    attention_max_group());
    if (d.d_model % 8 || d.d_ffn % 8 || (d.n_q_heads * d.head_dim) % 8)
        return fail(SPEC_ERR_SHAPE, "d_model, d_ffn and n_q_heads*head_dim must be multiples of 8");
    if (d.d_model > 16384) return fail(SPEC_ERR_UNSUPPORTED, "d_model %d > 16384", d.d_model);
    if (d.vocab % 2) return fail(SPEC_ERR_SHAPE, "vocab must be even");
    if (d.has_qkv_bias && !w->bqkv) return fail(SPEC_ERR_INVALID_ARG, "has_qkv_bias but bqkv is NULL");
    if (!w->embed || !w->attn_norm || !w->wqkv || !w->wo || !w->ffn_norm || !w->w_gate_up || !w->w_down ||
        !w->final_norm || !w->lm_head)
        return fail(SPEC_ERR_INVALID_ARG, "a weight pointer is NULL");
    if (!(d.rms_eps > 0.f) || !(d.rope_theta > 1.f)) return fail(SPEC_ERR_INVALID_ARG, "rms_eps / rope_theta");
    spec_model *m = new spec_model;
    m->d = d;
    m->w = *w;
    if (!d.has_qkv_bias) m->w.bqkv = nullptr;
    m->D = (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim;
    m->qd = d.n_q_heads * d.head_dim;
    m->xs = d.dtype == SPEC_BF16 ? 2 : 4;
    *out = m;
    return SPEC_OK;
}

void spec_model_destroy(spec_model *m) { delete m; }

spec_status spec_check_pair(const spec_model *draft, const spec_model *base) {
    if (!draft || !base) return fail(SPEC_ERR_INVALID_ARG, "NULL model");
    if (draft->d.vocab != base->d.vocab)
        return fail(SPEC_ERR_VOCAB_MISMATCH, "draft vocab %d != base vocab %d", draft->d.vocab, base->d.vocab);
    return SPEC_OK;
}

spec_status spec_default_group_plan(int L, int N, int32_t *offs, int max_offsets, int *n_stages_out) {
    if (L < 1 || N < 1 || !offs || !n_stages_out) return fail(SPEC_ERR_INVALID_ARG, "bad plan arguments");
    // set starts: layer 0, every intermediate layer l with l / N != (l - 1) / N
    // (and layer 1), the last layer; then the end marker L
    std::vector<int32_t> u;
    u.push_back(0);
    for (int l = 1; l < L - 1; ++l)
        if (l == 1 || l / N != (l - 1) / N) u.push_back(l);
    if (L > 1) u.push_back(L - 1);
    u.push_back(L);
    if ((int)u.size() > max_offsets) return fail(SPEC_ERR_INVALID_ARG, "offsets buffer too small (%zu)", u.size());
    for (size_t i = 0; i < u.size(); ++i) offs[i] = u[i];
    *n_stages_out = (int)u.size() - 1;
    return SPEC_OK;
}

size_t spec_workspace_bytes(const spec_model *m, int batch, int max_m, int max_group) {
    if (!m || batch < 1 || max_m < 1 || max_group < 1) return 0;
    return carve(m, batch, max_m, max_group).total;
}

// Plan check shared by the layer-parallel entry points; *G = largest set.
static spec_status check_plan(const spec_model *draft, const int32_t *plan_offsets, int n_stages, int flags,
                              int *G) {
    if (!plan_offsets || n_stages < 1) return fail(SPEC_ERR_PLAN, "empty plan");
    if (flags != SPEC_MLP_SEQUENTIAL && flags != SPEC_MLP_PARALLEL) return fail(SPEC_ERR_INVALID_ARG, "flags %d", flags);
    if (plan_offsets[0] != 0 || plan_offsets[n_stages] != draft->d.n_layers)
        return fail(SPEC_ERR_PLAN, "plan must cover layers 0..%d", draft->d.n_layers - 1);
    *G = 1;
    for (int s = 0; s < n_stages; ++s) {
        const int n = plan_offsets[s + 1] - plan_offsets[s];
        if (n < 1) return fail(SPEC_ERR_PLAN, "stage %d is empty or out of order", s);
        if (n > *G) *G = n;
    }
    if (flags == SPEC_MLP_PARALLEL && *G > kMaxSel)
        return fail(SPEC_ERR_UNSUPPORTED, "parallel MLPs support sets of at most %d layers", kMaxSel);
    return SPEC_OK;
}

spec_status spec_draft_attention_cosine(const spec_model *draft, const spec_kv *kv, const int32_t *plan_offsets,
                                        int n_stages, int batch, const int32_t *tokens, int tokens_stride,
                                        const int32_t *positions, int max_pos, float *cos_out, int cos_stride,
                                        void *workspace, size_t ws_bytes, void *stream) {
    spec_status st = check_model(draft, kv, batch);
    if (st) return st;
    int G = 1;
    if ((st = check_plan(draft, plan_offsets, n_stages, SPEC_MLP_SEQUENTIAL, &G))) return st;
    if (!tokens || !positions || !cos_out) return fail(SPEC_ERR_INVALID_ARG, "NULL tokens/positions/cos_out");
    if (tokens_stride < 1 || cos_stride < draft->d.n_layers)
        return fail(SPEC_ERR_INVALID_ARG, "tokens_stride >= 1 and cos_stride >= n_layers required");
    if (max_pos < 0 || max_pos >= kv->capacity)
        return fail(SPEC_ERR_CAPACITY, "max_pos %d outside KV capacity %d", max_pos, kv->capacity);
    if ((st = check_ws(draft, batch, 1, G, workspace, ws_bytes))) return st;
    Fwd f{draft, kv, batch, 1, max_pos, RowMap{positions, nullptr, 1, kv->capacity}, workspace,
          carve(draft, batch, 1, G), (hipStream_t)stream, {0}};
    hipError_t e = run_embed(f, tokens, tokens_stride, 0);
    if (e != hipSuccess) return hip_fail(e, "embed");
    for (int s = 0; s < n_stages; ++s) {
        e = run_stage(f, plan_offsets[s], plan_offsets[s + 1] - plan_offsets[s], SPEC_MLP_SEQUENTIAL, NextNorm{},
                      cos_out, cos_stride);
        if (e != hipSuccess) return hip_fail(e, "cosine stage");
    }
    return SPEC_OK;
}

spec_status spec_draft_group_step(const spec_model *draft, const spec_kv *kv, const int32_t *plan_offsets,
                                  int n_stages, int flags, int batch, const int32_t *tokens, int tokens_stride,
                                  const int32_t *positions, int max_pos, float inv_temperature, uint64_t seed,
                                  float *logits_out, int64_t logits_stride, int32_t *token_out,
                                  int token_out_stride, void *workspace, size_t ws_bytes, void *stream) {
    spec_status st = check_model(draft, kv, batch);
    if (st) return st;
    int G = 1;
    if ((st = check_plan(draft, plan_offsets, n_stages, flags, &G))) return st;
    if (!tokens || !positions || !token_out) return fail(SPEC_ERR_INVALID_ARG, "NULL tokens/positions/token_out");
    if (tokens_stride < 1 || token_out_stride < 1) return fail(SPEC_ERR_INVALID_ARG, "strides must be >= 1");
    if (logits_out && logits_stride < draft->d.vocab) return fail(SPEC_ERR_INVALID_ARG, "logits_stride < vocab");
    if (max_pos < 0 || max_pos >= kv->capacity)
        return fail(SPEC_ERR_CAPACITY, "max_pos %d outside KV capacity %d", max_pos, kv->capacity);
    if (!(inv_temperature >= 0.f)) return fail(SPEC_ERR_INVALID_ARG, "inv_temperature must be >= 0");
    if ((st = check_ws(draft, batch, 1, G, workspace, ws_bytes))) return st;

    Fwd f{draft, kv, batch, 1, max_pos, RowMap{positions, nullptr, 1, kv->capacity}, workspace,
          carve(draft, batch, 1, G), (hipStream_t)stream, {0}};
    hipError_t e = run_embed(f, tokens, tokens_stride, 0);
    if (e != hipSuccess) return hip_fail(e, "embed");
    for (int s = 0; s < n_stages; ++s) {
        const NextNorm nn = s + 1 < n_stages ? next_qkv(draft, plan_offsets[s + 1], plan_offsets[s + 2] - plan_offsets[s + 1])
                                             : head_norm(draft, EPI_LOGITS);
        e = run_stage(f, plan_offsets[s], plan_offsets[s + 1] - plan_offsets[s], flags, nn);
        if (e != hipSuccess) return hip_fail(e, "draft stage");
    }
    // the sampled token is the one at position positions[b] + 1
    e = run_head(f, false, nullptr, logits_out, logits_stride, inv_temperature, seed, positions, nullptr, 1,
                 token_out, token_out_stride);
    if (e != hipSuccess) return hip_fail(e, "draft head");
    return SPEC_OK;
}

spec_status spec_draft_group_step_noalloc(const spec_model *draft, const spec_kv *kv, const int32_t *plan_offsets,
                                          int n_stages, int flags, int batch, const int32_t *tokens, int tokens_stride,
                                          const int32_t *positions, int max_pos, float inv_temperature, uint64_t seed,
                                          float *logits_out, int64_t logits_stride, int32_t *token_out,
                                          int token_out_stride, void *stream) {
    // the size check needs the plan's largest set; the full argument checks
    // run again in spec_draft_group_step before anything is launched
    spec_status st = check_model(draft, kv, batch);
    if (st) return st;
    int G = 1;
    if ((st = check_plan(draft, plan_offsets, n_stages, flags, &G))) return st;
    const size_t need = spec_workspace_bytes(draft, batch, 1, G);
    if (need > SPEC_SCRATCH_BYTES)
        return fail(SPEC_ERR_WORKSPACE, "draft step needs %zu bytes of workspace > scratch array %zu", need,
                    (size_t)SPEC_SCRATCH_BYTES);
    void *ws = nullptr;
    if ((st = scratch_address(&ws))) return st;
    return spec_draft_group_step(draft, kv, plan_offsets, n_stages, flags, batch, tokens, tokens_stride, positions,
                                 max_pos, inv_temperature, seed, logits_out, logits_stride, token_out,
                                 token_out_stride, ws, SPEC_SCRATCH_BYTES, stream);
}

static spec_status precise_forward(const spec_model *m, const spec_kv *kv, int batch, const int32_t *tokens,
                                   int tokens_stride, const int32_t *start_pos, const int32_t *n_tokens, int mseq,
                                   int max_pos,
                                   void *ws, hipStream_t s, Fwd &f, const NextNorm &head) {
    f = Fwd{m, kv, batch, mseq, max_pos, RowMap{start_pos, n_tokens, mseq, kv->capacity}, ws,
            carve(m, batch, mseq, 1), s, {0}};
    hipError_t e = run_embed(f, tokens, tokens_stride, 1);
    if (e != hipSuccess) return hip_fail(e, "embed");
    for (int l = 0; l < m->d.n_layers; ++l) {
        e = run_stage(f, l, 1, SPEC_MLP_SEQUENTIAL, l + 1 < m->d.n_layers ? next_qkv(m, l + 1, 1) : head);
        if (e != hipSuccess) return hip_fail(e, "layer");
    }
    return SPEC_OK;
}

spec_status spec_calibrate_kv(const spec_model *draft, const spec_kv *kv, int batch, const int32_t *tokens,
                              int tokens_stride, const int32_t *start_pos, const int32_t *n_tokens, int max_m,
                              int max_pos,
                              float inv_temperature, uint64_t seed, float *last_logits_out, int64_t logits_stride,
                              int32_t *token_out, int token_out_stride, void *workspace, size_t ws_bytes,
                              void *stream) {
    spec_status st = check_model(draft, kv, batch);
    if (st) return st;
    if (!tokens || !start_pos || !token_out) return fail(SPEC_ERR_INVALID_ARG, "NULL tokens/start_pos/token_out");
    if (max_m < 1) return fail(SPEC_ERR_INVALID_ARG, "max_m %d < 1", max_m);
    if (tokens_stride < max_m) return fail(SPEC_ERR_INVALID_ARG, "tokens_stride %d < max_m %d", tokens_stride, max_m);
    if (token_out_stride < 1) return fail(SPEC_ERR_INVALID_ARG, "token_out_stride < 1");
    if (last_logits_out && logits_stride < draft->d.vocab) return fail(SPEC_ERR_INVALID_ARG, "logits_stride < vocab");
    if (max_pos < 0 || max_pos >= kv->capacity)
        return fail(SPEC_ERR_CAPACITY, "max_pos %d outside KV capacity %d", max_pos, kv->capacity);
    if (!(inv_temperature >= 0.f)) return fail(SPEC_ERR_INVALID_ARG, "inv_temperature must be >= 0");
    if ((st = check_ws(draft, batch, max_m, 1, workspace, ws_bytes))) return st;
    Fwd f;
    // the head reads each sequence's last valid row: no operand to prepare
    if ((st = precise_forward(draft, kv, batch, tokens, tokens_stride, start_pos, n_tokens, max_m, max_pos,
                              workspace, (hipStream_t)stream, f, NextNorm{})))
        return st;
    // the sampled token is the one after the last calibrated position:
    // start_pos[b] + n_tokens[b] (n_tokens NULL: every sequence has max_m)
    hipError_t e = run_head(f, true, n_tokens, last_logits_out, logits_stride, inv_temperature, seed, start_pos,
                            n_tokens, max_m, token_out, token_out_stride);
    if (e != hipSuccess) return hip_fail(e, "calibrate head");
    return SPEC_OK;
}

spec_status spec_verify_forward(const spec_model *base, const spec_kv *kv, int batch, const int32_t *tokens,
                                const int32_t *start_pos, int m, int max_pos, float *logits_out, void *workspace,
                                size_t ws_bytes, void *stream) {
    spec_status st = check_model(base, kv, batch);
    if (st) return st;
    if (!tokens || !start_pos) return fail(SPEC_ERR_INVALID_ARG, "NULL tokens/start_pos");
    if (m < 1) return fail(SPEC_ERR_INVALID_ARG, "m %d < 1", m);
    if (max_pos < 0 || max_pos >= kv->capacity)
        return fail(SPEC_ERR_CAPACITY, "max_pos %d outside KV capacity %d", max_pos, kv->capacity);
    if ((st = check_ws(base, batch, m, 1, workspace, ws_bytes))) return st;
    Fwd f;
    if ((st = precise_forward(base, kv, batch, tokens, m, start_pos, nullptr, m, max_pos, workspace,
                              (hipStream_t)stream, f, logits_out ? head_norm(base, EPI_STORE) : NextNorm{})))
        return st;
    if (logits_out) {
        hipError_t e = run_head(f, false, nullptr, logits_out, base->d.vocab, 0.f, 0, nullptr, nullptr, 0, nullptr, 1);
        if (e != hipSuccess) return hip_fail(e, "verify head");
    }
    return SPEC_OK;
}

size_t spec_accept_workspace_bytes(int batch, int k, int vocab) {
    if (batch < 1 || k < 0 || vocab < 2) return 0;
    const size_t nch = accept_chunks(vocab);
    size_t t = 0;
    t += align_up((size_t)batch * (2 * k + 1) * nch * 2 * 4);
    t += align_up((size_t)batch * (2 * k + 1) * nch * 4);
    t += align_up((size_t)batch * nch * 2 * 4);
    t += align_up((size_t)batch * nch * 2 * 4);
    t += align_up((size_t)batch * 2 * 4);
    return t;
}

spec_status spec_accept_resample(int batch, int k, int vocab, const float *p_logits, const float *q_logits,
                                 const int32_t *draft_tokens, int draft_stride, const int32_t *round_pos,
                                 float inv_temperature, uint64_t seed, int32_t *n_accepted_out, int32_t *next_token_out,
                                 int next_token_stride, int32_t *commit_out, void *workspace, size_t ws_bytes,
                                 void *stream) {
    if (batch < 1 || k < 0 || vocab < 2) return fail(SPEC_ERR_SHAPE, "batch %d, k %d, vocab %d", batch, k, vocab);
    if (k > 64) return fail(SPEC_ERR_UNSUPPORTED, "k %d > 64", k);
    if (!p_logits || !round_pos || !n_accepted_out || !next_token_out)
        return fail(SPEC_ERR_INVALID_ARG, "NULL p_logits/round_pos/outputs");
    if (k > 0 && !draft_tokens) return fail(SPEC_ERR_INVALID_ARG, "NULL draft_tokens");
    if (k > 0 && draft_stride < k) return fail(SPEC_ERR_INVALID_ARG, "draft_stride %d < k %d", draft_stride, k);
    if (k > 0 && inv_temperature != 0.f && !q_logits) return fail(SPEC_ERR_INVALID_ARG, "NULL q_logits");
    if (!(inv_temperature >= 0.f)) return fail(SPEC_ERR_INVALID_ARG, "inv_temperature must be >= 0");
    if (next_token_stride < 1) return fail(SPEC_ERR_INVALID_ARG, "next_token_stride < 1");
    const size_t need = spec_accept_workspace_bytes(batch, k, vocab);
    if (!workspace || ws_bytes < need) return fail(SPEC_ERR_WORKSPACE, "workspace %zu < %zu", ws_bytes, need);
    AcceptParams p{};
    p.batch = batch; p.k = k; p.vocab = vocab; p.nchunk = accept_chunks(vocab);
    p.p_logits = p_logits; p.q_logits = q_logits; p.drafts = draft_tokens; p.draft_stride = draft_stride; p.round_pos = round_pos;
    p.inv_temp = inv_temperature; p.seed = seed;
    size_t off = 0;
    const size_t nch = p.nchunk;
    p.stats = at<float>(workspace, off); off += align_up((size_t)batch * (2 * k + 1) * nch * 2 * 4);
    p.stats_idx = at<int32_t>(workspace, off); off += align_up((size_t)batch * (2 * k + 1) * nch * 4);
    p.cand_val = at<float>(workspace, off); off += align_up((size_t)batch * nch * 2 * 4);
    p.cand_idx = at<int32_t>(workspace, off); off += align_up((size_t)batch * nch * 2 * 4);
    p.decision = at<int32_t>(workspace, off);
    p.n_acc_out = n_accepted_out; p.next_out = next_token_out; p.next_stride = next_token_stride;
    p.commit_out = commit_out;
    hipError_t e = launch_accept(p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "accept");
    return SPEC_OK;
}

}  // extern "C"
