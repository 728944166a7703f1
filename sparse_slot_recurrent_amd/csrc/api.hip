// C ABI of the RAM-Net layer (declared in include/ramnet.h): host-side
// validation, workspace layout and kernel dispatch.  Nothing here touches
// the GPU until every argument has been checked.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "launch.h"
#include "ramnet.h"

namespace {

thread_local std::string g_last_error;

ramnet_status fail(ramnet_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

ramnet_status ok() {
    g_last_error.clear();
    return RAMNET_OK;
}

constexpr int64_t kMaxSlots = int64_t(1) << 30;
constexpr int64_t kMaxTokenHeads = int64_t(1) << 40;

ramnet_status check_params(const ramnet_params *p, bool step) {
    if (!p) return fail(RAMNET_EINVAL, "params is NULL");
    if (p->B < 0 || p->T < 0 || p->H < 0)
        return fail(RAMNET_EINVAL, "B, T, H must be >= 0 (got %d, %d, %d)", p->B, p->T, p->H);
    if (step && p->T != 1) return fail(RAMNET_EINVAL, "a decode step needs T == 1 (got %d)", p->T);
    if (static_cast<int64_t>(p->B) * p->T * p->H > kMaxTokenHeads)
        return fail(RAMNET_EINVAL, "B*T*H exceeds 2^40");
    if (p->d_p < 2 || p->U < 1) return fail(RAMNET_EINVAL, "need d_p >= 2 and U >= 1");
    int64_t M = 1;
    for (int u = 0; u < p->U; ++u) {
        M *= p->d_p;
        if (M > kMaxSlots) return fail(RAMNET_EINVAL, "d_p^U exceeds 2^30 slots");
    }
    if (p->M != M)
        return fail(RAMNET_EINVAL, "M = %lld but d_p^U = %lld", static_cast<long long>(p->M),
                    static_cast<long long>(M));
    if (p->K < 1 || p->K > M) return fail(RAMNET_EINVAL, "K = %d outside [1, M]", p->K);
    if (p->d_v < 1) return fail(RAMNET_EINVAL, "d_v must be >= 1");
    if (p->in_dtype != RAMNET_F32 && p->in_dtype != RAMNET_BF16)
        return fail(RAMNET_EINVAL, "unknown in_dtype %d", p->in_dtype);
    if (p->state_dtype != RAMNET_F32 && p->state_dtype != RAMNET_BF16)
        return fail(RAMNET_EINVAL, "unknown state_dtype %d", p->state_dtype);
    if (p->cape < 0 || p->cape > 3) return fail(RAMNET_EINVAL, "cape must be 0, 1, 2 or 3");
    if (!(p->eps_gsu >= 0.f) || !isfinite(p->eps_gsu) || !(p->eps_norm >= 0.f) ||
        !isfinite(p->eps_norm))
        return fail(RAMNET_EINVAL, "eps_gsu and eps_norm must be finite and >= 0");
    if (p->K > RAMNET_KMAX)
        return fail(RAMNET_EUNSUPPORTED, "K = %d exceeds RAMNET_KMAX = %d", p->K, RAMNET_KMAX);
    if (p->d_p > 8) return fail(RAMNET_EUNSUPPORTED, "d_p = %d > 8 is not built", p->d_p);
    if (p->d_v % 64 != 0 || p->d_v > 256)
        return fail(RAMNET_EUNSUPPORTED, "d_v = %d: only 64, 128, 192, 256 are built", p->d_v);
    return RAMNET_OK;
}

struct Span {
    const char *name;
    uintptr_t lo, hi;  // [lo, hi)
};

Span span(const char *name, const void *p, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Span{name, lo, lo + bytes};
}

bool overlaps(const Span &a, const Span &b) {
    return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi;
}

ramnet_status check_ptr(const char *name, const void *p, bool required) {
    if (!p) {
        if (required) return fail(RAMNET_EINVAL, "%s is NULL", name);
        return RAMNET_OK;
    }
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
        return fail(RAMNET_EINVAL, "%s is not 16-byte aligned", name);
    return RAMNET_OK;
}

// Written buffers must not overlap each other or any other buffer.
ramnet_status check_overlaps(const Span *spans, int n, int first_written) {
    for (int i = first_written; i < n; ++i)
        for (int j = 0; j < n; ++j)
            if (i != j && overlaps(spans[i], spans[j]))
                return fail(RAMNET_EINVAL, "%s overlaps %s", spans[i].name, spans[j].name);
    return RAMNET_OK;
}

size_t in_bytes(const ramnet_params *p) { return p->in_dtype == RAMNET_BF16 ? 2 : 4; }
size_t st_bytes(const ramnet_params *p) { return p->state_dtype == RAMNET_BF16 ? 2 : 4; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// How a layer call runs and what scratch it needs.
struct LayerPlan {
    bool chunked;
    ramnet::ChunkPlan cp;
    size_t addr_bytes;   // decoded addresses kept in the workspace
    size_t fails_bytes;  // the decoder's failure words
    size_t chunk_bytes;  // chunked-path scratch
    size_t total() const { return addr_bytes + fails_bytes + chunk_bytes; }
};


// addr_in_ws: the decoded addresses are kept in the workspace; decodes: the
// call decodes q and k (no addr_in).
LayerPlan plan_layer(const ramnet_params *p, bool step, bool addr_in_ws, bool decodes) {
    LayerPlan lp{};
    const int64_t n = static_cast<int64_t>(p->B) * p->T * p->H;
    const bool sbf = p->state_dtype == RAMNET_BF16;
    lp.chunked = false;
    if (!step) {
        lp.cp = ramnet::plan_chunked(p->M, p->K, p->d_v, p->B, p->T, p->H, p->in_dtype == RAMNET_BF16, sbf);
        lp.chunked = lp.cp.ok;
    }
    // The fused decoding step keeps its addresses on chip.
    const bool fused_step = step && ramnet::step_fused_supported(p->K, p->d_p, p->U, p->d_v, p->state_dtype == RAMNET_BF16);
    lp.addr_bytes = addr_in_ws && !fused_step ? 4 * align256(static_cast<size_t>(n) * p->K * 4) : 0;
    lp.fails_bytes = decodes && !fused_step && p->K <= 32 ? align256(ramnet::decode_fails_bytes(n)) : 0;
    lp.chunk_bytes = lp.chunked ? ramnet::chunk_workspace_bytes(lp.cp) : 0;
    return lp;
}

ramnet_addr carve_addr(void *ws, int64_t n, int K) {
    const size_t one = align256(static_cast<size_t>(n) * K * 4);
    char *base = static_cast<char *>(ws);
    return ramnet_addr{reinterpret_cast<int32_t *>(base), reinterpret_cast<float *>(base + one),
                       reinterpret_cast<int32_t *>(base + 2 * one),
                       reinterpret_cast<float *>(base + 3 * one)};
}

ramnet_status check_addr(const char *what, const ramnet_addr *a) {
    ramnet_status s;
    std::string nm = what;
    if ((s = check_ptr((nm + ".w_idx").c_str(), a->w_idx, true))) return s;
    if ((s = check_ptr((nm + ".w_wt").c_str(), a->w_wt, true))) return s;
    if ((s = check_ptr((nm + ".r_idx").c_str(), a->r_idx, true))) return s;
    if ((s = check_ptr((nm + ".r_wt").c_str(), a->r_wt, true))) return s;
    return RAMNET_OK;
}

ramnet_status hip_status(hipError_t e, const char *where) {
    if (e == hipSuccess) return ok();
    return fail(RAMNET_EHIP, "%s: %s", where, hipGetErrorString(e));
}

ramnet::DecodeArgs decode_args(const ramnet_params *p, const void *q, const void *k,
                               const int32_t *pos0, int64_t n, int T, const ramnet_addr &o) {
    ramnet::DecodeArgs d{};
    d.q = q;
    d.k = k;
    d.n = n;
    d.T = T;
    d.H = p->H;
    d.U = p->U;
    d.K = p->K;
    d.d_p = p->d_p;
    d.pos0 = pos0;
    d.cape = p->cape;
    d.content_heads = p->content_heads;
    d.M = p->M;
    d.in_bf16 = p->in_dtype == RAMNET_BF16;
    d.w_idx = o.w_idx;
    d.w_wt = o.w_wt;
    d.r_idx = o.r_idx;
    d.r_wt = o.r_wt;
    return d;
}

// Elements between consecutive tokens (b, t) of each layer input; 0 means
// the contiguous layout of the public entry points.  The whole-layer path
// reads all five from one packed projection buffer.
struct Strides {
    int64_t qk = 0, v = 0, g = 0, gamma = 0;
};

// Bytes a [B*T rows] input with `width` elements per head spans.
size_t in_span(const ramnet_params *p, int64_t ld, size_t width) {
    const size_t rows = static_cast<size_t>(p->B) * p->T;
    const size_t hw = static_cast<size_t>(p->H) * width;
    if (!ld) return rows * hw * in_bytes(p);
    return ((rows - 1) * static_cast<size_t>(ld) + hw) * in_bytes(p);
}

// Shared body of prefill (T tokens) and the decode step (T = 1).
ramnet_status run_layer(const ramnet_params *p, bool step, const void *q, const void *k,
                        const void *v, const void *gamma, const void *g, const float *norm_w,
                        const int32_t *pos, void *S, float *mass, void *out,
                        const ramnet_addr *addr_in, const ramnet_addr *addr_out, void *ws,
                        size_t ws_bytes, void *stream, void *out_bf16 = nullptr,
                        const Strides &sd = Strides{}) {
    ramnet_status s = check_params(p, step);
    if (s) return s;
    const int64_t n = static_cast<int64_t>(p->B) * p->T * p->H;
    const int64_t units = static_cast<int64_t>(p->B) * p->H;
    const bool decode = addr_in == nullptr;
    if (n == 0) return ok();
    if (decode) {
        if ((s = check_ptr("q", q, true)) || (s = check_ptr("k", k, true))) return s;
        if (step && p->cape && !pos) return fail(RAMNET_EINVAL, "pos is required when cape != 0");
        if ((s = check_ptr(step ? "pos" : "pos0", pos, false))) return s;
    } else if ((s = check_addr("addr_in", addr_in))) {
        return s;
    }
    if ((s = check_ptr("v", v, true)) || (s = check_ptr("gamma", gamma, true)) ||
        (s = check_ptr("g", g, true)) || (s = check_ptr("norm_w", norm_w, false)) ||
        (s = check_ptr("S", S, true)) || (s = check_ptr("mass", mass, true)) ||
        (s = check_ptr("out", out, true)))
        return s;
    if (addr_out && (s = check_addr("addr_out", addr_out))) return s;

    const size_t L = static_cast<size_t>(p->U) * p->d_p;
    const size_t nK4 = static_cast<size_t>(n) * p->K * 4;
    Span sp[16];
    int ns = 0;
    // read-only buffers first
    if (decode) {
        sp[ns++] = span("q", q, in_span(p, sd.qk, L));
        sp[ns++] = span("k", k, in_span(p, sd.qk, L));
        if (pos) sp[ns++] = span(step ? "pos" : "pos0", pos, p->B * sizeof(int32_t));
    } else {
        sp[ns++] = span("addr_in.w_idx", addr_in->w_idx, nK4);
        sp[ns++] = span("addr_in.w_wt", addr_in->w_wt, nK4);
        sp[ns++] = span("addr_in.r_idx", addr_in->r_idx, nK4);
        sp[ns++] = span("addr_in.r_wt", addr_in->r_wt, nK4);
    }
    sp[ns++] = span("v", v, in_span(p, sd.v, p->d_v));
    sp[ns++] = span("gamma", gamma, in_span(p, sd.gamma, 1));
    sp[ns++] = span("g", g, in_span(p, sd.g, p->d_v));
    if (norm_w) sp[ns++] = span("norm_w", norm_w, p->d_v * sizeof(float));
    const int first_written = ns;
    sp[ns++] = span("S", S, units * p->M * p->d_v * st_bytes(p));
    sp[ns++] = span("mass", mass, units * p->M * sizeof(float));
    sp[ns++] = span("out", out, n * p->d_v * st_bytes(p));
    if (addr_out) {
        sp[ns++] = span("addr_out.w_idx", addr_out->w_idx, nK4);
        sp[ns++] = span("addr_out.w_wt", addr_out->w_wt, nK4);
        sp[ns++] = span("addr_out.r_idx", addr_out->r_idx, nK4);
        sp[ns++] = span("addr_out.r_wt", addr_out->r_wt, nK4);
    }
    const LayerPlan lp = plan_layer(p, step, decode && !addr_out, decode);
    const size_t need = lp.total();
    if (need > 0) {
        if (!ws || ws_bytes < need)
            return fail(RAMNET_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                        ws ? ws_bytes : size_t(0));
        if ((s = check_ptr("workspace", ws, true))) return s;
        sp[ns++] = span("workspace", ws, need);
    }
    if ((s = check_overlaps(sp, ns, first_written))) return s;

    hipStream_t st = static_cast<hipStream_t>(stream);
    if (step && ramnet::step_fused_supported(p->K, p->d_p, p->U, p->d_v, p->state_dtype == RAMNET_BF16)) {
        ramnet::StepArgs sa{};
        sa.B = p->B;
        sa.H = p->H;
        sa.M = p->M;
        sa.K = p->K;
        sa.d_v = p->d_v;
        sa.U = p->U;
        sa.d_p = p->d_p;
        sa.cape = p->cape;
        sa.content_heads = p->content_heads;
        sa.in_bf16 = p->in_dtype == RAMNET_BF16;
        sa.state_bf16 = p->state_dtype == RAMNET_BF16;
        sa.q = q;
        sa.k = k;
        sa.v = v;
        sa.gamma = gamma;
        sa.g = g;
        sa.norm_w = norm_w;
        sa.pos = pos;
        sa.S = S;
        sa.mass = mass;
        sa.out = out;
        sa.out_idx[0] = addr_out ? addr_out->w_idx : nullptr;
        sa.out_idx[1] = addr_out ? addr_out->r_idx : nullptr;
        sa.out_wt[0] = addr_out ? addr_out->w_wt : nullptr;
        sa.out_wt[1] = addr_out ? addr_out->r_wt : nullptr;
        sa.eps_gsu = p->eps_gsu;
        sa.eps_norm = p->eps_norm;
        sa.ld_qk = sd.qk;
        sa.ld_v = sd.v;
        sa.ld_g = sd.g;
        sa.ld_gamma = sd.gamma;
        hipError_t e = ramnet::launch_step_fused(sa, st);
        if (e == hipSuccess && out_bf16)
            e = ramnet::launch_to_bf16(static_cast<const float *>(out), out_bf16, n * p->d_v, st);
        return hip_status(e, "decode step launch");
    }
    ramnet_addr addr;
    // Addresses kept in the workspace for the slot-grouped path are laid out
    // [B,H,T,K], so that each head's chunk of addresses is contiguous.
    bool unit_major = false;
    if (decode) {
        addr = lp.addr_bytes ? carve_addr(ws, n, p->K) : *addr_out;
        ramnet::DecodeArgs da = decode_args(p, q, k, pos, n, p->T, addr);
        unit_major = da.unit_major = lp.addr_bytes && lp.chunked;
        da.ld = sd.qk;
        if (lp.fails_bytes)
            da.fails = reinterpret_cast<unsigned long long *>(static_cast<char *>(ws) + lp.addr_bytes);
        hipError_t e = ramnet::launch_decode(da, st);
        if (e != hipSuccess) return hip_status(e, "address decoder launch");
    } else {
        addr = *addr_in;
    }
    ramnet::ScanArgs a{};
    a.B = p->B;
    a.T = p->T;
    a.H = p->H;
    a.M = p->M;
    a.K = p->K;
    a.d_v = p->d_v;
    a.in_bf16 = p->in_dtype == RAMNET_BF16;
    a.state_bf16 = p->state_dtype == RAMNET_BF16;
    a.v = v;
    a.gamma = gamma;
    a.g = g;
    a.norm_w = norm_w;
    a.w_idx = addr.w_idx;
    a.w_wt = addr.w_wt;
    a.r_idx = addr.r_idx;
    a.r_wt = addr.r_wt;
    a.addr_unit_major = unit_major;
    a.S = S;
    a.mass = mass;
    a.out = out;
    a.eps_gsu = p->eps_gsu;
    a.eps_norm = p->eps_norm;
    a.ld_v = sd.v;
    a.ld_g = sd.g;
    a.ld_gamma = sd.gamma;
    hipError_t e;
    if (lp.chunked) {
        ramnet::ChunkArgs c{};
        static_cast<ramnet::ScanArgs &>(c) = a;
        c.p = lp.cp;
        char *cw = static_cast<char *>(ws) + lp.addr_bytes + lp.fails_bytes;
        if (lp.cp.ws_rbuf) {
            c.rbuf = reinterpret_cast<float *>(cw);
            cw += lp.cp.ws_rbuf;
        } else {
            c.rbuf = static_cast<float *>(out);  // fp32 output holds r until normalised
        }
        c.sumsq = reinterpret_cast<float *>(cw);
        cw += lp.cp.ws_sumsq;
        c.mass_ws = reinterpret_cast<float *>(cw);
        cw += lp.cp.ws_mass;
        c.plan = reinterpret_cast<unsigned char *>(cw);
        cw += lp.cp.ws_plan;
        c.partial = reinterpret_cast<float *>(cw);
        cw += lp.cp.ws_partial;
        c.spill = cw;
        c.out_bf16 = out_bf16;  // the epilogue writes bf16 directly
        e = ramnet::launch_scan_chunked(c, st);
    } else {
        e = ramnet::launch_scan_serial(a, st);
        if (e == hipSuccess && out_bf16)
            e = ramnet::launch_to_bf16(static_cast<const float *>(out), out_bf16, n * p->d_v, st);
    }
    if (e != hipSuccess) return hip_status(e, "scan launch");
    if (!decode && addr_out) {
        for (int i = 0; i < 4; ++i) {
            void *dst = i == 0 ? static_cast<void *>(addr_out->w_idx)
                      : i == 1 ? static_cast<void *>(addr_out->w_wt)
                      : i == 2 ? static_cast<void *>(addr_out->r_idx)
                               : static_cast<void *>(addr_out->r_wt);
            const void *src = i == 0 ? static_cast<const void *>(addr_in->w_idx)
                            : i == 1 ? static_cast<const void *>(addr_in->w_wt)
                            : i == 2 ? static_cast<const void *>(addr_in->r_idx)
                                     : static_cast<const void *>(addr_in->r_wt);
            e = hipMemcpyAsync(dst, src, nK4, hipMemcpyDeviceToDevice, st);
            if (e != hipSuccess) return hip_status(e, "address export copy");
        }
    }
    return ok();
}

// ---------------------------------------------------------------- whole layer

ramnet::PackLayout layout_of(const ramnet_params *p, int32_t d_model) {
    return ramnet::pack_layout(p->H, p->U * p->d_p, p->d_v, d_model);
}

// Workspace of the projected layer: the packed input weights (unless the
// caller packed them), hipBLASLt scratch, the packed projections [rows, N],
// the layer output (and its bf16 copy when the state is fp32), then the
// layer's own workspace.
struct FwdPlan {
    size_t o_pack, o_gemm, o_proj, o_out, o_out16, o_layer, total;
};

FwdPlan plan_forward(const ramnet_params *p, int32_t d_model, bool step) {
    FwdPlan f{};
    const ramnet::PackLayout pl = layout_of(p, d_model);
    const size_t rows = static_cast<size_t>(p->B) * p->T;
    const size_t n = rows * p->H;
    size_t o = 0;
    f.o_pack = o; o += align256(static_cast<size_t>(pl.D) * pl.N * 2);
    f.o_gemm = o; o += ramnet::kGemmWorkspace;
    f.o_proj = o; o += align256(rows * pl.N * 2);
    f.o_out = o; o += align256(n * p->d_v * st_bytes(p));
    f.o_out16 = o; o += p->state_dtype == RAMNET_BF16 ? 0 : align256(n * p->d_v * 2);
    f.o_layer = o; o += plan_layer(p, step, true, true).total();
    f.total = o;
    return f;
}

constexpr int32_t kMaxDModel = 1 << 16;

ramnet_status check_d_model(const ramnet_params *p, int32_t d_model) {
    if (p->in_dtype != RAMNET_BF16)
        return fail(RAMNET_EUNSUPPORTED, "the projections need in_dtype = RAMNET_BF16");
    if (d_model < 8 || d_model > kMaxDModel || d_model % 8)
        return fail(RAMNET_EINVAL, "d_model = %d: must be a multiple of 8 in [8, %d]", d_model,
                    kMaxDModel);
    return RAMNET_OK;
}

// The separate input weights (needed unless a packed matrix is given).
ramnet_status check_input_weights(const ramnet_proj *w) {
    ramnet_status s;
    if ((s = check_ptr("w_q", w->w_q, true)) || (s = check_ptr("w_k", w->w_k, true)) ||
        (s = check_ptr("w_v", w->w_v, true)) || (s = check_ptr("w_g", w->w_g, true)) ||
        (s = check_ptr("w_gamma", w->w_gamma, true)) || (s = check_ptr("alpha", w->alpha, false)))
        return s;
    return RAMNET_OK;
}

ramnet_status check_proj(const ramnet_params *p, const ramnet_proj *w, bool need_o) {
    if (!w) return fail(RAMNET_EINVAL, "w is NULL");
    ramnet_status s;
    if ((s = check_d_model(p, w->d_model))) return s;
    if (w->w_in_packed) {
        if ((s = check_ptr("w_in_packed", w->w_in_packed, true))) return s;
    } else if ((s = check_input_weights(w))) {
        return s;
    }
    if (need_o && (s = check_ptr("w_o", w->w_o, true))) return s;
    return RAMNET_OK;
}

// Read-only spans of the weights a call uses.
int weight_spans(const ramnet_params *p, const ramnet_proj *w, bool with_o, Span *sp) {
    const size_t D = w->d_model;
    const ramnet::PackLayout pl = layout_of(p, w->d_model);
    int ns = 0;
    if (w->w_in_packed) {
        sp[ns++] = span("w_in_packed", w->w_in_packed, D * pl.N * 2);
    } else {
        sp[ns++] = span("w_q", w->w_q, D * pl.HL * 2);
        sp[ns++] = span("w_k", w->w_k, D * pl.HL * 2);
        sp[ns++] = span("w_v", w->w_v, D * pl.HV * 2);
        sp[ns++] = span("w_g", w->w_g, D * pl.HV * 2);
        sp[ns++] = span("w_gamma", w->w_gamma, D * p->H * 2);
        if (w->alpha) sp[ns++] = span("alpha", w->alpha, p->H * sizeof(float));
    }
    if (with_o) sp[ns++] = span("w_o", w->w_o, static_cast<size_t>(pl.HV) * D * 2);
    return ns;
}

// Validates every GEMM shape of the call (creating the handle), so that a
// failure is reported before anything is enqueued.
ramnet_status prepare_gemms(const ramnet_params *p, const ramnet_proj *w, int64_t rows,
                            bool with_o) {
    const ramnet::PackLayout pl = layout_of(p, w->d_model);
    std::string err;
    if (!ramnet::gemm_prepare(rows, pl.N, w->d_model, err) ||
        (with_o && !ramnet::gemm_prepare(rows, w->d_model, pl.HV, err)))
        return fail(RAMNET_EHIP, "%s", err.c_str());
    return RAMNET_OK;
}

// Enqueues the packing of the input weights (unless given packed) and the
// one input GEMM into proj [rows, N].
ramnet_status enqueue_inputs(const ramnet_params *p, const ramnet_proj *w, const void *x,
                             int64_t rows, void *proj, char *ws, const FwdPlan &f,
                             hipStream_t st) {
    const ramnet::PackLayout pl = layout_of(p, w->d_model);
    const void *packed = w->w_in_packed;
    if (!packed) {
        const hipError_t e = ramnet::launch_pack(w->w_q, w->w_k, w->w_v, w->w_g, w->w_gamma,
                                                 w->alpha, ws + f.o_pack, pl, st);
        if (e != hipSuccess) return hip_status(e, "weight packing launch");
        packed = ws + f.o_pack;
    }
    std::string err;
    if (!ramnet::gemm_bf16(x, packed, proj, rows, pl.N, w->d_model, ws + f.o_gemm, st, err))
        return fail(RAMNET_EHIP, "%s", err.c_str());
    return RAMNET_OK;
}

ramnet_status check_workspace(size_t need, void *ws, size_t ws_bytes) {
    if (!ws || ws_bytes < need)
        return fail(RAMNET_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    ws ? ws_bytes : size_t(0));
    return check_ptr("workspace", ws, true);
}

ramnet_status run_whole_layer(const ramnet_params *p, bool step, const ramnet_proj *w,
                              const void *x, const float *norm_w, const int32_t *pos, void *S,
                              float *mass, void *y, const ramnet_addr *addr_out, void *ws,
                              size_t ws_bytes, void *stream) {
    ramnet_status s = check_params(p, step);
    if (s || (s = check_proj(p, w, true))) return s;
    const int64_t rows = static_cast<int64_t>(p->B) * p->T;
    const int64_t n = rows * p->H;
    if (n == 0) return ok();
    if (step && p->cape && !pos) return fail(RAMNET_EINVAL, "pos is required when cape != 0");
    if ((s = check_ptr("x", x, true)) || (s = check_ptr("norm_w", norm_w, false)) ||
        (s = check_ptr(step ? "pos" : "pos0", pos, false)) || (s = check_ptr("S", S, true)) ||
        (s = check_ptr("mass", mass, true)) || (s = check_ptr("y", y, true)))
        return s;
    if (addr_out && (s = check_addr("addr_out", addr_out))) return s;
    const FwdPlan f = plan_forward(p, w->d_model, step);
    if ((s = check_workspace(f.total, ws, ws_bytes))) return s;
    const size_t D = w->d_model;
    const size_t nK4 = static_cast<size_t>(n) * p->K * 4;
    Span sp[20];
    int ns = weight_spans(p, w, true, sp);
    sp[ns++] = span("x", x, rows * D * 2);
    if (norm_w) sp[ns++] = span("norm_w", norm_w, p->d_v * sizeof(float));
    if (pos) sp[ns++] = span(step ? "pos" : "pos0", pos, p->B * sizeof(int32_t));
    const int first_written = ns;
    sp[ns++] = span("S", S, static_cast<size_t>(p->B) * p->H * p->M * p->d_v * st_bytes(p));
    sp[ns++] = span("mass", mass, static_cast<size_t>(p->B) * p->H * p->M * sizeof(float));
    sp[ns++] = span("y", y, rows * D * 2);
    if (addr_out) {
        sp[ns++] = span("addr_out.w_idx", addr_out->w_idx, nK4);
        sp[ns++] = span("addr_out.w_wt", addr_out->w_wt, nK4);
        sp[ns++] = span("addr_out.r_idx", addr_out->r_idx, nK4);
        sp[ns++] = span("addr_out.r_wt", addr_out->r_wt, nK4);
    }
    sp[ns++] = span("workspace", ws, f.total);
    if ((s = check_overlaps(sp, ns, first_written))) return s;
    if ((s = prepare_gemms(p, w, rows, true))) return s;

    hipStream_t st = static_cast<hipStream_t>(stream);
    char *wsb = static_cast<char *>(ws);
    char *proj = wsb + f.o_proj;
    if ((s = enqueue_inputs(p, w, x, rows, proj, wsb, f, st))) return s;
    // the layer reads its five inputs in place from the packed projections
    const ramnet::PackLayout pl = layout_of(p, w->d_model);
    Strides sd;
    sd.qk = sd.v = sd.g = sd.gamma = pl.N;
    const bool st16 = p->state_dtype == RAMNET_BF16;
    void *out = wsb + f.o_out;
    void *out16 = st16 ? out : wsb + f.o_out16;
    s = run_layer(p, step, proj, proj + 2 * pl.o_k, proj + 2 * pl.o_v, proj + 2 * pl.o_gamma,
                  proj + 2 * pl.o_g, norm_w, pos, S, mass, out, nullptr, addr_out,
                  wsb + f.o_layer, f.total - f.o_layer, stream, st16 ? nullptr : out16, sd);
    if (s) return s;
    std::string err;
    if (!ramnet::gemm_bf16(out16, w->w_o, y, rows, w->d_model, pl.HV, wsb + f.o_gemm, st, err))
        return fail(RAMNET_EHIP, "%s", err.c_str());
    return ok();
}

}  // namespace

// Scratch of ramnet_scan_prefill_noalloc: a static device array that every
// GPU the library runs on holds until the process ends.  Host code never
// passes `scratch` itself to a kernel or a copy (on the host the name is only
// a stand-in for the symbol); it uses the device address that
// hipGetSymbolAddress gives on each device.
static __device__ __align__(256) unsigned char scratch[RAMNET_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device

// The current device's address of `scratch`, looked up once per device
// with that device current.
ramnet_status scratch_of_current_device(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(RAMNET_EUNSUPPORTED, "device %d: the static scratch is kept for devices 0..%d",
                    dev, kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(RAMNET_EHIP, "hipGetSymbolAddress(scratch) gave NULL");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return RAMNET_OK;
}

}  // namespace

// ---------------------------------------------------------------- tiered state

namespace {

// Validates a tiered state for p and appends its buffers to sp (all of them
// written: the step moves rows and counts, the upkeep calls the maps).
ramnet_status check_tier(const ramnet_params *p, const ramnet_tiered_state *ts, Span *sp, int &ns) {
    if (!ts) return fail(RAMNET_EINVAL, "ts is NULL");
    const int64_t lim = std::min<int64_t>(p->M, RAMNET_TIER_CMAX);
    if (ts->C < 1 || ts->C > lim)
        return fail(RAMNET_EINVAL, "C = %d outside [1, %lld]", ts->C, static_cast<long long>(lim));
    ramnet_status s;
    if ((s = check_ptr("ts->S_host", ts->S_host, true)) || (s = check_ptr("ts->cache", ts->cache, true)) ||
        (s = check_ptr("ts->line_slot", ts->line_slot, true)) ||
        (s = check_ptr("ts->slot_line", ts->slot_line, true)) || (s = check_ptr("ts->hits", ts->hits, true)))
        return s;
    const size_t units = static_cast<size_t>(p->B) * p->H;
    const size_t rb = static_cast<size_t>(p->d_v) * st_bytes(p);
    sp[ns++] = span("ts->S_host", ts->S_host, units * p->M * rb);
    sp[ns++] = span("ts->cache", ts->cache, units * ts->C * rb);
    sp[ns++] = span("ts->line_slot", ts->line_slot, units * ts->C * 4);
    sp[ns++] = span("ts->slot_line", ts->slot_line, units * p->M * 4);
    sp[ns++] = span("ts->hits", ts->hits, units * p->M * 4);
    return RAMNET_OK;
}

ramnet::TierArgs tier_args(const ramnet_params *p, const ramnet_tiered_state *ts) {
    ramnet::TierArgs a{};
    a.units = p->B * p->H;
    a.C = ts->C;
    a.d_v = p->d_v;
    a.M = p->M;
    a.state_bf16 = p->state_dtype == RAMNET_BF16;
    a.S_host = ts->S_host;
    a.cache = ts->cache;
    a.line_slot = ts->line_slot;
    a.slot_line = ts->slot_line;
    a.hits = ts->hits;
    return a;
}

ramnet_status tier_upkeep(const ramnet_params *p, const ramnet_tiered_state *ts, void *stream,
                          hipError_t (*launch)(const ramnet::TierArgs &, hipStream_t), const char *what) {
    ramnet_status s = check_params(p, true);
    if (s) return s;
    Span sp[8];
    int ns = 0;
    if ((s = check_tier(p, ts, sp, ns)) || (s = check_overlaps(sp, ns, 0))) return s;
    if (static_cast<int64_t>(p->B) * p->H == 0) return ok();
    return hip_status(launch(tier_args(p, ts), static_cast<hipStream_t>(stream)), what);
}

}  // namespace

extern "C" {

size_t ramnet_layer_workspace_bytes(const ramnet_params *p, int32_t d_model) {
    const std::string saved = g_last_error;
    ramnet_status s = check_params(p, p && p->T == 1);
    if (s == RAMNET_OK) s = check_d_model(p, d_model);
    g_last_error = saved;
    if (s != RAMNET_OK) return 0;
    const FwdPlan a = plan_forward(p, d_model, false);
    if (p->T != 1) return a.total;
    const FwdPlan b = plan_forward(p, d_model, true);
    return a.total > b.total ? a.total : b.total;
}

size_t ramnet_packed_weights_bytes(const ramnet_params *p, int32_t d_model) {
    const std::string saved = g_last_error;
    ramnet_status s = check_params(p, false);
    if (s == RAMNET_OK) s = check_d_model(p, d_model);
    g_last_error = saved;
    if (s != RAMNET_OK) return 0;
    const ramnet::PackLayout pl = layout_of(p, d_model);
    return static_cast<size_t>(pl.D) * pl.N * 2;
}

ramnet_status ramnet_pack_weights(const ramnet_params *p, const ramnet_proj *w, void *packed,
                                  size_t packed_bytes, void *stream) {
    ramnet_status s = check_params(p, false);
    if (s) return s;
    if (!w) return fail(RAMNET_EINVAL, "w is NULL");
    if ((s = check_d_model(p, w->d_model)) || (s = check_input_weights(w)) ||
        (s = check_ptr("packed", packed, true)))
        return s;
    const ramnet::PackLayout pl = layout_of(p, w->d_model);
    const size_t need = static_cast<size_t>(pl.D) * pl.N * 2;
    if (packed_bytes < need)
        return fail(RAMNET_EINVAL, "packed needs %zu bytes, %zu given", need, packed_bytes);
    ramnet_proj wi = *w;
    wi.w_in_packed = nullptr;
    Span sp[8];
    int ns = weight_spans(p, &wi, false, sp);
    const int first_written = ns;
    sp[ns++] = span("packed", packed, need);
    if ((s = check_overlaps(sp, ns, first_written))) return s;
    return hip_status(ramnet::launch_pack(w->w_q, w->w_k, w->w_v, w->w_g, w->w_gamma, w->alpha,
                                          packed, pl, static_cast<hipStream_t>(stream)),
                      "weight packing launch");
}

ramnet_status ramnet_project_inputs(const ramnet_params *p, const ramnet_proj *w, const void *x,
                                    void *q, void *k, void *v, void *gamma, void *g,
                                    void *workspace, size_t workspace_bytes, void *stream) {
    ramnet_status s = check_params(p, false);
    if (s || (s = check_proj(p, w, false))) return s;
    const int64_t rows = static_cast<int64_t>(p->B) * p->T;
    const int64_t n = rows * p->H;
    if (n == 0) return ok();
    if ((s = check_ptr("x", x, true)) || (s = check_ptr("q", q, true)) ||
        (s = check_ptr("k", k, true)) || (s = check_ptr("v", v, true)) ||
        (s = check_ptr("gamma", gamma, true)) || (s = check_ptr("g", g, true)))
        return s;
    const FwdPlan f = plan_forward(p, w->d_model, false);
    // the packed weights, the GEMM scratch and the packed projections
    const size_t need = f.o_out;
    if ((s = check_workspace(need, workspace, workspace_bytes))) return s;
    const size_t L = static_cast<size_t>(p->U) * p->d_p;
    Span sp[16];
    int ns = weight_spans(p, w, false, sp);
    sp[ns++] = span("x", x, rows * static_cast<size_t>(w->d_model) * 2);
    const int first_written = ns;
    sp[ns++] = span("q", q, n * L * 2);
    sp[ns++] = span("k", k, n * L * 2);
    sp[ns++] = span("v", v, n * p->d_v * 2);
    sp[ns++] = span("g", g, n * p->d_v * 2);
    sp[ns++] = span("gamma", gamma, n * 2);
    sp[ns++] = span("workspace", workspace, need);
    if ((s = check_overlaps(sp, ns, first_written))) return s;
    if ((s = prepare_gemms(p, w, rows, false))) return s;
    char *wsb = static_cast<char *>(workspace);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((s = enqueue_inputs(p, w, x, rows, wsb + f.o_proj, wsb, f, st))) return s;
    return hip_status(ramnet::launch_split(wsb + f.o_proj, q, k, v, g, gamma, rows,
                                           layout_of(p, w->d_model), st),
                      "projection split launch");
}

ramnet_status ramnet_layer_forward(const ramnet_params *p, const ramnet_proj *w, const void *x,
                                   const float *norm_w, const int32_t *pos0, void *S, float *mass,
                                   void *y, const ramnet_addr *addr_out, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    return run_whole_layer(p, false, w, x, norm_w, pos0, S, mass, y, addr_out, workspace,
                           workspace_bytes, stream);
}

ramnet_status ramnet_layer_step(const ramnet_params *p, const ramnet_proj *w, const void *x,
                                const float *norm_w, const int32_t *pos, void *S, float *mass,
                                void *y, const ramnet_addr *addr_out, void *workspace,
                                size_t workspace_bytes, void *stream) {
    return run_whole_layer(p, true, w, x, norm_w, pos, S, mass, y, addr_out, workspace,
                           workspace_bytes, stream);
}


ramnet_status ramnet_decode_addresses(const ramnet_params *p, const void *q, const void *k,
                                      const int32_t *pos0, const ramnet_addr *out,
                                      void *stream) {
    ramnet_status s = check_params(p, false);
    if (s) return s;
    const int64_t n = static_cast<int64_t>(p->B) * p->T * p->H;
    if (!out) return fail(RAMNET_EINVAL, "out is NULL");
    if (n == 0) return ok();
    if ((s = check_ptr("q", q, true)) || (s = check_ptr("k", k, true)) ||
        (s = check_ptr("pos0", pos0, false)) || (s = check_addr("out", out)))
        return s;
    const size_t L = static_cast<size_t>(p->U) * p->d_p;
    const size_t nK4 = static_cast<size_t>(n) * p->K * 4;
    Span sp[9];
    int ns = 0;
    sp[ns++] = span("q", q, n * L * in_bytes(p));
    sp[ns++] = span("k", k, n * L * in_bytes(p));
    if (pos0) sp[ns++] = span("pos0", pos0, p->B * sizeof(int32_t));
    const int first_written = ns;
    sp[ns++] = span("out.w_idx", out->w_idx, nK4);
    sp[ns++] = span("out.w_wt", out->w_wt, nK4);
    sp[ns++] = span("out.r_idx", out->r_idx, nK4);
    sp[ns++] = span("out.r_wt", out->r_wt, nK4);
    if ((s = check_overlaps(sp, ns, first_written))) return s;
    hipError_t e = ramnet::launch_decode(decode_args(p, q, k, pos0, n, p->T, *out),
                                         static_cast<hipStream_t>(stream));
    return hip_status(e, "address decoder launch");
}

size_t ramnet_workspace_bytes(const ramnet_params *p, int32_t op) {
    const std::string saved = g_last_error;
    const bool step = op == RAMNET_OP_STEP;
    const ramnet_status s = check_params(p, step);
    g_last_error = saved;
    if (s != RAMNET_OK) return 0;
    if (op == RAMNET_OP_DECODE) return 0;
    if (op == RAMNET_OP_BACKWARD)
        return ramnet::backward_supported(p->M, p->d_v, p->U, p->d_p, p->state_dtype == RAMNET_BF16)
                   ? ramnet::backward_workspace_bytes(p->B, p->T, p->H, p->K, p->M, p->d_v,
                                                      p->state_dtype == RAMNET_BF16)
                   : 0;
    if (op != RAMNET_OP_PREFILL && op != RAMNET_OP_STEP) return 0;
    return plan_layer(p, step, true, true).total();
}

ramnet_status ramnet_scan_backward(const ramnet_params *p, const void *q, const void *k,
                                   const void *v, const void *gamma, const void *g,
                                   const float *norm_w, const int32_t *pos0, const void *S0,
                                   const float *mass0, const ramnet_addr *addr, const float *dout,
                                   const float *dS_final, const float *dmass_final, float *dq,
                                   float *dk, float *dv, float *dgamma, float *dg, float *dnorm_w,
                                   float *dS0, float *dmass0, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    ramnet_status s = check_params(p, false);
    if (s) return s;
    if (!ramnet::backward_supported(p->M, p->d_v, p->U, p->d_p, p->state_dtype == RAMNET_BF16))
        return fail(RAMNET_EUNSUPPORTED, "the backward pass is built for U*d_p <= 64");
    const int64_t n = static_cast<int64_t>(p->B) * p->T * p->H;
    const int64_t units = static_cast<int64_t>(p->B) * p->H;
    if (n == 0) return ok();
    if (!addr) return fail(RAMNET_EINVAL, "addr is NULL");
    if ((s = check_ptr("v", v, true)) || (s = check_ptr("gamma", gamma, true)) ||
        (s = check_ptr("g", g, true)) || (s = check_ptr("norm_w", norm_w, false)) ||
        (s = check_ptr("pos0", pos0, false)) || (s = check_ptr("S0", S0, true)) ||
        (s = check_ptr("mass0", mass0, true)) || (s = check_addr("addr", addr)) ||
        (s = check_ptr("dout", dout, true)) || (s = check_ptr("dS_final", dS_final, false)) ||
        (s = check_ptr("dmass_final", dmass_final, false)) || (s = check_ptr("dq", dq, false)) ||
        (s = check_ptr("dk", dk, false)) || (s = check_ptr("dv", dv, true)) ||
        (s = check_ptr("dgamma", dgamma, true)) ||
        (s = check_ptr("dg", dg, true)) || (s = check_ptr("dnorm_w", dnorm_w, false)) ||
        (s = check_ptr("dS0", dS0, true)) || (s = check_ptr("dmass0", dmass0, true)))
        return s;
    if (dq && (s = check_ptr("q", q, true))) return s;
    if (dk && (s = check_ptr("k", k, true))) return s;
    const size_t need = ramnet::backward_workspace_bytes(p->B, p->T, p->H, p->K, p->M, p->d_v,
                                                         p->state_dtype == RAMNET_BF16);
    if (!workspace || workspace_bytes < need)
        return fail(RAMNET_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : size_t(0));
    if ((s = check_ptr("workspace", workspace, true))) return s;
    const size_t L = static_cast<size_t>(p->U) * p->d_p;
    const size_t nK4 = static_cast<size_t>(n) * p->K * 4;
    const size_t nv = static_cast<size_t>(n) * p->d_v;
    const size_t st = static_cast<size_t>(units) * p->M;
    Span sp[32];
    int ns = 0;
    if (dq) sp[ns++] = span("q", q, n * L * in_bytes(p));
    if (dk) sp[ns++] = span("k", k, n * L * in_bytes(p));
    sp[ns++] = span("v", v, nv * in_bytes(p));
    sp[ns++] = span("gamma", gamma, n * in_bytes(p));
    sp[ns++] = span("g", g, nv * in_bytes(p));
    if (norm_w) sp[ns++] = span("norm_w", norm_w, p->d_v * sizeof(float));
    if (pos0) sp[ns++] = span("pos0", pos0, p->B * sizeof(int32_t));
    sp[ns++] = span("S0", S0, st * p->d_v * st_bytes(p));
    sp[ns++] = span("mass0", mass0, st * 4);
    sp[ns++] = span("addr.w_idx", addr->w_idx, nK4);
    sp[ns++] = span("addr.w_wt", addr->w_wt, nK4);
    sp[ns++] = span("addr.r_idx", addr->r_idx, nK4);
    sp[ns++] = span("addr.r_wt", addr->r_wt, nK4);
    sp[ns++] = span("dout", dout, nv * 4);
    if (dS_final) sp[ns++] = span("dS_final", dS_final, st * p->d_v * 4);
    if (dmass_final) sp[ns++] = span("dmass_final", dmass_final, st * 4);
    const int first_written = ns;
    if (dq) sp[ns++] = span("dq", dq, n * L * 4);
    if (dk) sp[ns++] = span("dk", dk, n * L * 4);
    sp[ns++] = span("dv", dv, nv * 4);
    sp[ns++] = span("dgamma", dgamma, n * 4);
    sp[ns++] = span("dg", dg, nv * 4);
    if (dnorm_w) sp[ns++] = span("dnorm_w", dnorm_w, p->d_v * sizeof(float));
    sp[ns++] = span("dS0", dS0, st * p->d_v * 4);
    sp[ns++] = span("dmass0", dmass0, st * 4);
    sp[ns++] = span("workspace", workspace, need);
    if ((s = check_overlaps(sp, ns, first_written))) return s;

    ramnet::BwdArgs a{};
    a.B = p->B;
    a.T = p->T;
    a.H = p->H;
    a.M = p->M;
    a.K = p->K;
    a.U = p->U;
    a.d_p = p->d_p;
    a.d_v = p->d_v;
    a.cape = p->cape;
    a.content_heads = p->content_heads;
    a.in_bf16 = p->in_dtype == RAMNET_BF16;
    a.state_bf16 = p->state_dtype == RAMNET_BF16;
    a.eps_gsu = p->eps_gsu;
    a.eps_norm = p->eps_norm;
    a.q = q;
    a.k = k;
    a.v = v;
    a.gamma = gamma;
    a.g = g;
    a.norm_w = norm_w;
    a.pos0 = pos0;
    a.S0 = S0;
    a.mass0 = mass0;
    a.w_idx = addr->w_idx;
    a.w_wt = addr->w_wt;
    a.r_idx = addr->r_idx;
    a.r_wt = addr->r_wt;
    a.dout = dout;
    a.dS_final = dS_final;
    a.dmass_final = dmass_final;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dgamma = dgamma;
    a.dg = dg;
    a.dnorm_w = dnorm_w;
    a.dS0 = dS0;
    a.dmass0 = dmass0;
    char *w = static_cast<char *>(workspace);
    const size_t rows = align256(nK4 * p->d_v);
    a.rec_w = reinterpret_cast<float *>(w);
    a.rec_r = reinterpret_cast<float *>(w + rows);
    a.rec_m = reinterpret_cast<float *>(w + 2 * rows);
    a.dw = reinterpret_cast<float *>(w + 2 * rows + align256(nK4));
    a.drho = reinterpret_cast<float *>(w + 2 * rows + 2 * align256(nK4));
    a.dom_part = reinterpret_cast<float *>(w + 2 * rows + 3 * align256(nK4));
    char *w2 = w + 2 * rows + 3 * align256(nK4) + align256(static_cast<size_t>(units) * ramnet::kBwdOutBlocks * p->d_v * 4);
    a.dr = reinterpret_cast<float *>(w2);
    w2 += align256(nv * 4);
    a.dvk = reinterpret_cast<float *>(w2);
    w2 += rows;
    a.dgk = reinterpret_cast<float *>(w2);
    w2 += align256(nK4);
    if (!ramnet::backward_slot_owner(p->M, p->d_v)) {
        // the per-token walk's replayed state and mass
        a.Sw = w2;
        w2 += align256(st * p->d_v * st_bytes(p));
        a.mw = reinterpret_cast<float *>(w2);
    }
    return hip_status(ramnet::launch_backward(a, static_cast<hipStream_t>(stream)),
                      "backward launch");
}

ramnet_status ramnet_scan_prefill(const ramnet_params *p, const void *q, const void *k,
                                  const void *v, const void *gamma, const void *g,
                                  const float *norm_w, const int32_t *pos0, void *S, float *mass,
                                  void *out, const ramnet_addr *addr_in,
                                  const ramnet_addr *addr_out, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    return run_layer(p, false, q, k, v, gamma, g, norm_w, pos0, S, mass, out, addr_in, addr_out,
                     workspace, workspace_bytes, stream);
}

ramnet_status ramnet_scan_prefill_noalloc(const ramnet_params *p, const void *q, const void *k,
                                          const void *v, const void *gamma, const void *g,
                                          const float *norm_w, const int32_t *pos0, void *S,
                                          float *mass, void *out, const ramnet_addr *addr_in,
                                          const ramnet_addr *addr_out, void *stream) {
    ramnet_status s = check_params(p, false);
    if (s) return s;
    // the scratch need is known from the parameters: refuse a call that does
    // not fit before any HIP call is made
    const LayerPlan lp = plan_layer(p, false, addr_in == nullptr && addr_out == nullptr,
                                    addr_in == nullptr);
    if (lp.total() > RAMNET_NOALLOC_SCRATCH_BYTES)
        return fail(RAMNET_EWORKSPACE,
                    "this prefill needs %zu bytes of scratch; the static scratch of "
                    "ramnet_scan_prefill_noalloc holds %zu (call ramnet_scan_prefill with a "
                    "workspace, or split the batch)",
                    lp.total(), static_cast<size_t>(RAMNET_NOALLOC_SCRATCH_BYTES));
    void *ws = nullptr;
    if ((s = scratch_of_current_device(&ws))) return s;
    return run_layer(p, false, q, k, v, gamma, g, norm_w, pos0, S, mass, out, addr_in, addr_out, ws,
                     RAMNET_NOALLOC_SCRATCH_BYTES, stream);
}

ramnet_status ramnet_step_decode(const ramnet_params *p, const void *q, const void *k,
                                 const void *v, const void *gamma, const void *g,
                                 const float *norm_w, const int32_t *pos, void *S, float *mass,
                                 void *out, const ramnet_addr *addr_out, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    return run_layer(p, true, q, k, v, gamma, g, norm_w, pos, S, mass, out, nullptr, addr_out,
                     workspace, workspace_bytes, stream);
}

ramnet_status ramnet_host_alloc(size_t bytes, void **ptr) {
    if (!ptr) return fail(RAMNET_EINVAL, "ptr is NULL");
    *ptr = nullptr;
    void *h = nullptr;
    hipError_t e = hipHostMalloc(&h, bytes ? bytes : 1, hipHostMallocMapped | hipHostMallocPortable);
    if (e != hipSuccess) return hip_status(e, "hipHostMalloc");
    void *d = nullptr;
    e = hipHostGetDevicePointer(&d, h, 0);
    if (e != hipSuccess || d != h) {
        (void)hipHostFree(h);
        return e != hipSuccess ? hip_status(e, "hipHostGetDevicePointer")
                               : fail(RAMNET_EUNSUPPORTED, "pinned memory has another device address");
    }
    *ptr = h;
    return ok();
}

ramnet_status ramnet_host_free(void *ptr) {
    if (!ptr) return ok();
    return hip_status(hipHostFree(ptr), "hipHostFree");
}

ramnet_status ramnet_tier_reset(const ramnet_params *p, const ramnet_tiered_state *ts, void *stream) {
    return tier_upkeep(p, ts, stream, ramnet::launch_tier_reset, "tier reset launch");
}

ramnet_status ramnet_tier_rebalance(const ramnet_params *p, const ramnet_tiered_state *ts, void *stream) {
    return tier_upkeep(p, ts, stream, ramnet::launch_tier_rebalance, "tier rebalance launch");
}

ramnet_status ramnet_tier_flush(const ramnet_params *p, const ramnet_tiered_state *ts, void *stream) {
    return tier_upkeep(p, ts, stream, ramnet::launch_tier_flush, "tier flush launch");
}

ramnet_status ramnet_step_decode_tiered(const ramnet_params *p, const void *q, const void *k,
                                        const void *v, const void *gamma, const void *g,
                                        const float *norm_w, const int32_t *pos,
                                        const ramnet_tiered_state *ts, float *mass, void *out,
                                        const ramnet_addr *addr_out, void *stream) {
    ramnet_status s = check_params(p, true);
    if (s) return s;
    if (!ramnet::step_fused_supported(p->K, p->d_p, p->U, p->d_v, p->state_dtype == RAMNET_BF16))
        return fail(RAMNET_EUNSUPPORTED, "the tiered step takes the fused step's shapes (K <= 32, d_p <= 8)");
    const int64_t units = static_cast<int64_t>(p->B) * p->H;
    if ((s = check_ptr("q", q, true)) || (s = check_ptr("k", k, true)) || (s = check_ptr("v", v, true)) ||
        (s = check_ptr("gamma", gamma, true)) || (s = check_ptr("g", g, true)) ||
        (s = check_ptr("norm_w", norm_w, false)) || (s = check_ptr("pos", pos, false)) ||
        (s = check_ptr("mass", mass, true)) || (s = check_ptr("out", out, true)))
        return s;
    if (p->cape && !pos) return fail(RAMNET_EINVAL, "pos is required when cape != 0");
    if (addr_out && (s = check_addr("addr_out", addr_out))) return s;
    const size_t L = static_cast<size_t>(p->U) * p->d_p;
    const size_t nK4 = static_cast<size_t>(units) * p->K * 4;
    Span sp[24];
    int ns = 0;
    sp[ns++] = span("q", q, units * L * in_bytes(p));
    sp[ns++] = span("k", k, units * L * in_bytes(p));
    if (pos) sp[ns++] = span("pos", pos, p->B * sizeof(int32_t));
    sp[ns++] = span("v", v, units * p->d_v * in_bytes(p));
    sp[ns++] = span("gamma", gamma, units * in_bytes(p));
    sp[ns++] = span("g", g, units * p->d_v * in_bytes(p));
    if (norm_w) sp[ns++] = span("norm_w", norm_w, p->d_v * sizeof(float));
    const int first_written = ns;
    sp[ns++] = span("mass", mass, units * p->M * sizeof(float));
    sp[ns++] = span("out", out, units * p->d_v * st_bytes(p));
    if (addr_out) {
        sp[ns++] = span("addr_out.w_idx", addr_out->w_idx, nK4);
        sp[ns++] = span("addr_out.w_wt", addr_out->w_wt, nK4);
        sp[ns++] = span("addr_out.r_idx", addr_out->r_idx, nK4);
        sp[ns++] = span("addr_out.r_wt", addr_out->r_wt, nK4);
    }
    if ((s = check_tier(p, ts, sp, ns)) || (s = check_overlaps(sp, ns, first_written))) return s;
    if (units == 0) return ok();
    ramnet::StepArgs sa{};
    sa.B = p->B;
    sa.H = p->H;
    sa.M = p->M;
    sa.K = p->K;
    sa.d_v = p->d_v;
    sa.U = p->U;
    sa.d_p = p->d_p;
    sa.cape = p->cape;
    sa.content_heads = p->content_heads;
    sa.in_bf16 = p->in_dtype == RAMNET_BF16;
    sa.state_bf16 = p->state_dtype == RAMNET_BF16;
    sa.q = q;
    sa.k = k;
    sa.v = v;
    sa.gamma = gamma;
    sa.g = g;
    sa.norm_w = norm_w;
    sa.pos = pos;
    sa.S = ts->S_host;
    sa.mass = mass;
    sa.out = out;
    sa.out_idx[0] = addr_out ? addr_out->w_idx : nullptr;
    sa.out_idx[1] = addr_out ? addr_out->r_idx : nullptr;
    sa.out_wt[0] = addr_out ? addr_out->w_wt : nullptr;
    sa.out_wt[1] = addr_out ? addr_out->r_wt : nullptr;
    sa.eps_gsu = p->eps_gsu;
    sa.eps_norm = p->eps_norm;
    sa.cache = ts->cache;
    sa.slot_line = ts->slot_line;
    sa.hits = ts->hits;
    sa.C = ts->C;
    return hip_status(ramnet::launch_step_fused(sa, static_cast<hipStream_t>(stream)), "tiered step launch");
}

const char *ramnet_status_str(ramnet_status s) {
    switch (s) {
        case RAMNET_OK: return "ok";
        case RAMNET_EINVAL: return "invalid argument";
        case RAMNET_EUNSUPPORTED: return "unsupported configuration";
        case RAMNET_EWORKSPACE: return "workspace missing or too small";
        case RAMNET_EHIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *ramnet_last_error(void) { return g_last_error.c_str(); }

int32_t ramnet_version(void) { return RAMNET_VERSION; }

}  // extern "C"
