// Backward pass of the RAM-Net layer recurrence (the pages name training and
// prefill together in their GPU-execution paragraph; they give no backward
// formulas, so the adjoint below is the exact derivative of the forward
// steps, Top-K selection held fixed).
//
// For a state held in fp32 with d_v = 64 channels and M <= 1024 slots, one
// workgroup per (batch, head) unit, thread s owning slot s:
//
//   bwd_record_kernel   replays the forward from (S0, m0) and records, per
//                       token, each write's row and mass before the write
//                       and each read's row after the writes (fp32, in the
//                       workspace: 2 K d_v + K floats per token-head).
//   bwd_out_kernel      for all tokens at once (the recorded read rows are all
//                       it needs): out = y omega sigmoid(g), y = r / rms(r):
//                         dg, d omega, dr = (dy - y mean(dy y)) / rms(r);
//                         r = sum_k rho_k S_jk:  drho_k = <dr, S_jk>.
//   bwd_adjoint_kernel  walks the tokens backwards with thread s holding
//                       dS[s] (64 registers) and dm[s]; each token's inputs,
//                       dr and recorded write rows are loaded one token
//                       ahead and staged in LDS (double-buffered, one barrier
//                       per token):
//                         dS_jk += rho_k dr
//                         each write, S+ = S- + lam (v - S-),
//                         m+ = alpha m- + w, lam = w / (m+ + eps),
//                         alpha = (1 - w)^e, e = exp(gamma):
//                           dv += lam dS+, dlam = <dS+, v - S->,
//                           dS- = (1 - lam) dS+,
//                           dm+ total = dm+ - dlam w / (m+ + eps)^2,
//                           dw = dlam / (m+ + eps) + dm+ total
//                                - dm+ total m- e alpha / (1 - w),
//                           dgamma += dm+ total m- alpha log(1 - w) e,
//                           dm- = dm+ total alpha
//   bwd_logits_kernel   turns d w and d rho into logit gradients through the
//                       Product Softmax: w = prod_u p_u(a_u) gives
//                       dl_u,d = sum_k dw_k w_k ([d = a_u(k)] - p_u(d)), with
//                       a(k) the selected slot's content digits (CAPE undone).
//   bwd_omega_kernel    sums the units' d omega in unit order.
#include "device_common.h"
#include "launch.h"

namespace ramnet {
namespace {

constexpr int kBwdDv = 64;
constexpr int kBwdNT = 1024;
constexpr int kKMax = 64;

struct Row4 {
    float e[4];
};

// One token's staged inputs of the serial kernels (double-buffered by token
// parity, so one barrier per token suffices).
struct Staged {
    int w[kKMax], r[kKMax];
    float wt[kKMax], rt[kKMax], v[kBwdDv], dr[kBwdDv], mm[kKMax];
    float gam;
};

// The next token's inputs, loaded into registers one token ahead: thread
// s < K its address pair, s < 64 channel s of v (and of dr), thread 0 gamma.
struct Prefetch {
    int w = 0, r = 0;
    float wt = 0.f, rt = 0.f, v = 0.f, dr = 0.f, mm = 0.f, gam = 0.f;
};

template <typename TIn, bool ADJ>
__device__ __forceinline__ void prefetch_token(const BwdArgs &a, int64_t th, int64_t rec, int s,
                                               Prefetch &p) {
    const int K = a.K;
    if (s < K) {
        p.w = a.w_idx[th * K + s];
        p.wt = a.w_wt[th * K + s];
        p.r = a.r_idx[th * K + s];
        if (ADJ) {
            p.rt = a.r_wt[th * K + s];
            p.mm = a.rec_m[rec + s];
        }
    }
    if (s < kBwdDv) {
        p.v = to_f32(static_cast<const TIn *>(a.v)[th * kBwdDv + s]);
        if (ADJ) p.dr = a.dr[th * kBwdDv + s];
    }
    if (s == 0) p.gam = to_f32(static_cast<const TIn *>(a.gamma)[th]);
}

__device__ __forceinline__ void stage_token(Staged &st, const Prefetch &p, int s, int K) {
    if (s < K) {
        st.w[s] = p.w;
        st.wt[s] = p.wt;
        st.r[s] = p.r;
        st.rt[s] = p.rt;
        st.mm[s] = p.mm;
    }
    if (s < kBwdDv) {
        st.v[s] = p.v;
        st.dr[s] = p.dr;
    }
    if (s == 0) st.gam = p.gam;
}

template <typename TIn>
__global__ __launch_bounds__(kBwdNT) void bwd_record_kernel(BwdArgs a) {
    __shared__ Staged stg[2];
    const int unit = blockIdx.x, b = unit / a.H, h = unit % a.H;
    const int s = threadIdx.x, K = a.K, T = a.T;
    const int M = static_cast<int>(a.M);
    const bool own = s < M;
    float row[kBwdDv];
    float m = 0.f;
    if (own) {
        const Row4 *src = reinterpret_cast<const Row4 *>(a.S0 + (static_cast<int64_t>(unit) * M + s) * kBwdDv);
#pragma unroll
        for (int j = 0; j < kBwdDv / 4; ++j) {
            const Row4 x = src[j];
#pragma unroll
            for (int c = 0; c < 4; ++c) row[4 * j + c] = x.e[c];
        }
        m = a.mass0[static_cast<int64_t>(unit) * M + s];
    }
    auto th_of = [&](int t) { return (static_cast<int64_t>(b) * T + t) * a.H + h; };
    Prefetch pf;
    prefetch_token<TIn, false>(a, th_of(0), 0, s, pf);
    for (int t = 0; t < T; ++t) {
        Staged &st = stg[t & 1];
        stage_token(st, pf, s, K);
        if (t + 1 < T) prefetch_token<TIn, false>(a, th_of(t + 1), 0, s, pf);
        __syncthreads();
        if (own) {
            const int64_t rec = (static_cast<int64_t>(unit) * T + t) * K;
            for (int k = 0; k < K; ++k) {
                if (st.w[k] != s) continue;  // write slots are distinct: at most one
                Row4 *dst = reinterpret_cast<Row4 *>(a.rec_w + (rec + k) * kBwdDv);
#pragma unroll
                for (int j = 0; j < kBwdDv / 4; ++j)
                    dst[j] = Row4{{row[4 * j], row[4 * j + 1], row[4 * j + 2], row[4 * j + 3]}};
                a.rec_m[rec + k] = m;
                const float w = st.wt[k];
                if (w > 0.f) {
                    const float alpha = retention(w, expf(st.gam));
                    m = fmaf(alpha, m, w);
                    const float lam = w / (m + a.eps_gsu);
#pragma unroll
                    for (int c = 0; c < kBwdDv; ++c) row[c] = fmaf(lam, st.v[c] - row[c], row[c]);
                }
            }
            for (int k = 0; k < K; ++k) {
                if (st.r[k] != s) continue;
                Row4 *dst = reinterpret_cast<Row4 *>(a.rec_r + (rec + k) * kBwdDv);
#pragma unroll
                for (int j = 0; j < kBwdDv / 4; ++j)
                    dst[j] = Row4{{row[4 * j], row[4 * j + 1], row[4 * j + 2], row[4 * j + 3]}};
            }
        }
    }
}

// Output gate, RMSNorm and read, for all tokens at once (they need only the
// recorded read rows): one wave per token-head, lane c = channel c.  Writes
// dg, dr (the read's adjoint, for the serial kernel) and d rho; each wave
// sums its tokens' d omega, and the workgroup's sum goes to a partial.
constexpr int kOutWaves = 4, kOutBlocks = 16;

template <typename TIn>
__global__ __launch_bounds__(kOutWaves * kWave) void bwd_out_kernel(BwdArgs a) {
    __shared__ float sdom[kOutWaves][kBwdDv];
    const int unit = blockIdx.x, b = unit / a.H, h = unit % a.H;
    const int wave = threadIdx.x / kWave, c = threadIdx.x % kWave;
    const int K = a.K, T = a.T;
    const TIn *gg = static_cast<const TIn *>(a.g);
    const float om = a.norm_w ? a.norm_w[c] : 1.0f;
    float dom = 0.f;
    for (int t = blockIdx.y * kOutWaves + wave; t < T; t += kOutBlocks * kOutWaves) {
        const int64_t th = (static_cast<int64_t>(b) * T + t) * a.H + h;
        const float *rr = a.rec_r + (static_cast<int64_t>(unit) * T + t) * K * kBwdDv + c;
        float r = 0.f;
        for (int k = 0; k < K; ++k) r = fmaf(a.r_wt[th * K + k], rr[k * kBwdDv], r);
        const float den = wave_sum(r * r) / static_cast<float>(kBwdDv) + a.eps_norm;
        const float inv = den > 0.f ? 1.0f / sqrtf(den) : 0.f;  // zero read, eps 0
        const float y = r * inv;
        const float sg = sigmoid(to_f32(gg[th * kBwdDv + c]));
        const float d_o = a.dout[th * kBwdDv + c];
        a.dg[th * kBwdDv + c] = d_o * om * y * sg * (1.0f - sg);
        dom = fmaf(d_o * y, sg, dom);
        const float dy = d_o * om * sg;
        const float dyy = wave_sum(dy * y) / static_cast<float>(kBwdDv);
        const float dr = inv * (dy - y * dyy);
        a.dr[th * kBwdDv + c] = dr;
        for (int k = 0; k < K; ++k) {
            const float dk = wave_sum(dr * rr[k * kBwdDv]);
            if (c == 0) a.drho[th * K + k] = dk;
        }
    }
    sdom[wave][c] = dom;
    __syncthreads();
    if (wave == 0) {
        float acc = 0.f;
        for (int w2 = 0; w2 < kOutWaves; ++w2) acc += sdom[w2][c];
        a.dom_part[(static_cast<int64_t>(unit) * kOutBlocks + blockIdx.y) * kBwdDv + c] = acc;
    }
}

template <typename TIn>
__global__ __launch_bounds__(kBwdNT) void bwd_adjoint_kernel(BwdArgs a) {
    __shared__ Staged stg[2];
    // dynamic: per token parity q, the writes' rows before them [K][64],
    // lam dS+ per write [K][64], and the gamma terms [K]
    extern __shared__ float dyn[];
    const int unit = blockIdx.x, b = unit / a.H, h = unit % a.H;
    const int s = threadIdx.x, K = a.K, T = a.T;
    auto sSm = [&](int q, int k) { return dyn + (static_cast<int64_t>(q) * K + k) * kBwdDv; };
    auto sdv = [&](int q, int k) { return dyn + (static_cast<int64_t>(2 + q) * K + k) * kBwdDv; };
    float *sdgk = dyn + 4 * K * kBwdDv;  // [2][K]
    const int M = static_cast<int>(a.M);
    const bool own = s < M;
    const int64_t srow = (static_cast<int64_t>(unit) * M + s) * kBwdDv;
    float dS[kBwdDv];
    float dm = 0.f;
#pragma unroll
    for (int c = 0; c < kBwdDv; ++c) dS[c] = 0.f;
    if (own && a.dS_final) {
        const Row4 *src = reinterpret_cast<const Row4 *>(a.dS_final + srow);
#pragma unroll
        for (int j = 0; j < kBwdDv / 4; ++j) {
            const Row4 x = src[j];
#pragma unroll
            for (int c = 0; c < 4; ++c) dS[4 * j + c] = x.e[c];
        }
    }
    if (own && a.dmass_final) dm = a.dmass_final[static_cast<int64_t>(unit) * M + s];
    auto th_of = [&](int t) { return (static_cast<int64_t>(b) * T + t) * a.H + h; };
    auto rec_of = [&](int t) { return (static_cast<int64_t>(unit) * T + t) * K; };
    // the recorded rows of the writes: thread s < 16 K holds 16 bytes
    const bool rows_lane = s < K * (kBwdDv / 4);
    Row4 pf_row{};
    auto prefetch_rows = [&](int t) {
        if (rows_lane) pf_row = reinterpret_cast<const Row4 *>(a.rec_w + rec_of(t) * kBwdDv)[s];
    };
    // token t's sums of lam dS+ and of the gamma terms (wave 0, after the
    // next token's barrier)
    auto finish = [&](int t) {
        const int q = t & 1;
        const Staged &st = stg[q];
        const int64_t th = th_of(t);
        if (s < kBwdDv) {
            float acc = 0.f;
            for (int k = 0; k < K; ++k)
                if (st.wt[k] > 0.f && st.w[k] >= 0 && st.w[k] < M) acc += sdv(q, k)[s];
            a.dv[th * kBwdDv + s] = acc;
        }
        if (s == 0) {
            float acc = 0.f;
            for (int k = 0; k < K; ++k)
                if (st.wt[k] > 0.f && st.w[k] >= 0 && st.w[k] < M) acc += sdgk[q * K + k];
            a.dgamma[th] = acc;
        }
    };
    Prefetch pf;
    prefetch_token<TIn, true>(a, th_of(T - 1), rec_of(T - 1), s, pf);
    prefetch_rows(T - 1);
    for (int t = T - 1; t >= 0; --t) {
        const int q = t & 1;
        Staged &st = stg[q];
        stage_token(st, pf, s, K);
        if (rows_lane) {
            const int k = s / (kBwdDv / 4), j = s % (kBwdDv / 4);
            *reinterpret_cast<Row4 *>(sSm(q, k) + 4 * j) = pf_row;
        }
        if (t > 0) {
            prefetch_token<TIn, true>(a, th_of(t - 1), rec_of(t - 1), s, pf);
            prefetch_rows(t - 1);
        }
        __syncthreads();
        if (t + 1 < T) finish(t + 1);
        if (own) {
            const int64_t th = th_of(t);
            // the read came after the writes: its adjoint goes in first
            for (int k = 0; k < K; ++k) {
                if (st.r[k] != s) continue;
                const float rho = st.rt[k];
#pragma unroll
                for (int c = 0; c < kBwdDv; ++c) dS[c] = fmaf(rho, st.dr[c], dS[c]);
            }
            for (int k = K - 1; k >= 0; --k) {
                if (st.w[k] != s) continue;
                const float w = st.wt[k];
                float dw = 0.f, dgk = 0.f;
                if (w > 0.f) {
                    const float mm = st.mm[k];
                    const float e = expf(st.gam);
                    const float alpha = retention(w, e);
                    const float mp = fmaf(alpha, mm, w);
                    const float den = mp + a.eps_gsu;
                    const float lam = w / den;
                    float dl = 0.f;
                    {
                        const float *sm = sSm(q, k);
#pragma unroll
                        for (int c = 0; c < kBwdDv; ++c) dl = fmaf(dS[c], st.v[c] - sm[c], dl);
                    }
                    float *dvk = sdv(q, k);
#pragma unroll
                    for (int c = 0; c < kBwdDv; ++c) {
                        dvk[c] = lam * dS[c];
                        dS[c] *= 1.0f - lam;
                    }
                    const float dmt = dm - dl * w / (den * den);
                    const float dalpha = dmt * mm;
                    dm = dmt * alpha;
                    dw = dl / den + dmt;
                    if (w < 1.0f && alpha > 0.f) {
                        dw -= dalpha * e * alpha / (1.0f - w);
                        dgk = dalpha * alpha * log1pf(-w) * e;
                    }
                }
                sdgk[q * K + k] = dgk;
                a.dw[th * K + k] = dw;
            }
        }
    }
    __syncthreads();
    finish(0);
    if (own) {
        Row4 *dst = reinterpret_cast<Row4 *>(a.dS0 + srow);
#pragma unroll
        for (int j = 0; j < kBwdDv / 4; ++j)
            dst[j] = Row4{{dS[4 * j], dS[4 * j + 1], dS[4 * j + 2], dS[4 * j + 3]}};
        a.dmass0[static_cast<int64_t>(unit) * M + s] = dm;
    }
}

// The position whose CAPE move undoes the move at pos (forms 1 and 3: the
// negated position; form 2: the digit-wise negation of pos mod M).
__device__ __forceinline__ int64_t cape_inverse_pos(int64_t pos, int form, int dp, int U, int64_t M) {
    if (form != 2) return -pos;
    uint64_t p = static_cast<uint64_t>(((pos % M) + M) % M), inv = 0, place = 1;
    for (int u = 0; u < U; ++u) {
        inv += ((dp - p % dp) % dp) * place;
        p /= dp;
        place *= dp;
    }
    return static_cast<int64_t>(inv);
}

template <typename TIn>
__global__ __launch_bounds__(256) void bwd_logits_kernel(BwdArgs a) {
    constexpr int kMaxL = 64;
    const int64_t n = static_cast<int64_t>(a.B) * a.T * a.H;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const bool key = blockIdx.y == 0;
    float *out = key ? a.dk : a.dq;
    if (!out) return;
    const int U = a.U, dp = a.d_p, L = U * dp, K = a.K;
    const TIn *lg = static_cast<const TIn *>(key ? a.k : a.q) + i * L;
    const int32_t *idx = (key ? a.w_idx : a.r_idx) + i * K;
    const float *wt = (key ? a.w_wt : a.r_wt) + i * K;
    const float *gr = (key ? a.dw : a.drho) + i * K;
    float p[kMaxL], dl[kMaxL];
    for (int u = 0; u < U; ++u) {
        float mx = to_f32(lg[u * dp]);
        for (int d = 1; d < dp; ++d) mx = fmaxf(mx, to_f32(lg[u * dp + d]));
        float sum = 0.f;
        for (int d = 0; d < dp; ++d) {
            p[u * dp + d] = expf(to_f32(lg[u * dp + d]) - mx);
            sum += p[u * dp + d];
        }
        for (int d = 0; d < dp; ++d) {
            p[u * dp + d] /= sum;
            dl[u * dp + d] = 0.f;
        }
    }
    const int64_t b = i / (static_cast<int64_t>(a.T) * a.H), t = (i / a.H) % a.T;
    const int h = static_cast<int>(i % a.H);
    const int form = head_uses_cape(a.content_heads, h) ? a.cape : 0;
    const int64_t pos = (a.pos0 ? a.pos0[b] : 0) + t;
    const int64_t ipos = cape_inverse_pos(pos, form, dp, U, a.M);
    for (int k = 0; k < K; ++k) {
        const int slot = idx[k];
        if (slot < 0 || slot >= a.M) continue;
        const float coef = gr[k] * wt[k];
        int content = form ? cape_slot<0>(slot, ipos, U, dp, form, a.M) : slot;
        // digits from the least significant (u = U - 1) up
        for (int u = U - 1; u >= 0; --u) {
            const int digit = content % dp;
            content /= dp;
            for (int d = 0; d < dp; ++d) dl[u * dp + d] -= coef * p[u * dp + d];
            dl[u * dp + digit] += coef;
        }
    }
    for (int j = 0; j < L; ++j) out[i * L + j] = dl[j];
}

__global__ __launch_bounds__(kBwdDv) void bwd_omega_kernel(const float *part, int units,
                                                          float *out) {
    const int c = threadIdx.x;
    float acc = 0.f;
    for (int u = 0; u < units; ++u) acc += part[static_cast<int64_t>(u) * kBwdDv + c];
    out[c] = acc;
}

template <typename TIn>
hipError_t launch_in(const BwdArgs &a, hipStream_t st) {
    const int units = a.B * a.H;
    const int nt = static_cast<int>(((a.M + kWave - 1) / kWave) * kWave);
    const int threads = nt < kWave ? kWave : nt;
    hipLaunchKernelGGL(bwd_record_kernel<TIn>, dim3(units), dim3(threads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_out_kernel<TIn>, dim3(units, kOutBlocks), dim3(kOutWaves * kWave), 0,
                       st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = (4 * static_cast<size_t>(a.K) * kBwdDv + 2 * a.K) * sizeof(float);
    hipLaunchKernelGGL(bwd_adjoint_kernel<TIn>, dim3(units), dim3(threads), lds, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.dq || a.dk) {
        const int64_t n = static_cast<int64_t>(units) * a.T;
        hipLaunchKernelGGL(bwd_logits_kernel<TIn>, dim3(static_cast<unsigned>((n + 255) / 256), 2),
                           dim3(256), 0, st, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.dnorm_w) {
        hipLaunchKernelGGL(bwd_omega_kernel, dim3(1), dim3(kBwdDv), 0, st, a.dom_part,
                           units * kOutBlocks, a.dnorm_w);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

bool backward_supported(int64_t M, int d_v, int U, int d_p, bool state_bf16) {
    return !state_bf16 && d_v == kBwdDv && M <= kBwdNT && U * d_p <= 64;
}

size_t backward_workspace_bytes(int B, int T, int H, int K) {
    const size_t units = static_cast<size_t>(B) * H;
    const size_t n = units * T;
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    return 2 * al(n * K * kBwdDv * 4) + 3 * al(n * K * 4) + al(units * kOutBlocks * kBwdDv * 4) +
           al(n * kBwdDv * 4);
}

hipError_t launch_backward(const BwdArgs &a, hipStream_t st) {
    if (static_cast<int64_t>(a.B) * a.H * a.T == 0) return hipSuccess;
    return a.in_bf16 ? launch_in<bf16_t>(a, st) : launch_in<float>(a, st);
}

}  // namespace ramnet
