// Backward pass of the RAM-Net layer recurrence (the pages name training and
// prefill together in their GPU-execution paragraph; they give no backward
// formulas, so the adjoint below is the exact derivative of the forward
// steps, Top-K selection held fixed).
//
// For d_v = 64 channels and M <= 1024 slots, the state in fp32 or bf16 (the
// replay rounds it as the forward does; each rounding passes its gradient
// through; the adjoint runs in fp32).  A
// slot's adjoint depends only on its own events, so the two serial kernels
// give each (batch, head) unit up to eight workgroups of 128 slots, two or
// four adjacent threads sharing a slot (32 or 16 channels each; the one
// full-row dot product is combined across them):
//
//   bwd_record_kernel   replays the forward from (S0, m0) and records, per
//                       token, each write's row and mass before the write
//                       and each read's row after the writes (fp32, in the
//                       workspace: 2 K d_v + K floats per token-head).  The
//                       sequence goes in chunks whose events are grouped by
//                       slot, each thread walking its own slot's events.
//   bwd_out_kernel      for all tokens at once (the recorded read rows are all
//                       it needs): out = y omega sigmoid(g), y = r / rms(r):
//                         dg, d omega, dr = (dy - y mean(dy y)) / rms(r);
//                         r = sum_k rho_k S_jk:  drho_k = <dr, S_jk>.
//   bwd_adjoint_kernel  walks the chunks backwards, a slot's threads holding
//                       dS[s] (their channels) and dm[s] and walking its slot's
//                       events of the chunk in reverse time order:
//                         dS_jk += rho_k dr
//                         each write, S+ = S- + lam (v - S-),
//                         m+ = alpha m- + w, lam = w / (m+ + eps),
//                         alpha = (1 - w)^e, e = exp(gamma):
//                           dv += lam dS+, dlam = <dS+, v - S->,
//                           dS- = (1 - lam) dS+,   (lam dS+ per write
//                           goes out; bwd_sum_kernel adds a token's writes)
//                           dm+ total = dm+ - dlam w / (m+ + eps)^2,
//                           dw = dlam / (m+ + eps) + dm+ total
//                                - dm+ total m- e alpha / (1 - w),
//                           dgamma += dm+ total m- alpha log(1 - w) e,
//                           dm- = dm+ total alpha
//   bwd_logits_kernel   turns d w and d rho into logit gradients through the
//                       Product Softmax: w = prod_u p_u(a_u) gives
//                       dl_u,d = sum_k dw_k w_k ([d = a_u(k)] - p_u(d)), with
//                       a(k) the selected slot's content digits (CAPE undone).
//   bwd_sum_kernel      adds each token's lam dS+ and gamma terms over its
//                       writes, in write order.
//   bwd_omega_kernel    sums the d omega partials in a fixed order.
//
// Other shapes (d_v != 64, or M > 1024 with the rows in HBM) replace the two
// serial kernels by bwd_record_range_kernel and bwd_adjoint_range_kernel: a
// unit's slots split into eight ranges (slot mod 8), one workgroup per
// (unit, range) owning its slots for the whole sequence; per chunk the
// range's events are sorted by (slot, time) in LDS and a 16-lane group per
// slot walks them with the slot's row, mass or adjoint in registers and the
// state, its copy and its adjoint in HBM (the slot-range walk below).
#include "device_common.h"
#include "launch.h"

#include <algorithm>

namespace ramnet {
namespace {

constexpr int kBwdDv = 64;
constexpr int kBwdNT = 1024;  // largest M
// The serial kernels split a unit's slots over workgroups of kSlotsPerWG
// slots; HV adjacent lanes share a slot (HV = 2 or 4), each holding
// kBwdDv / HV of its channels.
constexpr int kSlotsPerWG = 128;
template <int HV> constexpr int kThreadsOf = kSlotsPerWG * HV;

struct Row4 {
    float e[4];
};

// ---------------------------------------------------------------- slot grouping
//
// Both serial kernels take the sequence in chunks of C tokens.  A chunk's
// 2 C K events (its writes and reads) are grouped by slot with a counting
// sort in LDS; the thread owning a slot then sorts its few events by time
// and walks them on its own, with no barrier between tokens (the project
// page's GPU-execution grouping of events by slot, here for the replay and
// the adjoint).  An event code is t << 7 | read << 6 | k: ascending order is
// the forward order (a token's write before its read).

// EVM: a chunk's event capacity (2 C K), 2048 or 4096.  The larger halves
// the chunks (and their barriers) at large K, but its LDS (83 KB) allows
// one workgroup per CU; it is used when the grid has no more than that.

template <int HV, int EVM>
struct ChunkLds {
    int cnt[kSlotsPerWG];  // events per slot, then their offsets
    int wtot[kThreadsOf<HV> / kWave];
    int list[EVM];
};

__device__ __forceinline__ int wave_incl_scan_i(int x) {
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(x, off, kWave);
        if (lane >= off) x += y;
    }
    return x;
}

// Exclusive prefix over the block's threads in thread order.
__device__ int block_excl_scan_i(int x, int *wtot) {
    const int nw = (blockDim.x + kWave - 1) / kWave;
    const int lane = lane_id(), wid = threadIdx.x / kWave;
    const int incl = wave_incl_scan_i(x);
    if (lane == kWave - 1) wtot[wid] = incl;
    lds_barrier();
    if (wid == 0) {
        int y = lane < nw ? wtot[lane] : 0;
        y = wave_incl_scan_i(y);
        if (lane < nw) wtot[lane] = y;
    }
    lds_barrier();
    const int base = wid > 0 ? wtot[wid - 1] : 0;
    lds_barrier();
    return base + incl - x;
}

// Groups the chunk's events on this workgroup's slots [slot0, slot0 +
// kSlotsPerWG) by slot: afterwards cnt[s] is slot slot0 + s's event count
// and its events are list[base, base + n) in arbitrary order; both threads
// of slot s get base (returned) and n.  widx/ridx: the chunk's staged write
// and read slots, [Cc K] each.
template <int HV, int EVM>
__device__ int group_events(ChunkLds<HV, EVM> &g, const int *widx, const int *ridx, int nev, int slot0,
                            int nslots, int &n) {
    constexpr int kBwdThreads = kThreadsOf<HV>;
    const int s = threadIdx.x / HV;
    const bool first = threadIdx.x % HV == 0;
    if (first) g.cnt[s] = 0;
    lds_barrier();
    constexpr int kPer = EVM / kBwdThreads;
    int slot[kPer], rank[kPer], code[kPer];
    const int K2 = 2 * nev;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int e = static_cast<int>(threadIdx.x) + j * kBwdThreads;
        slot[j] = -1;
        if (e < K2) {
            const bool rd = e >= nev;
            const int i = rd ? e - nev : e;
            const int sl = (rd ? ridx[i] : widx[i]) - slot0;
            if (sl >= 0 && sl < nslots) {
                slot[j] = sl;
                rank[j] = atomicAdd(&g.cnt[sl], 1);
                code[j] = i;  // t * K + k; the kind goes in below
                code[j] |= rd ? (1 << 30) : 0;
            }
        }
    }
    lds_barrier();
    n = g.cnt[s];
    const int pre = block_excl_scan_i(first ? n : 0, g.wtot);  // thread order: slot order
    if (first) g.cnt[s] = pre;
    lds_barrier();
    const int base = g.cnt[s];
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        if (slot[j] >= 0) g.list[g.cnt[slot[j]] + rank[j]] = code[j];
    lds_barrier();
    return base;
}

// Event i = t * K + k, read flag in bit 30 -> sort key t << 7 | read << 6 | k.
__device__ __forceinline__ int ev_key(int code, int K) {
    const int i = code & ((1 << 30) - 1), t = i / K, k = i - t * K;
    return (t << 7) | ((code >> 30) & 1) << 6 | k;
}

// Insertion sort of a thread's own event keys (ascending), in place.
__device__ __forceinline__ void sort_keys(int *p, int n) {
    for (int i = 1; i < n; ++i) {
        const int x = p[i];
        int j = i - 1;
        while (j >= 0 && p[j] > x) {
            p[j + 1] = p[j];
            --j;
        }
        p[j + 1] = x;
    }
}

// Tokens per chunk: at most 64, and C K write events at most EVM / 2.
constexpr int kChunkMax = 64;
__host__ __device__ inline int bwd_chunk(int K, int EVM) {
    int c = kChunkMax;
    while (c > 1 && c * K > EVM / 2) c /= 2;
    return c;
}

// A chunk's staged token data.
template <int EVM>
struct ChunkTok {
    int widx[EVM / 2], ridx[EVM / 2];
    float wt[EVM / 2], rt[EVM / 2];
    float v[kChunkMax][kBwdDv];
    float dr[kChunkMax][kBwdDv];
    float gam[kChunkMax];
};

// The same data for the next chunk, loaded into registers while this chunk
// is walked (thread i takes entries i, i + NT, ...).
template <int HV, int EVM>
struct ChunkPf {
    static constexpr int kPfA = EVM / 2 / kThreadsOf<HV>;
    static constexpr int kPfV = kChunkMax * kBwdDv / kThreadsOf<HV>;
    int w[kPfA], r[kPfA];
    float wt[kPfA], rt[kPfA], v[kPfV], dr[kPfV], gam;
};

template <typename TIn, bool ADJ, int HV, int EVM>
__device__ __forceinline__ void load_chunk(const BwdArgs &a, ChunkPf<HV, EVM> &p, int b, int h, int t0,
                                           int Cc) {
    constexpr int kBwdThreads = kThreadsOf<HV>, kPfA = ChunkPf<HV, EVM>::kPfA,
                  kPfV = ChunkPf<HV, EVM>::kPfV;
    const int K = a.K, s = threadIdx.x;
    const TIn *v = static_cast<const TIn *>(a.v);
    const TIn *gam = static_cast<const TIn *>(a.gamma);
#pragma unroll
    for (int j = 0; j < kPfA; ++j) {
        const int i = s + j * kBwdThreads;
        if (i < Cc * K) {
            const int t = i / K, k = i - t * K;
            const int64_t e = ((static_cast<int64_t>(b) * a.T + t0 + t) * a.H + h) * K + k;
            p.w[j] = a.w_idx[e];
            p.wt[j] = a.w_wt[e];
            p.r[j] = a.r_idx[e];
            if (ADJ) p.rt[j] = a.r_wt[e];
        }
    }
#pragma unroll
    for (int j = 0; j < kPfV; ++j) {
        const int i = s + j * kBwdThreads;
        if (i < Cc * kBwdDv) {
            const int t = i / kBwdDv, c = i - t * kBwdDv;
            const int64_t th = (static_cast<int64_t>(b) * a.T + t0 + t) * a.H + h;
            p.v[j] = to_f32(v[th * kBwdDv + c]);
            if (ADJ) p.dr[j] = a.dr[th * kBwdDv + c];
        }
    }
    if (s < Cc) p.gam = to_f32(gam[(static_cast<int64_t>(b) * a.T + t0 + s) * a.H + h]);
}

template <bool ADJ, int HV, int EVM>
__device__ __forceinline__ void store_chunk(ChunkTok<EVM> &ct, const ChunkPf<HV, EVM> &p, int Cc, int K) {
    constexpr int kBwdThreads = kThreadsOf<HV>, kPfA = ChunkPf<HV, EVM>::kPfA,
                  kPfV = ChunkPf<HV, EVM>::kPfV;
    const int s = threadIdx.x;
#pragma unroll
    for (int j = 0; j < kPfA; ++j) {
        const int i = s + j * kBwdThreads;
        if (i < Cc * K) {
            ct.widx[i] = p.w[j];
            ct.wt[i] = p.wt[j];
            ct.ridx[i] = p.r[j];
            if (ADJ) ct.rt[i] = p.rt[j];
        }
    }
#pragma unroll
    for (int j = 0; j < kPfV; ++j) {
        const int i = s + j * kBwdThreads;
        if (i < Cc * kBwdDv) {
            ct.v[i / kBwdDv][i % kBwdDv] = p.v[j];
            if (ADJ) ct.dr[i / kBwdDv][i % kBwdDv] = p.dr[j];
        }
    }
    if (s < Cc) ct.gam[s] = p.gam;
}

// Both serial kernels: thread HV s + hf of a workgroup serves slot slot0 + s,
// channels [hf kCh, hf kCh + kCh); the slot's first thread sorts its
// events, then all HV walk them.
template <typename TIn, typename TS, int HV, int EVM>
__global__ __launch_bounds__(kThreadsOf<HV>) void bwd_record_kernel(BwdArgs a) {
    constexpr int kCh = kBwdDv / HV;
    __shared__ ChunkLds<HV, EVM> g;
    __shared__ ChunkTok<EVM> ct;
    const int unit = blockIdx.x, b = unit / a.H, h = unit % a.H;
    const int s = threadIdx.x / HV, c0 = (threadIdx.x % HV) * kCh;
    const bool first = c0 == 0;
    const int K = a.K, T = a.T;
    const int M = static_cast<int>(a.M);
    const int slot0 = blockIdx.y * kSlotsPerWG, slot = slot0 + s;
    const int nslots = min(kSlotsPerWG, M - slot0);
    const bool own = s < nslots;
    const int C = bwd_chunk(K, EVM);
    float row[kCh];
    float m = 0.f;
    if (own) {
        const TS *src = static_cast<const TS *>(a.S0) + (static_cast<int64_t>(unit) * M + slot) * kBwdDv + c0;
#pragma unroll
        for (int c = 0; c < kCh; ++c) row[c] = to_f32(src[c]);
        m = a.mass0[static_cast<int64_t>(unit) * M + slot];
    }
    ChunkPf<HV, EVM> pf;
    load_chunk<TIn, false, HV, EVM>(a, pf, b, h, 0, min(C, T));
    for (int t0 = 0; t0 < T; t0 += C) {
        const int Cc = min(C, T - t0), nev = Cc * K;
        store_chunk<false, HV, EVM>(ct, pf, Cc, K);
        lds_barrier();
        if (t0 + C < T) load_chunk<TIn, false, HV, EVM>(a, pf, b, h, t0 + C, min(C, T - t0 - C));
        int n;
        const int base = group_events(g, ct.widx, ct.ridx, nev, slot0, nslots, n);
        int *ev = g.list + base;
        if (own && first) {
            for (int i = 0; i < n; ++i) ev[i] = ev_key(ev[i], K);
            sort_keys(ev, n);
        }
        lds_barrier();
        if (own) {
            for (int i = 0; i < n; ++i) {
                const int key = ev[i], t = key >> 7, k = key & 63, e = t * K + k;
                const int64_t rec = (static_cast<int64_t>(unit) * T + t0 + t) * K + k;
                Row4 *dst = reinterpret_cast<Row4 *>((key & 64 ? a.rec_r : a.rec_w) + rec * kBwdDv + c0);
#pragma unroll
                for (int j = 0; j < kCh / 4; ++j)
                    dst[j] = Row4{{row[4 * j], row[4 * j + 1], row[4 * j + 2], row[4 * j + 3]}};
                if (key & 64) continue;  // a read: recorded
                if (first) a.rec_m[rec] = m;
                const float w = ct.wt[e];
                if (w > 0.f) {
                    const float alpha = retention(w, expf(ct.gam[t]));
                    m = fmaf(alpha, m, w);
                    const float lam = w / (m + a.eps_gsu);
#pragma unroll
                    for (int c = 0; c < kCh; ++c)
                        row[c] = stored<TS>(fmaf(lam, ct.v[t][c0 + c] - row[c], row[c]));
                }
            }
        }
        lds_barrier();
    }
}

// Output gate, RMSNorm and read, for all tokens at once (they need only the
// recorded read rows): one wave per token-head, lane c holding channels
// c, c + 64, ... (DV / 64 of them).  Writes dg, dr (the read's adjoint, for
// the serial kernel) and d rho; each wave sums its tokens' d omega, and the
// workgroup's sum goes to a partial.
constexpr int kOutWaves = 16, kOutBlocks = kBwdOutBlocks;

template <typename TIn, int DV>
__global__ __launch_bounds__(kOutWaves * kWave) void bwd_out_kernel(BwdArgs a) {
    constexpr int CPL = DV / kWave;
    __shared__ float sdom[kOutWaves][DV];
    const int unit = blockIdx.x, b = unit / a.H, h = unit % a.H;
    const int wave = threadIdx.x / kWave, c = threadIdx.x % kWave;
    const int K = a.K, T = a.T;
    const TIn *gg = static_cast<const TIn *>(a.g);
    float om[CPL], dom[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        om[i] = a.norm_w ? a.norm_w[c + kWave * i] : 1.0f;
        dom[i] = 0.f;
    }
    for (int t = blockIdx.y * kOutWaves + wave; t < T; t += kOutBlocks * kOutWaves) {
        const int64_t th = (static_cast<int64_t>(b) * T + t) * a.H + h;
        const float *rr = a.rec_r + (static_cast<int64_t>(unit) * T + t) * K * DV + c;
        // lane k holds rho_k; rows load eight at a time (K <= 64)
        const float rw = a.r_wt[th * K + (c < K ? c : 0)];
        float r[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) r[i] = 0.f;
        for (int k0 = 0; k0 < K; k0 += 8) {
            float x[8][CPL];
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int i = 0; i < CPL; ++i) x[j][i] = k0 + j < K ? rr[(k0 + j) * DV + kWave * i] : 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (k0 + j < K) {
                    const float rho = bcast(rw, k0 + j);
#pragma unroll
                    for (int i = 0; i < CPL; ++i) r[i] = fmaf(rho, x[j][i], r[i]);
                }
        }
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) ss = fmaf(r[i], r[i], ss);
        const float den = wave_sum(ss) / static_cast<float>(DV) + a.eps_norm;
        const float inv = den > 0.f ? 1.0f / sqrtf(den) : 0.f;  // zero read, eps 0
        float y[CPL], dy[CPL], dr[CPL];
        float dyy = 0.f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int64_t o = th * DV + c + kWave * i;
            y[i] = r[i] * inv;
            const float sg = sigmoid(to_f32(gg[o]));
            const float d_o = a.dout[o];
            a.dg[o] = d_o * om[i] * y[i] * sg * (1.0f - sg);
            dom[i] = fmaf(d_o * y[i], sg, dom[i]);
            dy[i] = d_o * om[i] * sg;
            dyy = fmaf(dy[i], y[i], dyy);
        }
        dyy = wave_sum(dyy) / static_cast<float>(DV);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            dr[i] = inv * (dy[i] - y[i] * dyy);
            a.dr[th * DV + c + kWave * i] = dr[i];
        }
        if (K >= 16) {
            // lane k takes <dr, S_jk> over its recorded row, dr broadcast
            // channel by channel (cheaper than K wave reductions)
            const int kk = c < K ? c : 0;
            const Row4 *rk = reinterpret_cast<const Row4 *>(rr - c + kk * DV);
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < CPL; ++i)
#pragma unroll
                for (int j = 0; j < kWave / 4; ++j) {
                    const Row4 x = rk[i * (kWave / 4) + j];
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc = fmaf(bcast(dr[i], 4 * j + q), x.e[q], acc);
                }
            if (c < K) a.drho[th * K + c] = acc;
        } else {
            for (int k0 = 0; k0 < K; k0 += 8) {
                float x[8][CPL];
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int i = 0; i < CPL; ++i) x[j][i] = k0 + j < K ? rr[(k0 + j) * DV + kWave * i] : 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (k0 + j < K) {
                        float part = 0.f;
#pragma unroll
                        for (int i = 0; i < CPL; ++i) part = fmaf(dr[i], x[j][i], part);
                        const float dk = wave_sum(part);
                        if (c == 0) a.drho[th * K + k0 + j] = dk;
                    }
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) sdom[wave][c + kWave * i] = dom[i];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            float acc = 0.f;
            for (int w2 = 0; w2 < kOutWaves; ++w2) acc += sdom[w2][c + kWave * i];
            a.dom_part[(static_cast<int64_t>(unit) * kOutBlocks + blockIdx.y) * DV + c + kWave * i] = acc;
        }
    }
}

template <typename TIn, int HV, int EVM>
__global__ __launch_bounds__(kThreadsOf<HV>) void bwd_adjoint_kernel(BwdArgs a) {
    constexpr int kCh = kBwdDv / HV;
    __shared__ ChunkLds<HV, EVM> g;
    __shared__ ChunkTok<EVM> ct;
    const int unit = blockIdx.x, b = unit / a.H, h = unit % a.H;
    const int s = threadIdx.x / HV, c0 = (threadIdx.x % HV) * kCh;
    const bool first = c0 == 0;
    const int K = a.K, T = a.T;
    const int M = static_cast<int>(a.M);
    const int slot0 = blockIdx.y * kSlotsPerWG, slot = slot0 + s;
    const int nslots = min(kSlotsPerWG, M - slot0);
    const bool own = s < nslots;
    const int C = bwd_chunk(K, EVM);
    const int64_t srow = (static_cast<int64_t>(unit) * M + slot) * kBwdDv + c0;
    float dS[kCh];
    float dm = 0.f;
#pragma unroll
    for (int c = 0; c < kCh; ++c) dS[c] = 0.f;
    if (own && a.dS_final) {
        const Row4 *src = reinterpret_cast<const Row4 *>(a.dS_final + srow);
#pragma unroll
        for (int j = 0; j < kCh / 4; ++j) {
            const Row4 x = src[j];
#pragma unroll
            for (int c = 0; c < 4; ++c) dS[4 * j + c] = x.e[c];
        }
    }
    if (own && a.dmass_final) dm = a.dmass_final[static_cast<int64_t>(unit) * M + slot];
    const int nch = (T + C - 1) / C;
    ChunkPf<HV, EVM> pf;
    load_chunk<TIn, true, HV, EVM>(a, pf, b, h, (nch - 1) * C, T - (nch - 1) * C);
    for (int ci = nch - 1; ci >= 0; --ci) {
        const int t0 = ci * C, Cc = min(C, T - t0), nev = Cc * K;
        store_chunk<true, HV, EVM>(ct, pf, Cc, K);
        lds_barrier();
        if (ci > 0) load_chunk<TIn, true, HV, EVM>(a, pf, b, h, t0 - C, C);
        int n;
        const int base = group_events(g, ct.widx, ct.ridx, nev, slot0, nslots, n);
        int *ev = g.list + base;
        if (own && first) {
            for (int i = 0; i < n; ++i) ev[i] = ev_key(ev[i], K);
            sort_keys(ev, n);
        }
        lds_barrier();
        if (own) {
            // backwards: a token's read before its write
            for (int i = n - 1; i >= 0; --i) {
                const int key = ev[i], t = key >> 7, k = key & 63, e = t * K + k;
                if (key & 64) {
                    const float rho = ct.rt[e];
#pragma unroll
                    for (int c = 0; c < kCh; ++c) dS[c] = fmaf(rho, ct.dr[t][c0 + c], dS[c]);
                    continue;
                }
                const int64_t rec = (static_cast<int64_t>(unit) * T + t0 + t) * K + k;
                const float w = ct.wt[e];
                float dw = 0.f, dgk = 0.f;
                float *dvk = a.dvk + rec * kBwdDv + c0;
                if (w > 0.f) {
                    const float mm = a.rec_m[rec];
                    const float eg = expf(ct.gam[t]);
                    const float alpha = retention(w, eg);
                    const float mp = fmaf(alpha, mm, w);
                    const float den = mp + a.eps_gsu;
                    const float lam = w / den;
                    const Row4 *sm = reinterpret_cast<const Row4 *>(a.rec_w + rec * kBwdDv + c0);
                    float dl = 0.f;
#pragma unroll
                    for (int j = 0; j < kCh / 4; ++j) {
                        const Row4 x = sm[j];
#pragma unroll
                        for (int c = 0; c < 4; ++c) dl = fmaf(dS[4 * j + c], ct.v[t][c0 + 4 * j + c] - x.e[c], dl);
                    }
                    // the lanes' parts of <dS+, v - S-> (a butterfly: every lane of
                    // the slot gets the same sum)
#pragma unroll
                    for (int o = 1; o < HV; o <<= 1) dl += __shfl_xor(dl, o, kWave);
#pragma unroll
                    for (int j = 0; j < kCh / 4; ++j) {
                        reinterpret_cast<Row4 *>(dvk)[j] =
                            Row4{{lam * dS[4 * j], lam * dS[4 * j + 1], lam * dS[4 * j + 2], lam * dS[4 * j + 3]}};
#pragma unroll
                        for (int c = 0; c < 4; ++c) dS[4 * j + c] *= 1.0f - lam;
                    }
                    const float dmt = dm - dl * w / (den * den);
                    const float dalpha = dmt * mm;
                    dm = dmt * alpha;
                    dw = dl / den + dmt;
                    if (w < 1.0f && alpha > 0.f) {
                        dw -= dalpha * eg * alpha / (1.0f - w);
                        dgk = dalpha * alpha * log1pf(-w) * eg;
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < kCh / 4; ++j) reinterpret_cast<Row4 *>(dvk)[j] = Row4{{0.f, 0.f, 0.f, 0.f}};
                }
                if (first) {
                    a.dgk[rec] = dgk;
                    a.dw[((static_cast<int64_t>(b) * T + t0 + t) * a.H + h) * K + k] = dw;
                }
            }
        }
        lds_barrier();
    }
    if (own) {
        Row4 *dst = reinterpret_cast<Row4 *>(a.dS0 + srow);
#pragma unroll
        for (int j = 0; j < kCh / 4; ++j)
            dst[j] = Row4{{dS[4 * j], dS[4 * j + 1], dS[4 * j + 2], dS[4 * j + 3]}};
        if (first) a.dmass0[static_cast<int64_t>(unit) * M + slot] = dm;
    }
}

// dv and dgamma of every token: the sums over its writes of lam dS+ and of
// the gamma terms, in write order (one wave per token-head, lane c holding
// channels c, c + 64, ...).
template <int DV>
__global__ __launch_bounds__(256) void bwd_sum_kernel(BwdArgs a) {
    constexpr int CPL = DV / kWave;
    const int64_t n = static_cast<int64_t>(a.B) * a.T * a.H;
    const int64_t th = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
    const int c = threadIdx.x % kWave, K = a.K;
    if (th >= n) return;
    const int64_t b = th / (static_cast<int64_t>(a.T) * a.H), t = (th / a.H) % a.T;
    const int h = static_cast<int>(th % a.H);
    const int64_t rec = ((b * a.H + h) * a.T + t) * K;
    // lane k tells whether write k counts; the mask is the same in every
    // lane, so the row loads below go out together (K <= 64)
    const int kk = c < K ? c : 0;
    const int slot = a.w_idx[th * K + kk];
    const bool mine = c < K && a.w_wt[th * K + kk] > 0.f && slot >= 0 && slot < a.M;
    const uint64_t ok = __ballot(mine);
    const float gk = mine ? a.dgk[rec + kk] : 0.f;
    const float *dv = a.dvk + rec * DV + c;
    float acc[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[i] = 0.f;
    for (int k0 = 0; k0 < K; k0 += 8) {
        float x[8][CPL];
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int i = 0; i < CPL; ++i)
                x[j][i] = k0 + j < K ? dv[static_cast<int64_t>(k0 + j) * DV + kWave * i] : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if ((ok >> (k0 + j)) & 1u)
#pragma unroll
                for (int i = 0; i < CPL; ++i) acc[i] += x[j][i];
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) a.dv[th * DV + c + kWave * i] = acc[i];
    const float gacc = wave_sum(gk);
    if (c == 0) a.dgamma[th] = gacc;
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

// One thread per (token-head, q or k), a wave per 64 token-heads.  The
// wave's slots and coefficients d_w * w are first staged in LDS with
// coalesced loads (rows of K + 1 entries, so that the lanes' reads of their
// own rows do not collide in banks).  Then slot after slot: the content
// index is formed once, and the slot's digits are peeled from the last
// level up (a compile-time base), each adding to its level's d_p
// gradients.  The levels live in registers indexed from the last one (level
// U - 1 - j is entry j), U * d_p <= 64; every (level, digit) sum still runs
// over the slots in rank order.
template <typename TIn, int DP>
__global__ __launch_bounds__(kWave) void bwd_logits_kernel(BwdArgs a) {
    constexpr int UMAX = 64 / DP;
    extern __shared__ unsigned char smem[];
    const int64_t n = static_cast<int64_t>(a.B) * a.T * a.H;
    const bool key = blockIdx.y == 0;
    float *out = key ? a.dk : a.dq;
    if (!out) return;
    const int U = a.U, K = a.K, KS = K + 1;
    const int64_t i0 = static_cast<int64_t>(blockIdx.x) * kWave;
    const int nb = static_cast<int>(min<int64_t>(kWave, n - i0));
    int *sidx = reinterpret_cast<int *>(smem);
    float *scoef = reinterpret_cast<float *>(smem + static_cast<size_t>(kWave) * KS * 4);
    {
        const int32_t *gidx = (key ? a.w_idx : a.r_idx) + i0 * K;
        const float *gwt = (key ? a.w_wt : a.r_wt) + i0 * K;
        const float *ggr = (key ? a.dw : a.drho) + i0 * K;
        // e / K as mulhi(e, ceil(2^32 / K)): exact for e < 4096 (K = 1 apart)
        const unsigned mk = K > 1 ? 0xffffffffu / static_cast<unsigned>(K) + 1u : 0u;
        for (int e = threadIdx.x; e < nb * K; e += kWave) {
            const int r = K > 1 ? static_cast<int>(__umulhi(static_cast<unsigned>(e), mk)) : e;
            const int c = e - r * K;
            sidx[r * KS + c] = gidx[e];
            scoef[r * KS + c] = ggr[e] * gwt[e];
        }
    }
    __syncthreads();
    if (static_cast<int>(threadIdx.x) >= nb) return;
    const int64_t i = i0 + threadIdx.x;
    const TIn *lg = static_cast<const TIn *>(key ? a.k : a.q) + i * U * DP;
    const int *idx = sidx + threadIdx.x * KS;
    const float *coefs = scoef + threadIdx.x * KS;
    const int64_t b = i / (static_cast<int64_t>(a.T) * a.H), t = (i / a.H) % a.T;
    const int h = static_cast<int>(i % a.H);
    const int form = head_uses_cape(a.content_heads, h) ? a.cape : 0;
    const int64_t pos = (a.pos0 ? a.pos0[b] : 0) + t;
    const CapeShift sh = cape_shift<DP>(cape_inverse_pos(pos, form, DP, U, a.M), DP, a.M);
    float p[UMAX][DP], dl[UMAX][DP];
#pragma unroll
    for (int j = 0; j < UMAX; ++j) {
        if (j < U) {
            const TIn *l = lg + (U - 1 - j) * DP;
            float mx = to_f32(l[0]);
#pragma unroll
            for (int d = 1; d < DP; ++d) mx = fmaxf(mx, to_f32(l[d]));
            float sum = 0.f;
#pragma unroll
            for (int d = 0; d < DP; ++d) {
                p[j][d] = expf(to_f32(l[d]) - mx);
                sum += p[j][d];
                dl[j][d] = 0.f;
            }
#pragma unroll
            for (int d = 0; d < DP; ++d) p[j][d] /= sum;
        }
    }
    for (int k = 0; k < K; ++k) {
        const int slot = idx[k];
        if (slot < 0 || slot >= a.M) continue;
        const float coef = coefs[k];
        unsigned c = static_cast<unsigned>(form ? cape_slot_at<DP>(slot, sh, U, DP, form, a.M) : slot);
#pragma unroll
        for (int j = 0; j < UMAX; ++j) {
            if (j < U) {
                const unsigned digit = c % DP;
                c /= DP;
#pragma unroll
                for (int d = 0; d < DP; ++d)
                    dl[j][d] = fmaf(-coef, p[j][d], dl[j][d] + (static_cast<unsigned>(d) == digit ? coef : 0.f));
            }
        }
    }
#pragma unroll
    for (int j = 0; j < UMAX; ++j) {
        if (j < U) {
#pragma unroll
            for (int d = 0; d < DP; ++d) out[i * U * DP + (U - 1 - j) * DP + d] = dl[j][d];
        }
    }
}

template <typename TIn>
hipError_t launch_logits(const BwdArgs &a, dim3 grid, hipStream_t st) {
    const size_t lds = static_cast<size_t>(kWave) * (a.K + 1) * 8;  // slots and coefficients
    switch (a.d_p) {
#define RAMNET_LOGITS_DP(D) \
    case D: hipLaunchKernelGGL((bwd_logits_kernel<TIn, D>), grid, dim3(kWave), lds, st, a); break;
        RAMNET_LOGITS_DP(2) RAMNET_LOGITS_DP(3) RAMNET_LOGITS_DP(4) RAMNET_LOGITS_DP(5)
        RAMNET_LOGITS_DP(6) RAMNET_LOGITS_DP(7) RAMNET_LOGITS_DP(8)
#undef RAMNET_LOGITS_DP
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Sums the partials [n][DV] in a fixed order: 16 groups of 64 threads take
// interleaved partials, then group 0 adds the 16 group sums in order.
template <int DV>
__global__ __launch_bounds__(1024) void bwd_omega_kernel(const float *part, int n, float *out) {
    constexpr int CPL = DV / kWave;
    __shared__ float gsum[16][DV];
    const int c = threadIdx.x % kWave, grp = threadIdx.x / kWave;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        float acc = 0.f;
        for (int u = grp; u < n; u += 16) acc += part[static_cast<int64_t>(u) * DV + c + kWave * i];
        gsum[grp][c + kWave * i] = acc;
    }
    __syncthreads();
    if (grp == 0) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            float tot = 0.f;
            for (int j = 0; j < 16; ++j) tot += gsum[j][c + kWave * i];
            out[c + kWave * i] = tot;
        }
    }
}

// ---------------------------------------------------------------- rows in HBM
//
// A row of DV channels is moved by kRowLanes lanes, DV / kRowLanes adjacent
// channels each (fp32, or bf16 in 8-byte pieces).
constexpr int kRowLanes = 16;

typedef float bnt_f32x4 __attribute__((ext_vector_type(4)));
// fp32 records, written once and read once: non-temporal
template <int CPL>
__device__ __forceinline__ void nt_load_rec(const float *p, float (&x)[CPL]) {
#pragma unroll
    for (int j = 0; j < CPL / 4; ++j) {
        const bnt_f32x4 f = __builtin_nontemporal_load(reinterpret_cast<const bnt_f32x4 *>(p) + j);
        x[4 * j] = f.x;
        x[4 * j + 1] = f.y;
        x[4 * j + 2] = f.z;
        x[4 * j + 3] = f.w;
    }
}
template <int CPL>
__device__ __forceinline__ void nt_store_rec(float *p, const float (&x)[CPL]) {
#pragma unroll
    for (int j = 0; j < CPL / 4; ++j) {
        bnt_f32x4 f;
        f.x = x[4 * j];
        f.y = x[4 * j + 1];
        f.z = x[4 * j + 2];
        f.w = x[4 * j + 3];
        __builtin_nontemporal_store(f, reinterpret_cast<bnt_f32x4 *>(p) + j);
    }
}

template <typename TS, int CPL>
__device__ __forceinline__ void load_cpl(const TS *p, float (&x)[CPL]) {
    if constexpr (sizeof(TS) == 4) {
#pragma unroll
        for (int j = 0; j < CPL / 4; ++j) {
            const float4 f = reinterpret_cast<const float4 *>(p)[j];
            x[4 * j] = f.x;
            x[4 * j + 1] = f.y;
            x[4 * j + 2] = f.z;
            x[4 * j + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < CPL / 4; ++j) {
            const uint2 u = reinterpret_cast<const uint2 *>(p)[j];
            x[4 * j] = __uint_as_float(u.x << 16);
            x[4 * j + 1] = __uint_as_float(u.x & 0xffff0000u);
            x[4 * j + 2] = __uint_as_float(u.y << 16);
            x[4 * j + 3] = __uint_as_float(u.y & 0xffff0000u);
        }
    }
}
// x holds values already representable in TS.
template <typename TS, int CPL>
__device__ __forceinline__ void store_cpl(TS *p, const float (&x)[CPL]) {
    if constexpr (sizeof(TS) == 4) {
#pragma unroll
        for (int j = 0; j < CPL / 4; ++j)
            reinterpret_cast<float4 *>(p)[j] = make_float4(x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]);
    } else {
#pragma unroll
        for (int j = 0; j < CPL / 4; ++j)
            reinterpret_cast<uint2 *>(p)[j] =
                make_uint2((__float_as_uint(x[4 * j]) >> 16) | (__float_as_uint(x[4 * j + 1]) & 0xffff0000u),
                           (__float_as_uint(x[4 * j + 2]) >> 16) | (__float_as_uint(x[4 * j + 3]) & 0xffff0000u));
    }
}

// ---------------------------------------------------------------- slot-range walk
//
// Any d_v and any number of slots, many tokens per step: a unit's slots are
// split into kBR ranges (slot mod kBR), one workgroup per (unit, range), which
// owns its slots for the whole sequence, so the workgroups never wait for one
// another.  The sequence goes in chunks of br_chunk(K) tokens.  Per chunk:
//   * the chunk's events on the range (writes and reads) are listed in LDS
//     with the key slot << 32 | t << 7 | read << 6 | k and sorted (bitonic
//     network): a slot's events end up together, in forward order (a
//     token's writes before its reads, writes in address order);
//   * one group of lanes per slot (kBRLanes) walks its events with the
//     slot's row and mass (the replay, forwards: the row and mass before each
//     write and the row at each read are recorded) or its adjoint dS and dm
//     (the adjoint, backwards) in registers; an event's inputs (weights,
//     gamma, v, dr, the recorded row and mass) are gathered by token, all
//     requested before any is used.
// An event whose slot is outside [0, M) belongs to no range: the workgroup of
// range k mod kBR writes its zero records or gradients.
constexpr int kBR = 8;
constexpr int kBRThreads = 1024;
// lanes per row in the walk: 8 at d_v 64 (8 channels each), else 16
template <int DV> constexpr int kBRLanes = DV == 64 ? 8 : kRowLanes;
constexpr int kBRCap = 4096;  // events of a chunk (writes and reads)
constexpr int kBRPer = kBRCap / kBRThreads;  // list positions per thread in the segment scan

__host__ __device__ inline int br_chunk(int K) {
    int c = 64;
    while (c > 1 && 2 * c * K > kBRCap) c /= 2;
    return c;
}

struct BRLds {
    unsigned long long key[kBRCap];
    int seg[kBRCap + 1];
    int wtot[kBRThreads / kWave];
    int cnt, nseg;
};

// Lists the range's events of tokens [t0, t0 + Cc), sorts them, and finds
// the slot segments: afterwards g.seg[0 .. nseg] bound them.  inv(t, k, read)
// is called for the invalid events this range answers for.
template <typename Inv>
__device__ __forceinline__ void br_group(const BwdArgs &a, BRLds &g, int b, int h, int r, int t0, int Cc,
                                         Inv inv) {
    const int K = a.K, tid = threadIdx.x;
    const int64_t M = a.M;
    if (tid == 0) g.cnt = 0;
    __syncthreads();
    const int nw = Cc * K;
    for (int e = tid; e < 2 * nw; e += kBRThreads) {
        const bool rd = e >= nw;
        const int i = rd ? e - nw : e, t = i / K, k = i - t * K;
        const int64_t th = (static_cast<int64_t>(b) * a.T + t0 + t) * a.H + h;
        const int s = (rd ? a.r_idx : a.w_idx)[th * K + k];
        if (s >= 0 && static_cast<int64_t>(s) < M) {
            if ((s & (kBR - 1)) == r) {
                const int pos = atomicAdd(&g.cnt, 1);
                g.key[pos] = (static_cast<unsigned long long>(s) << 32) |
                             static_cast<unsigned long long>((t << 7) | ((rd ? 1 : 0) << 6) | k);
            }
        } else if ((k & (kBR - 1)) == r) {
            inv(t, k, rd);
        }
    }
    __syncthreads();
    const int n = g.cnt;
    int np = 1;
    while (np < n) np <<= 1;
    for (int i = n + tid; i < np; i += kBRThreads) g.key[i] = ~0ull;
    __syncthreads();
    for (int kk = 2; kk <= np; kk <<= 1) {
        for (int j = kk >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < np; i += kBRThreads) {
                const int ij = i ^ j;
                if (ij > i) {
                    const unsigned long long x = g.key[i], y = g.key[ij];
                    const bool up = (i & kk) == 0;
                    if ((x > y) == up) {
                        g.key[i] = y;
                        g.key[ij] = x;
                    }
                }
            }
            __syncthreads();
        }
    }
    // segment starts, in list order: thread i takes positions kBRPer i ..
    int f[kBRPer], nf = 0;
#pragma unroll
    for (int q = 0; q < kBRPer; ++q) {
        const int i = kBRPer * tid + q;
        f[q] = i < n && (i == 0 || (g.key[i] >> 32) != (g.key[i - 1] >> 32)) ? 1 : 0;
        nf += f[q];
    }
    const int lane = tid % kWave, wid = tid / kWave;
    int incl = nf;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += y;
    }
    if (lane == kWave - 1) g.wtot[wid] = incl;
    __syncthreads();
    int base = 0, tot = 0;
    for (int w = 0; w < kBRThreads / kWave; ++w) {
        const int c = g.wtot[w];
        base += w < wid ? c : 0;
        tot += c;
    }
    int at = base + incl - nf;
#pragma unroll
    for (int q = 0; q < kBRPer; ++q) {
        if (f[q]) g.seg[at] = kBRPer * tid + q;
        at += f[q];
    }
    if (tid == 0) {
        g.nseg = tot;
        g.seg[tot] = n;
    }
    __syncthreads();
}

template <typename TIn, typename TS, int DV>
__global__ __launch_bounds__(kBRThreads) void bwd_record_range_kernel(BwdArgs a) {
    constexpr int LPR = kBRLanes<DV>, CPL = DV / LPR, kBRGroups = kBRThreads / LPR;
    __shared__ BRLds g;
    const int unit = blockIdx.x, r = blockIdx.y, b = unit / a.H, h = unit % a.H;
    const int K = a.K, T = a.T;
    const int64_t M = a.M;
    const int grp = threadIdx.x / LPR, gl = threadIdx.x % LPR, c0 = gl * CPL;
    const int glead = (threadIdx.x % kWave) - gl;
    const int C = br_chunk(K);
    TS *Su = static_cast<TS *>(a.Sw) + static_cast<int64_t>(unit) * M * DV;
    float *mu = a.mw + static_cast<int64_t>(unit) * M;
    const TIn *vin = static_cast<const TIn *>(a.v);
    const TIn *gam = static_cast<const TIn *>(a.gamma);
    for (int t0 = 0; t0 < T; t0 += C) {
        const int Cc = min(C, T - t0);
        br_group(a, g, b, h, r, t0, Cc, [&](int t, int k, bool rd) {
            const int64_t rec = (static_cast<int64_t>(unit) * T + t0 + t) * K + k;
            float *dst = (rd ? a.rec_r : a.rec_w) + rec * DV;
            for (int c = 0; c < DV; ++c) dst[c] = 0.f;
            if (!rd) a.rec_m[rec] = 0.f;
        });
        const int nseg = g.nseg;
        for (int sg = grp; sg < nseg; sg += kBRGroups) {
            const int lo = g.seg[sg], hi = g.seg[sg + 1];
            const int slot = static_cast<int>(g.key[lo] >> 32);
            TS *row = Su + static_cast<int64_t>(slot) * DV + c0;
            float x[CPL];
            load_cpl<TS, CPL>(row, x);
            const float m0 = gl == 0 ? mu[slot] : 0.f;
            float m = __shfl(m0, glead, kWave);
            for (int i = lo; i < hi; ++i) {
                const int ek = static_cast<int>(g.key[i] & 0xffffffffu);
                const int t = ek >> 7, k = ek & 63;
                const int64_t rec = (static_cast<int64_t>(unit) * T + t0 + t) * K + k;
                if (ek & 64) {
                    nt_store_rec<CPL>(a.rec_r + rec * DV + c0, x);
                    continue;
                }
                // the event's inputs, all requested before any is used
                const int64_t th = (static_cast<int64_t>(b) * T + t0 + t) * a.H + h;
                const float w = a.w_wt[th * K + k];
                const TIn gt = gam[th];
                float vr[CPL];
                load_cpl<TIn, CPL>(vin + th * DV + c0, vr);
                nt_store_rec<CPL>(a.rec_w + rec * DV + c0, x);
                if (gl == 0) a.rec_m[rec] = m;
                if (w > 0.f) {
                    const float alpha = retention(w, expf(to_f32(gt)));
                    m = fmaf(alpha, m, w);
                    const float lam = w / (m + a.eps_gsu);
#pragma unroll
                    for (int c = 0; c < CPL; ++c) x[c] = stored<TS>(fmaf(lam, vr[c] - x[c], x[c]));
                }
            }
            store_cpl<TS, CPL>(row, x);
            if (gl == 0) mu[slot] = m;
        }
        __syncthreads();  // the rows written here may be another group's next chunk
    }
}

template <typename TIn, int DV>
__global__ __launch_bounds__(kBRThreads) void bwd_adjoint_range_kernel(BwdArgs a) {
    constexpr int LPR = kBRLanes<DV>, CPL = DV / LPR, kBRGroups = kBRThreads / LPR;
    __shared__ BRLds g;
    const int unit = blockIdx.x, r = blockIdx.y, b = unit / a.H, h = unit % a.H;
    const int K = a.K, T = a.T;
    const int64_t M = a.M;
    const int grp = threadIdx.x / LPR, gl = threadIdx.x % LPR, c0 = gl * CPL;
    const int glead = (threadIdx.x % kWave) - gl;
    const int C = br_chunk(K);
    float *dSu = a.dS0 + static_cast<int64_t>(unit) * M * DV;
    float *dmu = a.dmass0 + static_cast<int64_t>(unit) * M;
    const TIn *vin = static_cast<const TIn *>(a.v);
    const TIn *gam = static_cast<const TIn *>(a.gamma);
    const int nch = (T + C - 1) / C;
    for (int ci = nch - 1; ci >= 0; --ci) {
        const int t0 = ci * C, Cc = min(C, T - t0);
        br_group(a, g, b, h, r, t0, Cc, [&](int t, int k, bool rd) {
            if (rd) return;
            const int64_t rec = (static_cast<int64_t>(unit) * T + t0 + t) * K + k;
            for (int c = 0; c < DV; ++c) a.dvk[rec * DV + c] = 0.f;
            a.dgk[rec] = 0.f;
            a.dw[((static_cast<int64_t>(b) * T + t0 + t) * a.H + h) * K + k] = 0.f;
        });
        const int nseg = g.nseg;
        for (int sg = grp; sg < nseg; sg += kBRGroups) {
            const int lo = g.seg[sg], hi = g.seg[sg + 1];
            const int slot = static_cast<int>(g.key[lo] >> 32);
            float *row = dSu + static_cast<int64_t>(slot) * DV + c0;
            float d[CPL];
            load_cpl<float, CPL>(row, d);
            const float dm0 = gl == 0 ? dmu[slot] : 0.f;
            float dm = __shfl(dm0, glead, kWave);
            for (int i = hi - 1; i >= lo; --i) {
                const int ek = static_cast<int>(g.key[i] & 0xffffffffu);
                const int t = ek >> 7, k = ek & 63;
                const int64_t th = (static_cast<int64_t>(b) * T + t0 + t) * a.H + h;
                if (ek & 64) {
                    const float rho = a.r_wt[th * K + k];
                    float dr[CPL];
                    load_cpl<float, CPL>(a.dr + th * DV + c0, dr);
#pragma unroll
                    for (int c = 0; c < CPL; ++c) d[c] = fmaf(rho, dr[c], d[c]);
                    continue;
                }
                const int64_t rec = (static_cast<int64_t>(unit) * T + t0 + t) * K + k;
                float *dvk = a.dvk + rec * DV + c0;
                // the event's inputs, all requested before any is used
                const float w = a.w_wt[th * K + k];
                float sm[CPL];
                nt_load_rec<CPL>(a.rec_w + rec * DV + c0, sm);
                float vr[CPL];
                load_cpl<TIn, CPL>(vin + th * DV + c0, vr);
                const float mm = a.rec_m[rec];
                const TIn gt = gam[th];
                float dw = 0.f, dgk = 0.f;
                if (w > 0.f) {
                    const float eg = expf(to_f32(gt));
                    const float alpha = retention(w, eg);
                    const float mp = fmaf(alpha, mm, w);
                    const float den = mp + a.eps_gsu;
                    const float lam = w / den;
                    float dl = 0.f;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) dl = fmaf(d[c], vr[c] - sm[c], dl);
#pragma unroll
                    for (int o = 1; o < LPR; o <<= 1) dl += __shfl_xor(dl, o, kWave);
                    float dv[CPL];
#pragma unroll
                    for (int c = 0; c < CPL; ++c) {
                        dv[c] = lam * d[c];
                        d[c] *= 1.0f - lam;
                    }
                    nt_store_rec<CPL>(dvk, dv);
                    const float dmt = dm - dl * w / (den * den);
                    const float dalpha = dmt * mm;
                    dw = dl / den + dmt;
                    if (w < 1.0f && alpha > 0.f) {
                        dw -= dalpha * eg * alpha / (1.0f - w);
                        dgk = dalpha * alpha * log1pf(-w) * eg;
                    }
                    dm = dmt * alpha;
                } else {
                    float z[CPL];
#pragma unroll
                    for (int c = 0; c < CPL; ++c) z[c] = 0.f;
                    nt_store_rec<CPL>(dvk, z);
                }
                if (gl == 0) {
                    a.dgk[rec] = dgk;
                    a.dw[th * K + k] = dw;
                }
            }
            store_cpl<float, CPL>(row, d);
            if (gl == 0) dmu[slot] = dm;
        }
        __syncthreads();
    }
}

// dst[i] = src ? src[i] : 0 over n floats (the walk's starting buffers).
__global__ __launch_bounds__(256) void bwd_copy_kernel(float *dst, const float *src, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * 256)
        dst[i] = src ? src[i] : 0.f;
}
__global__ __launch_bounds__(256) void bwd_copy16_kernel(uint16_t *dst, const uint16_t *src, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * 256)
        dst[i] = src[i];
}

// The slot-range walk for any d_v and any M: the starting buffers, the
// replay, the output/read kernel, the adjoint.
template <typename TIn, int DV>
hipError_t launch_walk(const BwdArgs &a, hipStream_t st) {
    const int units = a.B * a.H;
    const int64_t ns = static_cast<int64_t>(units) * a.M;
    auto grid_of = [](int64_t n) { return dim3(static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 4096))); };
    if (a.state_bf16)
        hipLaunchKernelGGL(bwd_copy16_kernel, grid_of(ns * DV), dim3(256), 0, st,
                           static_cast<uint16_t *>(a.Sw), static_cast<const uint16_t *>(a.S0), ns * DV);
    else
        hipLaunchKernelGGL(bwd_copy_kernel, grid_of(ns * DV), dim3(256), 0, st, static_cast<float *>(a.Sw),
                           static_cast<const float *>(a.S0), ns * DV);
    hipLaunchKernelGGL(bwd_copy_kernel, grid_of(ns), dim3(256), 0, st, a.mw, a.mass0, ns);
    hipLaunchKernelGGL(bwd_copy_kernel, grid_of(ns * DV), dim3(256), 0, st, a.dS0, a.dS_final, ns * DV);
    hipLaunchKernelGGL(bwd_copy_kernel, grid_of(ns), dim3(256), 0, st, a.dmass0, a.dmass_final, ns);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.state_bf16)
        hipLaunchKernelGGL((bwd_record_range_kernel<TIn, bf16_t, DV>), dim3(units, kBR), dim3(kBRThreads), 0, st, a);
    else
        hipLaunchKernelGGL((bwd_record_range_kernel<TIn, float, DV>), dim3(units, kBR), dim3(kBRThreads), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_out_kernel<TIn, DV>), dim3(units, kOutBlocks), dim3(kOutWaves * kWave), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_adjoint_range_kernel<TIn, DV>), dim3(units, kBR), dim3(kBRThreads), 0, st, a);
    return hipGetLastError();
}

template <int DV>
hipError_t launch_tail(const BwdArgs &a, hipStream_t st) {
    const int units = a.B * a.H;
    const int64_t n = static_cast<int64_t>(units) * a.T;
    hipLaunchKernelGGL((bwd_sum_kernel<DV>), dim3(static_cast<unsigned>((n + 3) / 4)), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.dq || a.dk) {
        e = a.in_bf16 ? launch_logits<bf16_t>(a, dim3(static_cast<unsigned>((n + kWave - 1) / kWave), 2), st)
                      : launch_logits<float>(a, dim3(static_cast<unsigned>((n + kWave - 1) / kWave), 2), st);
        if (e != hipSuccess) return e;
    }
    if (a.dnorm_w) {
        hipLaunchKernelGGL((bwd_omega_kernel<DV>), dim3(1), dim3(1024), 0, st, a.dom_part, units * kOutBlocks,
                           a.dnorm_w);
        e = hipGetLastError();
    }
    return e;
}

template <typename TIn>
hipError_t launch_in(const BwdArgs &a, hipStream_t st) {
    if (!backward_slot_owner(a.M, a.d_v)) {
        hipError_t e;
        switch (a.d_v) {
            case 64: e = launch_walk<TIn, 64>(a, st); break;
            case 128: e = launch_walk<TIn, 128>(a, st); break;
            case 192: e = launch_walk<TIn, 192>(a, st); break;
            case 256: e = launch_walk<TIn, 256>(a, st); break;
            default: return hipErrorInvalidValue;
        }
        if (e != hipSuccess) return e;
        switch (a.d_v) {
            case 64: return launch_tail<64>(a, st);
            case 128: return launch_tail<128>(a, st);
            case 192: return launch_tail<192>(a, st);
            default: return launch_tail<256>(a, st);
        }
    }
    const int units = a.B * a.H;
    const dim3 grid(units, static_cast<unsigned>((a.M + kSlotsPerWG - 1) / kSlotsPerWG));
    // Whether the grid has at most one workgroup per CU: then the adjoint
    // takes four lanes per slot (at 185 registers one workgroup fits a CU)
    // and both serial kernels take 4096-event chunks; otherwise two lanes
    // and 2048 events, two workgroups per CU.  The replay always takes four
    // lanes per slot.
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        ncu = 0;
    const bool wide = static_cast<int64_t>(grid.x) * grid.y <= ncu;
    if (a.state_bf16) {
        if (wide)
            hipLaunchKernelGGL((bwd_record_kernel<TIn, bf16_t, 4, 4096>), grid, dim3(kThreadsOf<4>), 0, st, a);
        else
            hipLaunchKernelGGL((bwd_record_kernel<TIn, bf16_t, 4, 2048>), grid, dim3(kThreadsOf<4>), 0, st, a);
    } else {
        if (wide)
            hipLaunchKernelGGL((bwd_record_kernel<TIn, float, 4, 4096>), grid, dim3(kThreadsOf<4>), 0, st, a);
        else
            hipLaunchKernelGGL((bwd_record_kernel<TIn, float, 4, 2048>), grid, dim3(kThreadsOf<4>), 0, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_out_kernel<TIn, kBwdDv>), dim3(units, kOutBlocks), dim3(kOutWaves * kWave), 0,
                       st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (wide)
        hipLaunchKernelGGL((bwd_adjoint_kernel<TIn, 4, 4096>), grid, dim3(kThreadsOf<4>), 0, st, a);
    else
        hipLaunchKernelGGL((bwd_adjoint_kernel<TIn, 2, 2048>), grid, dim3(kThreadsOf<2>), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_tail<kBwdDv>(a, st);
}

}  // namespace

bool backward_slot_owner(int64_t M, int d_v) { return d_v == kBwdDv && M <= kBwdNT; }

bool backward_supported(int64_t, int d_v, int U, int d_p, bool) {
    return d_v % kWave == 0 && d_v <= 256 && U * d_p <= 64;
}

size_t backward_workspace_bytes(int B, int T, int H, int K, int64_t M, int d_v, bool state_bf16) {
    const size_t units = static_cast<size_t>(B) * H;
    const size_t n = units * T;
    const size_t dv = static_cast<size_t>(d_v);
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    size_t bytes = 3 * al(n * K * dv * 4) + 4 * al(n * K * 4) + al(units * kOutBlocks * dv * 4) + al(n * dv * 4);
    if (!backward_slot_owner(M, d_v))
        bytes += al(units * static_cast<size_t>(M) * dv * (state_bf16 ? 2 : 4)) + al(units * static_cast<size_t>(M) * 4);
    return bytes;
}

hipError_t launch_backward(const BwdArgs &a, hipStream_t st) {
    if (static_cast<int64_t>(a.B) * a.H * a.T == 0) return hipSuccess;
    return a.in_bf16 ? launch_in<bf16_t>(a, st) : launch_in<float>(a, st);
}

}  // namespace ramnet
