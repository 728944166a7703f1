// One decoding step for gfx950, fused: address decoding, CAPE, the Gated
// Sparse Update, the read, RMSNorm and the gate for one token of each of B
// sequences (RAM-Net project page, GPU-execution paragraphs: decoding
// accesses the current token's slots directly, with no pass over the state).
//
// One wave serves UPW = 32 / KP (batch, head) units, KP = K rounded up to a
// power of two.
//  * Decoding: each of the wave's 2 * UPW addresses (key -> write, query ->
//    read) gets KP lanes; lane r holds entry r of the kept prefixes (sorted
//    by weight desc, prefix asc).  Per level, lane r's candidates are its
//    prefix extended by each digit value; candidate list a (prefix x p_u[a])
//    is sorted across the lanes because the prefixes are.  The next beam is
//    the first K entries of the merge of the d_p lists, built by a tree of
//    bitonic merges: list B reversed against list A, the better of each
//    pair, then log2(KP) compare-exchange stages.  This replaces K serial
//    merge steps per level by log2(KP) parallel ones.  At the first levels,
//    where every candidate can have a lane of its own (beam entries x d_p
//    <= KP), one bitonic sort of the candidates gives the same beam in
//    fewer stages.  Candidates rank by the sum of their digits' logits in
//    fp64 (a slot's weight is exp(that sum - the levels' log-normalisers),
//    the normalisers being common to all candidates), ties by the smaller
//    prefix, as in the prefill's decoder; the weights are formed at the end.
//    Every level's log-normaliser is computed first, one (address, level)
//    per lane, and kept in LDS.
//  * Update and read, one round trip to HBM: the masses of the write slots
//    and every write row and read row of the wave's units are loaded at
//    once.  Rows move in 16-byte pieces (12 where 16 would not tile a wave):
//    LPR lanes per row, 64 / LPR rows per load instruction.  The read is
//    taken from the rows as they were before this token's writes, plus, for
//    each write slot, the read's weight on that slot times the change the
//    write made; this equals the read after the writes without a second
//    pass over memory (non-temporal: a row piece is touched once per step).
//    Every load is consumed before the first store.  The
//    sub-row partial reads are summed through LDS; RMSNorm over d_v by a
//    wave reduction; the gate.
//  * Tiered state (TIER): the rows live in host memory except each unit's
//    cached ones (AI Radio page, deployment remark: only frequently accessed
//    slots in VRAM).  The decoding phase also fetches each address's cache
//    line and counts the access; the row phase takes each row where it
//    lives.  Nothing else changes, so the results are those of the
//    all-in-HBM step bit for bit.
#include "device_common.h"
#include "launch.h"

namespace ramnet {
namespace {

// Most digits an address has: U * d_p with d_p^U <= 2^30 peaks at 80 (d_p 8).
constexpr int kMaxDigits = 80;

// CPL adjacent channels of one row as a single vector access.
template <typename T, int CPL>
struct RowVec {
    T e[CPL];
};

// (logit sum, prefix) entries; invalid entries have sum -inf and prefix -1.
struct Ent {
    double w;
    int p;
};

// Logit sum desc (weight desc), then prefix asc.  An invalid entry's sum is
// -inf and its prefix the largest unsigned value, so invalid entries rank
// last.
// Branch-free: both comparisons are evaluated.
__device__ __forceinline__ bool better(const Ent &a, const Ent &b) {
    const bool gt = a.w > b.w, eq = a.w == b.w;
    const bool lt = static_cast<unsigned>(a.p) < static_cast<unsigned>(b.p);
    return gt | (eq & lt);
}

// Value of lane (r ^ J) within groups of KP lanes (lane_xor), or, for
// J == KP - 1, of the mirrored lane (row mirrors, plus the xor-16 swizzle
// for 32-lane groups).
template <int KP, int J>
__device__ __forceinline__ int xchg(int v) {
    if constexpr (J == 7 && KP == 8) return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);
    else if constexpr (J == 15 && KP == 16) return __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false);
    else if constexpr (J == 31 && KP == 32)
        return lane_xor<16>(__builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false));
    else return lane_xor<J>(v);
}

template <int KP, int J>
__device__ __forceinline__ Ent xchg_e(const Ent &e) {
    Ent o;
    const int lo = xchg<KP, J>(__double2loint(e.w));
    const int hi = xchg<KP, J>(__double2hiint(e.w));
    o.w = __hiloint2double(hi, lo);
    o.p = xchg<KP, J>(e.p);
    return o;
}

template <int KP, int J>
__device__ __forceinline__ Ent bitonic_stage(Ent e, int r) {
    const Ent o = xchg_e<KP, J>(e);
    const bool keep_better = (r & J) == 0;
    const bool ob = better(o, e);
    return (keep_better == ob) ? o : e;
}

// Sorts a bitonic sequence held one entry per lane across KP lanes into
// rank order (best at r = 0).
template <int KP>
__device__ __forceinline__ Ent bitonic_finish(Ent e, int r) {
    if constexpr (KP >= 32) e = bitonic_stage<KP, 16>(e, r);
    if constexpr (KP >= 16) e = bitonic_stage<KP, 8>(e, r);
    if constexpr (KP >= 8) e = bitonic_stage<KP, 4>(e, r);
    e = bitonic_stage<KP, 2>(e, r);
    e = bitonic_stage<KP, 1>(e, r);
    return e;
}

// First KP entries, in rank order, of two rank-ordered lists A and B held
// one entry per lane.
template <int KP>
__device__ __forceinline__ Ent merge_top(const Ent &a, const Ent &b, int r) {
    const Ent brev = xchg_e<KP, KP - 1>(b);   // lane r sees B[KP-1-r]
    const Ent c = better(brev, a) ? brev : a;  // bitonic: the top KP of A u B
    return bitonic_finish<KP>(c, r);
}

// Value of the lane mirrored within its block of S lanes (lane i of the
// block sees lane S - 1 - i): quad permute, row half mirror, row mirror,
// and for 32 lanes the row mirror of the other row.
template <int S>
__device__ __forceinline__ int mirror(int v) {
    static_assert(S == 2 || S == 4 || S == 8 || S == 16 || S == 32, "mirror");
    if constexpr (S == 2) return lane_xor<1>(v);
    else if constexpr (S == 4) return __builtin_amdgcn_mov_dpp(v, 0x1B, 0xF, 0xF, false);
    else if constexpr (S == 8) return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);
    else if constexpr (S == 16) return __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false);
    else return lane_xor<16>(__builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false));
}
template <int S>
__device__ __forceinline__ Ent mirror_e(const Ent &e) {
    Ent o;
    const int lo = mirror<S>(__double2loint(e.w));
    const int hi = mirror<S>(__double2hiint(e.w));
    o.w = __hiloint2double(hi, lo);
    o.p = mirror<S>(e.p);
    return o;
}
// Two rank-ordered runs of S / 2 lanes in each block of S lanes: the first
// half keeps the better of each mirrored pair (the top S / 2, bitonic), the
// second half the worse.
template <int S>
__device__ __forceinline__ Ent mirror_stage(Ent e, int r) {
    const Ent o = mirror_e<S>(e);
    const bool keep_better = (r & (S / 2)) == 0;
    return (keep_better == better(o, e)) ? o : e;
}
// Sorts the entries of each block of S lanes into rank order (best first):
// runs of 2, 4, ... S lanes, each merge a mirror stage and the halving
// stages of the bitonic finish.
template <int KP, int S>
__device__ __forceinline__ Ent bitonic_sort(Ent e, int r) {
    e = mirror_stage<2>(e, r);
    if constexpr (S >= 4) {
        e = mirror_stage<4>(e, r);
        e = bitonic_stage<KP, 1>(e, r);
    }
    if constexpr (S >= 8) {
        e = mirror_stage<8>(e, r);
        e = bitonic_stage<KP, 2>(e, r);
        e = bitonic_stage<KP, 1>(e, r);
    }
    if constexpr (S >= 16) {
        e = mirror_stage<16>(e, r);
        e = bitonic_stage<KP, 4>(e, r);
        e = bitonic_stage<KP, 2>(e, r);
        e = bitonic_stage<KP, 1>(e, r);
    }
    if constexpr (S >= 32) {
        e = mirror_stage<32>(e, r);
        e = bitonic_stage<KP, 8>(e, r);
        e = bitonic_stage<KP, 4>(e, r);
        e = bitonic_stage<KP, 2>(e, r);
        e = bitonic_stage<KP, 1>(e, r);
    }
    return e;
}

// Row access geometry for d_v channels of type TS: each lane moves VW bytes
// of one row (16, or 12 where 16-byte pieces would not tile the wave), LPR
// lanes cover a row and one instruction moves RPI = 64 / LPR rows.
template <typename TS, int DV>
struct RowGeom {
    static constexpr int kRowBytes = DV * static_cast<int>(sizeof(TS));
    static constexpr int VW = (kWave % (kRowBytes / 16) == 0) ? 16 : 12;
    static constexpr int NW = VW / 4;
    static constexpr int LPR = kRowBytes / VW;
    static constexpr int RPI = kWave / LPR;
    static constexpr int CPL = VW / static_cast<int>(sizeof(TS));
    static_assert(kRowBytes % VW == 0 && kWave % LPR == 0, "row geometry");
};

// Row registers one unit needs per address kind, and how many units are held
// at once (rows of at most 128 registers in flight per lane).
template <typename TS, int KP, int DV>
struct RowPlan {
    using G = RowGeom<TS, DV>;
    static constexpr int UPW = kWave / (2 * KP);
    static constexpr int NJ = (KP + G::RPI - 1) / G::RPI;  // row loads per unit and kind
    static constexpr int PER = NJ * G::NW;
    static constexpr bool kFits = PER <= 64;
    static constexpr int UB = PER <= 16 ? (UPW < 4 ? UPW : 4) : PER <= 32 ? (UPW < 2 ? UPW : 2) : 1;
};

template <int NW>
struct alignas(NW == 4 ? 16 : 4) Words {
    uint32_t w[NW];
};

typedef unsigned int ntu32x4 __attribute__((ext_vector_type(4)));
// Row pieces are touched once per step: loads and stores that do not keep
// them in the caches.
template <int NW>
__device__ __forceinline__ Words<NW> nt_load(const void *p) {
    if constexpr (NW == 4) {
        const ntu32x4 v = __builtin_nontemporal_load(static_cast<const ntu32x4 *>(p));
        Words<NW> x;
        x.w[0] = v.x; x.w[1] = v.y; x.w[2] = v.z; x.w[3] = v.w;
        return x;
    } else {
        return *static_cast<const Words<NW> *>(p);
    }
}
template <int NW>
__device__ __forceinline__ void nt_store(void *p, const Words<NW> &x) {
    if constexpr (NW == 4) {
        ntu32x4 v;
        v.x = x.w[0]; v.y = x.w[1]; v.z = x.w[2]; v.w = x.w[3];
        __builtin_nontemporal_store(v, static_cast<ntu32x4 *>(p));
    } else {
        *static_cast<Words<NW> *>(p) = x;
    }
}

template <typename TS, int NW>
__device__ __forceinline__ void unpack(const Words<NW> &x, float *f) {
    if constexpr (sizeof(TS) == 2) {
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            f[2 * i] = __uint_as_float(x.w[i] << 16);
            f[2 * i + 1] = __uint_as_float(x.w[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < NW; ++i) f[i] = __uint_as_float(x.w[i]);
    }
}

// Rounds to TS; f is replaced by the stored values.
template <typename TS, int NW>
__device__ __forceinline__ Words<NW> pack(float *f) {
    Words<NW> x;
    if constexpr (sizeof(TS) == 2) {
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const uint32_t lo = bf16_rne(f[2 * i]).bits, hi = bf16_rne(f[2 * i + 1]).bits;
            x.w[i] = lo | (hi << 16);
            f[2 * i] = __uint_as_float(lo << 16);
            f[2 * i + 1] = __uint_as_float(hi << 16);
        }
    } else {
#pragma unroll
        for (int i = 0; i < NW; ++i) x.w[i] = __float_as_uint(f[i]);
    }
    return x;
}

// Byte offsets of the kernel's LDS arrays.
struct StepLds {
    int idx, wt, lg, pr, lam, cr, red, ln, total;
};
__host__ __device__ constexpr StepLds step_lds(int UPW, int K, int L, int RPI, int DV) {
    StepLds o{};
    o.idx = 0;                                   // int   [UPW][2][K]
    o.wt = o.idx + UPW * 2 * K * 4;              // float [UPW][2][K]
    o.lg = o.wt + UPW * 2 * K * 4;               // float [UPW][2][L]
    o.pr = (o.lg + UPW * 2 * L * 4 + 7) & ~7;    // double[UPW][2][U]: the levels' log-normalisers
    o.lam = o.pr + UPW * 2 * L * 8;              // float [UPW][K]
    o.cr = o.lam + UPW * K * 4;                  // float [UPW][K]
    o.red = o.cr + UPW * K * 4;                  // float [RPI][DV]
    o.ln = o.red + RPI * DV * 4;                 // int   [UPW][2][K]: cache lines (tiered state)
    o.total = o.ln + UPW * 2 * K * 4;
    return o;
}

// TIER: the rows of cached slots live in a.cache (line a.slot_line[slot]),
// the others in a.S (host memory); each accessed slot's count is raised.
template <typename TIn, typename TS, int KP, int DV, bool TIER>
__global__ __launch_bounds__(kWave) void step_fused_kernel(StepArgs a) {
    using G = RowGeom<TS, DV>;
    using P = RowPlan<TS, KP, DV>;
    constexpr int UPW = P::UPW, NW = G::NW, CPL = G::CPL, LPR = G::LPR, RPI = G::RPI;
    constexpr int NJ = P::NJ, UB = P::UB;
    constexpr int CPO = DV / kWave;  // output channels per lane
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x;
    const int K = a.K, U = a.U, dp = a.d_p;
    const int64_t M = a.M;
    const int units = a.B * a.H;
    const int u0 = blockIdx.x * UPW;
    const int nu = min(UPW, units - u0);
    const int L = U * dp;
    const StepLds lo = step_lds(UPW, K, L, RPI, DV);
    int *sidx = reinterpret_cast<int *>(smem + lo.idx);
    float *swt = reinterpret_cast<float *>(smem + lo.wt);
    float *slg = reinterpret_cast<float *>(smem + lo.lg);
    double *slse = reinterpret_cast<double *>(smem + lo.pr);
    float *slam = reinterpret_cast<float *>(smem + lo.lam);
    float *scr = reinterpret_cast<float *>(smem + lo.cr);
    float *sred = reinterpret_cast<float *>(smem + lo.red);
    int *sline = reinterpret_cast<int *>(smem + lo.ln);

    // the gates and norm weights of the wave's units do not depend on the
    // addresses: their loads go out first and land during the decoding
    const TIn *gg = static_cast<const TIn *>(a.g);
    float gpre[UPW][CPO], ompre[CPO];
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
        const int unit = min(u0 + i, units - 1);
        const TIn *gu = gg + static_cast<int64_t>(unit / a.H) * a.ld_g + (unit % a.H) * DV + lane * CPO;
#pragma unroll
        for (int c = 0; c < CPO; ++c) gpre[i][c] = to_f32(gu[c]);
    }
#pragma unroll
    for (int c = 0; c < CPO; ++c) ompre[c] = a.norm_w ? a.norm_w[lane * CPO + c] : 1.0f;

    // every logit the wave decodes, fetched at once
    for (int i = lane; i < UPW * 2 * L; i += kWave) {
        const int g = i / L, e = i - g * L;
        const int unit = min(u0 + g / 2, units - 1);
        const TIn *src = static_cast<const TIn *>(g % 2 ? a.q : a.k);
        slg[i] = to_f32(src[(unit / a.H) * a.ld_qk + (unit % a.H) * L + e]);
    }
    __syncthreads();
    // every level's log-normaliser, one (address, level) per lane:
    // max + log(sum exp(l - max)), the sum in fp64 in digit order
    for (int i = lane; i < UPW * 2 * U; i += kWave) {
        const float *lv = slg + i * dp;
        float mx = lv[0];
        for (int d = 1; d < dp; ++d) mx = fmaxf(mx, lv[d]);
        double sum = 0.0;
        for (int d = 0; d < dp; ++d) sum += exp(static_cast<double>(lv[d]) - static_cast<double>(mx));
        slse[i] = static_cast<double>(mx) + log(sum);
    }
    __syncthreads();

    // ---------------- decoding: group g = address, lane r = beam rank
    {
        const int g = lane / KP, r = lane % KP;
        const int ul = g / 2, which = g % 2;  // which 0: key -> write, 1: query -> read
        const int unit = min(u0 + ul, units - 1);  // spare groups decode a copy, never stored
        const float *pg = slg + g * L;
        Ent beam;
        beam.w = r == 0 ? 0.0 : -__builtin_inf();
        beam.p = r == 0 ? 0 : -1;
        int nb = 1;  // entries of the beam (the same in every lane)
        for (int u = 0; u < U; ++u) {
            const int nc = nb * dp;  // candidates
            if (nc <= KP) {
                // every candidate has a lane of its own: lane r extends
                // beam entry r / d_p by digit r % d_p, and one bitonic sort
                // orders them (fewer stages than merging d_p lists)
                const int bi = r / dp, d = r - bi * dp;
                const int src = lane - r + (bi < nb ? bi : 0);
                Ent c;
                c.w = __hiloint2double(__shfl(__double2hiint(beam.w), src), __shfl(__double2loint(beam.w), src));
                c.p = __shfl(beam.p, src);
                const bool ok = r < nc;
                c.w = ok ? c.w + static_cast<double>(pg[u * dp + (ok ? d : 0)]) : -__builtin_inf();
                c.p = ok ? c.p * dp + d : -1;
                Ent res;
                if (nc <= 2) res = bitonic_sort<KP, 2>(c, r);
                else if (nc <= 4) res = bitonic_sort<KP, 4>(c, r);
                else if (KP >= 8 && nc <= 8) res = bitonic_sort<KP, (KP >= 8 ? 8 : 2)>(c, r);
                else if (KP >= 16 && nc <= 16) res = bitonic_sort<KP, (KP >= 16 ? 16 : 2)>(c, r);
                else res = bitonic_sort<KP, KP>(c, r);
                if (r >= K) {
                    res.w = -__builtin_inf();
                    res.p = -1;
                }
                beam = res;
                nb = min(K, nc);
                continue;
            }
            double lgd[8];
#pragma unroll
            for (int d = 0; d < 8; ++d) lgd[d] = d < dp ? static_cast<double>(pg[u * dp + d]) : 0.0;
            // candidate lists and their merge tree
            Ent lst[8];
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const bool ok = beam.p >= 0 && d < dp;
                lst[d].w = ok ? beam.w + lgd[d] : -__builtin_inf();
                lst[d].p = ok ? beam.p * dp + d : -1;
            }
            Ent res = merge_top<KP>(lst[0], lst[1], r);
            if (dp > 2) res = merge_top<KP>(res, merge_top<KP>(lst[2], lst[3], r), r);
            if (dp > 4)
                res = merge_top<KP>(res, merge_top<KP>(merge_top<KP>(lst[4], lst[5], r),
                                                       merge_top<KP>(lst[6], lst[7], r), r), r);
            if (r >= K) {  // keep K entries
                res.w = -__builtin_inf();
                res.p = -1;
            }
            beam = res;
            nb = min(K, nc);
        }
        // CAPE and hand-off
        const int b = unit / a.H;
        const int64_t pos = a.pos ? a.pos[b] : 0;
        if (u0 + ul < units && r < K) {
            const int form = head_uses_cape(a.content_heads, unit % a.H) ? a.cape : 0;
            const int slot = form ? cape_slot<0>(beam.p, pos, U, dp, form, M) : beam.p;
            // the weight exp(logit sum - the levels' log-normalisers)
            double lse_sum = 0.0;
            for (int u = 0; u < U; ++u) lse_sum += slse[g * U + u];
            const float wt = static_cast<float>(exp(beam.w - lse_sum));
            sidx[(ul * 2 + which) * K + r] = slot;
            swt[(ul * 2 + which) * K + r] = wt;
            if constexpr (TIER) {
                const int64_t si = static_cast<int64_t>(unit) * M + slot;
                sline[(ul * 2 + which) * K + r] = a.slot_line[si];
                atomicAdd(&a.hits[si], 1u);
            }
            if (a.out_idx[which]) {
                a.out_idx[which][static_cast<int64_t>(unit) * K + r] = slot;
                a.out_wt[which][static_cast<int64_t>(unit) * K + r] = wt;
            }
        }
    }
    __syncthreads();

    const TIn *v = static_cast<const TIn *>(a.v);
    const TIn *gam = static_cast<const TIn *>(a.gamma);
    TS *S = static_cast<TS *>(a.S);
    TS *out = static_cast<TS *>(a.out);
    const int npair = nu * K;  // <= 32
    // where the row of address (ul, which, k) lives
    auto row_of = [&](int ul, int which, int k) -> TS * {
        const int i = (ul * 2 + which) * K + k;
        const int64_t un = u0 + ul;
        if constexpr (TIER) {
            const int ln = sline[i];
            if (static_cast<unsigned>(ln) < static_cast<unsigned>(a.C))
                return static_cast<TS *>(a.cache) + (un * a.C + ln) * DV;
        }
        return S + (un * M + sidx[i]) * DV;
    };

    // ---------------- mass of every write pair: lane l < npair holds pair
    // (unit l / K, rank l % K); the load is issued before the row loads
    const int pu = lane / K, pk = lane - (lane / K) * K;
    float wgt = 0.f, mold = 0.f;
    float *mp = nullptr;
    int wsl = 0;
    if (lane < npair) {
        wsl = sidx[(pu * 2) * K + pk];
        wgt = swt[(pu * 2) * K + pk];
        if (wgt > 0.f) {  // w = 0: alpha = 1, lambda = 0, nothing changes
            mp = a.mass + static_cast<int64_t>(u0 + pu) * M + wsl;
            mold = *mp;
        }
    }

    // row lanes: sub-row `sub` of each row instruction, channels c0..c0+CPL
    const int sub = lane / LPR, c0 = (lane - sub * LPR) * CPL;

#pragma unroll
    for (int b0 = 0; b0 < UPW; b0 += UB) {
        // ---- every write row and read row of UB units, in flight at once
        Words<NW> wrow[UB][NJ], rrow[UB][NJ];
        float vin[UB][CPL];
#pragma unroll
        for (int i = 0; i < UB; ++i) {
            const int ul = b0 + i;
            if (ul < nu) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int k = j * RPI + sub;
                    if (k < K) {
                        wrow[i][j] = nt_load<NW>(row_of(ul, 0, k) + c0);
                        rrow[i][j] = nt_load<NW>(row_of(ul, 1, k) + c0);
                    }
                }
                const int un = u0 + ul;
                const TIn *vu = v + static_cast<int64_t>(un / a.H) * a.ld_v + (un % a.H) * DV + c0;
#pragma unroll
                for (int c = 0; c < CPL; ++c) vin[i][c] = to_f32(vu[c]);
            }
        }

        if (b0 == 0) {
            // ---- masses and rates (pair lanes); the read's weight on each
            // write slot of its unit, for the read-after-write correction
            float lam = 0.f, cr = 0.f;
            if (lane < npair) {
                if (wgt > 0.f) {
                    const int un = u0 + pu;
                    const float eg = expf(to_f32(gam[static_cast<int64_t>(un / a.H) * a.ld_gamma + un % a.H]));
                    const float mnew = fmaf(retention_fast(wgt, eg), mold, wgt);
                    *mp = mnew;
                    lam = wgt * __builtin_amdgcn_rcpf(mnew + a.eps_gsu);
                }
                const int rb = (pu * 2 + 1) * K;
                for (int kk = 0; kk < K; ++kk)
                    if (sidx[rb + kk] == wsl) cr += swt[rb + kk];
                slam[lane] = lam;
                scr[lane] = cr;
            }
            __syncthreads();
        }

        // ---- per unit: the read of the old contents, the update, the
        // read's share of the change, RMSNorm and the gate
#pragma unroll
        for (int i = 0; i < UB; ++i) {
            const int ul = b0 + i;
            if (ul >= nu) break;
            float acc[CPL];
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
            // all loads are consumed before the first store of the unit
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int k = j * RPI + sub;
                if (k < K) {
                    const float rho = swt[(ul * 2 + 1) * K + k];
                    float x[CPL];
                    unpack<TS, NW>(rrow[i][j], x);
#pragma unroll
                    for (int c = 0; c < CPL; ++c) acc[c] = fmaf(rho, x[c], acc[c]);
                }
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int k = j * RPI + sub;
                if (k < K) {
                    const float lam = slam[ul * K + k];
                    if (lam != 0.f) {
                        const float cr = scr[ul * K + k];
                        float x[CPL], y[CPL];
                        unpack<TS, NW>(wrow[i][j], x);
#pragma unroll
                        for (int c = 0; c < CPL; ++c) y[c] = fmaf(lam, vin[i][c] - x[c], x[c]);
                        const Words<NW> nw = pack<TS, NW>(y);
                        nt_store<NW>(row_of(ul, 0, k) + c0, nw);
#pragma unroll
                        for (int c = 0; c < CPL; ++c) acc[c] = fmaf(cr, y[c] - x[c], acc[c]);
                    }
                }
            }
            // sum over the RPI sub-rows, then one lane per CPO output channels
#pragma unroll
            for (int c = 0; c < CPL; ++c) sred[sub * DV + c0 + c] = acc[c];
            __syncthreads();
            const int unit = u0 + ul;
            float r[CPO];
            float ss = 0.f;
#pragma unroll
            for (int c = 0; c < CPO; ++c) {
                const int ch = lane * CPO + c;
                float t = 0.f;
#pragma unroll
                for (int s2 = 0; s2 < RPI; ++s2) t += sred[s2 * DV + ch];
                r[c] = t;
                ss = fmaf(t, t, ss);
            }
            __syncthreads();
            ss = wave_sum(ss);
            const float den = ss / static_cast<float>(DV) + a.eps_norm;
            const float inv = den > 0.f ? 1.0f / sqrtf(den) : 0.f;  // zero read, eps 0
            TS *ou = out + static_cast<int64_t>(unit) * DV + lane * CPO;
#pragma unroll
            for (int c = 0; c < CPO; ++c) {
                ou[c] = from_f32<TS>(r[c] * inv * ompre[c] * sigmoid(gpre[ul][c]));
            }
        }
    }
}

template <typename TIn, typename TS, int KP, int DV>
hipError_t launch_kd(const StepArgs &a, hipStream_t st) {
    using P = RowPlan<TS, KP, DV>;
    if constexpr (!P::kFits) {
        return hipErrorInvalidValue;
    } else {
        constexpr int UPW = P::UPW;
        const StepLds lo = step_lds(UPW, a.K, a.U * a.d_p, RowGeom<TS, DV>::RPI, DV);
        const int units = a.B * a.H;
        const unsigned grid = static_cast<unsigned>((units + UPW - 1) / UPW);
        if (a.cache)
            hipLaunchKernelGGL((step_fused_kernel<TIn, TS, KP, DV, true>), dim3(grid), dim3(kWave),
                               static_cast<size_t>(lo.total), st, a);
        else
            hipLaunchKernelGGL((step_fused_kernel<TIn, TS, KP, DV, false>), dim3(grid), dim3(kWave),
                               static_cast<size_t>(lo.total), st, a);
        return hipGetLastError();
    }
}

template <typename TIn, typename TS, int KP>
hipError_t launch_k(const StepArgs &a, hipStream_t st) {
    switch (a.d_v) {
        case 64: return launch_kd<TIn, TS, KP, 64>(a, st);
        case 128: return launch_kd<TIn, TS, KP, 128>(a, st);
        case 192: return launch_kd<TIn, TS, KP, 192>(a, st);
        case 256: return launch_kd<TIn, TS, KP, 256>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <typename TIn, typename TS>
hipError_t launch_ts(const StepArgs &a, hipStream_t st) {
    if (a.K <= 8) return launch_k<TIn, TS, 8>(a, st);
    if (a.K <= 16) return launch_k<TIn, TS, 16>(a, st);
    return launch_k<TIn, TS, 32>(a, st);
}

template <typename TS, int KP>
constexpr bool fits_any(int d_v) {
    return d_v == 64    ? RowPlan<TS, KP, 64>::kFits
           : d_v == 128 ? RowPlan<TS, KP, 128>::kFits
           : d_v == 192 ? RowPlan<TS, KP, 192>::kFits
                        : RowPlan<TS, KP, 256>::kFits;
}

template <typename TS>
bool fits(int K, int d_v) {
    return K <= 8 ? fits_any<TS, 8>(d_v) : K <= 16 ? fits_any<TS, 16>(d_v) : fits_any<TS, 32>(d_v);
}

}  // namespace

bool step_fused_supported(int K, int d_p, int U, int d_v, bool state_bf16) {
    if (K < 1 || K > 32 || d_p > 8 || U * d_p > kMaxDigits) return false;
    if (d_v != 64 && d_v != 128 && d_v != 192 && d_v != 256) return false;
    return state_bf16 ? fits<bf16_t>(K, d_v) : fits<float>(K, d_v);
}

hipError_t launch_step_fused(const StepArgs &args, hipStream_t st) {
    if (static_cast<int64_t>(args.B) * args.H == 0) return hipSuccess;
    if (!step_fused_supported(args.K, args.d_p, args.U, args.d_v, args.state_bf16))
        return hipErrorInvalidValue;
    StepArgs a = args;
    if (!a.ld_qk) a.ld_qk = static_cast<int64_t>(a.H) * a.U * a.d_p;
    if (!a.ld_v) a.ld_v = static_cast<int64_t>(a.H) * a.d_v;
    if (!a.ld_g) a.ld_g = static_cast<int64_t>(a.H) * a.d_v;
    if (!a.ld_gamma) a.ld_gamma = a.H;
    if (a.in_bf16)
        return a.state_bf16 ? launch_ts<bf16_t, bf16_t>(a, st) : launch_ts<bf16_t, float>(a, st);
    return a.state_bf16 ? launch_ts<float, bf16_t>(a, st) : launch_ts<float, float>(a, st);
}

}  // namespace ramnet
