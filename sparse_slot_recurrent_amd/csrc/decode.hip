// Address Decoder for gfx950: Product Softmax + exact prefix-tree Top-K +
// CAPE, one address per lane.
//
// RAM-Net project page, "Product Softmax" / "Multilevel Decision Tree" and
// the exact Top-K paragraph: each level fixes one more digit (most
// significant first); extending the K kept prefixes by the d_p values of the
// next digit gives K*d_p candidates, of which the K best are kept.  A prefix
// that drops out already trails K others that share every later factor, so
// the search returns the exact Top-K of all M slots.
//
// Design: the kept prefixes are held sorted (weight desc, prefix asc).  The
// candidates form d_p sorted lists (the beam times one digit's probability),
// and the new beam is the first K entries of their merge.  Each lane merges
// its own lists: a step takes the best list head, then advances that list
// alone, its beam position and probability gathered by selects, so that
// lanes choosing different lists never diverge.  The beams live in LDS,
// column-interleaved by lane ([rank][lane]), so the data-dependent rank
// index never causes a bank conflict.
//
// The decision ranks candidates by their exact weight, ties by the smaller
// prefix.  Two searches reach it:
//   * fp64 (decode_kernel): candidates ranked by their logit sums (below).
//   * fixed point (decode_fast_kernel, bf16 logits, K <= 32): a candidate is
//     one 64-bit key (its drop below the best prefix as an exact 32-bit
//     integer, its prefix), so a merge step compares once per list and the
//     merge orders candidates exactly.  Where the logits span too many
//     binary orders for exact 32-bit drops, rounded drops are used and each
//     cut is checked against their error; an address with a near-tie inside
//     it is marked and searched in fp64 (decode_fallback_kernel).
#include "device_common.h"
#include "launch.h"

namespace ramnet {
namespace {

// Digit u's logits as fp32, their max, and the level's log-normaliser
// max + log(sum exp(l - max)) in fp64 (a digit's probability is
// exp(l - lse)).  Both searches take them from here.
template <int DP, typename TIn>
__device__ __forceinline__ void level_logits(const TIn *lg, int u, float (&l)[DP], float &mx, double &lse) {
#pragma unroll
    for (int d = 0; d < DP; ++d) l[d] = to_f32(lg[u * DP + d]);
    mx = l[0];
#pragma unroll
    for (int d = 1; d < DP; ++d) mx = fmaxf(mx, l[d]);
    double sum = 0.0;
#pragma unroll
    for (int d = 0; d < DP; ++d) sum += exp(static_cast<double>(l[d]) - static_cast<double>(mx));
    lse = static_cast<double>(mx) + log(sum);
}

// ---------------------------------------------------------------- fp64 search

// A slot's weight is the product of its digits' probabilities, that is
// exp(sum of its digits' logits - sum of the levels' log-normalisers); the
// normalisers are common to every candidate of a level, so candidates rank
// by the sum of their digits' logits.  The fp64 search ranks by that sum
// (exact in fp64 for logits whose binary exponents span less than about 29
// bits, as bf16 logits always do) and forms the weights at the end.

// Branch-free: both comparisons are evaluated and combined bitwise, so the
// compiler emits no exec-mask branches inside the merge step.
__device__ __forceinline__ bool ranks_before(double sa, int ia, double sb, int ib) {
    return (sa > sb) | ((sa == sb) & (ia < ib));
}

// Digit u's logits in fp64 sorted by (logit desc, value asc), with a
// stable insertion network over compile-time positions, and the level's
// log-normaliser.
template <int DP, typename TIn>
__device__ __forceinline__ void digit_logits(const TIn *lg, int u, double (&sl)[DP], int (&dg)[DP],
                                             double &lse) {
    float l[DP], mx;
    level_logits<DP>(lg, u, l, mx, lse);
#pragma unroll
    for (int d = 0; d < DP; ++d) {
        sl[d] = l[d];
        dg[d] = d;
    }
#pragma unroll
    for (int i = 1; i < DP; ++i) {
#pragma unroll
        for (int j = i; j > 0; --j) {
            const bool sw = sl[j] > sl[j - 1];
            const double tp = sl[j];
            const int td = dg[j];
            sl[j] = sw ? sl[j - 1] : sl[j];
            dg[j] = sw ? dg[j - 1] : dg[j];
            sl[j - 1] = sw ? tp : sl[j - 1];
            dg[j - 1] = sw ? td : dg[j - 1];
        }
    }
}

// The fp64 search of one address.  KC: beam capacity (K rounded up to 8,
// 16, 32 or 64).  The beam being read lives in LDS (bs/bp: [bufs][KC][64],
// logit sums and prefixes); up to KC = 32 the beam being built is held in
// registers (nxs/nxp: its rank index is a compile-time constant of the
// unrolled merge), above that in a second LDS buffer, and `cur` gives the
// buffer holding the result.  lse_sum: the sum of the levels'
// log-normalisers (a slot's weight is exp(its logit sum - lse_sum)).
template <int DP, int KC, typename TIn>
__device__ __forceinline__ void search64(const TIn *lg, int U, int K, double *bs, int32_t *bp,
                                         int lane, double (&nxs)[KC <= 32 ? KC : 1],
                                         int32_t (&nxp)[KC <= 32 ? KC : 1], int &cur,
                                         double &lse_sum) {
    constexpr bool kRegs = KC <= 32;
    auto BS = [&](int buf, int r) -> double & { return bs[(buf * KC + r) * kWave + lane]; };
    auto BP = [&](int buf, int r) -> int32_t & { return bp[(buf * KC + r) * kWave + lane]; };
    cur = 0;
    lse_sum = 0.0;
    int nb = 1;
    for (int u = 0; u < U; ++u) {
        double sl[DP];
        int dg[DP];
        double lse;
        digit_logits<DP>(lg, u, sl, dg, lse);
        lse_sum += lse;
        const int nn = min(K, nb * DP);  // the same in every lane
        const int rd = kRegs ? 0 : cur;
        const int nxt = cur ^ 1;
        if (u == 0) {
            // The first digit's beam is its sorted values themselves.
#pragma unroll
            for (int r = 0; r < (DP < KC ? DP : KC); ++r) {
                if (r < nn) {
                    if constexpr (kRegs) {
                        nxs[r] = sl[r];
                        nxp[r] = dg[r];
                        if (U > 1) {
                            BS(0, r) = sl[r];
                            BP(0, r) = dg[r];
                        }
                    } else {
                        BS(nxt, r) = sl[r];
                        BP(nxt, r) = dg[r];
                    }
                }
            }
            if constexpr (!kRegs) cur = nxt;
            nb = nn;
            continue;
        }
        // List d (beam entries plus the digit of rank d) has its head at
        // beam entry h[d]; (cs, cp) is that head's candidate.
        int h[DP];
        double cs[DP];
        int cp[DP];
        const double b0 = BS(rd, 0);
        const int p0 = BP(rd, 0);
#pragma unroll
        for (int d = 0; d < DP; ++d) {
            h[d] = 0;
            cs[d] = b0 + sl[d];
            cp[d] = p0 * DP + dg[d];
        }
        auto step = [&](double &os, int32_t &op) {
            int best = 0;
            double bsv = cs[0];
            int bpv = cp[0];
#pragma unroll
            for (int d = 1; d < DP; ++d) {
                const bool bt = ranks_before(cs[d], cp[d], bsv, bpv);
                best = bt ? d : best;
                bsv = bt ? cs[d] : bsv;
                bpv = bt ? cp[d] : bpv;
            }
            os = bsv;
            op = bpv;
            int hb = h[0], db = dg[0];
            double lb = sl[0];
#pragma unroll
            for (int d = 1; d < DP; ++d) {
                const bool sel = best == d;
                hb = sel ? h[d] : hb;
                db = sel ? dg[d] : db;
                lb = sel ? sl[d] : lb;
            }
            ++hb;
            // the entry is loaded from a valid position even when the list
            // is exhausted (sum -inf), so no branch guards the loads
            const int hc = hb < nb ? hb : nb - 1;
            const double ncs = hb < nb ? BS(rd, hc) + lb : -__builtin_inf();
            const int ncp = BP(rd, hc) * DP + db;
#pragma unroll
            for (int d = 0; d < DP; ++d) {
                const bool sel = best == d;
                h[d] = sel ? hb : h[d];
                cs[d] = sel ? ncs : cs[d];
                cp[d] = sel ? ncp : cp[d];
            }
        };
        if constexpr (kRegs) {
#pragma unroll
            for (int r = 0; r < KC; ++r)
                if (r < nn) step(nxs[r], nxp[r]);
            if (u + 1 < U) {
#pragma unroll
                for (int r = 0; r < KC; ++r) {
                    if (r < nn) {
                        BS(0, r) = nxs[r];
                        BP(0, r) = nxp[r];
                    }
                }
            }
        } else {
            for (int r = 0; r < nn; ++r) step(BS(nxt, r), BP(nxt, r));
            cur = nxt;
        }
        nb = nn;
    }
}

// ---------------------------------------------------------------- fixed-point search

// A candidate's drop T: the sum over its digits of (level max - logit),
// >= 0; candidates rank by T ascending, exactly as by weight descending
// (T = the levels' maxima minus the logit sum).  Every logit of an address
// is a multiple of 2^e (e: the lowest set bit over its logits), so every
// drop is an integer number of 2^e; while the largest possible T stays
// below 2^(e + 30) every drop is held exactly as a 32-bit integer (for
// bf16 logits all but about one address in 10^5).
//
// A candidate as one key: the high word is T / 2^e, the low word the
// prefix.  The smaller key ranks first: the order (weight desc, prefix asc)
// in one unsigned compare.
__device__ __forceinline__ uint64_t mk_key(uint32_t t, uint32_t prefix) {
    return (static_cast<uint64_t>(t) << 32) | prefix;
}
__device__ __forceinline__ uint32_t key_t(uint64_t k) { return static_cast<uint32_t>(k >> 32); }
__device__ __forceinline__ uint32_t key_prefix(uint64_t k) { return static_cast<uint32_t>(k); }
// An exhausted list: T = 3 2^30, above every real candidate (T < 2^30) also
// once a drop (< 2^30) is added.
constexpr uint64_t kSentinel = static_cast<uint64_t>(0xc0000000u) << 32;

// Beam key k extended by digit value d whose drop is dl.
template <int DP>
__device__ __forceinline__ uint64_t extend(uint64_t k, uint32_t dl, uint32_t d) {
    return mk_key(key_t(k) + dl, static_cast<uint32_t>(k) * DP + d);
}

// Exponent of the lowest set bit of a finite fp32 x != 0 (x = n 2^e, n odd).
__device__ __forceinline__ int low_bit_exp(float x) {
    const uint32_t b = __float_as_uint(x);
    const int be = static_cast<int>((b >> 23) & 0xffu);
    const uint32_t sig = be ? ((b & 0x7fffffu) | 0x800000u) : (b & 0x7fffffu);
    return (be ? be - 127 : -126) - 23 + __builtin_ctz(sig);
}

// The sum of prefix x's digit logits (u + 1 digits) in fp64, and whether
// every addition was exact (the TwoSum error of each is zero): then it
// orders candidates as their exact weights do.
template <int DP, typename TIn>
__device__ double exact_logit_sum(uint32_t x, int u, const TIn *lg, bool &exact) {
    double s = 0.0;
    for (int v = u; v >= 0; --v, x /= DP) {
        const double l = to_f32(lg[v * DP + x % DP]);
        const double t = s + l;
        const double bb = t - s;
        exact = exact && ((s - (t - bb)) + (l - bb)) == 0.0;
        s = t;
    }
    return s;
}

// The most candidates a near-tie check walks on either side of a cut.
constexpr int kMaxBand = 16;

// The fixed-point path serves U <= kMaxUFix levels.
constexpr int kMaxUFix = 16;

// A lane's beam in LDS (KC + 1 entries: the beam and its sentinel), entry r
// of lane l at index r * 64 + l.  Wide: 64-bit keys.  Narrow (every prefix
// below 2^16, i.e. M <= 65536): the drops in a 32-bit array and the prefixes
// in a 16-bit one after it, 6 bytes an entry instead of 8, so that 12 waves
// fit a compute unit's LDS instead of 9.
template <int KC, bool NARROW>
struct Beam {
    unsigned char *base;
    int lane;
    static constexpr size_t bytes() { return static_cast<size_t>(KC + 1) * kWave * (NARROW ? 6 : 8); }
    __device__ __forceinline__ uint64_t ld(int r) const {
        const int i = r * kWave + lane;
        if constexpr (NARROW) {
            const uint32_t t = reinterpret_cast<const uint32_t *>(base)[i];
            const uint32_t px = reinterpret_cast<const uint16_t *>(base + (KC + 1) * kWave * 4)[i];
            return mk_key(t, px);
        } else {
            return reinterpret_cast<const uint64_t *>(base)[i];
        }
    }
    __device__ __forceinline__ void st(int r, uint64_t k) const {
        const int i = r * kWave + lane;
        if constexpr (NARROW) {
            reinterpret_cast<uint32_t *>(base)[i] = key_t(k);
            reinterpret_cast<uint16_t *>(base + (KC + 1) * kWave * 4)[i] = static_cast<uint16_t>(key_prefix(k));
        } else {
            reinterpret_cast<uint64_t *>(base)[i] = k;
        }
    }
};

// The fixed-point search of one address (KC <= 32), its beam in bkl.  The
// result is left in `out` (keys, heaviest first), with the drop unit 2^e
// (unit) and lnz, the sum of the levels' log(sum exp(l - max)) in fp64 (a
// slot's weight is exp(-T unit - lnz)).  Where the logits span too many
// binary orders for exact 32-bit drops, the drops are rounded and every cut
// must clear the rounding error.  Returns false where that fails (a
// near-tie within the error) or a logit is not finite.
template <int DP, int KC, bool NARROW, typename TIn>
__device__ __forceinline__ bool search_fix(const TIn *lg, int U, int K, Beam<KC, NARROW> bkl,
                                           uint64_t (&out)[KC], double &unit, double &lnz) {
    // the drop unit and the largest possible T, from every logit
    int e = 1 << 20;
    double tmax = 0.0;  // exact: a sum of at most kMaxUFix fp32 differences
    bool finite = true;
    lnz = 0.0;
    for (int u = 0; u < U; ++u) {
        float l[DP], mx;
        double lse;
        level_logits<DP>(lg, u, l, mx, lse);
        lnz += lse - static_cast<double>(mx);
        float mn = l[0];
#pragma unroll
        for (int d = 0; d < DP; ++d) {
            mn = fminf(mn, l[d]);
            finite = finite && isfinite(l[d]);
            if (l[d] != 0.f) e = min(e, low_bit_exp(l[d]));
        }
        tmax += static_cast<double>(mx) - static_cast<double>(mn);
    }
    if (!finite || !(tmax < 0x1p100)) return false;
    if (e == 1 << 20) e = 0;  // every logit is 0: every drop is 0
    // Drops too fine for 32 bits: round them to multiples of 2^e with
    // tmax < 2^(e + 30) instead; every cut is then checked below.
    const bool rounded = !(tmax < __hiloint2double((1023 + e + 30) << 20, 0));
    if (rounded) e = static_cast<int>((__double_as_longlong(tmax) >> 52) & 0x7ff) - 1023 - 29;
    // 2^-e and 2^e as fp64 (-1022 < e < 1023 here)
    const double scale = __hiloint2double((1023 - e) << 20, 0);
    unit = __hiloint2double((1023 + e) << 20, 0);

    // the beam before the first digit: one entry of drop 0, prefix 0
    bkl.st(0, mk_key(0u, 0u));
    bkl.st(1, kSentinel);
    int nb = 1;
    for (int u = 0; u < U; ++u) {
        uint32_t dl[DP];
        {
            float l[DP];
#pragma unroll
            for (int d = 0; d < DP; ++d) l[d] = to_f32(lg[u * DP + d]);
            float mx = l[0];
#pragma unroll
            for (int d = 1; d < DP; ++d) mx = fmaxf(mx, l[d]);
            // (mx - l) 2^-e: exact in fp64, an integer below 2^30 (rounded to
            // the nearest one for rounded drops)
#pragma unroll
            for (int d = 0; d < DP; ++d)
                dl[d] = static_cast<uint32_t>(rint((static_cast<double>(mx) - static_cast<double>(l[d])) * scale));
        }
        const int nn = min(K, nb * DP);  // the same in every lane
        // list d: the beam extended by digit value d; its head is beam
        // entry hi[d]
        uint64_t hk[DP];
        int hi[DP];
        {
            const uint64_t k0 = bkl.ld(0);
#pragma unroll
            for (int d = 0; d < DP; ++d) {
                hk[d] = extend<DP>(k0, dl[d], d);
                hi[d] = 0;
            }
        }
        // takes the best head (c[d]: list d beat every list before it) and
        // advances its list (the winner is the last list that beat all
        // before it)
        auto pop = [&]() -> uint64_t {
            uint64_t bk = hk[0];
            int bi = hi[0];
            uint32_t bdl = dl[0];
            uint32_t bd = 0;
            bool c[DP];
#pragma unroll
            for (int d = 1; d < DP; ++d) {
                c[d] = hk[d] < bk;
                bk = c[d] ? hk[d] : bk;
                bi = c[d] ? hi[d] : bi;
                bdl = c[d] ? dl[d] : bdl;
                bd = c[d] ? static_cast<uint32_t>(d) : bd;
            }
            const int ni = bi + 1;
            const uint64_t nk = extend<DP>(bkl.ld(ni), bdl, bd);
            bool later = false;
#pragma unroll
            for (int d = DP - 1; d >= 0; --d) {
                const bool win = (d == 0 || c[d]) && !later;
                hk[d] = win ? nk : hk[d];
                hi[d] = win ? ni : hi[d];
                if (d > 0) later = later || c[d];
            }
            return bk;
        };
        uint64_t last = 0;  // ends as the last kept key
#pragma unroll
        for (int r = 0; r < KC; ++r) {
            if (r < nn) {
                out[r] = pop();
                last = out[r];
            }
        }
        // Rounded drops: a candidate's T is within (u + 1) / 2 units of
        // exact, so a cut holds where the best dropped candidate trails the
        // last kept one by more than u + 1 units.  Otherwise the candidates
        // within that distance of the cut are ordered by their exact logit
        // sums: the worst kept must still rank before the best dropped.
        const uint32_t err = static_cast<uint32_t>(u + 1);
        bool near = false;
        uint32_t td = 0;
        double ds = 0.0, ks = 0.0;
        uint32_t dpx = 0, kpx = 0;
        bool ok = true, have_d = false, have_k = false;
        if (rounded && nn < nb * DP) {
            uint64_t bk = hk[0];
#pragma unroll
            for (int d = 1; d < DP; ++d) bk = hk[d] < bk ? hk[d] : bk;
            td = key_t(bk);
            near = !(td - key_t(last) > err);
            for (int np = 0; near && ok; ++np) {
                bk = hk[0];
#pragma unroll
                for (int d = 1; d < DP; ++d) bk = hk[d] < bk ? hk[d] : bk;
                if (key_t(bk) > key_t(last) + err) break;
                if (np == kMaxBand) {
                    ok = false;
                    break;
                }
                const uint32_t px = key_prefix(bk);
                const double sx = exact_logit_sum<DP>(px, u, lg, ok);
                if (!have_d || sx > ds || (sx == ds && px < dpx)) {
                    ds = sx;
                    dpx = px;
                    have_d = true;
                }
                pop();
            }
        }
        // the new beam and its sentinel
        if (u + 1 < U || near) {
#pragma unroll
            for (int r = 0; r < KC; ++r)
                if (r < nn) bkl.st(r, out[r]);
            bkl.st(nn, kSentinel);
        }
        if (near && ok) {
            for (int r = nn - 1; r >= 0 && ok; --r) {
                const uint64_t k = bkl.ld(r);
                if (key_t(k) + err < td) break;
                if (r == nn - 1 - kMaxBand) {
                    ok = false;
                    break;
                }
                const uint32_t px = key_prefix(k);
                const double sx = exact_logit_sum<DP>(px, u, lg, ok);
                if (!have_k || sx < ks || (sx == ks && px > kpx)) {
                    ks = sx;
                    kpx = px;
                    have_k = true;
                }
            }
            ok = ok && have_d && have_k && (ks > ds || (ks == ds && kpx < dpx));
        }
        if (!ok) return false;
        nb = nn;
    }
    return true;
}

// ---------------------------------------------------------------- kernels

// The arguments every decode kernel takes.
struct DecodeK {
    const void *q, *k;
    int64_t n;
    int T, H, U, K;
    const int32_t *pos0;
    int cape;
    uint64_t content_heads;
    int64_t M;
    bool unit_major;
    int64_t ld;
    int32_t *w_idx, *r_idx;
    float *w_wt, *r_wt;
    // one word per wave of the fixed-point kernel (keys' waves, then
    // queries'): bit i set where lane i's address is left to the fp64 search
    unsigned long long *fails;
    int64_t waves;  // waves per side
};

template <typename TIn>
__device__ __forceinline__ const TIn *logits_of(const DecodeK &d, int64_t a, bool key, int DP) {
    return static_cast<const TIn *>(key ? d.k : d.q) + (a / d.H) * d.ld + (a % d.H) * (d.U * DP);
}

// The i-th address in launch order: token-major ([B,T,H], the address
// index itself), or, for head-major output ([B,H,T]), a head's tokens one
// after another, so that a wave's stores fill consecutive rows.
__device__ __forceinline__ int64_t address_of(const DecodeK &d, int64_t i) {
    if (!d.unit_major) return i;
    const int64_t T = d.T, H = d.H;
    const int64_t b = i / (H * T), h = (i / T) % H, t = i % T;
    return (b * T + t) * H + h;
}

// Stores one address's K slots (moved by CAPE) and weights, heaviest first;
// at(r, slot, w) gives the r-th pre-CAPE slot and its weight.
template <int DP, int KC, typename At>
__device__ __forceinline__ void write_address(const DecodeK &d, int64_t a, bool key, At at) {
    const int64_t T = d.T, H = d.H;
    const int64_t b = a / (T * H);
    const int64_t t = (a / H) % T;
    const int64_t pos = (d.pos0 ? d.pos0[b] : 0) + t;
    const int form = head_uses_cape(d.content_heads, static_cast<int>(a % H)) ? d.cape : 0;
    const CapeShift sh = cape_shift<DP>(pos, DP, d.M);
    // [B,T,H,K], or [B,H,T,K] so that a head's addresses are contiguous
    const int64_t o = d.unit_major ? ((b * H + a % H) * T + t) : a;
    const int K = d.K;
    int32_t *oi = (key ? d.w_idx : d.r_idx) + o * K;
    float *ow = (key ? d.w_wt : d.r_wt) + o * K;
    auto moved = [&](int slot) { return form ? cape_slot_at<DP>(slot, sh, d.U, DP, form, d.M) : slot; };
    if (KC <= 32 && K % 4 == 0) {
        // whole 16-byte pieces: a lane's row goes out in K/4 stores instead
        // of K, so rows are complete sooner
#pragma unroll
        for (int r = 0; r < (KC <= 32 ? KC : 0); r += 4) {
            if (r < K) {
                int s[4];
                float w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) at(r + i, s[i], w[i]);
                *reinterpret_cast<int4 *>(oi + r) = make_int4(moved(s[0]), moved(s[1]), moved(s[2]), moved(s[3]));
                *reinterpret_cast<float4 *>(ow + r) = make_float4(w[0], w[1], w[2], w[3]);
            }
        }
    } else if (KC <= 32) {
#pragma unroll
        for (int r = 0; r < KC; ++r) {
            if (r < K) {
                int s;
                float w;
                at(r, s, w);
                oi[r] = moved(s);
                ow[r] = w;
            }
        }
    } else {
        for (int r = 0; r < K; ++r) {
            int s;
            float w;
            at(r, s, w);
            oi[r] = moved(s);
            ow[r] = w;
        }
    }
}

// LDS bytes per wave of the fp64 search (beam buffers, lane-interleaved) and
// of the fixed-point search (the beam and its sentinel).
template <int KC>
constexpr size_t lds64_bytes() {
    return static_cast<size_t>(KC <= 32 ? 1 : 2) * KC * kWave * (sizeof(double) + sizeof(int32_t));
}

// The fp64 search of address a and its stores.
template <int DP, int KC, typename TIn>
__device__ __forceinline__ void decode64(const DecodeK &d, int64_t a, bool key, unsigned char *smem) {
    const int lane = threadIdx.x;
    double *bs = reinterpret_cast<double *>(smem);
    int32_t *bp = reinterpret_cast<int32_t *>(bs + (KC <= 32 ? 1 : 2) * KC * kWave);
    double nxs[KC <= 32 ? KC : 1];
    int32_t nxp[KC <= 32 ? KC : 1];
    int cur;
    double lse_sum;
    search64<DP, KC>(logits_of<TIn>(d, a, key, DP), d.U, d.K, bs, bp, lane, nxs, nxp, cur, lse_sum);
    write_address<DP, KC>(d, a, key, [&](int r, int &s, float &w) {
        if constexpr (KC <= 32) {
            s = nxp[r];
            w = static_cast<float>(exp(nxs[r] - lse_sum));
        } else {
            s = bp[(cur * KC + r) * kWave + lane];
            w = static_cast<float>(exp(bs[(cur * KC + r) * kWave + lane] - lse_sum));
        }
    });
}

// One address per lane in fp64 (blockIdx.y: 0 keys, 1 queries).
template <int DP, int KC, typename TIn>
__global__ __launch_bounds__(kWave) void decode_kernel(DecodeK d) {
    extern __shared__ unsigned char smem[];
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kWave + threadIdx.x;
    if (i >= d.n) return;  // no barrier below: lanes are independent
    decode64<DP, KC, TIn>(d, address_of(d, i), blockIdx.y == 0, smem);
}

// One address per lane in fixed point: an address whose drops fit 32 bits
// is stored, the others are marked in the wave's failure word for the fp64
// search.  Every wave of the grid has its lane 0 (a < n), which writes the
// word.
template <int DP, int KC, bool NARROW, typename TIn>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(3))) void decode_fast_kernel(DecodeK d) {
    extern __shared__ unsigned char smem[];
    const int lane = threadIdx.x;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kWave + lane;
    if (i >= d.n) return;
    const int64_t a = address_of(d, i);
    const bool key = blockIdx.y == 0;
    uint64_t out[KC];
    double unit, lnz;
    const TIn *lg = logits_of<TIn>(d, a, key, DP);
    const bool ok = search_fix<DP, KC>(lg, d.U, d.K, Beam<KC, NARROW>{smem, lane}, out, unit, lnz);
    if (ok) {
        // a slot's weight exp(-T - lnz), T = its drop (exact)
        write_address<DP, KC>(d, a, key, [&](int r, int &s, float &w) {
            s = static_cast<int>(key_prefix(out[r]));
            w = static_cast<float>(exp(-static_cast<double>(key_t(out[r])) * unit - lnz));
        });
    }
    const unsigned long long failed = __ballot(!ok);
    if (lane == 0) d.fails[blockIdx.y * d.waves + blockIdx.x] = failed;
}

// The addresses the fixed-point kernel left, in fp64: one failure word per
// lane, its addresses one after another (almost every word is 0).
template <int DP, int KC, typename TIn>
__global__ __launch_bounds__(kWave) void decode_fallback_kernel(DecodeK d) {
    extern __shared__ unsigned char smem[];
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kWave + threadIdx.x;
    if (i >= 2 * d.waves) return;
    const bool key = i < d.waves;
    const int64_t w0 = (key ? i : i - d.waves) * kWave;
    for (unsigned long long f = d.fails[i]; f != 0; f &= f - 1)
        decode64<DP, KC, TIn>(d, address_of(d, w0 + __builtin_ctzll(f)), key, smem);
}

template <typename K>
hipError_t set_lds(K kern, size_t lds) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
}

// fp64 for every address; or, with failure words (bf16 logits, KC <= 32,
// U <= kMaxUFix), the fixed-point search, then fp64 for the addresses it
// left.
template <int DP, int KC, typename TIn>
hipError_t launch_kc(const DecodeArgs &a, hipStream_t st) {
    const int64_t waves = (a.n + kWave - 1) / kWave;
    DecodeK d{a.q, a.k, a.n, a.T, a.H, a.U, a.K, a.pos0, a.cape, a.content_heads, a.M, a.unit_major,
              a.ld ? a.ld : static_cast<int64_t>(a.H) * a.U * a.d_p, a.w_idx, a.r_idx, a.w_wt, a.r_wt,
              a.fails, waves};
    const dim3 grid(static_cast<unsigned>(waves), 2);
    constexpr size_t lds64 = lds64_bytes<KC>();
    hipError_t e;
    if constexpr (KC <= 32) {
        if (a.fails && a.in_bf16 && a.U <= kMaxUFix) {
            // every prefix of the beam is below d_p^U
            int64_t span = 1;
            for (int u = 0; u < a.U && span <= 65536; ++u) span *= a.d_p;
            const bool narrow = span <= 65536;
            const size_t ldsfix = narrow ? Beam<KC, true>::bytes() : Beam<KC, false>::bytes();
            auto fast = narrow ? decode_fast_kernel<DP, KC, true, TIn> : decode_fast_kernel<DP, KC, false, TIn>;
            if ((e = set_lds(fast, ldsfix)) != hipSuccess) return e;
            hipLaunchKernelGGL(fast, grid, dim3(kWave), ldsfix, st, d);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            auto slow = decode_fallback_kernel<DP, KC, TIn>;
            if ((e = set_lds(slow, lds64)) != hipSuccess) return e;
            hipLaunchKernelGGL(slow, dim3(static_cast<unsigned>((2 * waves + kWave - 1) / kWave)), dim3(kWave),
                               lds64, st, d);
            return hipGetLastError();
        }
    }
    auto kern = decode_kernel<DP, KC, TIn>;
    if ((e = set_lds(kern, lds64)) != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(kWave), lds64, st, d);
    return hipGetLastError();
}

template <int DP, typename TIn>
hipError_t launch_dp(const DecodeArgs &d, hipStream_t st) {
    if (d.K <= 8) return launch_kc<DP, 8, TIn>(d, st);
    if (d.K <= 16) return launch_kc<DP, 16, TIn>(d, st);
    if (d.K <= 32) return launch_kc<DP, 32, TIn>(d, st);
    return launch_kc<DP, 64, TIn>(d, st);
}

template <typename TIn>
hipError_t launch_in(const DecodeArgs &d, hipStream_t st) {
    switch (d.d_p) {
        case 2: return launch_dp<2, TIn>(d, st);
        case 3: return launch_dp<3, TIn>(d, st);
        case 4: return launch_dp<4, TIn>(d, st);
        case 5: return launch_dp<5, TIn>(d, st);
        case 6: return launch_dp<6, TIn>(d, st);
        case 7: return launch_dp<7, TIn>(d, st);
        case 8: return launch_dp<8, TIn>(d, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t decode_fails_bytes(int64_t n) {
    return sizeof(unsigned long long) * 2 * static_cast<size_t>((n + kWave - 1) / kWave);
}

hipError_t launch_decode(const DecodeArgs &d, hipStream_t st) {
    if (d.n == 0) return hipSuccess;
    return d.in_bf16 ? launch_in<bf16_t>(d, st) : launch_in<float>(d, st);
}

}  // namespace ramnet
