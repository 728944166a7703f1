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
// Design: the kept prefixes are held sorted (weight desc, prefix asc).  With
// the next digit's probabilities sorted the same way, the candidates form
// d_p sorted lists (one per digit value), and the new beam is the first K
// entries of their merge; the first digit's beam is its sorted values.  Each
// lane merges its own lists: a step takes the best list head, then advances
// that list alone, its beam position, probability and digit gathered by
// selects, so that lanes choosing different lists never diverge.  The beams
// live in LDS, column-interleaved by lane ([buffer][rank][lane]), so the
// data-dependent rank index never causes a bank conflict.  The decision is
// taken in fp64 so that it agrees with an fp64 reference except at exact
// ties.
#include "device_common.h"
#include "launch.h"

namespace ramnet {
namespace {

// Branch-free: both comparisons are evaluated and combined bitwise, so the
// compiler emits no exec-mask branches inside the merge step.
template <typename WT>
__device__ __forceinline__ bool ranks_before(WT wa, int ia, WT wb, int ib) {
    return (wa > wb) | ((wa == wb) & (ia < ib));
}

__device__ __forceinline__ double wexp(double x) { return exp(x); }

// KC: beam capacity (K rounded up to 8, 16, 32 or 64).  The beam being read
// lives in LDS, column-interleaved by lane; up to KC = 32 the beam being
// built is held in registers (its rank index is a compile-time constant of
// the unrolled merge), which halves the LDS a wave needs and so doubles the
// waves a CU can hold.
template <int DP, int KC, typename WT, typename TIn>
__global__ __launch_bounds__(kWave) void decode_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, int64_t n, int T, int H,
    int U, int K, const int32_t *__restrict__ pos0, int cape, uint64_t content_heads,
    int64_t M, bool unit_major, int64_t ld,
    int32_t *__restrict__ w_idx, float *__restrict__ w_wt,
    int32_t *__restrict__ r_idx, float *__restrict__ r_wt) {
    constexpr bool kRegs = KC <= 32;
    extern __shared__ unsigned char smem[];
    const int lane = threadIdx.x;
    WT *bw = reinterpret_cast<WT *>(smem);                                      // [bufs][KC][64]
    int32_t *bp = reinterpret_cast<int32_t *>(bw + (kRegs ? 1 : 2) * KC * kWave);  // [bufs][KC][64]
    const int64_t a = static_cast<int64_t>(blockIdx.x) * kWave + lane;
    if (a >= n) return;  // no barrier below: lanes are independent
    const bool key = blockIdx.y == 0;
    const TIn *lg = (key ? k : q) + (a / H) * ld + (a % H) * (U * DP);
    auto BW = [&](int buf, int r) -> WT & { return bw[(buf * KC + r) * kWave + lane]; };
    auto BP = [&](int buf, int r) -> int32_t & { return bp[(buf * KC + r) * kWave + lane]; };

    WT nxw[kRegs ? KC : 1];
    int32_t nxp[kRegs ? KC : 1];
    int cur = 0, nb = 1;
    for (int u = 0; u < U; ++u) {
        // Digit u's distribution: softmax over its d_p logits.
        WT pr[DP];
        int dg[DP];
        float l[DP];
#pragma unroll
        for (int d = 0; d < DP; ++d) l[d] = to_f32(lg[u * DP + d]);
        float mx = l[0];
#pragma unroll
        for (int d = 1; d < DP; ++d) mx = fmaxf(mx, l[d]);
        WT sum = 0;
#pragma unroll
        for (int d = 0; d < DP; ++d) {
            pr[d] = wexp(static_cast<WT>(l[d]) - static_cast<WT>(mx));
            sum += pr[d];
        }
#pragma unroll
        for (int d = 0; d < DP; ++d) {
            pr[d] /= sum;
            dg[d] = d;
        }
        // Sort digit values by (probability desc, value asc); stable
        // insertion network over compile-time positions.
#pragma unroll
        for (int i = 1; i < DP; ++i) {
#pragma unroll
            for (int j = i; j > 0; --j) {
                const bool sw = pr[j] > pr[j - 1];
                const WT tp = pr[j];
                const int td = dg[j];
                pr[j] = sw ? pr[j - 1] : pr[j];
                dg[j] = sw ? dg[j - 1] : dg[j];
                pr[j - 1] = sw ? tp : pr[j - 1];
                dg[j - 1] = sw ? td : dg[j - 1];
            }
        }
        const int nn = min(K, nb * DP);  // the same in every lane
        const int rd = kRegs ? 0 : cur;
        const int nxt = cur ^ 1;
        if (u == 0) {
            // The first digit's beam is its sorted values themselves.
#pragma unroll
            for (int r = 0; r < (DP < KC ? DP : KC); ++r) {
                if (r < nn) {
                    if constexpr (kRegs) {
                        nxw[r] = pr[r];
                        nxp[r] = dg[r];
                        if (U > 1) {
                            BW(0, r) = pr[r];
                            BP(0, r) = dg[r];
                        }
                    } else {
                        BW(nxt, r) = pr[r];
                        BP(nxt, r) = dg[r];
                    }
                }
            }
            if constexpr (!kRegs) cur = nxt;
            nb = nn;
            continue;
        }
        // Merge the d_p candidate lists into the next beam.
        // List d (beam entries times the digit of rank d) has its head at
        // beam entry h[d]; (cw, cp) is that head's candidate.  A step takes
        // the best head, then gathers that list's entry, probability and
        // digit by selects and loads only its next beam entry, so that no
        // lane-divergent per-list branch is needed.
        int h[DP];
        WT cw[DP];
        int cp[DP];
        const WT b0 = BW(rd, 0);
        const int p0 = BP(rd, 0);
#pragma unroll
        for (int d = 0; d < DP; ++d) {
            h[d] = 0;
            cw[d] = b0 * pr[d];
            cp[d] = p0 * DP + dg[d];
        }
        auto step = [&](WT &ow, int32_t &op) {
            int best = 0;
            WT bwv = cw[0];
            int bpv = cp[0];
#pragma unroll
            for (int d = 1; d < DP; ++d) {
                const bool bt = ranks_before(cw[d], cp[d], bwv, bpv);
                best = bt ? d : best;
                bwv = bt ? cw[d] : bwv;
                bpv = bt ? cp[d] : bpv;
            }
            ow = bwv;
            op = bpv;
            int hb = h[0], db = dg[0];
            WT pb = pr[0];
#pragma unroll
            for (int d = 1; d < DP; ++d) {
                const bool sel = best == d;
                hb = sel ? h[d] : hb;
                db = sel ? dg[d] : db;
                pb = sel ? pr[d] : pb;
            }
            ++hb;
            // the entry is loaded from a valid position even when the list
            // is exhausted (weight -1), so no branch guards the loads
            const int hc = hb < nb ? hb : nb - 1;
            const WT ncw = hb < nb ? BW(rd, hc) * pb : WT(-1);
            const int ncp = BP(rd, hc) * DP + db;
#pragma unroll
            for (int d = 0; d < DP; ++d) {
                const bool sel = best == d;
                h[d] = sel ? hb : h[d];
                cw[d] = sel ? ncw : cw[d];
                cp[d] = sel ? ncp : cp[d];
            }
        };
        if constexpr (kRegs) {
#pragma unroll
            for (int r = 0; r < KC; ++r)
                if (r < nn) step(nxw[r], nxp[r]);
            if (u + 1 < U) {
#pragma unroll
                for (int r = 0; r < KC; ++r) {
                    if (r < nn) {
                        BW(0, r) = nxw[r];
                        BP(0, r) = nxp[r];
                    }
                }
            }
        } else {
            for (int r = 0; r < nn; ++r) step(BW(nxt, r), BP(nxt, r));
            cur = nxt;
        }
        nb = nn;
    }

    const int64_t b = a / (static_cast<int64_t>(T) * H);
    const int64_t t = (a / H) % T;
    const int64_t pos = (pos0 ? pos0[b] : 0) + t;
    const int form = head_uses_cape(content_heads, static_cast<int>(a % H)) ? cape : 0;
    const CapeShift sh = cape_shift<DP>(pos, DP, M);
    // [B,T,H,K], or [B,H,T,K] so that a head's addresses are contiguous
    const int64_t o = unit_major ? ((b * H + a % H) * T + t) : a;
    int32_t *oi = (key ? w_idx : r_idx) + o * K;
    float *ow = (key ? w_wt : r_wt) + o * K;
    if constexpr (kRegs) {
        if (K % 4 == 0) {
            // whole 16-byte pieces: a lane's row goes out in K/4 stores
            // instead of K, so rows are complete sooner
#pragma unroll
            for (int r = 0; r < KC; r += 4) {
                if (r < K) {
                    int4 vi;
                    float4 vw;
                    vi.x = form ? cape_slot_at<DP>(nxp[r], sh, U, DP, form, M) : nxp[r];
                    vi.y = form ? cape_slot_at<DP>(nxp[r + 1], sh, U, DP, form, M) : nxp[r + 1];
                    vi.z = form ? cape_slot_at<DP>(nxp[r + 2], sh, U, DP, form, M) : nxp[r + 2];
                    vi.w = form ? cape_slot_at<DP>(nxp[r + 3], sh, U, DP, form, M) : nxp[r + 3];
                    vw.x = static_cast<float>(nxw[r]);
                    vw.y = static_cast<float>(nxw[r + 1]);
                    vw.z = static_cast<float>(nxw[r + 2]);
                    vw.w = static_cast<float>(nxw[r + 3]);
                    *reinterpret_cast<int4 *>(oi + r) = vi;
                    *reinterpret_cast<float4 *>(ow + r) = vw;
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < KC; ++r) {
                if (r < K) {
                    oi[r] = form ? cape_slot_at<DP>(nxp[r], sh, U, DP, form, M) : nxp[r];
                    ow[r] = static_cast<float>(nxw[r]);
                }
            }
        }
    } else {
        for (int r = 0; r < K; ++r) {
            const int slot = BP(cur, r);
            oi[r] = form ? cape_slot_at<DP>(slot, sh, U, DP, form, M) : slot;
            ow[r] = static_cast<float>(BW(cur, r));
        }
    }
}

template <int DP, int KC, typename TIn>
hipError_t launch_kc(const DecodeArgs &d, hipStream_t st) {
    using WT = double;
    constexpr int bufs = KC <= 32 ? 1 : 2;
    const size_t lds = static_cast<size_t>(bufs) * KC * kWave * (sizeof(WT) + sizeof(int32_t));
    auto kern = decode_kernel<DP, KC, WT, TIn>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    dim3 grid(static_cast<unsigned>((d.n + kWave - 1) / kWave), 2);
    hipLaunchKernelGGL(kern, grid, dim3(kWave), lds, st,
                       static_cast<const TIn *>(d.q), static_cast<const TIn *>(d.k), d.n,
                       d.T, d.H, d.U, d.K, d.pos0, d.cape, d.content_heads, d.M, d.unit_major,
                       d.ld ? d.ld : static_cast<int64_t>(d.H) * d.U * d.d_p, d.w_idx, d.w_wt, d.r_idx, d.r_wt);
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

hipError_t launch_decode(const DecodeArgs &d, hipStream_t st) {
    if (d.n == 0) return hipSuccess;
    return d.in_bf16 ? launch_in<bf16_t>(d, st) : launch_in<float>(d, st);
}

}  // namespace ramnet
