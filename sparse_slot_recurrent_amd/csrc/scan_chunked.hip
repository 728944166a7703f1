// Slot-grouped prefill recurrence for gfx950, with every slot row on chip
// (M <= 1024 slots: one scan thread per slot).  Rows in HBM (more slots)
// take the slot-range path of scan_ranges.hip.
//
// RAM-Net project page, GPU-execution paragraphs: with every token's
// addresses known, events are grouped by slot, each slot applies its own
// events in causal order, different slots and channels run in parallel and
// untouched slots cost nothing.  The Gated Sparse Update and the read are
// those of the "Gated Sparse Update" and "three stages" paragraphs.
//
// The sequence of each (batch, head) unit is cut into chunks of C tokens.
//
// plan_kernel: one workgroup per (unit, chunk), all chunks at once, since
// grouping does not depend on the state.
//   * Every valid write (slot in [0, M), weight > 0) and read (slot in
//     [0, M)) finds its slot's entry in an LDS table indexed by slot;
//     entries count their writes.
//   * Entries are numbered in table order and given the offsets of their
//     write lists; writes are bucketed, then put in causal order by counting
//     the bucket's earlier tokens.  Each write gets its retention
//     alpha = (1 - w)^exp(gamma_t).
//   * Each read is resolved to the version of its slot it sees: the row
//     before the chunk (version 0) or after the chunk's i-th write to the
//     slot (version i).  Only versions that some read sees get a row in the
//     scan's version buffer.
//   * Where a chunk writes each slot at least twice on average, the slots
//     with more than n0 writes are listed busiest first for the scan's
//     helpers (hand-off below), as many as the version rows left free hold.
// scan_kernel: one workgroup per (unit, slice of CG channels), chunk after
// chunk.
//   * The plan and the slice's values are staged in LDS (loaded one chunk
//     ahead into registers).
//   * The owner of each touched slot stores version 0 if a read sees it,
//     then applies the slot's writes in order (mass, lambda, row), storing
//     the versions reads see.  Thread s owns slot s and keeps its row slice
//     and mass in registers for the whole sequence.
//   * Hand-off: a listed slot's owner applies its first n0
//     writes and parks the row in a free version row; a helper, one lane per
//     16-byte piece of the row, applies the rest; the owner takes it back.
//     A wave then no longer waits for its busiest slot's whole chain.
//   * The reads: lanes of a token sum rho * version over its K reads in
//     address order, one 16-byte piece of every row each where a row slice
//     has several, else splitting the reads and combining them by a fixed
//     butterfly; r and the slice's sum of squares go to global memory.
// rms_gate_kernel: sums the slices' squares per token, applies RMSNorm and
// the gate, and copies the final mass.
#include "chunk_common.h"
#include "device_common.h"
#include "launch.h"

#include <algorithm>
#include <type_traits>

namespace ramnet {
namespace {

constexpr int kHBins = 32;                          // write-count bins of the hand-off order

// LDS rows are stored in 16-byte chunks whose order is XOR-swizzled by the
// row index, so that lanes touching different rows spread over the banks
// instead of all landing on the first chunk's banks.
template <typename T, int CG>
__device__ __forceinline__ int row_swz(int64_t row) {
    constexpr int nch = CG * static_cast<int>(sizeof(T)) / 16;
    return nch > 1 ? static_cast<int>((row >> 1) & (nch - 1)) : 0;
}
// Element c of row `row` in a swizzled [rows][CG] array of T.
template <typename T, int CG>
__device__ __forceinline__ int64_t swz_index(int64_t row, int c) {
    constexpr int epc = 16 / static_cast<int>(sizeof(T));
    return row * CG + ((c / epc) ^ row_swz<T, CG>(row)) * epc + (c % epc);
}

// A row slice of CG channels between LDS and registers (fp32 values).
template <int CG>
__device__ __forceinline__ void load_row(const float *p, int swz, float (&x)[CG]) {
#pragma unroll
    for (int j = 0; j < CG / 4; ++j) {
        const float4 f = reinterpret_cast<const float4 *>(p)[j ^ swz];
        x[4 * j] = f.x;
        x[4 * j + 1] = f.y;
        x[4 * j + 2] = f.z;
        x[4 * j + 3] = f.w;
    }
}
template <int CG>
__device__ __forceinline__ void load_row(const bf16_t *p, int swz, float (&x)[CG]) {
#pragma unroll
    for (int j = 0; j < CG / 8; ++j) {
        const uint4 u = reinterpret_cast<const uint4 *>(p)[j ^ swz];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            x[8 * j + 2 * q] = __uint_as_float(w[q] << 16);
            x[8 * j + 2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
        }
    }
}
template <int CG>
__device__ __forceinline__ void store_row(float *p, int swz, const float (&x)[CG]) {
#pragma unroll
    for (int j = 0; j < CG / 4; ++j)
        reinterpret_cast<float4 *>(p)[j ^ swz] =
            make_float4(x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]);
}
template <int CG>
__device__ __forceinline__ void store_row(bf16_t *p, int swz, const float (&x)[CG]) {
#pragma unroll
    for (int j = 0; j < CG / 8; ++j) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            w[q] = static_cast<uint32_t>(bf16_rne(x[8 * j + 2 * q]).bits) |
                   (static_cast<uint32_t>(bf16_rne(x[8 * j + 2 * q + 1]).bits) << 16);
        reinterpret_cast<uint4 *>(p)[j ^ swz] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// LDS of the plan kernel (byte offsets).
struct PlanLds {
    size_t cf, wo, bk, sk, sa, need, wtot, hist, total;
};
__host__ __device__ inline PlanLds plan_lds(const ChunkPlan &p, int64_t M) {
    PlanLds L{};
    const size_t ht = static_cast<size_t>(M);  // the table is indexed by slot
    size_t o = 0;
    L.cf = o; o = al16(o + ht * 4);                                       // writes | read flag; entry id
    L.wo = o; o = al16(o + static_cast<size_t>(p.ENT + 1) * 4);          // entry -> write offset
    L.bk = o; o = al16(o + static_cast<size_t>(p.EV) * 4);                // writes, arrival order
    L.sk = o; o = al16(o + static_cast<size_t>(p.EV) * 4);                // writes, causal order
    L.sa = o; o = al16(o + static_cast<size_t>(p.EV) * 4);                // staged write retention
    L.need = o; o = al16(o + static_cast<size_t>(p.ENT + p.EV + 1) * 4);  // versions read
    L.wtot = o; o = al16(o + 32 * 4);
    L.hist = o; o = al16(o + (2 * kHBins + 1) * 4);                       // hand-off bins, offsets, total
    L.total = o;
    return L;
}

// Header of a (unit, chunk) plan record.
struct PlanHdr {
    int nt;    // touched slots (entries)
    int nver;  // version rows
    int nwt;   // valid writes
    int nh;    // slots handed off after their first n0 writes
};

template <typename TIn, int EPW>
__global__ __launch_bounds__(kPT) void plan_kernel(ChunkArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const ChunkPlan &P = a.p;
    const int tid = threadIdx.x;
    // the heads of one (sequence, chunk) are neighbours: their addresses
    // share cache lines
    const int h = static_cast<int>(blockIdx.x % a.H);
    const int chunk = static_cast<int>((blockIdx.x / a.H) % P.n_chunks);
    const int b = static_cast<int>(blockIdx.x / a.H / P.n_chunks);
    const int unit = b * a.H + h;
    const int t0 = chunk * P.C, Cc = min(P.C, a.T - t0);
    const int K = a.K, nev = Cc * K;
    const int M = static_cast<int>(a.M);
    const int HT = M;  // table position = slot
    const uint64_t kdiv = ((uint64_t(1) << 32) + K - 1) / K;
    const PlanLds L = plan_lds(P, a.M);
    int *tcf = reinterpret_cast<int *>(smem + L.cf);
    int *ewo = reinterpret_cast<int *>(smem + L.wo);
    int *bk = reinterpret_cast<int *>(smem + L.bk);
    int *sk = reinterpret_cast<int *>(smem + L.sk);
    int *need = reinterpret_cast<int *>(smem + L.need);
    int *sa = reinterpret_cast<int *>(smem + L.sa);
    int *wtot = reinterpret_cast<int *>(smem + L.wtot);
    int *hist = reinterpret_cast<int *>(smem + L.hist);  // [kHBins] counts, offsets, total

    unsigned char *rec = a.plan + (static_cast<int64_t>(unit) * P.n_chunks + chunk) * P.rec_bytes;
    int *dwo = reinterpret_cast<int *>(rec + P.o_map);  // per slot: write
    int *dnx = dwo + M;                                 // offset; writes | (version-0 row + 1) << 16
    int *hl = reinterpret_cast<int *>(rec + P.o_hl);    // handed-off slots: rest offset | rest << 16
    int *wtv = reinterpret_cast<int *>(rec + P.o_wtv);
    float *ww = reinterpret_cast<float *>(rec + P.o_ww);
    float *wa = reinterpret_cast<float *>(rec + P.o_wa);
    int *rv = reinterpret_cast<int *>(rec + P.o_rv);
    float *rr = reinterpret_cast<float *>(rec + P.o_rr);
    const int64_t th0 = static_cast<int64_t>(b) * a.T * a.H + h;  // token 0 of the unit
    const TIn *gam = static_cast<const TIn *>(a.gamma) + static_cast<int64_t>(b) * a.T * a.ld_gamma + h;

    // ---- 0. this thread's events, e = tid + j * kPT (index t * K + k within
    //         the chunk), writes and reads alike; the loads go out first
    int ws[EPW], rs[EPW];
    float wt[EPW], rt[EPW], eg[EPW];
#pragma unroll
    for (int j = 0; j < EPW; ++j) {
        const int e = tid + j * kPT;
        ws[j] = -1;
        rs[j] = -1;
        if (e < nev) {
            const int t = div_by(e, kdiv), k = e - t * K;
            const int64_t th = th0 + static_cast<int64_t>(t0 + t) * a.H;
            const int64_t ai = (a.addr_unit_major ? static_cast<int64_t>(unit) * a.T + t0 + t : th) * K + k;
            ws[j] = a.w_idx[ai];
            wt[j] = a.w_wt[ai];
            rs[j] = a.r_idx[ai];
            rt[j] = a.r_wt[ai];
            eg[j] = to_f32(gam[static_cast<int64_t>(t0 + t) * a.ld_gamma]);
        }
    }
    for (int i = tid; i < HT; i += kPT) tcf[i] = 0;
    for (int i = tid; i <= P.ENT + P.EV; i += kPT) need[i] = 0;
    if (tid < 2 * kHBins) hist[tid] = 0;
    lds_barrier();

    // ---- 1. every event finds its slot's entry; writes count, reads flag.
    //         A zero-weight write changes nothing (alpha = 1, lambda = 0); a
    //         slot outside [0, M) (caller-given addresses) is skipped, and a
    //         skipped read contributes nothing.
    auto entry_of = [&](int s) -> int { return s; };
    int wpos[EPW], ar[EPW], rpos[EPW];
    float al[EPW];
#pragma unroll
    for (int j = 0; j < EPW; ++j) {
        wpos[j] = -1;
        rpos[j] = -1;
        ar[j] = 0;
        al[j] = 0.f;
        if (static_cast<uint32_t>(ws[j]) < static_cast<uint32_t>(M) && wt[j] > 0.f) {
            wpos[j] = entry_of(ws[j]);
            ar[j] = atomicAdd(&tcf[wpos[j]], 1) & (kReadFlag - 1);
            al[j] = retention_fast(wt[j], expf(eg[j]));
        }
        if (static_cast<uint32_t>(rs[j]) < static_cast<uint32_t>(M)) {
            rpos[j] = entry_of(rs[j]);
            atomicOr(&tcf[rpos[j]], kReadFlag);
        }
    }
    lds_barrier();

    // ---- 2. entries in table order: ids and write offsets from one scan of
    //         (1 + writes << 16) over the touched positions
    int nt, nwt;
    {
        const int per = (HT + kPT - 1) / kPT;
        const int lo = min(tid * per, HT), hi = min(lo + per, HT);
        int local = 0;
        for (int p = lo; p < hi; ++p) {
            const int c = tcf[p];
            if (c) local += 1 + ((c & (kReadFlag - 1)) << 16);
        }
        int total;
        int base = block_excl_scan<kPT>(local, wtot, total);
        for (int p = lo; p < hi; ++p) {
            const int c = tcf[p];
            int eid = -1;
            if (c) {
                const int nw = c & (kReadFlag - 1);
                eid = base & 0xffff;
                const int wo = base >> 16;
                ewo[eid] = wo;
                base += 1 + (nw << 16);
            }
            tcf[p] = eid;  // -1: untouched
        }
        nt = total & 0xffff;
        nwt = total >> 16;
        if (tid == 0) ewo[nt] = nwt;
    }
    lds_barrier();

    // ---- 3. writes into their entries' buckets, arrival order ...
#pragma unroll
    for (int j = 0; j < EPW; ++j)
        if (wpos[j] >= 0) bk[ewo[tcf[wpos[j]]] + ar[j]] = tid + j * kPT;
    lds_barrier();
    // ... then causal order: a write's rank is the number of the bucket's
    // writes with a smaller event index (token-major; one write per slot and
    // token)
    int spos[EPW];
#pragma unroll
    for (int j = 0; j < EPW; ++j) {
        spos[j] = -1;
        if (wpos[j] >= 0) {
            const int e = tid + j * kPT;
            const int eid = tcf[wpos[j]];
            const int wo = ewo[eid], n = ewo[eid + 1] - wo;
            int r = 0;
            for (int i = 0; i < n; ++i) r += bk[wo + i] < e ? 1 : 0;
            spos[j] = wo + r;
            sk[wo + r] = e;
        }
    }
    lds_barrier();

    // ---- 4. each read sees version c of its slot: c = the number of the
    //         slot's writes at tokens <= its own (writes come first within a
    //         token).  Entry eid's versions are numbered ewo[eid] + eid + c.
    int gv[EPW];
#pragma unroll
    for (int j = 0; j < EPW; ++j) {
        gv[j] = -1;
        if (rpos[j] >= 0) {
            const int eid = tcf[rpos[j]];
            const int wo = ewo[eid], n = ewo[eid + 1] - wo;
            const int tr = div_by(tid + j * kPT, kdiv);
            int c = 0;
            while (c < n && div_by(sk[wo + c], kdiv) <= tr) ++c;
            gv[j] = wo + eid + c;
            need[gv[j]] = 1;
        }
    }
    lds_barrier();

    // ---- 5. version rows: exclusive scan of the flags over nt + nwt + 1
    //         positions; version g has a row iff need[g + 1] > need[g]
    const int nver = block_scan_array<kPT>(need, nt + nwt + 1, wtot);
    lds_barrier();

    // ---- 6. the record: entries, writes staged in LDS in causal order, then
    //         everything stored with consecutive lanes on consecutive words
    int nh = 0;
    if (P.HMAX == 0) {
        for (int p = tid; p < M; p += kPT) {
            const int eid = tcf[p];
            int wo = 0, nx = 0;
            if (eid >= 0) {
                const int g = ewo[eid] + eid;
                wo = ewo[eid];
                nx = (ewo[eid + 1] - wo) | ((need[g + 1] > need[g] ? need[g] + 1 : 0) << 16);
            }
            dwo[p] = wo;
            dnx[p] = nx;
        }
    } else {
        // Hand-off: the slots with more than n0 writes, busiest first (bins
        // of the write count, the last bin holding every count beyond it),
        // as many as there are spare rows at the end of the scan's version
        // buffer and helper threads.  Positions within a bin come from LDS
        // atomics, so they vary from run to run; a position decides only
        // which thread applies a slot's writes, never the arithmetic.
        constexpr int kSP = (kNT + kPT - 1) / kPT;  // slots per thread (M <= kNT)
        int hbin[kSP], hrank[kSP];
#pragma unroll
        for (int j = 0; j < kSP; ++j) {
            const int p = tid + j * kPT;
            hbin[j] = -1;
            if (P.HMAX > 0 && p < M && tcf[p] >= 0) {
                const int nw = ewo[tcf[p] + 1] - ewo[tcf[p]];
                if (nw > P.n0) {
                    hbin[j] = kHBins - 1 - min(nw - P.n0 - 1, kHBins - 1);
                    hrank[j] = atomicAdd(&hist[hbin[j]], 1);
                }
            }
        }
        lds_barrier();
        if (tid < kWave) {  // offsets of the bins: one wave's prefix sum
            const int c = tid < kHBins ? hist[tid] : 0;
            const int inc = wave_incl_scan(c);
            if (tid < kHBins) hist[kHBins + tid] = inc - c;
            if (tid == kWave - 1) hist[2 * kHBins] = inc;  // total
        }
        lds_barrier();
        nh = min(hist[2 * kHBins], min(P.HMAX, P.EV - nver));
#pragma unroll
        for (int j = 0; j < kSP; ++j) {
            const int p = tid + j * kPT;
            if (p < M) {
                const int eid = tcf[p];
                int wo = 0, nx = 0;
                if (eid >= 0) {
                    const int g = ewo[eid] + eid;
                    const int nw = ewo[eid + 1] - ewo[eid];
                    wo = ewo[eid];
                    nx = nw | ((need[g + 1] > need[g] ? need[g] + 1 : 0) << 16);
                    if (hbin[j] >= 0) {
                        const int pos = hist[kHBins + hbin[j]] + hrank[j];
                        if (pos < nh) {
                            hl[pos] = (wo + P.n0) | ((nw - P.n0) << 16);
                            wo |= (pos + 1) << 16;
                        }
                    }
                }
                dwo[p] = wo;
                dnx[p] = nx;
            }
        }
    }
    if (tid == 0) {
        PlanHdr hd{nt, nver, nwt, nh};
        *reinterpret_cast<PlanHdr *>(rec) = hd;
    }
#pragma unroll
    for (int j = 0; j < EPW; ++j) {
        const int e = tid + j * kPT;
        if (spos[j] >= 0) {
            const int eid = tcf[wpos[j]];
            const int wo = ewo[eid];
            const int g = wo + eid + (spos[j] - wo) + 1;  // version after this write
            const int vr = need[g + 1] > need[g] ? need[g] : -1;
            bk[spos[j]] = div_by(e, kdiv) | ((vr + 1) << 10);
            sk[spos[j]] = __float_as_int(wt[j]);
            sa[spos[j]] = __float_as_int(al[j]);
        }
        if (e < nev) {
            rv[e] = gv[j] >= 0 ? need[gv[j]] : -1;
            rr[e] = gv[j] >= 0 ? rt[j] : 0.f;
        }
    }
    lds_barrier();
    for (int i = tid; i < nwt; i += kPT) {
        wtv[i] = bk[i];
        ww[i] = __int_as_float(sk[i]);
        wa[i] = __int_as_float(sa[i]);
    }
}

// LDS of the scan kernel (byte offsets).
struct ScanLds {
    size_t v, wtv, wwa, rv, rr, ver, hm, total;
};
__host__ __device__ inline size_t al256d(size_t x) { return (x + 255) & ~size_t(255); }
__host__ __device__ inline ScanLds scan_lds(const ChunkPlan &p, int64_t M, int sbytes, int vbytes) {
    ScanLds L{};
    size_t o = 0;
    L.v = o; o = al16(o + static_cast<size_t>(p.C) * (p.CG * vbytes + 16));  // values, rows padded by 16 B
    L.wtv = o; o = al16(o + static_cast<size_t>(p.EV) * 4);                 // write: token | row
    L.wwa = o; o = al16(o + static_cast<size_t>(p.EV) * 8);                 // write: weight, retention
    L.rv = o; o = al16(o + static_cast<size_t>(p.EV) * 4);                  // read: version row
    L.rr = o; o = al16(o + static_cast<size_t>(p.EV) * 4);                  // read weight
    L.ver = o = al256d(o); o = al16(o + static_cast<size_t>(p.EV) * p.CG * sbytes);  // version rows
    L.hm = o; o = al16(o + static_cast<size_t>(p.HMAX) * 4);                        // handed-off masses
    L.total = o;
    return L;
}

// Version row `r` ([rows][CG] TS at a row-size-aligned LDS byte offset, 16-byte
// chunks XOR-swizzled by the row): chunk j is at the returned offset ^ (j << 4).
template <typename T, int CG>
__device__ __forceinline__ uint32_t row_chunk0(uint32_t base, int r) {
    return base + static_cast<uint32_t>(r) * (CG * sizeof(T)) + (row_swz<T, CG>(r) << 4);
}
template <int CG>
__device__ __forceinline__ void store_row_x(unsigned char *lds, uint32_t a0, const float (&x)[CG], float) {
#pragma unroll
    for (int j = 0; j < CG / 4; ++j)
        *reinterpret_cast<float4 *>(lds + (a0 ^ (j << 4))) =
            make_float4(x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]);
}
template <int CG>
__device__ __forceinline__ void store_row_x(unsigned char *lds, uint32_t a0, const float (&x)[CG], bf16_t) {
#pragma unroll
    for (int j = 0; j < CG / 8; ++j) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            w[q] = static_cast<uint32_t>(bf16_rne(x[8 * j + 2 * q]).bits) |
                   (static_cast<uint32_t>(bf16_rne(x[8 * j + 2 * q + 1]).bits) << 16);
        *reinterpret_cast<uint4 *>(lds + (a0 ^ (j << 4))) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

template <int CG>
__device__ __forceinline__ void load_row_x(const unsigned char *lds, uint32_t a0, float (&x)[CG], float) {
#pragma unroll
    for (int j = 0; j < CG / 4; ++j) {
        const uint4 u = *reinterpret_cast<const uint4 *>(lds + (a0 ^ (j << 4)));
        float f[4];
        unpack_chunk(u, f);
#pragma unroll
        for (int q = 0; q < 4; ++q) x[4 * j + q] = f[q];
    }
}
template <int CG>
__device__ __forceinline__ void load_row_x(const unsigned char *lds, uint32_t a0, float (&x)[CG], bf16_t) {
#pragma unroll
    for (int j = 0; j < CG / 8; ++j) {
        const uint4 u = *reinterpret_cast<const uint4 *>(lds + (a0 ^ (j << 4)));
        float f[8];
        unpack_chunk(u, f);
#pragma unroll
        for (int q = 0; q < 8; ++q) x[8 * j + q] = f[q];
    }
}

// Value row t of the chunk (fp32 or bf16 in LDS, rows padded by 16 B), as fp32.
template <int CG>
__device__ __forceinline__ void value_row(const float *vbuf, int t, float (&vt)[CG]) {
    const float4 *r = reinterpret_cast<const float4 *>(vbuf + t * (CG + 4));
#pragma unroll
    for (int j = 0; j < CG / 4; ++j) {
        const float4 f = r[j];
        vt[4 * j] = f.x;
        vt[4 * j + 1] = f.y;
        vt[4 * j + 2] = f.z;
        vt[4 * j + 3] = f.w;
    }
}
template <int CG>
__device__ __forceinline__ void value_row(const bf16_t *vbuf, int t, float (&vt)[CG]) {
    const uint4 *r = reinterpret_cast<const uint4 *>(vbuf + t * (CG + 8));
#pragma unroll
    for (int j = 0; j < CG / 8; ++j) {
        const uint4 u = r[j];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            vt[8 * j + 2 * q] = __uint_as_float(w[q] << 16);
            vt[8 * j + 2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
        }
    }
}

// Applies one touched slot's chunk: version 0 if a read sees it, then the
// writes in causal order (mass, lambda, row), storing the versions reads see.
template <typename TS, int CG, typename TV>
__device__ __forceinline__ void walk_slot(int wo, int nw, int x0r, float (&x)[CG], float &m,
                                          float eps, const int *wtv, const float2 *wwa,
                                          const TV *vbuf, unsigned char *lds, uint32_t ver_off) {
    if (x0r >= 0) store_row_x<CG>(lds, row_chunk0<TS, CG>(ver_off, x0r), x, TS{});
    for (int i = 0; i < nw; ++i) {
        const int tv = wtv[wo + i];
        const int t = tv & 1023, vr = (tv >> 10) - 1;
        const float2 wa = wwa[wo + i];  // weight, retention
        m = fmaf(wa.y, m, wa.x);
        const float lam = wa.x * __builtin_amdgcn_rcpf(m + eps);
        float vt[CG];
        value_row<CG>(vbuf, t, vt);
#pragma unroll
        for (int c = 0; c < CG; ++c) x[c] = stored<TS>(fmaf(lam, vt[c] - x[c], x[c]));
        if (vr >= 0) store_row_x<CG>(lds, row_chunk0<TS, CG>(ver_off, vr), x, TS{});
    }
}

// One 16-byte piece of a row slice (CP = 16 / sizeof(TS) channels) between
// LDS and registers; piece h of the row whose piece 0 is at a0 is at a0 ^ (h << 4).
template <int CP>
__device__ __forceinline__ void load_piece(const unsigned char *lds, uint32_t a, float (&x)[CP]) {
    unpack_chunk(*reinterpret_cast<const uint4 *>(lds + a), x);
}
__device__ __forceinline__ void store_piece(unsigned char *lds, uint32_t a, const float (&x)[4]) {
    *reinterpret_cast<float4 *>(lds + a) = make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void store_piece(unsigned char *lds, uint32_t a, const float (&x)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        w[q] = static_cast<uint32_t>(bf16_rne(x[2 * q]).bits) | (static_cast<uint32_t>(bf16_rne(x[2 * q + 1]).bits) << 16);
    *reinterpret_cast<uint4 *>(lds + a) = make_uint4(w[0], w[1], w[2], w[3]);
}
// walk_slot for piece h of a row slice: the LH = CG / CP lanes that share a
// slot each apply its writes to their own piece (each computing the same
// mass and rate) and store their piece of the versions reads see.
template <typename TS, int CG, typename TV>
__device__ __forceinline__ void walk_piece(int wo, int nw, int h, float (&xp)[16 / sizeof(TS)], float &m,
                                           float eps, const int *wtv, const float2 *wwa, const TV *vbuf,
                                           unsigned char *lds, uint32_t ver_off) {
    constexpr int CP = 16 / static_cast<int>(sizeof(TS));
    constexpr int VROW = CG + 16 / static_cast<int>(sizeof(TV));
    int tvn = 0;
    float2 wan = make_float2(0.f, 0.f);
    if (nw > 0) {
        tvn = wtv[wo];
        wan = wwa[wo];
    }
    for (int i = 0; i < nw; ++i) {
        const int tv = tvn;
        const int t = tv & 1023, vr = (tv >> 10) - 1;
        const float2 wa = wan;
        float vt[CP];
        value_part<CP>(vbuf, t * VROW + h * CP, vt);
        if (i + 1 < nw) {
            tvn = wtv[wo + i + 1];
            wan = wwa[wo + i + 1];
        }
        m = fmaf(wa.y, m, wa.x);
        const float lam = wa.x * __builtin_amdgcn_rcpf(m + eps);
#pragma unroll
        for (int c = 0; c < CP; ++c) xp[c] = stored<TS>(fmaf(lam, vt[c] - xp[c], xp[c]));
        if (vr >= 0) store_piece(lds, row_chunk0<TS, CG>(ver_off, vr) ^ (h << 4), xp);
    }
}

// CG values of a row slice in HBM.
template <typename TS, int CG>
struct HRow {
    TS e[CG];
};

// VT: the value rows' type in LDS: fp32 (converted once at staging), or the
// bf16 input itself (half the LDS, which buys a longer chunk, at a
// conversion per write); the planner picks per configuration.
// HAND: the hand-off of the busiest slots (P.HMAX > 0).
template <typename TIn, typename TS, int CG, typename VT, bool HAND, int EVT>
__global__ __launch_bounds__(kNT) void scan_kernel(ChunkArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const ChunkPlan &P = a.p;
    const int tid = threadIdx.x;
    const int ncg = P.ncg;
    const int units = a.B * a.H;
    int unit, cg;
    {
        const int bid = blockIdx.x;
        if (units % 8 == 0) {  // keep the slices of one unit on one XCD
            const int xcd = bid % 8, j = bid / 8;
            unit = (j / ncg) * 8 + xcd;
            cg = j % ncg;
        } else {
            unit = bid / ncg;
            cg = bid % ncg;
        }
    }
    const int b = unit / a.H, h = unit % a.H;
    const int M = static_cast<int>(a.M);
    const int K = a.K, C = P.C, d_v = a.d_v, EV = P.EV;
    const int nchunks = static_cast<int>(P.n_chunks);
    const ScanLds L = scan_lds(P, a.M, sizeof(TS), sizeof(VT));
    VT *vbuf = reinterpret_cast<VT *>(smem + L.v);
    constexpr int VROW = CG + 16 / static_cast<int>(sizeof(VT));  // padded value row
    int *s_wtv = reinterpret_cast<int *>(smem + L.wtv);
    float2 *s_wwa = reinterpret_cast<float2 *>(smem + L.wwa);
    const uint32_t ver_off = static_cast<uint32_t>(L.ver);
    int *s_rv = reinterpret_cast<int *>(smem + L.rv);
    float *s_rr = reinterpret_cast<float *>(smem + L.rr);
    float *s_hm = reinterpret_cast<float *>(smem + L.hm);
    constexpr int kCP = 16 / static_cast<int>(sizeof(TS));  // channels per 16-byte piece
    constexpr int kLH = CG / kCP;                            // lanes per handed-off slot

    // this unit's token 0 in the values
    const TIn *v = static_cast<const TIn *>(a.v) + static_cast<int64_t>(b) * a.T * a.ld_v + h * d_v;
    TS *S = static_cast<TS *>(a.S);
    const int64_t th_unit = static_cast<int64_t>(b) * a.T * a.H + h;  // token 0 of the unit
    const unsigned char *plan0 = a.plan + static_cast<int64_t>(unit) * P.n_chunks * P.rec_bytes;

    // Resident state: thread s owns slot s's row slice and mass.
    float x[CG];
    float m = 0.f;
    if (tid < M) {
        const HRow<TS, CG> r = *reinterpret_cast<const HRow<TS, CG> *>(
            S + (static_cast<int64_t>(unit) * M + tid) * d_v + cg * CG);
#pragma unroll
        for (int c = 0; c < CG; ++c) x[c] = to_f32(r.e[c]);
        m = a.mass[static_cast<int64_t>(unit) * M + tid];
    }

    // The next chunk's plan and values, loaded one chunk ahead.
    constexpr int VPT = (CG * 512 + kNT - 1) / kNT;
    // value element tid + j NT of a chunk's slice is token vt0 + j TPJ,
    // channel vcc: the thread's column is fixed and its rows step by TPJ
    constexpr int TPJ = kNT / CG;
    const int vt0 = static_cast<int>(static_cast<unsigned>(tid) / CG);
    const int vcc = static_cast<int>(static_cast<unsigned>(tid) % CG);
    const TIn *vcol = v + cg * CG + vcc;
    const uint32_t ldv32 = static_cast<uint32_t>(a.ld_v);  // the launcher checks ld_v < 2^32
    int pf_wtv[EVT], pf_rv[EVT];
    float pf_ww[EVT], pf_wa[EVT], pf_rr[EVT];
    TIn pf_v[VPT];  // raw: converting at load time would wait for each load
    int pf_dwo = 0, pf_dnx = 0;  // resident: this slot's write offset, writes | x0
    int pf_nh = 0, pf_hl = 0;               // resident: slots handed off; this thread's one
    auto prefetch = [&](int c) {
        const unsigned char *rec = plan0 + static_cast<int64_t>(c) * P.rec_bytes;
        const int t0 = c * C, Cc = min(C, a.T - t0), nev = Cc * K;
        const int *wtv = reinterpret_cast<const int *>(rec + P.o_wtv);
        const float *ww = reinterpret_cast<const float *>(rec + P.o_ww);
        const float *wa = reinterpret_cast<const float *>(rec + P.o_wa);
        const int *rv = reinterpret_cast<const int *>(rec + P.o_rv);
        const float *rr = reinterpret_cast<const float *>(rec + P.o_rr);
        if (HAND) pf_nh = reinterpret_cast<const PlanHdr *>(rec)->nh;
        // every load is independent of every other (no wait on the header):
        // the write list is read to its capacity, entries past its end are
        // never used
#pragma unroll
        for (int j = 0; j < EVT; ++j) {
            const int i = tid + j * kNT;
            if (i < EV) {
                pf_wtv[j] = wtv[i];
                pf_ww[j] = ww[i];
                pf_wa[j] = wa[i];
            }
            if (i < nev) {
                pf_rv[j] = rv[i];
                pf_rr[j] = rr[i];
            }
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int t = min(vt0 + j * TPJ, Cc - 1);  // in range; extra lanes unused
            pf_v[j] = vcol[static_cast<uint64_t>(static_cast<uint32_t>(t0 + t)) * ldv32];
        }
        {
            if (tid < M) {
                pf_dwo = reinterpret_cast<const int *>(rec + P.o_map)[tid];
                pf_dnx = reinterpret_cast<const int *>(rec + P.o_map)[M + tid];
            }
            // read to capacity like the write list; entries past nh unused
            if (HAND && tid / kLH < P.HMAX) pf_hl = reinterpret_cast<const int *>(rec + P.o_hl)[tid / kLH];
        }
    };

    prefetch(0);
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C, Cc = min(C, a.T - t0), nev = Cc * K;
        // ---- 1. stage this chunk's plan and values
#pragma unroll
        for (int j = 0; j < EVT; ++j) {
            const int i = tid + j * kNT;
            if (i < EV) {
                s_wtv[i] = pf_wtv[j];
                s_wwa[i] = make_float2(pf_ww[j], pf_wa[j]);
                s_rv[i] = pf_rv[j];
                s_rr[i] = pf_rr[j];
            }
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int t = vt0 + j * TPJ;
            if (t < Cc) {
                if constexpr (std::is_same_v<VT, TIn>) vbuf[t * VROW + vcc] = pf_v[j];
                else vbuf[t * VROW + vcc] = to_f32(pf_v[j]);
            }
        }
        const int my_wo = HAND ? pf_dwo & 0xffff : pf_dwo, my_nx = pf_dnx;
        const int my_hp = HAND ? static_cast<int>(static_cast<uint32_t>(pf_dwo) >> 16) - 1 : -1;  // hand-off row
        const int nh = HAND ? pf_nh : 0, my_hl = pf_hl;
        lds_barrier();
        // ---- 2. the next chunk's loads go out now and land during the walk
        if (c + 1 < nchunks) prefetch(c + 1);
        // ---- 3. walk the touched slots
        {
            // the owner applies its slot's first writes (all of them unless
            // the slot is handed off) ...
            if (tid < M && my_nx != 0) {
                const int nw = my_nx & 0xffff;
                walk_slot<TS, CG>(my_wo, HAND && my_hp >= 0 ? P.n0 : nw, (my_nx >> 16) - 1, x, m, a.eps_gsu, s_wtv,
                                  s_wwa, vbuf, smem, ver_off);
                if (HAND && my_hp >= 0) {
                    store_row_x<CG>(smem, row_chunk0<TS, CG>(ver_off, EV - 1 - my_hp), x, TS{});
                    s_hm[my_hp] = m;
                }
            }
            // ... then helper j applies the rest of the j-th busiest slot's
            // writes to its row, parked in version row EV - 1 - j (the plan
            // leaves those rows free), and the owner takes the row back
            if (HAND && nh > 0) {
                lds_barrier();
                const int j = tid / kLH, hp = tid % kLH;  // helper j, piece hp
                if (j < nh) {
                    const uint32_t a0 = row_chunk0<TS, CG>(ver_off, EV - 1 - j) ^ (hp << 4);
                    float xp[kCP];
                    load_piece<kCP>(smem, a0, xp);
                    float mm = s_hm[j];
                    walk_piece<TS, CG>(my_hl & 0xffff, my_hl >> 16, hp, xp, mm, a.eps_gsu, s_wtv, s_wwa, vbuf,
                                       smem, ver_off);
                    store_piece(smem, a0, xp);
                    if (hp == 0) s_hm[j] = mm;
                }
                lds_barrier();
                if (my_hp >= 0) {
                    load_row_x<CG>(smem, row_chunk0<TS, CG>(ver_off, EV - 1 - my_hp), x, TS{});
                    m = s_hm[my_hp];
                }
            }
        }
        lds_barrier();
        // ---- 4. reads: r = sum_k rho_k * version_k over the slice; G = P.RG
        //         lanes share a token.  With 1 < NCH <= G (NCH: pieces per row), lane
        //         g takes piece g % NCH of reads k = g / NCH, g / NCH + G / NCH,
        //         ... in order, and the G / NCH lanes of a piece are combined
        //         by a butterfly; the lanes of a token then read neighbouring
        //         pieces of one row.  Otherwise lane g takes whole rows of
        //         reads k = g, g + G, ...  r and the slice's sum of squares go
        //         to global memory.
        {
            constexpr int EPC = 16 / static_cast<int>(sizeof(TS));  // channels per 16-byte piece
            constexpr int NCH = CG / EPC;                            // pieces per row
            const int G = P.RG;
            if (NCH > 1 && G >= NCH) {
                const int GR = G / NCH;  // lanes per piece
                for (int i = tid; i < Cc * G; i += kNT) {
                    const int g = i % G, t = i / G;
                    const int jc = g % NCH, kr = g / NCH;
                    float r[EPC];
#pragma unroll
                    for (int cc = 0; cc < EPC; ++cc) r[cc] = 0.f;
                    for (int k = kr; k < K; k += GR) {
                        // skipped reads have no row; a zero weight adds nothing
                        const int row = t * K + k;
                        const int vr = s_rv[row];
                        const float rw = s_rr[row];
                        if (vr >= 0 && rw != 0.f) {
                            const uint4 u = *reinterpret_cast<const uint4 *>(
                                smem + (row_chunk0<TS, CG>(ver_off, vr) ^ (jc << 4)));
                            float sv[EPC];
                            unpack_chunk(u, sv);
#pragma unroll
                            for (int cc = 0; cc < EPC; ++cc) r[cc] = fmaf(rw, sv[cc], r[cc]);
                        }
                    }
#pragma unroll
                    for (int cc = 0; cc < EPC; ++cc) {
                        if (NCH <= 1 && G > 1) r[cc] += lane_xor<1>(r[cc]);
                        if (NCH <= 2 && G > 2) r[cc] += lane_xor<2>(r[cc]);
                        if (NCH <= 4 && G > 4) r[cc] += lane_xor<4>(r[cc]);
                        if (NCH <= 8 && G > 8) r[cc] += lane_xor<8>(r[cc]);
                    }
                    const int64_t th = th_unit + static_cast<int64_t>(t0 + t) * a.H;
                    float ss = 0.f;
#pragma unroll
                    for (int cc = 0; cc < EPC; ++cc) ss = fmaf(r[cc], r[cc], ss);
                    if (NCH > 1) ss += lane_xor<1>(ss);
                    if (NCH > 2) ss += lane_xor<2>(ss);
                    if (NCH > 4) ss += lane_xor<4>(ss);
                    if (kr == 0) {
                        float *dst = a.rbuf + th * d_v + cg * CG + jc * EPC;
#pragma unroll
                        for (int cc = 0; cc < EPC; cc += 4)
                            *reinterpret_cast<float4 *>(dst + cc) = make_float4(r[cc], r[cc + 1], r[cc + 2], r[cc + 3]);
                        if (jc == 0) a.sumsq[th * ncg + cg] = ss;
                    }
                }
            } else {
                for (int i = tid; i < Cc * G; i += kNT) {
                    const int g = i % G, t = i / G;
                    float r[CG];
#pragma unroll
                    for (int cc = 0; cc < CG; ++cc) r[cc] = 0.f;
                    for (int k = g; k < K; k += G) {
                        // skipped reads have no row; a zero weight adds nothing
                        const int row = t * K + k;
                        const int vr = s_rv[row];
                        const float rw = s_rr[row];
                        if (vr >= 0 && rw != 0.f) {
                            const uint32_t a0 = row_chunk0<TS, CG>(ver_off, vr);
#pragma unroll
                            for (int j = 0; j < NCH; ++j) {
                                const uint4 u = *reinterpret_cast<const uint4 *>(smem + (a0 ^ (j << 4)));
                                float sv[EPC];
                                unpack_chunk(u, sv);
#pragma unroll
                                for (int cc = 0; cc < EPC; ++cc) r[j * EPC + cc] = fmaf(rw, sv[cc], r[j * EPC + cc]);
                            }
                        }
                    }
#pragma unroll
                    for (int cc = 0; cc < CG; ++cc) {
                        if (G > 1) r[cc] += lane_xor<1>(r[cc]);
                        if (G > 2) r[cc] += lane_xor<2>(r[cc]);
                        if (G > 4) r[cc] += lane_xor<4>(r[cc]);
                        if (G > 8) r[cc] += lane_xor<8>(r[cc]);
                    }
                    const int64_t th = th_unit + static_cast<int64_t>(t0 + t) * a.H;
                    float *dst = a.rbuf + th * d_v + cg * CG;
#pragma unroll
                    for (int j = 0; j < NCH; ++j) {
                        if (j % G == g) {
#pragma unroll
                            for (int cc = 0; cc < EPC; cc += 4)
                                *reinterpret_cast<float4 *>(dst + j * EPC + cc) =
                                    make_float4(r[j * EPC + cc], r[j * EPC + cc + 1], r[j * EPC + cc + 2],
                                                r[j * EPC + cc + 3]);
                        }
                    }
                    if (g == 0) {
                        float ss = 0.f;
#pragma unroll
                        for (int cc = 0; cc < CG; ++cc) ss = fmaf(r[cc], r[cc], ss);
                        a.sumsq[th * ncg + cg] = ss;
                    }
                }
            }
        }
        (void)nev;
        lds_barrier();
    }

    if (tid < M) {
        HRow<TS, CG> o;
#pragma unroll
        for (int cc = 0; cc < CG; ++cc) o.e[cc] = from_f32<TS>(x[cc]);
        *reinterpret_cast<HRow<TS, CG> *>(S + (static_cast<int64_t>(unit) * M + tid) * d_v + cg * CG) = o;
        // Other slices of this unit may not have read the initial mass
        // yet; the epilogue copies slice 0's final mass over.
        if (cg == 0) a.mass_ws[static_cast<int64_t>(unit) * M + tid] = m;
    }
}

// Four values of type T as one vector access.
template <typename T>
struct alignas(4 * sizeof(T)) Quad {
    T e[4];
};

// Four read sums in, four outputs out, each touched once: non-temporal.
typedef float nt_f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int nt_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ Quad<float> nt_load_quad(const float *p) {
    const nt_f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_f32x4 *>(p));
    Quad<float> q;
    q.e[0] = v.x;
    q.e[1] = v.y;
    q.e[2] = v.z;
    q.e[3] = v.w;
    return q;
}
__device__ __forceinline__ void nt_store_quad(float *p, const Quad<float> &q) {
    nt_f32x4 v;
    v.x = q.e[0];
    v.y = q.e[1];
    v.z = q.e[2];
    v.w = q.e[3];
    __builtin_nontemporal_store(v, reinterpret_cast<nt_f32x4 *>(p));
}
__device__ __forceinline__ void nt_store_quad(bf16_t *p, const Quad<bf16_t> &q) {
    nt_u32x2 v;
    v.x = static_cast<uint32_t>(q.e[0].bits) | (static_cast<uint32_t>(q.e[1].bits) << 16);
    v.y = static_cast<uint32_t>(q.e[2].bits) | (static_cast<uint32_t>(q.e[3].bits) << 16);
    __builtin_nontemporal_store(v, reinterpret_cast<nt_u32x2 *>(p));
}

// out = r / sqrt(mean(r^2) + eps) * omega * sigmoid(g), four channels per
// thread; the per-token square sums of the channel slices are added in
// slice order.  With an fp32 output, r is held in `out` itself (rbuf ==
// out): each thread reads its own four values before it writes them, and
// neither pointer is declared restrict.
template <typename TIn, typename TO>
__global__ __launch_bounds__(256) void rms_gate_kernel(const float *rbuf,
                                                       const float *__restrict__ sumsq, int ncg,
                                                       const TIn *__restrict__ g, int H,
                                                       int64_t ld_g,
                                                       const float *__restrict__ norm_w,
                                                       TO *out, int64_t n, int d_v, float eps,
                                                       const float *__restrict__ mass_ws,
                                                       int mass_stride, float *__restrict__ mass,
                                                       int64_t n_mass) {
    const int q4 = d_v / 4;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n_mass) mass[i] = mass_ws[i * mass_stride];
    if (i >= n * q4) return;
    const int64_t th = i / q4;
    const int c0 = static_cast<int>(i - th * q4) * 4;
    float tot = 0.f;
    for (int j = 0; j < ncg; ++j) tot += sumsq[th * ncg + j];
    const float den = tot / static_cast<float>(d_v) + eps;
    const float inv = den > 0.f ? 1.0f / sqrtf(den) : 0.f;  // zero read, eps 0
    const Quad<float> r = nt_load_quad(rbuf + th * d_v + c0);
    const Quad<TIn> gv = *reinterpret_cast<const Quad<TIn> *>(g + (th / H) * ld_g + (th % H) * d_v + c0);
    Quad<TO> o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float om = norm_w ? norm_w[c0 + j] : 1.0f;
        o.e[j] = from_f32<TO>(r.e[j] * inv * om * sigmoid(to_f32(gv.e[j])));
    }
    nt_store_quad(out + th * d_v + c0, o);
}

template <typename K>
hipError_t set_lds(K kern, size_t lds) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
}

using ScanFn = void (*)(ChunkArgs);
template <typename TIn, typename TS, int CG, typename VB, int EVT>
ScanFn pick_scan(const ChunkPlan &P) {
    return P.HMAX > 0 ? (P.raw_values ? scan_kernel<TIn, TS, CG, VB, true, EVT>
                                      : scan_kernel<TIn, TS, CG, float, true, EVT>)
                      : (P.raw_values ? scan_kernel<TIn, TS, CG, VB, false, EVT>
                                      : scan_kernel<TIn, TS, CG, float, false, EVT>);
}

template <typename TIn, typename TS, int CG>
hipError_t launch_cfg(const ChunkArgs &a, hipStream_t st) {
    const ChunkPlan &P = a.p;
    const int64_t units = static_cast<int64_t>(a.B) * a.H;
    const int tier = (P.EV + 1023) / 1024;  // 1..4
    if (tier < 1 || tier > kMaxEV / 1024) return hipErrorInvalidValue;
    auto pk = tier <= 2 ? plan_kernel<TIn, 2048 / kPT> : tier == 3 ? plan_kernel<TIn, 3072 / kPT>
                                                                      : plan_kernel<TIn, 4096 / kPT>;
    hipError_t e = set_lds(pk, P.lds_plan);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(pk, dim3(static_cast<unsigned>(units * P.n_chunks)), dim3(kPT), P.lds_plan, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    using VB = std::conditional_t<std::is_same_v<TIn, bf16_t>, bf16_t, float>;
    const ScanFn sk = tier <= 2 ? pick_scan<TIn, TS, CG, VB, 2>(P)
                      : tier == 3 ? pick_scan<TIn, TS, CG, VB, 3>(P)
                                  : pick_scan<TIn, TS, CG, VB, 4>(P);
    if (!sk) return hipErrorInvalidValue;
    e = set_lds(sk, P.lds_scan);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sk, dim3(static_cast<unsigned>(units * P.ncg)), dim3(kNT), P.lds_scan, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = units * a.T;
    const int64_t n_mass = units * a.M;
    const int64_t work = std::max<int64_t>(n * (a.d_v / 4), n_mass);
    const unsigned g2 = static_cast<unsigned>((work + 255) / 256);
    if (a.out_bf16)
        hipLaunchKernelGGL((rms_gate_kernel<TIn, bf16_t>), dim3(g2), dim3(256), 0, st, a.rbuf,
                           a.sumsq, P.ncg, static_cast<const TIn *>(a.g), a.H, a.ld_g, a.norm_w,
                           static_cast<bf16_t *>(a.out_bf16), n, a.d_v, a.eps_norm, a.mass_ws,
                           1, a.mass, n_mass);
    else
        hipLaunchKernelGGL((rms_gate_kernel<TIn, TS>), dim3(g2), dim3(256), 0, st, a.rbuf,
                           a.sumsq, P.ncg, static_cast<const TIn *>(a.g), a.H, a.ld_g, a.norm_w,
                           static_cast<TS *>(a.out), n, a.d_v, a.eps_norm, a.mass_ws,
                           1, a.mass, n_mass);
    return hipGetLastError();
}

template <typename TIn, typename TS>
hipError_t launch_cg(const ChunkArgs &a, hipStream_t st) {
    switch (a.p.CG) {
        case 8: return launch_cfg<TIn, TS, 8>(a, st);
        case 16: return launch_cfg<TIn, TS, 16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

namespace {
ChunkPlan plan_with(int64_t M, int K, int d_v, int B, int T, int H, bool state_bf16, int vbytes) {
    ChunkPlan p{};
    p.ok = false;
    const int sbytes = state_bf16 ? 2 : 4;
    const int64_t units = static_cast<int64_t>(B) * H;
    // Plan entries pack the token in 10 bits and table sums in 16; thread s
    // of the scan owns slot s (rows in HBM take the slot-range path).
    if (T < 32 || units == 0 || K > 63 || M > kNT) return p;
    p.resident = true;
    // Largest channel slice that still gives about one workgroup per CU,
    // then the longest chunk (a multiple of 32 tokens) whose plan and
    // version rows fit LDS.
    const int cgs[2] = {16, 8};
    for (int ci = 0; ci < 2; ++ci) {
        const int CG = cgs[ci];
        if (d_v % CG || CG * sbytes < 16) continue;
        const bool last = ci == 1;
        if (!last && units * (d_v / CG) < 256) continue;
        for (int C = 512; C >= 32; C -= 32) {
            const int EV = C * K;
            if (EV > kMaxEV) continue;
            ChunkPlan q = p;
            q.CG = CG;
            q.C = C;
            q.EV = EV;
            q.ENT = static_cast<int>(std::min<int64_t>(M, 2 * EV));
            q.HT = 0;  // the plan's table is indexed by slot
            q.ncg = d_v / CG;
            // lanes per token in the read reduction: enough to keep the
            // workgroup busy, within one 16-lane row
            {
                int g = 1;
                while (g < 16 && g < K && static_cast<int64_t>(C) * g * 2 <= kNT) g *= 2;
                q.RG = g;
            }
            q.n0 = 1;
            q.HMAX = 0;
            q.lds_plan = plan_lds(q, M).total;
            q.lds_scan = scan_lds(q, M, sbytes, vbytes).total;
            q.raw_values = vbytes == 2;
            if (q.lds_plan > kChunkLdsLimit || q.lds_scan > kChunkLdsLimit) continue;
            if (static_cast<int64_t>(C) * K >= 2 * M) {
                // helpers for the busiest slots, where a chunk writes each
                // slot at least twice on average (below that the hand-off's
                // barriers cost about what it saves: Top-8, 1.75 writes per
                // slot, ran 1-3% slower with it, Top-32, 3 writes, 7%
                // faster): as many masses as the LDS left over holds, at
                // most one helper group per thread group and slot
                const size_t spare = (kChunkLdsLimit - q.lds_scan) / 16 * 4;  // whole 16-byte pieces
                const int lh = CG * sbytes / 16;  // lanes per handed-off slot, one 16-byte piece each
                q.HMAX = static_cast<int>(std::min<int64_t>(std::min<int64_t>(M, kNT / lh), static_cast<int64_t>(spare)));
                q.lds_scan = scan_lds(q, M, sbytes, vbytes).total;
                if (q.lds_scan > kChunkLdsLimit) q.HMAX = 0, q.lds_scan = scan_lds(q, M, sbytes, vbytes).total;
            }
            q.n_chunks = (T + C - 1) / C;
            size_t o = 256;  // header
            q.ENTA = (q.ENT + 63) & ~63;
            q.o_ent = o;
            q.o_map = o; o += al256(static_cast<size_t>(M) * 8);
            q.o_hl = o; o += al256(static_cast<size_t>(q.HMAX) * 4);
            q.o_wtv = o; o += al256(static_cast<size_t>(EV) * 4);
            q.o_ww = o; o += al256(static_cast<size_t>(EV) * 4);
            q.o_wa = o; o += al256(static_cast<size_t>(EV) * 4);
            q.o_rv = o; o += al256(static_cast<size_t>(EV) * 4);
            q.o_rr = o; o += al256(static_cast<size_t>(EV) * 4);
            q.rec_bytes = o;
            const size_t n = static_cast<size_t>(units) * T;
            q.ws_rbuf = state_bf16 ? al256(n * d_v * 4) : 0;
            q.ws_sumsq = al256(n * q.ncg * 4);
            q.ws_mass = al256(static_cast<size_t>(units) * M * 4);
            q.ws_plan = al256(static_cast<size_t>(units) * q.n_chunks * q.rec_bytes);
            q.ok = true;
            return q;
        }
    }
    return p;
}

}  // namespace

ChunkPlan plan_chunked(int64_t M, int K, int d_v, int B, int T, int H, bool in_bf16, bool state_bf16) {
    if (M > kNT) return plan_ranges(M, K, d_v, B, T, H, in_bf16, state_bf16);  // rows in HBM
    const ChunkPlan f = plan_with(M, K, d_v, B, T, H, state_bf16, 4);
    if (!in_bf16) return f;
    const ChunkPlan r = plan_with(M, K, d_v, B, T, H, state_bf16, 2);
    return (r.ok && (!f.ok || r.C > f.C)) ? r : f;
}

size_t chunk_workspace_bytes(const ChunkPlan &p) {
    return p.ws_rbuf + p.ws_sumsq + p.ws_mass + p.ws_plan + p.ws_partial + p.ws_spill;
}

hipError_t launch_scan_chunked(const ChunkArgs &args, hipStream_t st) {
    if (static_cast<int64_t>(args.B) * args.H * args.T == 0) return hipSuccess;
    if (!args.p.ok) return hipErrorInvalidValue;
    if (!args.p.resident) return launch_scan_ranges(args, st);
    ChunkArgs a = args;
    if (!a.ld_v) a.ld_v = static_cast<int64_t>(a.H) * a.d_v;
    if (a.ld_v > 0xffffffffll) return hipErrorInvalidValue;  // the scan's row steps are 32-bit
    if (!a.ld_g) a.ld_g = static_cast<int64_t>(a.H) * a.d_v;
    if (!a.ld_gamma) a.ld_gamma = a.H;
    if (a.in_bf16)
        return a.state_bf16 ? launch_cg<bf16_t, bf16_t>(a, st) : launch_cg<bf16_t, float>(a, st);
    return a.state_bf16 ? launch_cg<float, bf16_t>(a, st) : launch_cg<float, float>(a, st);
}

}  // namespace ramnet
