// Slot-grouped prefill recurrence with the state rows in HBM (M > 1024),
// for gfx950.
//
// RAM-Net project page, GPU-execution paragraphs: with every token's
// addresses known, events are grouped by slot, each slot applies its own
// events in causal order, different slots run in parallel and untouched
// slots cost nothing.  The Gated Sparse Update and the read are those of the
// "Gated Sparse Update" and "three stages" paragraphs.
//
// A unit's (batch, head) slots are split into kRanges ranges by slot mod
// kRanges, and its sequence into chunks of C tokens.
//
// plan_range_kernel: the (unit, chunk) items are planned all at once
// (grouping does not depend on the state), by as many workgroups as fit the
// chip, each looping over items with the next item's events in flight.
// Every valid event finds its slot's entry in an LDS table (the slot itself,
// or a double-hashed table for a large state); entries are numbered range by
// range, so that
// each range's entries, its write list (in (slot, token) order, each write
// with its retention alpha = (1 - w)^exp(gamma_t)), the versions its reads
// see and its reads (grouped by token) are contiguous sections of the record.
// A read sees the row before the chunk (version 0) or after the slot's i-th
// write in the chunk; only versions some read sees get a row.
//
// scan_range_kernel: one workgroup per (unit, range), chunk after chunk.
//   * The range's write and read lists and the chunk's value rows are staged
//     in LDS (loaded one chunk ahead).
//   * Walk: every touched slot's row is gathered whole from HBM, one 16-byte
//     piece per lane (the first round's rows during the previous chunk's
//     reads); the range's masses stay in LDS where they fit.  The lanes of a
//     slot each apply its writes to their piece (each computing the same
//     mass and rate), two pieces per lane in step, store the versions reads
//     see in LDS (later ones in a spill area) and write the row and mass
//     back.  A slot belongs to one range, so the mass is updated in place.
//   * Reads: per token, four channels per lane, the range's reads summed in
//     address order (rho * version); every token's partial (zero when the
//     range holds none of its reads) goes to the workspace, in fp16 where the
//     state is bf16.
// gate_partials_kernel: one wave per token-head adds the kRanges partials in
// range order, then RMSNorm over d_v and the sigmoid gate.
#include "chunk_common.h"
#include "device_common.h"
#include "launch.h"

#include <algorithm>
#include <type_traits>

namespace ramnet {
namespace {

// Address-space qualifiers for the version rows: LDS and global memory are
// named in the pointer types, so that no access to them is generic (the
// host pass sees plain pointers).
#if defined(__HIP_DEVICE_COMPILE__)
#define RN_LDS __attribute__((address_space(3)))
#define RN_GLB __attribute__((address_space(1)))
#define RN_CONST __attribute__((address_space(4)))
#else
#define RN_LDS
#define RN_GLB
#define RN_CONST
#endif
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Four channels of storage type T as one vector access.
template <typename T> struct Vec4Of;
template <> struct Vec4Of<float> { using type = u32x4; };
template <> struct Vec4Of<bf16_t> { using type = u32x2; };
template <typename T> using VecOf = typename Vec4Of<T>::type;

constexpr int kR = kRanges;
// The scan kernel runs kRT threads per (unit, range): one workgroup per
// compute unit at the benchmark's size, 16 waves to hide the latency of the
// row gathers.
constexpr int kRT = 1024;
constexpr int kPTW = 4;  // walk tasks (16-byte row pieces) per scan thread and round
constexpr int kLW = 1;   // list entries per kind and thread staged (CAPW = CAPR = kLW * kRT)
constexpr int kIL = 2;   // row pieces whose write chains a lane walks together

__device__ __forceinline__ int range_of(int slot) { return slot & (kR - 1); }

// Waits for every vector memory access in flight (s_waitcnt vmcnt(0)).
// Placed where the loads in flight are known to have arrived, or inside a
// rarely taken branch that loads from global memory, so that the code after
// it has no such load pending: the compiler then adds no wait there (a wait
// it adds after stores covers the stores too).
__device__ __forceinline__ void wait_vm_loads() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// LDS of the plan kernel (byte offsets).
struct RPlanLds {
    size_t key, cf, wo, bk, sk, sa, need, rg, rt, misc, total;
};
// The plan kernel of the HBM-row path runs kPRT threads; its slot table has
// at most kPlanSteps * kPRT positions.
constexpr int kPRT = 1024;
constexpr int kPlanSteps = 8;
__host__ __device__ inline RPlanLds rplan_lds(const ChunkPlan &p, int64_t M) {
    RPlanLds L{};
    const size_t ht = p.HT ? static_cast<size_t>(p.HT) : static_cast<size_t>(M);
    const size_t need = std::max<size_t>(static_cast<size_t>(p.ENT) + p.EV + 1, kR * kPRT);
    const size_t ev = al16(static_cast<size_t>(p.EV) * 4);
    size_t o = 0;
    // the hash keys are dead once the entries are numbered (step 2); the
    // write lists (bk, sk, sa: step 3 on) share their space
    L.key = o;                                                    // slot of a hash entry
    L.bk = o; L.sk = o + ev; L.sa = o + 2 * ev;                   // writes: arrival, causal order; staging
    o = al16(o + std::max<size_t>(p.HT ? ht * 4 : 0, 3 * ev));
    L.cf = o; o = al16(o + ht * 4);                               // writes | read flag; entry id
    L.wo = o; o = al16(o + static_cast<size_t>(p.ENT + 1) * 4);  // entry -> writes, then offset
    L.need = o; o = al16(o + need * 4);                           // (range, thread) counts; versions read
    L.rg = o; o = al16(o + static_cast<size_t>(p.EV) * 4);        // range of each read (-1: skipped)
    L.rt = o; o = al16(o + static_cast<size_t>(kR * p.C + 1) * 4);  // reads per (range, token)
    L.misc = o; o = al16(o + (32 + 3 * (kR + 1)) * 4);            // scan totals; range bases, counts
    L.total = o;
    return L;
}

// Record header: per range r (and r = kR for the end), the first entry,
// write, read and version row of the range.
struct RangeHdr {
    int ebase[kR + 1], wbase[kR + 1], rbase[kR + 1], vbase[kR + 1];
};
static_assert(sizeof(RangeHdr) == 4 * 4 * (kR + 1), "RangeHdr: four int arrays, no padding");

template <typename TIn, int EPW>
__global__ __launch_bounds__(kPRT) void plan_range_kernel(ChunkArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const ChunkPlan &P = a.p;
    const int tid = threadIdx.x;
    const int C = P.C, K = a.K;
    const int M = static_cast<int>(a.M);
    const bool hashed = P.HT != 0;
    const int HT = hashed ? P.HT : M;
    const int hsh = 32 - (__ffs(HT) - 1);  // hashed: HT is a power of two
    const uint64_t kdiv = ((uint64_t(1) << 32) + K - 1) / K;
    const RPlanLds L = rplan_lds(P, a.M);
    int *tkey = reinterpret_cast<int *>(smem + L.key);
    int *tcf = reinterpret_cast<int *>(smem + L.cf);
    int *ewo = reinterpret_cast<int *>(smem + L.wo);
    int *bk = reinterpret_cast<int *>(smem + L.bk);
    int *sk = reinterpret_cast<int *>(smem + L.sk);
    int *sa = reinterpret_cast<int *>(smem + L.sa);
    int *need = reinterpret_cast<int *>(smem + L.need);
    int *rg = reinterpret_cast<int *>(smem + L.rg);
    int *rt = reinterpret_cast<int *>(smem + L.rt);
    int *wtot = reinterpret_cast<int *>(smem + L.misc);
    int *rs0 = wtot + 32;       // first entry id of range r, r <= kR
    int *vb = rs0 + (kR + 1);   // first version row of range r, r <= kR

    // A workgroup plans (unit, chunk) items wi = blockIdx.x, + gridDim.x,
    // ...; the heads of one (sequence, chunk) are neighbouring items (their
    // addresses share cache lines).  The next item's events are requested
    // while this one is planned.
    const int64_t nwork = static_cast<int64_t>(a.B) * a.H * P.n_chunks;
    // this thread's events of an item, e = tid + j * kPRT (index t * K + k
    // within the chunk), writes and reads alike
    struct Events {
        int ws[EPW], rs[EPW];
        float wt[EPW], rtw[EPW];
        TIn eg[EPW];  // (as stored: a conversion here would wait for the load)
    };
    auto load_events = [&](int64_t wi, Events &ev) {
        const int h = static_cast<int>(wi % a.H);
        const int chunk = static_cast<int>((wi / a.H) % P.n_chunks);
        const int b = static_cast<int>(wi / a.H / P.n_chunks);
        const int unit = b * a.H + h;
        const int t0 = chunk * C, nev = min(C, a.T - t0) * K;
        const int64_t th0 = static_cast<int64_t>(b) * a.T * a.H + h;
        const TIn *gam = static_cast<const TIn *>(a.gamma) + static_cast<int64_t>(b) * a.T * a.ld_gamma + h;
#pragma unroll
        for (int j = 0; j < EPW; ++j) {
            const int e = tid + j * kPRT;
            ev.ws[j] = -1;
            ev.rs[j] = -1;
            if (e < nev) {
                const int t = div_by(e, kdiv), k = e - t * K;
                const int64_t th = th0 + static_cast<int64_t>(t0 + t) * a.H;
                const int64_t ai = (a.addr_unit_major ? static_cast<int64_t>(unit) * a.T + t0 + t : th) * K + k;
                ev.ws[j] = a.w_idx[ai];
                ev.wt[j] = a.w_wt[ai];
                ev.rs[j] = a.r_idx[ai];
                ev.rtw[j] = a.r_wt[ai];
                ev.eg[j] = gam[static_cast<int64_t>(t0 + t) * a.ld_gamma];
            }
        }
    };
    Events cur, nxt;
    if (static_cast<int64_t>(blockIdx.x) < nwork) load_events(blockIdx.x, cur);
    // (the first item's events are waited for here: otherwise every item's
    // first use of its events would also wait for the next item's loads)
    wait_vm_loads();
    for (int64_t wi = blockIdx.x; wi < nwork; wi += gridDim.x) {
    if (wi + gridDim.x < nwork) load_events(wi + gridDim.x, nxt);
    // (the thread index is taken afresh per item, so that the compiler does
    // not keep every address derived from it live across the loop)
    int tid = threadIdx.x;
    __asm__ volatile("" : "+v"(tid));
    const int h = static_cast<int>(wi % a.H);
    const int chunk = static_cast<int>((wi / a.H) % P.n_chunks);
    const int b = static_cast<int>(wi / a.H / P.n_chunks);
    const int unit = b * a.H + h;
    const int t0 = chunk * C, Cc = min(C, a.T - t0);
    const int nev = Cc * K;
    (void)t0;

    unsigned char *rec = a.plan + (static_cast<int64_t>(unit) * P.n_chunks + chunk) * P.rec_bytes;
    RangeHdr *hdr = reinterpret_cast<RangeHdr *>(rec);
    int *rtoff = reinterpret_cast<int *>(rec + P.o_rt);       // [kR][C + 1], per range
    int *ent_slot = reinterpret_cast<int *>(rec + P.o_ent);  // per entry: slot, write offset,
    int *ent_wo = ent_slot + P.ENTA;                          // writes | (version-0 row + 1) << 16
    int *ent_nx = ent_wo + P.ENTA;
    int *wtv = reinterpret_cast<int *>(rec + P.o_wtv);
    float *ww = reinterpret_cast<float *>(rec + P.o_ww);
    float *wa = reinterpret_cast<float *>(rec + P.o_wa);
    int *rv = reinterpret_cast<int *>(rec + P.o_rv);
    float *rr = reinterpret_cast<float *>(rec + P.o_rr);
    const int (&ws)[EPW] = cur.ws;
    const int (&rs)[EPW] = cur.rs;
    const float (&wt)[EPW] = cur.wt;
    const float (&rtw)[EPW] = cur.rtw;
    const TIn (&eg)[EPW] = cur.eg;

    for (int i = tid; i < HT; i += kPRT) {
        tcf[i] = 0;
        if (hashed) tkey[i] = -1;
    }
    for (int i = tid; i <= kR * C; i += kPRT) rt[i] = 0;
    lds_barrier();

    // ---- 1. every event finds its slot's entry; writes count, reads flag
    //         and count per (range, token).  A zero-weight write changes
    //         nothing (alpha = 1, lambda = 0); a slot outside [0, M)
    //         (caller-given addresses) is skipped, and a skipped read
    //         contributes nothing.
    auto entry_of = [&](int s) -> int {
        if (!hashed) return s;
        // double hashing: an odd step (from a second multiplicative hash)
        // visits every position of the power-of-two table, and probe runs
        // stay short at the table's load of up to 3/4, where linear probing
        // builds long clusters (a wave waits for its longest probe run)
        uint32_t hp = (static_cast<uint32_t>(s) * 2654435761u) >> hsh;
        const uint32_t step = ((static_cast<uint32_t>(s) * 0x85ebca6bu) >> hsh) | 1u;
        for (;;) {
            const int old = atomicCAS(&tkey[hp], -1, s);
            if (old == -1 || old == s) return static_cast<int>(hp);
            hp = (hp + step) & static_cast<uint32_t>(HT - 1);
        }
    };
    int wpos[EPW], ar[EPW], rpos[EPW];
    float al[EPW];
#pragma unroll
    for (int j = 0; j < EPW; ++j) {
        const int e = tid + j * kPRT;
        wpos[j] = -1;
        rpos[j] = -1;
        ar[j] = 0;
        al[j] = 0.f;
        if (static_cast<uint32_t>(ws[j]) < static_cast<uint32_t>(M) && wt[j] > 0.f) {
            wpos[j] = entry_of(ws[j]);
            ar[j] = atomicAdd(&tcf[wpos[j]], 1) & (kReadFlag - 1);
            al[j] = retention_fast(wt[j], expf(to_f32(eg[j])));
        }
        if (static_cast<uint32_t>(rs[j]) < static_cast<uint32_t>(M)) {
            rpos[j] = entry_of(rs[j]);
            atomicOr(&tcf[rpos[j]], kReadFlag);
            atomicAdd(&rt[range_of(rs[j]) * C + div_by(e, kdiv)], 1);
            rg[e] = range_of(rs[j]);
        } else if (e < nev) {
            rg[e] = -1;
        }
    }
    lds_barrier();

    // ---- 2. entry ids, range by range and, within a range, written slots
    //         before read-only ones (so that the scan's waves take either
    //         write chains or none): one scan of the (range, thread) counts
    //         of touched table positions, written and read-only counts packed
    //         in the low and high 16 bits.  Thread tid takes positions tid,
    //         tid + kPRT, ... (neighbouring lanes on neighbouring words) and
    //         numbers its entries in that order.  The entry's slot goes to
    //         the record; its write count to ewo.
    int *rsum = vb + (kR + 1);  // packed counts of the ranges before r, r <= kR
    // this thread's table positions tid + q kPRT (at most kPlanSteps), read
    // by each pass below with every load out before the first use
    const int nstep = (HT + kPRT - 1) / kPRT;
    auto read_positions = [&](int (&pc)[kPlanSteps], int (&pk)[kPlanSteps]) {
#pragma unroll
        for (int q = 0; q < kPlanSteps; ++q) {
            const int p = tid + q * kPRT;
            const bool in = q < nstep && p < HT;
            pc[q] = in ? tcf[p] : 0;
            pk[q] = in && hashed ? tkey[p] : p;
        }
    };
    {
        int pc[kPlanSteps], pk[kPlanSteps];
        read_positions(pc, pk);
        int cnt[kR];
#pragma unroll
        for (int r = 0; r < kR; ++r) cnt[r] = 0;
#pragma unroll
        for (int q = 0; q < kPlanSteps; ++q) {
            const int c = pc[q];
            if (c) {
                const int sr = range_of(pk[q]);
                const int inc = (c & (kReadFlag - 1)) ? 1 : 0x10000;
#pragma unroll
                for (int r = 0; r < kR; ++r) cnt[r] += sr == r ? inc : 0;
            }
        }
#pragma unroll
        for (int r = 0; r < kR; ++r) need[r * kPRT + tid] = cnt[r];
    }
    lds_barrier();
    const int ptot = block_scan_striped<kPRT>(need, kR * kPRT, wtot);
    lds_barrier();
    if (tid <= kR) rsum[tid] = tid < kR ? need[tid * kPRT] : ptot;
    lds_barrier();
    const int nt = (ptot & 0xffff) + (ptot >> 16);
    {
        int nx0[kR], nx1[kR];  // this thread's next written / read-only id per range
#pragma unroll
        for (int r = 0; r < kR; ++r) {
            const int pr = rsum[r], pn = rsum[r + 1], mine = need[r * kPRT + tid];
            const int base = (pr & 0xffff) + (pr >> 16);          // entries of earlier ranges
            const int wr = (pn & 0xffff) - (pr & 0xffff);          // written entries of range r
            nx0[r] = base + (mine & 0xffff) - (pr & 0xffff);
            nx1[r] = base + wr + (mine >> 16) - (pr >> 16);
        }
        int pc[kPlanSteps], pk[kPlanSteps];
        read_positions(pc, pk);
#pragma unroll
        for (int q = 0; q < kPlanSteps; ++q) {
            const int p = tid + q * kPRT;
            if (q >= nstep || p >= HT) break;
            const int c = pc[q];
            const int slot = pk[q];
            const int sr = range_of(slot);
            const bool written = (c & (kReadFlag - 1)) != 0;
            // the range's next written or read-only id, by selects (no
            // branch per range)
            int eid = -1;
#pragma unroll
            for (int r = 0; r < kR; ++r) {
                const bool m0 = c != 0 && sr == r && written;
                const bool m1 = c != 0 && sr == r && !written;
                eid = m0 ? nx0[r] : m1 ? nx1[r] : eid;
                nx0[r] += m0 ? 1 : 0;
                nx1[r] += m1 ? 1 : 0;
            }
            if (c) {
                ewo[eid] = c & (kReadFlag - 1);
                ent_slot[eid] = slot;
            }
            tcf[p] = eid;  // -1: untouched
        }
        if (tid <= kR) rs0[tid] = (rsum[tid] & 0xffff) + (rsum[tid] >> 16);
    }
    lds_barrier();
    // write offsets in entry order (range by range)
    const int nwt = block_scan_striped<kPRT>(ewo, nt, wtot);
    lds_barrier();
    if (tid == 0) ewo[nt] = nwt;
    for (int i = tid; i <= nt + nwt; i += kPRT) need[i] = 0;
    lds_barrier();

    // ---- 3. writes into their entries' buckets, arrival order ...
#pragma unroll
    for (int j = 0; j < EPW; ++j)
        if (wpos[j] >= 0) bk[ewo[tcf[wpos[j]]] + ar[j]] = tid + j * kPRT;
    lds_barrier();
    // ... then causal order: a write's rank is the number of the bucket's
    // writes with a smaller event index (one write per slot and token)
    int spos[EPW];
#pragma unroll
    for (int j = 0; j < EPW; ++j) {
        spos[j] = -1;
        if (wpos[j] >= 0) {
            const int e = tid + j * kPRT;
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
            const int tr = div_by(tid + j * kPRT, kdiv);
            int c = 0;
            while (c < n && div_by(sk[wo + c], kdiv) <= tr) ++c;
            gv[j] = wo + eid + c;
            need[gv[j]] = 1;
        }
    }
    lds_barrier();

    // ---- 5. version rows: exclusive scan of the flags over nt + nwt + 1
    //         positions (range by range, as the entries); version g has a row
    //         iff need[g + 1] > need[g].  Range r's rows start at vb[r]; the
    //         scan gives reads, per (range, token), their list offsets.
    const int nver = block_scan_striped<kPRT>(need, nt + nwt + 1, wtot);
    lds_barrier();
    const int nrd = block_scan_striped<kPRT>(rt, kR * C, wtot);
    lds_barrier();
    if (tid <= kR) {
        const int e0 = rs0[tid];
        vb[tid] = tid < kR ? need[ewo[e0] + e0] : nver;
    }
    if (tid == 0) rt[kR * C] = nrd;
    lds_barrier();
    // the next item's events have long arrived: take them now, before this
    // item's record stores go out (later, the wait would cover those stores)
    wait_vm_loads();

    // ---- 6. the record: header, per-range token offsets of the reads,
    //         entries, then writes and reads staged in LDS in list order and
    //         stored with consecutive lanes on consecutive words (non-temporal:
    //         the scan reads the record once, long after)
    if (tid == 0) {
        RangeHdr hd;
        for (int r = 0; r <= kR; ++r) {
            hd.ebase[r] = rs0[r];
            hd.wbase[r] = ewo[rs0[r]];
            hd.rbase[r] = r < kR ? rt[r * C] : nrd;
            hd.vbase[r] = vb[r];
        }
        *hdr = hd;
    }
    for (int i = tid; i < kR * (C + 1); i += kPRT) {
        const int r = i / (C + 1), t = i - r * (C + 1);
        __builtin_nontemporal_store(rt[r * C + t] - rt[r * C], rtoff + i);  // t == C: the next range's start (or nrd)
    }
    for (int eid = tid; eid < nt; eid += kPRT) {
        int r = 0;
#pragma unroll
        for (int q = 1; q < kR; ++q) r += eid >= rs0[q] ? 1 : 0;
        const int g = ewo[eid] + eid;
        __builtin_nontemporal_store(ewo[eid], ent_wo + eid);
        const int x0 = need[g + 1] > need[g] ? need[g] - vb[r] : -1;
        __builtin_nontemporal_store((ewo[eid + 1] - ewo[eid]) | ((x0 + 1) << 16), ent_nx + eid);
    }
    // reads: list position and (range-local version row, weight).  A read's
    // rank among its token's reads of the same range: where K divides the
    // wave, a token's K reads sit on K aligned lanes of one wave, and the
    // rank is a popcount of the range's ballot below the lane.
    const bool token_in_wave = (kWave % K) == 0;
    int rp[EPW], rvv[EPW];
#pragma unroll
    for (int j = 0; j < EPW; ++j) {
        rp[j] = -1;
        const int e = tid + j * kPRT;
        const int t = div_by(e, kdiv), k = e - t * K;
        const int r = gv[j] >= 0 ? range_of(rs[j]) : -1;
        int rank = 0;
        if (token_in_wave) {
            const int lane = tid & (kWave - 1);
            const uint64_t below = ((uint64_t(1) << lane) - 1) & ~((uint64_t(1) << (lane - k)) - 1);
            uint64_t same = 0;
#pragma unroll
            for (int q = 0; q < kR; ++q) {
                const uint64_t bq = __ballot(r == q);
                same = r == q ? bq : same;
            }
            rank = __popcll(same & below);
        } else if (r >= 0) {
            for (int q = 0; q < k; ++q) rank += rg[t * K + q] == r ? 1 : 0;
        }
        if (r >= 0) {
            rp[j] = rt[r * C + t] + rank;
            rvv[j] = need[gv[j]] - vb[r];
        }
    }
#pragma unroll
    for (int j = 0; j < EPW; ++j) {
        if (spos[j] >= 0) {
            const int e = tid + j * kPRT;
            const int eid = tcf[wpos[j]];
            const int wo = ewo[eid];
            const int g = wo + eid + (spos[j] - wo) + 1;  // version after this write
            const int vr = need[g + 1] > need[g] ? need[g] - vb[range_of(ws[j])] : -1;
            bk[spos[j]] = div_by(e, kdiv) | ((vr + 1) << 10);
            sk[spos[j]] = __float_as_int(wt[j]);
            sa[spos[j]] = __float_as_int(al[j]);
        }
    }
    lds_barrier();
    for (int i = tid; i < nwt; i += kPRT) {
        __builtin_nontemporal_store(bk[i], wtv + i);
        __builtin_nontemporal_store(__int_as_float(sk[i]), ww + i);
        __builtin_nontemporal_store(__int_as_float(sa[i]), wa + i);
    }
    lds_barrier();
#pragma unroll
    for (int j = 0; j < EPW; ++j) {
        if (rp[j] >= 0) {
            bk[rp[j]] = rvv[j];
            sk[rp[j]] = __float_as_int(rtw[j]);
        }
    }
    lds_barrier();
    for (int i = tid; i < nrd; i += kPRT) {
        __builtin_nontemporal_store(bk[i], rv + i);
        __builtin_nontemporal_store(__int_as_float(sk[i]), rr + i);
    }
    // the LDS tables are set up again for the next item
    lds_barrier();
    cur = nxt;
    }
}

// LDS of the scan kernel (byte offsets).
struct RScanLds {
    size_t v, wtv, wwa, rv, rr, rt, ms, ver, total;
};
__host__ __device__ inline RScanLds rscan_lds(const ChunkPlan &p, int d_v, int sbytes, int vbytes) {
    RScanLds L{};
    size_t o = 0;
    L.v = o; o = al16(o + static_cast<size_t>(p.C) * (d_v * vbytes + 16));  // values, rows padded by 16 B
    L.wtv = o; o = al16(o + static_cast<size_t>(p.CAPW) * 4);                // write: token | version row
    L.wwa = o; o = al16(o + static_cast<size_t>(p.CAPW) * 8);                // write: weight, retention
    L.rv = o; o = al16(o + static_cast<size_t>(p.CAPR) * 4);                 // read: version row
    L.rr = o; o = al16(o + static_cast<size_t>(p.CAPR) * 4);                 // read weight
    L.rt = o; o = al16(o + static_cast<size_t>(p.C + 1) * 4);                // reads per token
    L.ms = o; o = al16(o + static_cast<size_t>(p.MSL) * 4);                  // the range's masses
    L.ver = o = (o + 255) & ~size_t(255);
    o += static_cast<size_t>(p.VCAP) * d_v * sbytes;                        // version rows
    L.total = o;
    return L;
}

// Four channels of a version row as fp32 (8 bytes of bf16, 16 of fp32), from
// LDS or from the spill area (Q: the pointer's address-space qualifier).
template <typename Q>
__device__ __forceinline__ void load4q(const Q *p, float (&x)[4], float) {
    const u32x4 u = *p;
    x[0] = __uint_as_float(u.x);
    x[1] = __uint_as_float(u.y);
    x[2] = __uint_as_float(u.z);
    x[3] = __uint_as_float(u.w);
}
template <typename Q>
__device__ __forceinline__ void load4q(const Q *p, float (&x)[4], bf16_t) {
    const u32x2 u = *p;
    x[0] = __uint_as_float(u.x << 16);
    x[1] = __uint_as_float(u.x & 0xffff0000u);
    x[2] = __uint_as_float(u.y << 16);
    x[3] = __uint_as_float(u.y & 0xffff0000u);
}

// Value words of a 16-byte row piece's CP channels (CP * sizeof(TIn) / 4
// words), loaded as they are stored.
template <typename TIn, int NW>
__device__ __forceinline__ void value_words(const TIn *vbuf, int off, uint32_t (&w)[NW]) {
    if constexpr (NW % 4 == 0) {
#pragma unroll
        for (int k = 0; k < NW / 4; ++k) {
            const u32x4 x = reinterpret_cast<const u32x4 *>(vbuf + off)[k];
            w[4 * k] = x.x;
            w[4 * k + 1] = x.y;
            w[4 * k + 2] = x.z;
            w[4 * k + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < NW / 2; ++k) {
            const u32x2 x = reinterpret_cast<const u32x2 *>(vbuf + off)[k];
            w[2 * k] = x.x;
            w[2 * k + 1] = x.y;
        }
    }
}
template <int NW> __device__ __forceinline__ float value_at(const uint32_t (&w)[NW], int q, float) {
    return __uint_as_float(w[q]);
}
template <int NW> __device__ __forceinline__ float value_at(const uint32_t (&w)[NW], int q, bf16_t) {
    return __uint_as_float((q & 1) ? (w[q >> 1] & 0xffff0000u) : (w[q >> 1] << 16));
}

// One write applied to a row piece held as its stored bits:
// x <- x + lambda (v - x), rounded to the storage type.
template <int NW, typename TIn>
__device__ __forceinline__ uint4 apply_piece(const uint4 &xr, float lam, const uint32_t (&vw)[NW], float, TIn) {
    const uint32_t w[4] = {xr.x, xr.y, xr.z, xr.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float x = __uint_as_float(w[k]);
        o[k] = __float_as_uint(fmaf(lam, value_at(vw, k, TIn{}) - x, x));
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}
template <int NW, typename TIn>
__device__ __forceinline__ uint4 apply_piece(const uint4 &xr, float lam, const uint32_t (&vw)[NW], bf16_t, TIn) {
    const uint32_t w[4] = {xr.x, xr.y, xr.z, xr.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float x0 = __uint_as_float(w[k] << 16), x1 = __uint_as_float(w[k] & 0xffff0000u);
        const float y0 = fmaf(lam, value_at(vw, 2 * k, TIn{}) - x0, x0);
        const float y1 = fmaf(lam, value_at(vw, 2 * k + 1, TIn{}) - x1, x1);
        o[k] = static_cast<uint32_t>(bf16_rne(y0).bits) | (static_cast<uint32_t>(bf16_rne(y1).bits) << 16);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// The partial reads' type: fp16 where the state (and so the output) is
// bf16, whose 8 significant bits the 11 of fp16 leave intact; else fp32.
template <typename TS>
using PartialOf = std::conditional_t<std::is_same_v<TS, bf16_t>, _Float16, float>;

// VPT: value elements per thread and chunk (C * d_v / kRT, at most VPT).
template <typename TIn, typename TS, int VPT>
__global__ __launch_bounds__(kRT) void scan_range_kernel(ChunkArgs a) {
    using TP = PartialOf<TS>;
    extern __shared__ __align__(16) unsigned char smem[];
    const ChunkPlan &P = a.p;
    const int tid = threadIdx.x;
    const int units = a.B * a.H;
    int unit, r;
    {
        const int bid = blockIdx.x;
        if (units % 8 == 0) {  // the ranges of one unit on one XCD (they share value rows)
            const int xcd = bid % 8, j = bid / 8;
            unit = (j / kR) * 8 + xcd;
            r = j % kR;
        } else {
            unit = bid / kR;
            r = bid % kR;
        }
    }
    const int b = unit / a.H, h = unit % a.H;
    const int M = static_cast<int>(a.M);
    const int d_v = a.d_v, C = P.C, EV = P.EV;
    const int nchunks = static_cast<int>(P.n_chunks);
    constexpr int CP = 16 / static_cast<int>(sizeof(TS));  // channels per 16-byte piece
    constexpr int VWP = CP * static_cast<int>(sizeof(TIn)) / 4;  // value words per piece
    const int NP = d_v / CP;                                // pieces per row
    // entry of a walk task (task = entry * NP + piece): a shift when NP is a
    // power of two (d_v 64, 128, 256)
    const int lnp = __ffs(NP) - 1;
    const bool np_pow2 = (NP & (NP - 1)) == 0;
    auto entry_of_task = [&](int task) { return np_pow2 ? task >> lnp : task / NP; };
    const int RL = d_v / 4;                                 // read lanes per token
    const int TPP = kRT / RL;                               // tokens per read pass
    constexpr int VPAD = 16 / static_cast<int>(sizeof(TIn));
    const int VROW = d_v + VPAD;                            // padded value row (elements)
    const RScanLds L = rscan_lds(P, d_v, sizeof(TS), sizeof(TIn));
    TIn *vbuf = reinterpret_cast<TIn *>(smem + L.v);
    RN_LDS int *s_wtv = (RN_LDS int *)(smem + L.wtv);
    RN_LDS f32x2 *s_wwa = (RN_LDS f32x2 *)(smem + L.wwa);
    RN_LDS int *s_rv = (RN_LDS int *)(smem + L.rv);
    RN_LDS float *s_rr = (RN_LDS float *)(smem + L.rr);
    RN_LDS float *ms = (RN_LDS float *)(smem + L.ms);  // mass of slot s: ms[s / kR] (MSL > 0)
    const int MSL = P.MSL;
    int *s_rt = reinterpret_cast<int *>(smem + L.rt);
    // version rows in LDS and the spill area in global memory, with their
    // address spaces in the type so that no access to either is generic
    // rows of 16-byte pieces (u32x4) in LDS and in the spill area
    RN_LDS unsigned char *ver = (RN_LDS unsigned char *)(smem + L.ver);
    const int CAPW = P.CAPW, CAPR = P.CAPR, VCAP = P.VCAP;

    TS *S = static_cast<TS *>(a.S) + static_cast<int64_t>(unit) * M * d_v;
    float *mass = a.mass + static_cast<int64_t>(unit) * M;
    RN_GLB unsigned char *spill =
        (RN_GLB unsigned char *)(static_cast<TS *>(a.spill) + (static_cast<int64_t>(unit) * kR + r) * EV * d_v);
    const int rowb = d_v * static_cast<int>(sizeof(TS));  // bytes per version row
    const TIn *v = static_cast<const TIn *>(a.v) + static_cast<int64_t>(b) * a.T * a.ld_v + h * d_v;
    const int64_t th_unit = static_cast<int64_t>(b) * a.T * a.H + h;  // token 0 of the unit
    const unsigned char *plan0 = a.plan + static_cast<int64_t>(unit) * P.n_chunks * P.rec_bytes;
    auto rec_of = [&](int c) { return plan0 + static_cast<int64_t>(c) * P.rec_bytes; };

    // Version row vr: the first VCAP rows in LDS, later ones in the spill
    // area.  The two are separate branches so that each access is a plain
    // LDS or global instruction (a pointer that may be either would be a
    // generic access, which waits for every load in flight).
    auto ver_store = [&](int vr, int c, const uint4 &u) {
        const u32x4 w = {u.x, u.y, u.z, u.w};
        const int off = c * static_cast<int>(sizeof(TS));
        if (vr < VCAP) *reinterpret_cast<RN_LDS u32x4 *>(ver + vr * rowb + off) = w;
        else *reinterpret_cast<RN_GLB u32x4 *>(spill + static_cast<int64_t>(vr) * rowb + off) = w;
    };

    // ---- the pipeline: chunk c + 1's lists, values and entries are loaded
    //      during chunk c's walk, its rows right after chunk c's write-backs
    //      (during chunk c's reads), and headers two chunks ahead
    // (the header's words are kept as loaded and the counts formed where
    // they are used)
    struct Hdr {
        int eb, ee, wb, we, rb, re;
        __device__ int ne() const { return ee - eb; }
        __device__ int nw() const { return we - wb; }
        __device__ int nr() const { return re - rb; }
    };
    // (the header is the same for the whole workgroup and is not written
    // while this kernel runs: scalar loads through the constant address
    // space keep it in scalar registers)
    auto load_header = [&](int c) {
        const RN_CONST int *hd = (const RN_CONST int *)rec_of(c);
        constexpr int E = 0, W = kR + 1, R = 2 * (kR + 1);  // RangeHdr's arrays
        Hdr x;
        x.eb = hd[E + r];
        x.ee = hd[E + r + 1];
        x.wb = hd[W + r];
        x.we = hd[W + r + 1];
        x.rb = hd[R + r];
        x.re = hd[R + r + 1];
        return x;
    };
    int pf_wtv[kLW], pf_rv[kLW], pf_rt = 0;
    float pf_ww[kLW], pf_wa[kLW], pf_rr[kLW];
    // values move as 32-bit words (two bf16 channels, or one fp32 channel):
    // row offsets and d_v are even, so every word is aligned
    constexpr int VE = 4 / static_cast<int>(sizeof(TIn));  // channels per word
    constexpr int VW = (VPT + VE - 1) / VE;                 // words per thread and chunk
    uint32_t pf_v[VW];
    const int vcol = tid % (d_v / VE), vrow0 = tid / (d_v / VE), vstep = kRT / (d_v / VE);
    auto load_values = [&](int c) {
        const int t0 = c * C, Cc = min(C, a.T - t0);
#pragma unroll
        for (int j = 0; j < VW; ++j) {
            const int t = vrow0 + j * vstep;  // word tid + j kRT of the chunk's [C][d_v]
            if (t < C)
                pf_v[j] = reinterpret_cast<const uint32_t *>(v + static_cast<int64_t>(t0 + min(t, Cc - 1)) * a.ld_v)[vcol];
        }
    };
    // the event lists are read once, here: non-temporal loads
    auto load_lists = [&](int c, const Hdr &hd) {
        const unsigned char *rec = rec_of(c);
#pragma unroll
        for (int j = 0; j < kLW; ++j) {
            const int i = tid + j * kRT;
            if (i < min(hd.nw(), CAPW)) {
                pf_wtv[j] = __builtin_nontemporal_load(reinterpret_cast<const int *>(rec + P.o_wtv) + hd.wb + i);
                pf_ww[j] = __builtin_nontemporal_load(reinterpret_cast<const float *>(rec + P.o_ww) + hd.wb + i);
                pf_wa[j] = __builtin_nontemporal_load(reinterpret_cast<const float *>(rec + P.o_wa) + hd.wb + i);
            }
            if (i < min(hd.nr(), CAPR)) {
                pf_rv[j] = __builtin_nontemporal_load(reinterpret_cast<const int *>(rec + P.o_rv) + hd.rb + i);
                pf_rr[j] = __builtin_nontemporal_load(reinterpret_cast<const float *>(rec + P.o_rr) + hd.rb + i);
            }
        }
        if (tid <= C) pf_rt = reinterpret_cast<const int *>(rec + P.o_rt)[r * (C + 1) + tid];
    };
    // entries of walk tasks task0 + tid + j kRT (task = entry * NP + piece):
    // slot, write offset, writes | (version-0 row + 1) << 16
    struct Ent {
        int slot[kPTW], wo[kPTW], nx[kPTW];
    };
    auto load_entries = [&](int c, int task0, const Hdr &hd, Ent &pe) {
        const int *ent = reinterpret_cast<const int *>(rec_of(c) + P.o_ent);
#pragma unroll
        for (int j = 0; j < kPTW; ++j) {
            const int e = entry_of_task(task0 + tid + j * kRT);
            pe.nx[j] = 0;
            if (e < hd.ne()) {
                const int eid = hd.eb + e;
                pe.slot[j] = ent[eid];
                pe.wo[j] = ent[P.ENTA + eid];
                pe.nx[j] = ent[2 * P.ENTA + eid];
            }
        }
    };
    // every row piece and mass of a round at once
    struct Rows {
        uint4 raw[kPTW];
        float m[kPTW];
    };
    // (branch-free row loads: a task past the range's entries loads row 0,
    // so that the loads go out back to back, with no wait between them)
    auto gather = [&](int task0, const Hdr &hd, const Ent &pe, Rows &rw) {
#pragma unroll
        for (int j = 0; j < kPTW; ++j) {
            const int task = task0 + tid + j * kRT;
            const int e = entry_of_task(task), piece = task - e * NP;
            const int slot = e < hd.ne() ? pe.slot[j] : 0;
            rw.raw[j] = *reinterpret_cast<const uint4 *>(S + static_cast<int64_t>(slot) * d_v + piece * CP);
        }
        if (!MSL) {
#pragma unroll
            for (int j = 0; j < kPTW; ++j) {
                const int e = entry_of_task(task0 + tid + j * kRT);
                if (e < hd.ne() && (pe.nx[j] & 0xffff)) rw.m[j] = mass[pe.slot[j]];
            }
        }
    };

    // the range's masses, in LDS for the whole sequence where they fit (they
    // are seen by the first staging barrier)
    for (int i = tid; i < MSL; i += kRT) {
        const int slot = i * kR + r;
        ms[i] = slot < M ? mass[slot] : 0.f;
    }
    Hdr h_cur = load_header(0), h_nxt{};
    Ent pe;
    Rows rw;
    load_values(0);
    load_lists(0, h_cur);
    load_entries(0, 0, h_cur, pe);
    gather(0, h_cur, pe, rw);
    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * C, Cc = min(C, a.T - t0);
        const Hdr hc = h_cur;
        // ---- 1. stage the lists, token offsets and values
#pragma unroll
        for (int j = 0; j < kLW; ++j) {
            const int i = tid + j * kRT;
            if (i < min(hc.nw(), CAPW)) {
                s_wtv[i] = pf_wtv[j];
                s_wwa[i] = f32x2{pf_ww[j], pf_wa[j]};
            }
            if (i < min(hc.nr(), CAPR)) {
                s_rv[i] = pf_rv[j];
                s_rr[i] = pf_rr[j];
            }
        }
        if (tid <= C) s_rt[tid] = pf_rt;
#pragma unroll
        for (int j = 0; j < VW; ++j) {
            const int t = vrow0 + j * vstep;
            if (t < Cc) reinterpret_cast<uint32_t *>(vbuf + t * VROW)[vcol] = pf_v[j];
        }
        lds_barrier();
        const unsigned char *rec = rec_of(c);
        const RN_GLB int *g_wtv = (const RN_GLB int *)(rec + P.o_wtv) + hc.wb;
        const RN_GLB float *g_ww = (const RN_GLB float *)(rec + P.o_ww) + hc.wb;
        const RN_GLB float *g_wa = (const RN_GLB float *)(rec + P.o_wa) + hc.wb;
        const RN_GLB int *g_rv = (const RN_GLB int *)(rec + P.o_rv) + hc.rb;
        const RN_GLB float *g_rr = (const RN_GLB float *)(rec + P.o_rr) + hc.rb;
        // ---- 2. chunk c + 1's header goes out now
        if (c + 1 < nchunks) h_nxt = load_header(c + 1);
        // ---- 3. walk the range's touched slots, kRT * kPTW row pieces per
        //         round: gather the round's pieces and masses at once, apply
        //         the writes, store the versions reads see, write back
        for (int task0 = 0; task0 < hc.ne() * NP; task0 += kRT * kPTW) {
            if (task0 > 0) {  // (the first round's rows were gathered during the last reads)
                load_entries(c, task0, hc, pe);
                gather(task0, hc, pe, rw);
            }
            // pairs of the lane's pieces advance together, one write each
            // per step, so that their loads overlap (each piece's writes
            // stay in order).  A piece stays in its stored bits (rw.raw).
#pragma unroll
            for (int jp = 0; jp < kPTW; jp += kIL) {
                float m[kIL];
                int n[kIL], i0[kIL], pc[kIL], nmax = 0;
#pragma unroll
                for (int u = 0; u < kIL; ++u) {
                    const int j = jp + u;
                    const int task = task0 + tid + j * kRT;
                    const int e = entry_of_task(task);
                    const bool live = e < hc.ne();
                    pc[u] = (task - e * NP) * CP;  // the piece's first channel
                    const int x0 = live ? (pe.nx[j] >> 16) - 1 : -1;
                    if (x0 >= 0) ver_store(x0, pc[u], rw.raw[j]);
                    n[u] = live ? pe.nx[j] & 0xffff : 0;
                    i0[u] = pe.wo[j] - hc.wb;  // range-local write list index
                    m[u] = 0.f;
                    if (n[u]) m[u] = MSL ? ms[pe.slot[j] / kR] : rw.m[j];
                    nmax = max(nmax, n[u]);
                }
                for (int st = 0; st < nmax; ++st) {
                    int tv[kIL];
                    f32x2 wa[kIL];
                    uint32_t vw[kIL][VWP];
#pragma unroll
                    for (int u = 0; u < kIL; ++u) {
                        // a piece with no write left reads write 0 and keeps its row
                        const int i = st < n[u] ? i0[u] + st : 0;
                        if (i < CAPW) {
                            tv[u] = s_wtv[i];
                            wa[u] = s_wwa[i];
                        } else {
                            tv[u] = g_wtv[i];
                            wa[u] = f32x2{g_ww[i], g_wa[i]};
                            wait_vm_loads();
                        }
                    }
#pragma unroll
                    for (int u = 0; u < kIL; ++u) value_words(vbuf, (tv[u] & 1023) * VROW + pc[u], vw[u]);
#pragma unroll
                    for (int u = 0; u < kIL; ++u) {
                        if (st >= n[u]) continue;
                        const int j = jp + u;
                        const int vr = (tv[u] >> 10) - 1;
                        m[u] = fmaf(wa[u].y, m[u], wa[u].x);
                        const float lam = wa[u].x * __builtin_amdgcn_rcpf(m[u] + a.eps_gsu);
                        rw.raw[j] = apply_piece(rw.raw[j], lam, vw[u], TS{}, TIn{});
                        if (vr >= 0) ver_store(vr, pc[u], rw.raw[j]);
                    }
                }
#pragma unroll
                for (int u = 0; u < kIL; ++u) {
                    const int j = jp + u;
                    if (n[u] == 0) continue;
                    *reinterpret_cast<uint4 *>(S + static_cast<int64_t>(pe.slot[j]) * d_v + pc[u]) = rw.raw[j];
                    if (pc[u] == 0) {
                        if (MSL) ms[pe.slot[j] / kR] = m[u];
                        else mass[pe.slot[j]] = m[u];
                    }
                }
            }
        }
        // ---- 4. chunk c + 1's values, lists and entries go out now (not
        //         before the walk: a write step waits for every load in
        //         flight, so the walk runs with none)
        if (c + 1 < nchunks) {
            load_values(c + 1);
            load_lists(c + 1, h_nxt);
            load_entries(c + 1, 0, h_nxt, pe);
        }
        // row write-backs and spilled versions visible to this workgroup
        __syncthreads();
        // ... and chunk c + 1's first rows, which may be rows chunk c just
        // wrote: they land during the reads
        if (c + 1 < nchunks) gather(0, h_nxt, pe, rw);
        // ---- 5. reads: lane q of a token sums channels [4q, 4q + 4) over the
        //         range's reads of that token in address order; the partial
        //         (zero if none) goes to the workspace.  A token with more
        //         than kHeavy reads here (a token's reads often share their
        //         low digits, and so a range) is summed by a whole wave
        //         instead: its lane groups take every G-th read and are added
        //         in a fixed order, so that no group waits on a long list.
        // (a read list or version row beyond LDS is loaded from global
        // memory and waited for in its own branch, so that the common path
        // does not wait for the next chunk's row gathers)
        {
            constexpr int kHeavy = 8;
            const int G = kWave / RL;  // lane groups of a wave
            auto entry = [&](int j, int &vr, float &rho) {
                if (j < CAPR) {
                    vr = s_rv[j];
                    rho = s_rr[j];
                } else {
                    vr = g_rv[j];
                    rho = g_rr[j];
                    wait_vm_loads();
                }
            };
            auto row = [&](int vr, int q, float (&x)[4]) {
                const int off = 4 * q * static_cast<int>(sizeof(TS));
                if (vr < VCAP) {
                    load4q(reinterpret_cast<const RN_LDS VecOf<TS> *>(ver + vr * rowb + off), x, TS{});
                } else {
                    load4q(reinterpret_cast<const RN_GLB VecOf<TS> *>(spill + static_cast<int64_t>(vr) * rowb + off),
                           x, TS{});
                    wait_vm_loads();
                }
            };
            auto store = [&](int t, int q, const float (&acc)[4]) {
                const int64_t th = th_unit + static_cast<int64_t>(t0 + t) * a.H;
                TP *dst = reinterpret_cast<TP *>(a.partial) + (th * kR + r) * d_v + 4 * q;
                // (read once, by the gate: non-temporal)
                if constexpr (std::is_same_v<TP, float>) {
                    typedef float pf32x4 __attribute__((ext_vector_type(4)));
                    pf32x4 v;
                    v.x = acc[0];
                    v.y = acc[1];
                    v.z = acc[2];
                    v.w = acc[3];
                    __builtin_nontemporal_store(v, reinterpret_cast<pf32x4 *>(dst));
                } else {
                    const _Float16 hv[4] = {static_cast<_Float16>(acc[0]), static_cast<_Float16>(acc[1]),
                                            static_cast<_Float16>(acc[2]), static_cast<_Float16>(acc[3])};
                    const uint2 u = __builtin_bit_cast(uint2, hv);
                    u32x2 v;
                    v.x = u.x;
                    v.y = u.y;
                    __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(dst));
                }
            };
            for (int tb = 0; tb < Cc; tb += TPP) {
                const int t = tb + tid / RL, q = tid % RL;
                if (t < Cc) {
                    const int j0 = s_rt[t], j1 = s_rt[t + 1];
                    if (G > 1 && j1 - j0 > kHeavy) continue;  // summed below
                    float acc[4] = {0.f, 0.f, 0.f, 0.f};
                    // two reads per step: their loads overlap; the sum keeps
                    // address order
                    int j = j0;
                    for (; j + 1 < j1; j += 2) {
                        int vr0, vr1;
                        float rho0, rho1, x0[4], x1[4];
                        entry(j, vr0, rho0);
                        entry(j + 1, vr1, rho1);
                        row(vr0, q, x0);
                        row(vr1, q, x1);
#pragma unroll
                        for (int u = 0; u < 4; ++u) acc[u] = fmaf(rho0, x0[u], acc[u]);
#pragma unroll
                        for (int u = 0; u < 4; ++u) acc[u] = fmaf(rho1, x1[u], acc[u]);
                    }
                    if (j < j1) {
                        int vr;
                        float rho, x[4];
                        entry(j, vr, rho);
                        row(vr, q, x);
#pragma unroll
                        for (int u = 0; u < 4; ++u) acc[u] = fmaf(rho, x[u], acc[u]);
                    }
                    store(t, q, acc);
                }
            }
            if (G > 1) {
                // heavy tokens in token order, the h-th to wave h mod (waves)
                const int lane = tid & (kWave - 1), wave = tid / kWave;
                const int gq = lane / RL, q = lane % RL;
                int h = 0;
                for (int tw = 0; tw < Cc; tw += kWave) {
                    const int tt = tw + lane;
                    uint64_t bits = __ballot(tt < Cc && s_rt[tt + 1] - s_rt[tt] > kHeavy);
                    while (bits) {
                        const int t = tw + __builtin_ctzll(bits);
                        bits &= bits - 1;
                        if (h++ % (kRT / kWave) != wave) continue;
                        float acc[4] = {0.f, 0.f, 0.f, 0.f};
                        const int j1 = s_rt[t + 1];
                        int j = s_rt[t] + gq;
                        for (; j + G < j1; j += 2 * G) {
                            int vr0, vr1;
                            float rho0, rho1, x0[4], x1[4];
                            entry(j, vr0, rho0);
                            entry(j + G, vr1, rho1);
                            row(vr0, q, x0);
                            row(vr1, q, x1);
#pragma unroll
                            for (int u = 0; u < 4; ++u) acc[u] = fmaf(rho0, x0[u], acc[u]);
#pragma unroll
                            for (int u = 0; u < 4; ++u) acc[u] = fmaf(rho1, x1[u], acc[u]);
                        }
                        if (j < j1) {
                            int vr;
                            float rho, x[4];
                            entry(j, vr, rho);
                            row(vr, q, x);
#pragma unroll
                            for (int u = 0; u < 4; ++u) acc[u] = fmaf(rho, x[u], acc[u]);
                        }
                        // the groups' sums, pairwise in a fixed order (each
                        // addition is commutative, so every lane holds the
                        // same bits)
                        for (int o = RL; o < kWave; o <<= 1) {
#pragma unroll
                            for (int u = 0; u < 4; ++u) acc[u] += __shfl_xor(acc[u], o, kWave);
                        }
                        if (gq == 0) store(t, q, acc);
                    }
                }
            }
        }
        // LDS is restaged and the spill area rewritten by the next chunk
        // (every load of this chunk's reads has been consumed by now)
        lds_barrier();
        h_cur = h_nxt;
    }
    for (int i = tid; i < MSL; i += kRT) {
        const int slot = i * kR + r;
        if (slot < M) mass[slot] = ms[i];
    }
}

// Four consecutive partial-read channels as fp32 (8 bytes of fp16, 16 of
// fp32), and four outputs stored at once; both are touched once, so the
// accesses are non-temporal.
__device__ __forceinline__ void load4p(const _Float16 *p, float (&x)[4]) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
    const uint2 u = make_uint2(v.x, v.y);
    const _Float16 *h = reinterpret_cast<const _Float16 *>(&u);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = static_cast<float>(h[i]);
}
typedef float ntf32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void load4p(const float *p, float (&x)[4]) {
    const ntf32x4 f = __builtin_nontemporal_load(reinterpret_cast<const ntf32x4 *>(p));
    x[0] = f.x;
    x[1] = f.y;
    x[2] = f.z;
    x[3] = f.w;
}
__device__ __forceinline__ void store4(float *p, const float (&x)[4]) {
    ntf32x4 f;
    f.x = x[0]; f.y = x[1]; f.z = x[2]; f.w = x[3];
    __builtin_nontemporal_store(f, reinterpret_cast<ntf32x4 *>(p));
}
__device__ __forceinline__ void store4(bf16_t *p, const float (&x)[4]) {
    const uint32_t w0 = static_cast<uint32_t>(bf16_rne(x[0]).bits) | (static_cast<uint32_t>(bf16_rne(x[1]).bits) << 16);
    const uint32_t w1 = static_cast<uint32_t>(bf16_rne(x[2]).bits) | (static_cast<uint32_t>(bf16_rne(x[3]).bits) << 16);
    u32x2 v;
    v.x = w0; v.y = w1;
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(p));
}

// out = r / sqrt(mean(r^2) + eps) * omega * sigmoid(g) with r the sum of the
// kRanges partials in range order.  A token-head takes d_v / 4 lanes of a
// group of G (a power of two), four consecutive channels per lane, so that
// every partial is read in 8- or 16-byte pieces; 64 / G token-heads per wave.
template <typename TIn, typename TO, typename TP, int G>
__global__ __launch_bounds__(256) void gate_partials_kernel(const TP *__restrict__ partial,
                                                            const TIn *__restrict__ g, int H,
                                                            int64_t ld_g,
                                                            const float *__restrict__ norm_w,
                                                            TO *__restrict__ out, int64_t n, int d_v,
                                                            float eps) {
    const int lane = threadIdx.x % kWave;
    const int64_t th = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / kWave * (kWave / G) + lane / G;
    const int q = lane % G, c = 4 * q;
    const bool act = th < n && c < d_v;
    float rv[4] = {0.f, 0.f, 0.f, 0.f};
    float ss = 0.f;
    if (act) {
        const TP *pp = partial + th * kR * d_v + c;
#pragma unroll
        for (int r = 0; r < kR; ++r) {
            float x[4];
            load4p(pp + r * d_v, x);
#pragma unroll
            for (int i = 0; i < 4; ++i) rv[i] += x[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) ss = fmaf(rv[i], rv[i], ss);
    }
    // (every lane takes part in the group's sum)
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, kWave);
    if (!act) return;
    const float den = ss / static_cast<float>(d_v) + eps;
    const float inv = den > 0.f ? 1.0f / sqrtf(den) : 0.f;  // zero read, eps 0
    const TIn *gp = g + (th / H) * ld_g + (th % H) * d_v + c;
    float o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float om = norm_w ? norm_w[c + i] : 1.0f;
        o[i] = rv[i] * inv * om * sigmoid(to_f32(gp[i]));
    }
    store4(out + th * d_v + c, o);
}

template <typename T> struct TypeTag { using type = T; };

template <typename K>
hipError_t set_lds(K kern, size_t lds) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                               hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
}

template <typename TIn, typename TS>
hipError_t launch_ranges_typed(const ChunkArgs &a, hipStream_t st) {
    const ChunkPlan &P = a.p;
    const int64_t units = static_cast<int64_t>(a.B) * a.H;
    auto pk = P.EV <= 2048 ? plan_range_kernel<TIn, 2048 / kPRT> : plan_range_kernel<TIn, 3072 / kPRT>;
    hipError_t e = set_lds(pk, P.lds_plan);
    if (e != hipSuccess) return e;
    // as many plan workgroups as fit the chip at once; each loops over items
    int dev = 0, ncu = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    const int64_t per_cu = std::max<int64_t>(1, static_cast<int64_t>(kChunkLdsLimit / std::max<size_t>(P.lds_plan, 1)));
    const int64_t nwork = units * P.n_chunks;
    const int64_t grid = std::min<int64_t>(nwork, std::max<int64_t>(1, ncu) * per_cu);
    hipLaunchKernelGGL(pk, dim3(static_cast<unsigned>(grid)), dim3(kPRT), P.lds_plan, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int vpt = (P.C * a.d_v + kRT - 1) / kRT;
    auto sk = vpt <= 4 ? scan_range_kernel<TIn, TS, 4>
            : vpt <= 6 ? scan_range_kernel<TIn, TS, 6>
            : vpt <= 8 ? scan_range_kernel<TIn, TS, 8> : scan_range_kernel<TIn, TS, 16>;
    if ((e = set_lds(sk, P.lds_scan)) != hipSuccess) return e;
    hipLaunchKernelGGL(sk, dim3(static_cast<unsigned>(units * kR)), dim3(kRT), P.lds_scan, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t n = units * a.T;
    using TP = PartialOf<TS>;
    const TP *part = reinterpret_cast<const TP *>(a.partial);
    // a token-head's lanes: d_v / 4, in a group of G (d_v is 64 ... 256)
    auto gate = [&](auto gt, auto out_t, void *o) {
        constexpr int G = decltype(gt)::value;
        using TO = typename decltype(out_t)::type;
        const int64_t waves = (n + kWave / G - 1) / (kWave / G);
        hipLaunchKernelGGL((gate_partials_kernel<TIn, TO, TP, G>), dim3(static_cast<unsigned>((waves * kWave + 255) / 256)),
                           dim3(256), 0, st, part, static_cast<const TIn *>(a.g), a.H, a.ld_g, a.norm_w,
                           static_cast<TO *>(o), n, a.d_v, a.eps_norm);
    };
    auto gate_out = [&](auto out_t, void *o) {
        if (a.d_v <= 64) gate(std::integral_constant<int, 16>{}, out_t, o);
        else if (a.d_v <= 128) gate(std::integral_constant<int, 32>{}, out_t, o);
        else gate(std::integral_constant<int, 64>{}, out_t, o);
    };
    if (a.out_bf16) gate_out(TypeTag<bf16_t>{}, a.out_bf16);
    else gate_out(TypeTag<TS>{}, a.out);
    return hipGetLastError();
}

}  // namespace

ChunkPlan plan_ranges(int64_t M, int K, int d_v, int B, int T, int H, bool in_bf16, bool state_bf16) {
    ChunkPlan p{};
    p.ok = false;
    const int sbytes = state_bf16 ? 2 : 4;
    const int vbytes = in_bf16 ? 2 : 4;
    const int64_t units = static_cast<int64_t>(B) * H;
    // plan entries pack the token in 10 bits; rows are whole 16-byte pieces
    if (T < 32 || units == 0 || K > 63 || M > (int64_t(1) << 22) || M < kR) return p;
    // value rows and read lanes tile a workgroup: d_v divides kRT
    if (d_v % 64 || d_v > 256 || kRT % d_v) return p;
    p.resident = false;
    ChunkPlan best{};
    best.ok = false;
    for (int C = 512; C >= 32; C -= 32) {
        const int EV = C * K;
        if (EV > kMaxEVHbm || static_cast<int64_t>(C) * d_v > 16 * kRT || C + 1 > kRT) continue;
        ChunkPlan q = p;
        q.C = C;
        q.EV = EV;
        q.CG = d_v;
        q.ncg = 1;
        q.ENT = static_cast<int>(std::min<int64_t>(M, 2 * EV));
        q.HT = 0;
        if (M > 4096) {  // hash table at most 3/4 full
            int ht = 1;
            while (ht * 3 < 2 * EV * 4) ht *= 2;
            q.HT = ht;
        }
        if ((q.HT ? q.HT : M) > kPlanSteps * kPRT) continue;  // (not reached: EV <= 3072, M <= 4096)
        q.CAPW = q.CAPR = std::min(EV, kLW * kRT);
        q.VCAP = 0;
        // the range's masses stay in LDS where they take at most 32 KiB
        q.MSL = (M + kR - 1) / kR * 4 <= 32 * 1024 ? static_cast<int>((M + kR - 1) / kR) : 0;
        q.lds_plan = rplan_lds(q, M).total;
        const size_t fixed = rscan_lds(q, d_v, sbytes, vbytes).total;
        if (q.lds_plan > kChunkLdsLimit || fixed > kChunkLdsLimit) continue;
        q.VCAP = static_cast<int>(std::min<size_t>(EV, (kChunkLdsLimit - fixed) / (static_cast<size_t>(d_v) * sbytes)));
        q.lds_scan = rscan_lds(q, d_v, sbytes, vbytes).total;
        q.n_chunks = (T + C - 1) / C;
        q.ENTA = (q.ENT + 63) & ~63;
        size_t o = al256(sizeof(RangeHdr));
        q.o_rt = o; o += al256(static_cast<size_t>(kR) * (C + 1) * 4);
        q.o_ent = o; o += al256(static_cast<size_t>(q.ENTA) * 12);
        q.o_map = q.o_hl = o;
        q.o_wtv = o; o += al256(static_cast<size_t>(EV) * 4);
        q.o_ww = o; o += al256(static_cast<size_t>(EV) * 4);
        q.o_wa = o; o += al256(static_cast<size_t>(EV) * 4);
        q.o_rv = o; o += al256(static_cast<size_t>(EV) * 4);
        q.o_rr = o; o += al256(static_cast<size_t>(EV) * 4);
        q.rec_bytes = o;
        const size_t n = static_cast<size_t>(units) * T;
        q.ws_rbuf = q.ws_sumsq = q.ws_mass = 0;
        q.ws_plan = al256(static_cast<size_t>(units) * q.n_chunks * q.rec_bytes);
        q.ws_partial = al256(n * kR * d_v * (state_bf16 ? 2 : 4));  // fp16 or fp32 partials
        q.ws_spill = al256(static_cast<size_t>(units) * kR * EV * d_v * sbytes);
        q.ok = true;
        // the longest chunk whose typical versions per range (2 EV / kR)
        // stay in LDS; else the longest that fits at all
        if (!best.ok) best = q;
        if (q.VCAP >= std::min(EV, 3 * EV / (2 * kR))) return q;
    }
    return best;
}

hipError_t launch_scan_ranges(const ChunkArgs &args, hipStream_t st) {
    if (static_cast<int64_t>(args.B) * args.H * args.T == 0) return hipSuccess;
    if (!args.p.ok || args.p.resident) return hipErrorInvalidValue;
    ChunkArgs a = args;
    if (!a.ld_v) a.ld_v = static_cast<int64_t>(a.H) * a.d_v;
    if (!a.ld_g) a.ld_g = static_cast<int64_t>(a.H) * a.d_v;
    if (!a.ld_gamma) a.ld_gamma = a.H;
    if (a.in_bf16)
        return a.state_bf16 ? launch_ranges_typed<bf16_t, bf16_t>(a, st) : launch_ranges_typed<bf16_t, float>(a, st);
    return a.state_bf16 ? launch_ranges_typed<float, bf16_t>(a, st) : launch_ranges_typed<float, float>(a, st);
}

}  // namespace ramnet
