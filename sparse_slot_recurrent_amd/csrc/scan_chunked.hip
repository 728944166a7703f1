// Slot-grouped prefill recurrence for gfx950.
//
// RAM-Net project page, GPU-execution paragraphs: with every token's
// addresses known, read and write events are grouped by slot; each slot
// replays its own events in causal order, different slots and channels run
// in parallel, and slots without events cost nothing.  The Gated Sparse
// Update and the read are those of the "Gated Sparse Update" and "three
// stages" paragraphs.
//
// Organisation.  One workgroup owns one (batch, head) unit and a slice of CG
// channels of its state; thread s holds slot s's row slice and mass in
// registers for the whole sequence.  The sequence is cut into chunks of C
// tokens.  Per chunk:
//   1. the chunk's values (this slice), exp(gamma) and read weights are
//      staged in LDS, and the chunk's 2*C*K events (K writes, then K reads
//      per token) are counted per slot;
//   2. the counts are scanned into bucket offsets and every event is
//      scattered into its slot's bucket; each event then counts the bucket's
//      keys below its own (token, write before read) and moves to that rank,
//      so every bucket is in causal order without a serial sort;
//   3. thread s replays its bucket: a write updates mass and row, a read
//      leaves a snapshot of the row (storage dtype) in the token's read
//      position;
//   4. one thread per (token, channel) sums rho_k * snapshot_k over the K
//      reads in rank order; r (fp32) and its sum of squares over the slice go
//      to global memory.
// The next chunk's addresses, values and gates are loaded during step 3.  The
// mass recurrence is the same in every channel slice, so each workgroup of a
// unit computes it.  A small second kernel sums the slices' squares per token
// and applies RMSNorm and the gate.
#include "device_common.h"
#include "launch.h"

namespace ramnet {
namespace {

constexpr int kNT = 1024;           // threads per workgroup
constexpr int kWavesPerBlock = kNT / kWave;

__device__ __forceinline__ int wave_incl_scan(int x) {
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(x, off, kWave);
        if (lane >= off) x += y;
    }
    return x;
}

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

// A 16-byte chunk of a row as fp32 values.
__device__ __forceinline__ void unpack_chunk(const uint4 &u, float (&v)[4]) {
    v[0] = __uint_as_float(u.x);
    v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z);
    v[3] = __uint_as_float(u.w);
}
__device__ __forceinline__ void unpack_chunk(const uint4 &u, float (&v)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        v[2 * q] = __uint_as_float(w[q] << 16);
        v[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    }
}

// floor(e / K) for 0 <= e < 2^24 with a precomputed m = ceil(2^32 / K).
__device__ __forceinline__ int div_by(uint32_t e, uint64_t m) {
    return static_cast<int>((static_cast<uint64_t>(e) * m) >> 32);
}

// One event of a slot's replay: a write updates mass and row; a read leaves
// a snapshot of the row (storage dtype) in its token's read position.
template <typename TS, int CG>
__device__ __forceinline__ void replay_event(uint32_t kk, float wv, int K, float eps,
                                             const float *egb, const float *vbuf, TS *snap,
                                             float (&x)[CG], float &m) {
    const int t = static_cast<int>(kk >> 7);
    if (kk & 64u) {
        const int row = t * K + static_cast<int>(kk & 63u);
        store_row<CG>(snap + row * CG, row_swz<TS, CG>(row), x);
    } else {
        const float alpha = retention_fast(wv, egb[t]);
        m = fmaf(alpha, m, wv);
        const float lam = wv * __builtin_amdgcn_rcpf(m + eps);
        float vt[CG];
        load_row<CG>(vbuf + t * CG, row_swz<float, CG>(t), vt);
#pragma unroll
        for (int c = 0; c < CG; ++c) x[c] = stored<TS>(fmaf(lam, vt[c] - x[c], x[c]));
    }
}

template <typename TIn, typename TS, int CG, int EPT, int NB>
__global__ __launch_bounds__(kNT) void scan_chunked_kernel(ChunkArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int wid = tid / kWave, lane = tid % kWave;
    const int ncg = a.d_v / CG;
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
    const int K = a.K, C = a.C, d_v = a.d_v;
    const uint64_t kdiv = ((uint64_t(1) << 32) + K - 1) / K;
    const ChunkLayout L = chunk_layout(M, CG, C, K, sizeof(TS));
    int *hist = reinterpret_cast<int *>(smem + L.h_off);
    uint32_t *ekey = reinterpret_cast<uint32_t *>(smem + L.k_off);
    float *ewt = reinterpret_cast<float *>(smem + L.w_off);
    float *vbuf = reinterpret_cast<float *>(smem + L.v_off);
    float *egb = reinterpret_cast<float *>(smem + L.e_off);
    float *rho = reinterpret_cast<float *>(smem + L.r_off);
    TS *snap = reinterpret_cast<TS *>(smem + L.n_off);
    int *wtot = reinterpret_cast<int *>(smem + L.x_off);  // per-wave totals

    const TIn *v = static_cast<const TIn *>(a.v);
    const TIn *gam = static_cast<const TIn *>(a.gamma);
    const int64_t th_unit = static_cast<int64_t>(b) * a.T * a.H + h;  // token 0 of the unit

    // Thread s owns slot s: its row slice and mass stay in registers for the
    // whole sequence.
    const bool owner = tid < M;
    float x[CG];
    float m = 0.f;
    {
        const TS *Sg = static_cast<const TS *>(a.S) + (static_cast<int64_t>(unit) * M + tid) * d_v + cg * CG;
        if (owner) {
            TS tmp[CG];
#pragma unroll
            for (int c = 0; c < CG; ++c) tmp[c] = Sg[c];
#pragma unroll
            for (int c = 0; c < CG; ++c) x[c] = to_f32(tmp[c]);
            m = a.mass[static_cast<int64_t>(unit) * M + tid];
        } else {
#pragma unroll
            for (int c = 0; c < CG; ++c) x[c] = 0.f;
        }
    }

    // Next chunk's inputs, loaded one chunk ahead into registers.
    constexpr int VPT = (CG * 512 + kNT - 1) / kNT;  // values per thread (C <= 512)
    int pf_slot[EPT];
    float pf_wt[EPT];
    float pf_v[VPT];
    float pf_g = 0.f;
    auto prefetch = [&](int t0) {
        const int Cc = min(C, a.T - t0);
        const int nw = Cc * K;
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const int e = tid + j * kNT;
            pf_slot[j] = -1;
            pf_wt[j] = 0.f;
            if (e < 2 * nw) {
                const bool rd = e >= nw;
                const int ee = rd ? e - nw : e;
                const int t = div_by(ee, kdiv), k = ee - t * K;
                const int64_t idx = (th_unit + static_cast<int64_t>(t0 + t) * a.H) * K + k;
                pf_slot[j] = rd ? a.r_idx[idx] : a.w_idx[idx];
                pf_wt[j] = rd ? a.r_wt[idx] : a.w_wt[idx];
            }
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int i = tid + j * kNT;
            pf_v[j] = 0.f;
            if (i < Cc * CG) {
                const int t = i / CG, c = i % CG;
                pf_v[j] = to_f32(v[(th_unit + static_cast<int64_t>(t0 + t) * a.H) * d_v + cg * CG + c]);
            }
        }
        if (tid < Cc) pf_g = to_f32(gam[th_unit + static_cast<int64_t>(t0 + tid) * a.H]);
    };

    for (int i = tid; i <= M; i += kNT) hist[i] = 0;
    prefetch(0);
    __syncthreads();

    for (int t0 = 0; t0 < a.T; t0 += C) {
        const int Cc = min(C, a.T - t0);
        const int nw = Cc * K;
        // ---- 1. stage values, gates and read weights; count events per slot
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int i = tid + j * kNT;
            if (i < Cc * CG) vbuf[swz_index<float, CG>(i / CG, i % CG)] = pf_v[j];
        }
        if (tid < Cc) egb[tid] = expf(pf_g);
        int erank[EPT];
        uint32_t ekk[EPT];
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const int e = tid + j * kNT;
            erank[j] = -1;
            ekk[j] = 0;
            if (e < 2 * nw) {
                const bool rd = e >= nw;
                const int ee = rd ? e - nw : e;
                const int t = div_by(ee, kdiv), k = ee - t * K;
                const int s = pf_slot[j];
                // A zero-weight write changes nothing (alpha = 1, lambda = 0);
                // a slot outside [0, M) (caller-given addresses) is skipped and
                // a skipped read contributes nothing.
                const bool ok = static_cast<uint32_t>(s) < static_cast<uint32_t>(M) && (rd || pf_wt[j] > 0.f);
                if (rd) rho[ee] = ok ? pf_wt[j] : 0.f;
                if (ok) {
                    ekk[j] = (((static_cast<uint32_t>(t) << 1) | (rd ? 1u : 0u)) << 6) |
                             static_cast<uint32_t>(k);
                    erank[j] = atomicAdd(&hist[s], 1);
                }
            }
        }
        __syncthreads();
        // ---- 2a. exclusive scan of the counts into bucket offsets
        {
            const int per = (M + kNT - 1) / kNT;
            const int lo = min(tid * per, M);
            const int hi = min(lo + per, M);
            int local = 0;
            for (int i = lo; i < hi; ++i) local += hist[i];
            const int incl = wave_incl_scan(local);
            if (lane == kWave - 1) wtot[wid] = incl;
            __syncthreads();
            if (wid == 0) {
                int y = lane < kWavesPerBlock ? wtot[lane] : 0;
                y = wave_incl_scan(y);
                if (lane < kWavesPerBlock) wtot[lane] = y;
            }
            __syncthreads();
            int base = (wid > 0 ? wtot[wid - 1] : 0) + incl - local;
            for (int i = lo; i < hi; ++i) {
                const int c = hist[i];
                hist[i] = base;
                base += c;
            }
            if (hi == M && lo < hi) hist[M] = base;
        }
        __syncthreads();
        // ---- 2b. scatter events into their buckets (arrival order) ...
#pragma unroll
        for (int j = 0; j < EPT; ++j)
            if (erank[j] >= 0) ekey[hist[pf_slot[j]] + erank[j]] = ekk[j];
        __syncthreads();
        // ---- 2c. ... then move each to its causal rank within the bucket:
        //          the number of the bucket's keys below its own (keys are
        //          unique within a slot: one write and one read per token)
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            if (erank[j] >= 0) {
                const int beg = hist[pf_slot[j]], n = hist[pf_slot[j] + 1] - beg;
                int r = 0;
                for (int i = 0; i < n; ++i) r += ekey[beg + i] < ekk[j] ? 1 : 0;
                erank[j] = beg + r;
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            if (erank[j] >= 0) {
                ekey[erank[j]] = ekk[j];
                ewt[erank[j]] = pf_wt[j];
            }
        }
        __syncthreads();
        // ---- 3. next chunk's loads go out now and land during the replay
        if (t0 + C < a.T) prefetch(t0 + C);
        // Replay: thread s applies its bucket, already in causal order, to
        // its row in registers.
        if (owner) {
            const int beg = hist[tid], n = hist[tid + 1] - beg;
            uint32_t kk[NB];
            float ww[NB];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                kk[i] = i < n ? ekey[beg + i] : 0u;
                ww[i] = i < n ? ewt[beg + i] : 0.f;
            }
#pragma unroll
            for (int i = 0; i < NB; ++i)
                if (i < n) replay_event<TS, CG>(kk[i], ww[i], K, a.eps_gsu, egb, vbuf, snap, x, m);
            for (int i = NB; i < n; ++i)
                replay_event<TS, CG>(ekey[beg + i], ewt[beg + i], K, a.eps_gsu, egb, vbuf, snap, x, m);
        }
        __syncthreads();
        // ---- 4. reads: r = sum_k rho_k * snapshot_k (k in rank order) for one
        //         16-byte chunk of channels per thread; r and the sum of
        //         squares over the slice go to global memory
        {
            constexpr int EPC = 16 / static_cast<int>(sizeof(TS));  // channels per chunk
            constexpr int NCH = CG / EPC;                            // chunks per row
            for (int i = tid; i < Cc * NCH; i += kNT) {
                const int t = i / NCH, j = i % NCH;
                float r[EPC];
#pragma unroll
                for (int c = 0; c < EPC; ++c) r[c] = 0.f;
                for (int k = 0; k < K; ++k) {
                    // A read with weight 0 adds nothing; skipped reads (slot
                    // outside [0, M)) have weight 0 and no snapshot.
                    const int row = t * K + k;
                    const float rw = rho[row];
                    if (rw != 0.f) {
                        const uint4 u = reinterpret_cast<const uint4 *>(snap + row * CG)[j ^ row_swz<TS, CG>(row)];
                        float sv[EPC];
                        unpack_chunk(u, sv);
#pragma unroll
                        for (int c = 0; c < EPC; ++c) r[c] = fmaf(rw, sv[c], r[c]);
                    }
                }
                const int64_t th = th_unit + static_cast<int64_t>(t0 + t) * a.H;
                float *dst = a.rbuf + th * d_v + cg * CG + j * EPC;
#pragma unroll
                for (int c = 0; c < EPC; c += 4)
                    *reinterpret_cast<float4 *>(dst + c) = make_float4(r[c], r[c + 1], r[c + 2], r[c + 3]);
                float ss = 0.f;
#pragma unroll
                for (int c = 0; c < EPC; ++c) ss = fmaf(r[c], r[c], ss);
#pragma unroll
                for (int off = NCH / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, kWave);
                if (j == 0) a.sumsq[th * ncg + cg] = ss;
            }
        }
        for (int i = tid; i <= M; i += kNT) hist[i] = 0;
        __syncthreads();
    }

    if (owner) {
        TS *Sg = static_cast<TS *>(a.S) + (static_cast<int64_t>(unit) * M + tid) * d_v + cg * CG;
#pragma unroll
        for (int c = 0; c < CG; ++c) Sg[c] = from_f32<TS>(x[c]);
        // The mass goes to the workspace: other slices of this unit may not
        // have read the initial mass yet; the epilogue kernel copies it over
        // once every slice has finished.
        if (cg == 0) a.mass_ws[static_cast<int64_t>(unit) * M + tid] = m;
    }
}

// out = r / sqrt(mean(r^2) + eps) * omega * sigmoid(g), four channels per
// thread; the per-token square sums of the channel slices are added in
// slice order.
template <typename TIn, typename TO>
__global__ __launch_bounds__(256) void rms_gate_kernel(const float *__restrict__ rbuf,
                                                       const float *__restrict__ sumsq, int ncg,
                                                       const TIn *__restrict__ g,
                                                       const float *__restrict__ norm_w,
                                                       TO *out, int64_t n, int d_v, float eps,
                                                       const float *__restrict__ mass_ws,
                                                       float *__restrict__ mass, int64_t n_mass) {
    const int q4 = d_v / 4;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n_mass) mass[i] = mass_ws[i];
    if (i >= n * q4) return;
    const int64_t th = i / q4;
    const int c0 = static_cast<int>(i - th * q4) * 4;
    float tot = 0.f;
    for (int j = 0; j < ncg; ++j) tot += sumsq[th * ncg + j];
    const float den = tot / static_cast<float>(d_v) + eps;
    const float inv = den > 0.f ? 1.0f / sqrtf(den) : 0.f;  // zero read, eps 0
    const float4 r = *reinterpret_cast<const float4 *>(rbuf + th * d_v + c0);
    const float rv[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float om = norm_w ? norm_w[c0 + j] : 1.0f;
        out[th * d_v + c0 + j] = from_f32<TO>(rv[j] * inv * om * sigmoid(to_f32(g[th * d_v + c0 + j])));
    }
}

template <typename TIn, typename TS, int CG, int EPT>
hipError_t launch_cfg(const ChunkArgs &a, hipStream_t st) {
    const size_t lds = chunk_layout(a.M, CG, a.C, a.K, sizeof(TS)).total;
    constexpr int NB = EPT >= 8 ? 16 : 8;  // bucket entries held in registers
    auto kern = scan_chunked_kernel<TIn, TS, CG, EPT, NB>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    const unsigned grid = static_cast<unsigned>(a.B) * a.H * (a.d_v / CG);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kNT), lds, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = static_cast<int64_t>(a.B) * a.T * a.H;
    const int64_t n_mass = static_cast<int64_t>(a.B) * a.H * a.M;
    const int64_t work = max(n * (a.d_v / 4), n_mass);
    const unsigned g2 = static_cast<unsigned>((work + 255) / 256);
    hipLaunchKernelGGL((rms_gate_kernel<TIn, TS>), dim3(g2), dim3(256), 0, st, a.rbuf, a.sumsq,
                       a.d_v / CG, static_cast<const TIn *>(a.g), a.norm_w,
                       static_cast<TS *>(a.out), n, a.d_v, a.eps_norm, a.mass_ws, a.mass,
                       n_mass);
    return hipGetLastError();
}

template <typename TIn, typename TS, int CG>
hipError_t launch_ept(const ChunkArgs &a, hipStream_t st) {
    switch (a.EPT) {
        case 2: return launch_cfg<TIn, TS, CG, 2>(a, st);
        case 4: return launch_cfg<TIn, TS, CG, 4>(a, st);
        case 8: return launch_cfg<TIn, TS, CG, 8>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <typename TIn, typename TS>
hipError_t launch_cg(const ChunkArgs &a, hipStream_t st) {
    switch (a.CG) {
        case 8: return launch_ept<TIn, TS, 8>(a, st);
        case 16: return launch_ept<TIn, TS, 16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

ChunkPlan plan_chunked(int64_t M, int K, int d_v, int B, int T, int H, bool state_bf16) {
    ChunkPlan p{};
    p.ok = false;
    const int sbytes = state_bf16 ? 2 : 4;
    const int64_t units = static_cast<int64_t>(B) * H;
    // Thread s owns slot s, so the whole slot array must fit one workgroup.
    if (T < 32 || units == 0 || M > kNT || K > 63) return p;
    // Largest channel slice that still gives about one workgroup per CU,
    // then the longest chunk (a multiple of 32 tokens) that fits LDS.
    const int cgs[2] = {16, 8};
    for (int ci = 0; ci < 2; ++ci) {
        const int CG = cgs[ci];
        if (d_v % CG || CG * sbytes < 16) continue;
        const bool last = ci == 1;
        if (!last && units * (d_v / CG) < 256) continue;
        for (int C = 512; C >= 32; C -= 32) {
            const int64_t ev = 2LL * C * K;
            if (ev > 8LL * kNT) continue;  // at most 8 events per thread
            const size_t lds = chunk_layout(M, CG, C, K, sbytes).total;
            if (lds > kChunkLdsLimit) continue;
            int ept = 1;
            while (static_cast<int64_t>(ept) * kNT < ev) ept *= 2;
            p.ok = true;
            p.CG = CG;
            p.C = C;
            p.EPT = ept < 2 ? 2 : ept;
            p.lds = lds;
            return p;
        }
    }
    return p;
}

size_t chunk_workspace_bytes(const ChunkPlan &p, int64_t n, int64_t units, int64_t M, int d_v,
                             bool state_bf16) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    size_t b = 0;
    if (state_bf16) b += al(static_cast<size_t>(n) * d_v * 4);
    b += al(static_cast<size_t>(n) * (d_v / p.CG) * 4);
    b += al(static_cast<size_t>(units) * M * 4);
    return b;
}

hipError_t launch_scan_chunked(const ChunkArgs &a, hipStream_t st) {
    if (static_cast<int64_t>(a.B) * a.H * a.T == 0) return hipSuccess;
    if (a.in_bf16)
        return a.state_bf16 ? launch_cg<bf16_t, bf16_t>(a, st) : launch_cg<bf16_t, float>(a, st);
    return a.state_bf16 ? launch_cg<float, bf16_t>(a, st) : launch_cg<float, float>(a, st);
}

}  // namespace ramnet
