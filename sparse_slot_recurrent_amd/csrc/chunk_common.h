// Helpers shared by the slot-grouped prefill kernels (scan_chunked.hip:
// state rows on chip; scan_ranges.hip: state rows in HBM): block-wide
// scans, the division by K, 16-byte row pieces and value rows in LDS.
#pragma once

#include "device_common.h"

namespace ramnet {

constexpr int kNT = 1024;  // threads per workgroup
constexpr int kWavesPerBlock = kNT / kWave;
constexpr int kMaxEV = 4096;                        // events of one kind per chunk
constexpr int kMaxEVHbm = 3072;                     // the same with slot rows in HBM
constexpr int kPT = 512;                            // plan kernel threads
// Events per plan thread (EPW) and plan entries per scan thread (EVT) are
// template parameters: EV / kPT and EV / kNT for chunks of at most 2048,
// 3072 or 4096 events (EV rounded up to a multiple of 1024).
constexpr int kReadFlag = 1 << 30;  // plan tables: a read touches the slot

__host__ __device__ inline size_t al16(size_t x) { return (x + 15) & ~size_t(15); }
inline size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

// Inclusive prefix sum over the 64 lanes of a wave, with DPP moves only
// (no LDS permutes): shifts right by 1, 2, 4 and 8 lanes within each row of
// 16 (a lane whose source lies outside its row adds 0), then row 0's last
// lane is added to row 1 and row 2's to row 3, and lane 31 to rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
    return x;
}

// Exclusive prefix of x over a block of NT threads (thread order); the block
// total goes to `total`.  Every thread must call it.
template <int NT>
__device__ int block_excl_scan(int x, int *wtot, int &total) {
    constexpr int NW = NT / kWave;
    const int lane = lane_id(), wid = threadIdx.x / kWave;
    const int incl = wave_incl_scan(x);
    if (lane == kWave - 1) wtot[wid] = incl;
    lds_barrier();
    if (wid == 0) {
        int y = lane < NW ? wtot[lane] : 0;
        y = wave_incl_scan(y);
        if (lane < NW) wtot[lane] = y;
    }
    lds_barrier();
    const int base = wid > 0 ? wtot[wid - 1] : 0;
    total = wtot[NW - 1];
    lds_barrier();
    return base + incl - x;
}

// In-place exclusive scan of a[0, n) by a block of NT threads, each taking
// a contiguous run; returns the sum.  Callers synchronise before reading a.
template <int NT>
__device__ int block_scan_array(int *a, int n, int *wtot) {
    const int per = (n + NT - 1) / NT;
    const int lo = min(static_cast<int>(threadIdx.x) * per, n), hi = min(lo + per, n);
    int local = 0;
    for (int i = lo; i < hi; ++i) local += a[i];
    int total;
    int base = block_excl_scan<NT>(local, wtot, total);
    for (int i = lo; i < hi; ++i) {
        const int c = a[i];
        a[i] = base;
        base += c;
    }
    return total;
}

// In-place exclusive scan of a[0, n) by a block of NT threads, returning the
// sum.  Wave w takes the w-th contiguous segment of the array and reads it
// 64 consecutive words at a time (lane i word i: no LDS bank conflicts),
// carrying its running total from one group of 64 to the next.  Callers
// synchronise before reading a.
template <int NT>
__device__ int block_scan_striped(int *a, int n, int *wtot) {
    constexpr int NW = NT / kWave;
    const int lane = lane_id(), wid = threadIdx.x / kWave;
    const int per = (n + NT - 1) / NT;  // groups of 64 per wave
    const int lo = min(wid * per * kWave, n), hi = min(lo + per * kWave, n);
    int tot = 0;
    for (int i = lo + lane; i < hi; i += kWave) tot += a[i];
    tot = wave_incl_scan(tot);
    if (lane == kWave - 1) wtot[wid] = tot;
    lds_barrier();
    if (wid == 0) {
        int y = lane < NW ? wtot[lane] : 0;
        y = wave_incl_scan(y);
        if (lane < NW) wtot[lane] = y;
    }
    lds_barrier();
    int carry = wid > 0 ? wtot[wid - 1] : 0;
    const int total = wtot[NW - 1];
    lds_barrier();
    for (int g = lo; g < hi; g += kWave) {
        const int i = g + lane;
        const int x = i < hi ? a[i] : 0;
        const int incl = wave_incl_scan(x);
        if (i < hi) a[i] = carry + incl - x;
        carry += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    return total;
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

// Channels [c0, c0 + CP) of value row t (rows of VROW elements), as fp32.
template <int CP>
__device__ __forceinline__ void value_part(const float *vbuf, int off, float (&vt)[CP]) {
#pragma unroll
    for (int j = 0; j < CP / 4; ++j) {
        const float4 f = reinterpret_cast<const float4 *>(vbuf + off)[j];
        vt[4 * j] = f.x;
        vt[4 * j + 1] = f.y;
        vt[4 * j + 2] = f.z;
        vt[4 * j + 3] = f.w;
    }
}
template <int CP>
__device__ __forceinline__ void value_part(const bf16_t *vbuf, int off, float (&vt)[CP]) {
#pragma unroll
    for (int j = 0; j < CP / 4; ++j) {
        const uint2 u = reinterpret_cast<const uint2 *>(vbuf + off)[j];
        vt[4 * j] = __uint_as_float(u.x << 16);
        vt[4 * j + 1] = __uint_as_float(u.x & 0xffff0000u);
        vt[4 * j + 2] = __uint_as_float(u.y << 16);
        vt[4 * j + 3] = __uint_as_float(u.y & 0xffff0000u);
    }
}

}  // namespace ramnet
