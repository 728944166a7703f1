// Internal launcher interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ramnet {

// Address Decoder over n = B*T*H addresses of both q (read) and k (write).
struct DecodeArgs {
    const void *q, *k;
    int64_t n;
    int T, H, U, K, d_p;
    const int32_t *pos0;  // position of token t of sequence b: pos0[b] + t
    int cape;
    bool in_bf16;
    int32_t *w_idx, *r_idx;
    float *w_wt, *r_wt;
};
hipError_t launch_decode(const DecodeArgs &d, hipStream_t st);

// Recurrence over T tokens for B*H units, given addresses.
struct ScanArgs {
    int B, T, H;
    int64_t M;
    int K, d_v;
    bool in_bf16, state_bf16;
    const void *v, *gamma, *g;
    const float *norm_w;
    const int32_t *w_idx, *r_idx;
    const float *w_wt, *r_wt;
    void *S;
    float *mass;
    void *out;
    float eps_gsu, eps_norm;
};
// LDS bytes the serial scan needs to keep one head's state on chip, and
// whether that fits a workgroup.
size_t scan_state_lds_bytes(int64_t M, int d_v, bool state_bf16);
bool scan_state_fits_lds(int64_t M, int d_v, bool state_bf16);
hipError_t launch_scan_serial(const ScanArgs &a, hipStream_t st);

// Slot-grouped chunked recurrence (state slice in LDS) + RMSNorm/gate
// epilogue.  r (fp32 [B,T,H,d_v]) and per-slice square sums
// ([B,T,H,d_v/CG]) pass through global memory between the two kernels.
struct ChunkArgs : ScanArgs {
    float *rbuf;     // may alias out when the output is fp32
    float *sumsq;
    float *mass_ws;  // final mass, copied to `mass` by the epilogue kernel
    int CG, C, EPT;
};



struct ChunkPlan {
    bool ok;
    int CG, C, EPT;
    size_t lds;
};

constexpr size_t kChunkLdsLimit = 160 * 1024;

// Workspace bytes of the chunked path beyond the addresses: r (when the
// output is not fp32), per-slice square sums, final mass.
size_t chunk_workspace_bytes(const ChunkPlan &p, int64_t n, int64_t units, int64_t M, int d_v,
                             bool state_bf16);

struct ChunkLayout {
    size_t h_off, k_off, w_off, v_off, e_off, r_off, n_off, x_off, total;
};

__host__ __device__ inline size_t chunk_align16(size_t x) { return (x + 15) & ~size_t(15); }

// LDS layout of one chunked-scan workgroup: bucket counts/offsets, event keys
// and weights, staged values, exp(gamma), read weights, read snapshots, scan
// scratch.
__host__ __device__ inline ChunkLayout chunk_layout(int64_t M, int CG, int C, int K, int sbytes) {
    ChunkLayout L;
    size_t o = 0;
    L.h_off = o; o = chunk_align16(o + static_cast<size_t>(M + 1) * 4);
    L.k_off = o; o = chunk_align16(o + static_cast<size_t>(2) * C * K * 4);
    L.w_off = o; o = chunk_align16(o + static_cast<size_t>(2) * C * K * 4);
    L.v_off = o; o = chunk_align16(o + static_cast<size_t>(C) * CG * 4);
    L.e_off = o; o = chunk_align16(o + static_cast<size_t>(C) * 4);
    L.r_off = o; o = chunk_align16(o + static_cast<size_t>(C) * K * 4);
    L.n_off = o; o = chunk_align16(o + static_cast<size_t>(C) * K * CG * sbytes);
    L.x_off = o; o = chunk_align16(o + 32 * 4);
    L.total = o;
    return L;
}

// One fused decoding step (decode + CAPE + GSU + read + norm + gate).
struct StepArgs {
    int B, H;
    int64_t M;
    int K, d_v, U, d_p, cape;
    bool in_bf16, state_bf16;
    const void *q, *k, *v, *gamma, *g;
    const float *norm_w;
    const int32_t *pos;
    void *S;
    float *mass;
    void *out;
    int32_t *out_idx[2];  // write, read addresses [B,H,K] or NULL
    float *out_wt[2];
    float eps_gsu, eps_norm;
};
bool step_fused_supported(int K, int d_p, int U, int d_v, bool state_bf16);
hipError_t launch_step_fused(const StepArgs &a, hipStream_t st);

ChunkPlan plan_chunked(int64_t M, int K, int d_v, int B, int T, int H, bool state_bf16);
hipError_t launch_scan_chunked(const ChunkArgs &a, hipStream_t st);

}  // namespace ramnet
