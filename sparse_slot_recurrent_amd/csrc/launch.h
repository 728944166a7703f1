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

}  // namespace ramnet
