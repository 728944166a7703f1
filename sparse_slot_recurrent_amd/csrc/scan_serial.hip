// Token-serial recurrence for gfx950: one wave per (batch, head) unit, lane c
// owns channels c, c+64, ... of every slot row.
//
// RAM-Net project page, "Gated Sparse Update" (four steps per addressed
// slot) and the read of the "three stages" paragraph.  Per token: the K
// writes (retention, mass, rate, content), then the read of the K read slots,
// RMSNorm over d_v and the sigmoid gate.
//
// Each lane only ever touches its own channels of the state, so every
// read-after-write is within one thread and needs no synchronisation; the
// per-slot scalars (mass, alpha, lambda) are computed identically by every
// lane.  The head's state sits in LDS when it fits (copied in and out once),
// else it is updated in place in HBM.
#include "device_common.h"
#include "launch.h"

namespace ramnet {
namespace {

constexpr size_t kLdsBytes = 160 * 1024;

template <typename TIn, typename TS, int CPL, bool IN_LDS>
__global__ __launch_bounds__(kWave) void scan_serial_kernel(ScanArgs a) {
    extern __shared__ unsigned char smem[];
    const int unit = blockIdx.x;
    const int b = unit / a.H, h = unit % a.H;
    const int lane = threadIdx.x;
    const int64_t M = a.M;
    const int d_v = a.d_v, K = a.K;
    TS *Sg = static_cast<TS *>(a.S) + static_cast<int64_t>(unit) * M * d_v;
    float *mg = a.mass + static_cast<int64_t>(unit) * M;
    TS *Su = Sg;
    float *mu = mg;
    const int64_t row_bytes = M * d_v * static_cast<int64_t>(sizeof(TS));
    if (IN_LDS) {
        Su = reinterpret_cast<TS *>(smem);
        mu = reinterpret_cast<float *>(smem + row_bytes);
        const uint4 *src = reinterpret_cast<const uint4 *>(Sg);
        uint4 *dst = reinterpret_cast<uint4 *>(Su);
        for (int64_t i = lane; i < row_bytes / 16; i += kWave) dst[i] = src[i];
        for (int64_t i = lane; i < M; i += kWave) mu[i] = mg[i];
        __syncthreads();
    }
    const TIn *v = static_cast<const TIn *>(a.v);
    const TIn *gam = static_cast<const TIn *>(a.gamma);
    const TIn *g = static_cast<const TIn *>(a.g);
    TS *out = static_cast<TS *>(a.out);
    float nw[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) nw[j] = a.norm_w ? a.norm_w[lane + kWave * j] : 1.0f;

    for (int t = 0; t < a.T; ++t) {
        const int64_t th = (static_cast<int64_t>(b) * a.T + t) * a.H + h;
        int wi = 0, ri = 0;
        float ww = 0.f, rw = 0.f;
        if (lane < K) {
            wi = a.w_idx[th * K + lane];
            ww = a.w_wt[th * K + lane];
            ri = a.r_idx[th * K + lane];
            rw = a.r_wt[th * K + lane];
        }
        const int64_t row = static_cast<int64_t>(b) * a.T + t;  // token (b, t)
        const float eg = expf(to_f32(gam[row * a.ld_gamma + h]));
        float vv[CPL], gg[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            vv[j] = to_f32(v[row * a.ld_v + h * d_v + lane + kWave * j]);
            gg[j] = to_f32(g[row * a.ld_g + h * d_v + lane + kWave * j]);
        }
        // Gated Sparse Update of the K write slots.
        for (int kk = 0; kk < K; ++kk) {
            const float w = bcast(ww, kk);
            const int i = bcast(wi, kk);
            // w = 0: alpha = 1, lambda = 0.  A slot outside [0, M) (only
            // possible with caller-given addresses) is ignored.
            if (!(w > 0.f) || static_cast<uint64_t>(i) >= static_cast<uint64_t>(M)) continue;
            const float alpha = retention(w, eg);
            const float m = fmaf(alpha, mu[i], w);
            mu[i] = m;
            const float lam = w / (m + a.eps_gsu);
            TS *row = Su + static_cast<int64_t>(i) * d_v;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = lane + kWave * j;
                const float s = to_f32(row[c]);
                row[c] = from_f32<TS>(fmaf(lam, vv[j] - s, s));
            }
        }
        // Read the K read slots, RMSNorm, gate.
        float r[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) r[j] = 0.f;
        for (int kk = 0; kk < K; ++kk) {
            const float rho = bcast(rw, kk);
            const int j_ = bcast(ri, kk);
            if (static_cast<uint64_t>(j_) >= static_cast<uint64_t>(M)) continue;
            const TS *row = Su + static_cast<int64_t>(j_) * d_v;
#pragma unroll
            for (int j = 0; j < CPL; ++j) r[j] = fmaf(rho, to_f32(row[lane + kWave * j]), r[j]);
        }
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) ss = fmaf(r[j], r[j], ss);
        ss = wave_sum(ss);
        const float den = ss / static_cast<float>(d_v) + a.eps_norm;
        const float inv = den > 0.f ? 1.0f / sqrtf(den) : 0.f;  // zero read, eps 0
#pragma unroll
        for (int j = 0; j < CPL; ++j)
            out[th * d_v + lane + kWave * j] =
                from_f32<TS>(r[j] * inv * nw[j] * sigmoid(gg[j]));
    }

    if (IN_LDS) {
        __syncthreads();
        const uint4 *src = reinterpret_cast<const uint4 *>(Su);
        uint4 *dst = reinterpret_cast<uint4 *>(Sg);
        for (int64_t i = lane; i < row_bytes / 16; i += kWave) dst[i] = src[i];
        for (int64_t i = lane; i < M; i += kWave) mg[i] = mu[i];
    }
}

template <typename TIn, typename TS, int CPL>
hipError_t launch_cpl(const ScanArgs &a, hipStream_t st) {
    const unsigned grid = static_cast<unsigned>(a.B) * a.H;
    // Holding the head on chip costs one read and one write of the whole
    // state; updating in HBM costs the touched rows (K written twice, K read)
    // per token.  Take the cheaper one.
    const double whole = 2.0 * static_cast<double>(scan_state_lds_bytes(a.M, a.d_v, a.state_bf16));
    const double rows = 3.0 * a.T * a.K * a.d_v * (a.state_bf16 ? 2.0 : 4.0);
    if (scan_state_fits_lds(a.M, a.d_v, a.state_bf16) && whole < rows) {
        const size_t lds = scan_state_lds_bytes(a.M, a.d_v, a.state_bf16);
        auto kern = scan_serial_kernel<TIn, TS, CPL, true>;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(grid), dim3(kWave), lds, st, a);
    } else {
        hipLaunchKernelGGL((scan_serial_kernel<TIn, TS, CPL, false>), dim3(grid), dim3(kWave),
                           0, st, a);
    }
    return hipGetLastError();
}

template <typename TIn, typename TS>
hipError_t launch_ts(const ScanArgs &a, hipStream_t st) {
    switch (a.d_v / kWave) {
        case 1: return launch_cpl<TIn, TS, 1>(a, st);
        case 2: return launch_cpl<TIn, TS, 2>(a, st);
        case 3: return launch_cpl<TIn, TS, 3>(a, st);
        case 4: return launch_cpl<TIn, TS, 4>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t scan_state_lds_bytes(int64_t M, int d_v, bool state_bf16) {
    return static_cast<size_t>(M) * d_v * (state_bf16 ? 2 : 4) + static_cast<size_t>(M) * 4;
}

bool scan_state_fits_lds(int64_t M, int d_v, bool state_bf16) {
    return scan_state_lds_bytes(M, d_v, state_bf16) <= kLdsBytes;
}

hipError_t launch_scan_serial(const ScanArgs &args, hipStream_t st) {
    if (static_cast<int64_t>(args.B) * args.H == 0) return hipSuccess;
    ScanArgs a = args;
    if (!a.ld_v) a.ld_v = static_cast<int64_t>(a.H) * a.d_v;
    if (!a.ld_g) a.ld_g = static_cast<int64_t>(a.H) * a.d_v;
    if (!a.ld_gamma) a.ld_gamma = a.H;
    if (a.in_bf16)
        return a.state_bf16 ? launch_ts<bf16_t, bf16_t>(a, st) : launch_ts<bf16_t, float>(a, st);
    return a.state_bf16 ? launch_ts<float, bf16_t>(a, st) : launch_ts<float, float>(a, st);
}

}  // namespace ramnet
