// Device-side helpers shared by the gfx950 kernels of the RAM-Net layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ramnet {

constexpr int kWave = 64;

// bf16 is carried as its 16-bit pattern.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (gfx950 converts in hardware,
// v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t bf16_rne(float x) {
    return bf16_t{__builtin_bit_cast(uint16_t, static_cast<__bf16>(x))};
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return bf16_rne(x); }

// Value after a round trip through storage type T.
template <typename T> __device__ __forceinline__ float stored(float x) {
    return to_f32(from_f32<T>(x));
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Workgroup barrier ordering LDS only: global loads in flight (prefetches)
// stay in flight across it.  Not for global-memory hand-offs between threads.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Broadcast from a lane chosen by a wave-uniform index.
__device__ __forceinline__ int bcast(int x, int lane) {
    return __builtin_amdgcn_readlane(x, lane);
}
__device__ __forceinline__ float bcast(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Value held by lane (lane ^ J), J in {1, 2, 4, 8, 16}: DPP inside 16-lane
// rows (xor 1 and 2: quad permutes; xor 4: row shift left or right by 4;
// xor 8: row rotate by 8), ds_swizzle across the two rows of a 32-lane half
// (xor 16).
template <int J>
__device__ __forceinline__ int lane_xor(int v) {
    static_assert(J == 1 || J == 2 || J == 4 || J == 8 || J == 16, "lane_xor");
    if constexpr (J == 1) return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
    else if constexpr (J == 2) return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
    else if constexpr (J == 4) {
        const int up = __builtin_amdgcn_mov_dpp(v, 0x104, 0xF, 0xF, false);  // lane i+4
        const int dn = __builtin_amdgcn_mov_dpp(v, 0x114, 0xF, 0xF, false);  // lane i-4
        return (__lane_id() & 4) ? dn : up;
    } else if constexpr (J == 8) return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false);
    else return __builtin_amdgcn_ds_swizzle(v, 0x401F);
}
template <int J>
__device__ __forceinline__ float lane_xor(float v) {
    return __int_as_float(lane_xor<J>(__float_as_int(v)));
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

// Retention of the Gated Sparse Update: (1 - w)^(exp(gamma)) for 0 < w,
// written as exp(exp(gamma) * log1p(-w)); 0 for w >= 1.
__device__ __forceinline__ float retention(float w, float exp_gamma) {
    if (w >= 1.0f) return 0.0f;
    return expf(exp_gamma * log1pf(-w));
}

__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + expf(-x)); }

// Retention with the hardware base-2 log and exp: (1 - w)^(exp(gamma)) =
// 2^(exp(gamma) * log2(1 - w)).  1 - w is rounded to u; the rounding error
// e = (1 - u) - w is exact (1 >= w), and log2(1 - w) = log2(u) + e / (u ln 2)
// to first order, which keeps the exponent accurate for small w.
__device__ __forceinline__ float retention_fast(float w, float exp_gamma) {
    if (w >= 1.0f) return 0.0f;
    const float u = 1.0f - w;
    const float e = (1.0f - u) - w;
    const float l2 = __builtin_amdgcn_logf(u) + e * __builtin_amdgcn_rcpf(u) * 1.44269504088896341f;
    return __builtin_amdgcn_exp2f(exp_gamma * l2);
}

// CAPE (project page, CAPE paragraph): the slot a content address moves to
// at position pos, by reading `form`: 1 every digit advances by pos mod dp;
// 2 digit u advances by digit u of pos (base dp, U digits, no carry); 3 the
// slot index advances by pos, wrapping over the M = dp^U slots.  Digits wrap
// within their dp values (M <= 2^30).  DP > 0 fixes the base at compile
// time.  cape_shift holds the position-dependent part (pos mod M, pos mod
// dp), so that callers moving many slots at one position reduce pos once.
struct CapeShift {
    unsigned pm, s1;
    unsigned dm;  // DP == 0: ceil(2^32 / dp), so that x / dp = mulhi(x, dm) for x < 2^30
};
template <int DP>
__device__ __forceinline__ CapeShift cape_shift(int64_t pos, int dp_rt, int64_t M) {
    const int dp = DP > 0 ? DP : dp_rt;
    CapeShift sh;
    if (pos >= 0 && pos <= 0xffffffffll) {  // the usual case, in 32-bit arithmetic
        const unsigned p = static_cast<unsigned>(pos);
        sh.pm = p % static_cast<unsigned>(M);
        sh.s1 = p % static_cast<unsigned>(dp);
    } else {
        sh.pm = static_cast<unsigned>(((pos % M) + M) % M);
        sh.s1 = static_cast<unsigned>(((pos % dp) + dp) % dp);
    }
    sh.dm = DP > 0 ? 0u : 0xffffffffu / static_cast<unsigned>(dp) + 1u;
    return sh;
}
// x / dp for x < 2^30 and 2 <= dp <= 8: e = dm * dp - 2^32 is at most 4 for
// these bases, so the error term x * e / 2^32 stays below 1 and the
// multiply-high is exact (checked for every such x and dp).
template <int DP>
__device__ __forceinline__ unsigned cape_div(unsigned x, const CapeShift &sh) {
    if constexpr (DP > 0) return x / DP;
    else return __umulhi(x, sh.dm);
}
// The slot content address `slot` (in [0, M)) moves to under shift sh.
template <int DP>
__device__ __forceinline__ int cape_slot_at(int slot, CapeShift sh, int U, int dp_rt, int form,
                                            int64_t M) {
    const unsigned dp = DP > 0 ? DP : dp_rt;
    if (form == 3) {
        const unsigned x = static_cast<unsigned>(slot) + sh.pm;  // both below M <= 2^30
        return static_cast<int>(x >= static_cast<unsigned>(M) ? x - static_cast<unsigned>(M) : x);
    }
    if (form == 1 && sh.s1 == 0) return slot;
    unsigned x = static_cast<unsigned>(slot), p = sh.pm, moved = 0, place = 1;
    for (int u = 0; u < U; ++u) {
        const unsigned xq = cape_div<DP>(x, sh), d = x - xq * dp;
        unsigned s = sh.s1;
        if (form == 2) {
            const unsigned pq = cape_div<DP>(p, sh);
            s = p - pq * dp;
            p = pq;
        }
        x = xq;
        const unsigned ds = d + s;  // below 2 dp
        moved += (ds >= dp ? ds - dp : ds) * place;
        place *= dp;
    }
    return static_cast<int>(moved);
}
template <int DP>
__device__ __forceinline__ int cape_slot(int slot, int64_t pos, int U, int dp_rt, int form, int64_t M) {
    return cape_slot_at<DP>(slot, cape_shift<DP>(pos, dp_rt, M), U, dp_rt, form, M);
}

// Whether head h uses CAPE: its bit of content_heads (bit 63 for h >= 63)
// is clear.
__device__ __forceinline__ bool head_uses_cape(uint64_t content_heads, int h) {
    return !((content_heads >> (h < 63 ? h : 63)) & 1u);
}

}  // namespace ramnet
