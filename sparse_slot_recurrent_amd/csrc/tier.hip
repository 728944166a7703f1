// Upkeep of a tiered slot state for gfx950: the rows in host memory, the
// most accessed ones of each (batch, head) unit cached in device memory
// (AI Radio page, deployment remark: the sparse access lets only the
// frequently accessed slots be cached in VRAM).  The decoding step reads and
// writes each row where it lives (step_fused.hip) and counts the accesses;
// these kernels empty the cache, re-choose its slots, and write it back.
//
// tier_rebalance_kernel: one workgroup per unit.
//   1. A 256-bin histogram of the key 2 * hits + cached (capped at 255) over
//      the unit's slots, and from it the threshold tau: slots above it are
//      all kept, slots at it are kept in slot order up to C lines in all
//      (tau = 0: none at it, key 0 is never cached).
//   2. Slots in order, a block's worth at a time (a block scan ranks the
//      slots at tau): the choice is marked in the count's top bit; a cached
//      slot not chosen is written back to host memory and its line freed.
//   3. The free lines, in line order, listed in LDS.
//   4. Slots in order again: a chosen slot without a line takes the next
//      free line, and its row is copied in from host memory.
//   5. Counts halved, marks cleared.
// Rows move in 16-byte pieces, 16 lanes per row.
#include "device_common.h"
#include "launch.h"

#include <algorithm>

namespace ramnet {
namespace {

constexpr int kTierThreads = 1024;
constexpr uint32_t kChosen = 0x80000000u;

__device__ __forceinline__ int tier_key(uint32_t hits, bool cached) {
    const uint32_t k = 2u * min(hits & ~kChosen, 1u << 20) + (cached ? 1u : 0u);
    return static_cast<int>(min(k, 255u));
}

// Exclusive prefix over the block's threads (thread order); total returned
// in `total`.  wtot: kTierThreads / 64 ints of LDS.
__device__ int tier_excl_scan(int x, int *wtot, int &total) {
    const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
    constexpr int nw = kTierThreads / kWave;
    int incl = x;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += y;
    }
    if (lane == kWave - 1) wtot[wid] = incl;
    __syncthreads();
    int base = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < nw; ++w) {
        const int c = wtot[w];
        base += w < wid ? c : 0;
        total += c;
    }
    __syncthreads();
    return base + incl - x;
}

// Copies one row of `bytes` bytes (a multiple of 16) with the 16 lanes of a
// group, lane gl taking pieces gl, gl + 16, ...
__device__ __forceinline__ void copy_row(void *dst, const void *src, int bytes, int gl) {
    const uint4 *s = static_cast<const uint4 *>(src);
    uint4 *d = static_cast<uint4 *>(dst);
    for (int i = gl; i < bytes / 16; i += 16) d[i] = s[i];
}

__global__ __launch_bounds__(kTierThreads) void tier_rebalance_kernel(TierArgs a) {
    __shared__ int hist[256];
    __shared__ int wtot[kTierThreads / kWave];
    __shared__ int sh[4];
    extern __shared__ int freelist[];  // [C]
    const int unit = blockIdx.x, tid = threadIdx.x;
    const int64_t M = a.M;
    const int C = a.C;
    const int rb = a.d_v * (a.state_bf16 ? 2 : 4);
    uint32_t *hits = a.hits + static_cast<int64_t>(unit) * M;
    int32_t *sl = a.slot_line + static_cast<int64_t>(unit) * M;
    int32_t *ls = a.line_slot + static_cast<int64_t>(unit) * C;
    char *cache = static_cast<char *>(a.cache) + static_cast<int64_t>(unit) * C * rb;
    char *host = static_cast<char *>(a.S_host) + static_cast<int64_t>(unit) * M * rb;

    // 1. histogram and threshold
    for (int i = tid; i < 256; i += kTierThreads) hist[i] = 0;
    __syncthreads();
    // a line outside [0, C) counts as no line
    auto line_of = [&](int64_t s) { const int l = sl[s]; return static_cast<unsigned>(l) < static_cast<unsigned>(C) ? l : -1; };
    for (int64_t s = tid; s < M; s += kTierThreads) atomicAdd(&hist[tier_key(hits[s], line_of(s) >= 0)], 1);
    __syncthreads();
    if (tid == 0) {
        int above = 0, tau = 0;
        for (int k = 255; k >= 1; --k) {
            if (above + hist[k] >= C) {
                tau = k;
                break;
            }
            above += hist[k];
        }
        // tau = 0: every slot with a nonzero key fits
        sh[0] = tau;
        sh[1] = tau ? C - above : 0;  // slots at tau to keep
    }
    __syncthreads();
    const int tau = sh[0], take = sh[1];

    // 2. choose; write back and free the lines of cached slots not chosen.
    //    A group of 16 lanes moves each such row.
    int ties_before = 0;
    for (int64_t s0 = 0; s0 < M; s0 += kTierThreads) {
        const int64_t s = s0 + tid;
        int key = 0, line = -1;
        uint32_t h = 0;
        if (s < M) {
            h = hits[s];
            line = line_of(s);
            key = tier_key(h, line >= 0);
        }
        const bool tie = tau > 0 && key == tau;
        int nties;
        const int r = tier_excl_scan(tie ? 1 : 0, wtot, nties) + ties_before;
        ties_before += nties;
        const bool chosen = s < M && key > 0 && (key > tau || (tie && r < take));
        if (chosen) hits[s] = h | kChosen;
        const bool evict = s < M && line >= 0 && !chosen;
        if (evict) {
            ls[line] = -1;
            sl[s] = -1;
        }
        // the evicted rows of this block, 16 lanes each: lanes of a wave
        // ballot their slots and the wave's groups take them in turn
        const uint64_t ev = __ballot(evict);
        const int lane = tid % kWave, g = lane / 16, gl = lane % 16;
        uint64_t rest = ev;
        int n = 0;
        while (rest) {
            const int src = __builtin_ctzll(rest);
            rest &= rest - 1;
            const int ln = __shfl(line, src, kWave);
            if (n % 4 == g) {
                const int64_t slot = s0 + (tid - lane) + src;
                copy_row(host + slot * rb, cache + static_cast<int64_t>(ln) * rb, rb, gl);
            }
            ++n;
        }
    }
    __syncthreads();

    // 3. free lines in line order
    int nfree_before = 0;
    for (int l0 = 0; l0 < C; l0 += kTierThreads) {
        const int l = l0 + tid;
        const bool fr = l < C && (ls[l] < 0 || ls[l] >= M);
        int nf;
        const int r = tier_excl_scan(fr ? 1 : 0, wtot, nf) + nfree_before;
        nfree_before += nf;
        if (fr) freelist[r] = l;
    }
    __syncthreads();

    // 4. entering slots take the free lines in slot order; their rows come in
    int nin_before = 0;
    for (int64_t s0 = 0; s0 < M; s0 += kTierThreads) {
        const int64_t s = s0 + tid;
        bool in = false;
        if (s < M) in = (hits[s] & kChosen) && line_of(s) < 0;
        int nin;
        const int r = tier_excl_scan(in ? 1 : 0, wtot, nin) + nin_before;
        nin_before += nin;
        int line = -1;
        if (in && r < nfree_before) {
            line = freelist[r];
            sl[s] = line;
            ls[line] = static_cast<int32_t>(s);
        }
        const uint64_t mv = __ballot(line >= 0);
        const int lane = tid % kWave, g = lane / 16, gl = lane % 16;
        uint64_t rest = mv;
        int n = 0;
        while (rest) {
            const int src = __builtin_ctzll(rest);
            rest &= rest - 1;
            const int ln = __shfl(line, src, kWave);
            if (n % 4 == g) {
                const int64_t slot = s0 + (tid - lane) + src;
                copy_row(cache + static_cast<int64_t>(ln) * rb, host + slot * rb, rb, gl);
            }
            ++n;
        }
    }
    __syncthreads();

    // 5. counts halved, marks cleared
    for (int64_t s = tid; s < M; s += kTierThreads) hits[s] = (hits[s] & ~kChosen) >> 1;
}

__global__ __launch_bounds__(256) void tier_reset_kernel(TierArgs a) {
    const int64_t ns = static_cast<int64_t>(a.units) * a.M, nl = static_cast<int64_t>(a.units) * a.C;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < ns;
         i += static_cast<int64_t>(gridDim.x) * 256) {
        a.slot_line[i] = -1;
        a.hits[i] = 0;
    }
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < nl;
         i += static_cast<int64_t>(gridDim.x) * 256)
        a.line_slot[i] = -1;
}

// One group of 16 lanes per line: a filled line's row goes back to host.
__global__ __launch_bounds__(256) void tier_flush_kernel(TierArgs a) {
    const int rb = a.d_v * (a.state_bf16 ? 2 : 4);
    const int64_t nl = static_cast<int64_t>(a.units) * a.C;
    const int gl = threadIdx.x % 16;
    for (int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) / 16; i < nl;
         i += static_cast<int64_t>(gridDim.x) * 16) {
        const int slot = a.line_slot[i];
        if (slot < 0 || slot >= a.M) continue;
        const int64_t unit = i / a.C;
        copy_row(static_cast<char *>(a.S_host) + (unit * a.M + slot) * rb,
                 static_cast<const char *>(a.cache) + i * rb, rb, gl);
    }
}

unsigned grid_of(int64_t n) { return static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 8192)); }

}  // namespace

hipError_t launch_tier_reset(const TierArgs &a, hipStream_t st) {
    if (a.units == 0) return hipSuccess;
    hipLaunchKernelGGL(tier_reset_kernel, dim3(grid_of(static_cast<int64_t>(a.units) * a.M)), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_tier_rebalance(const TierArgs &a, hipStream_t st) {
    if (a.units == 0) return hipSuccess;
    const size_t lds = static_cast<size_t>(a.C) * 4;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(tier_rebalance_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(tier_rebalance_kernel, dim3(a.units), dim3(kTierThreads), lds, st, a);
    return hipGetLastError();
}

hipError_t launch_tier_flush(const TierArgs &a, hipStream_t st) {
    if (a.units == 0) return hipSuccess;
    hipLaunchKernelGGL(tier_flush_kernel, dim3(grid_of(static_cast<int64_t>(a.units) * a.C * 16)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace ramnet
