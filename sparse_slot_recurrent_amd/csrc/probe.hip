// Device peak probes for the benchmark (not part of the RAM-Net C ABI):
// measured HBM copy bandwidth and LDS read bandwidth, against which the
// benchmark reports its roofline fractions next to the vendor's figures.
//
//   probe_hbm_copy: dst = src over n 16-byte words, a grid-stride copy with
//     one 16-byte load and store per lane and iteration (HBM bytes moved:
//     2 n 16, read and write).
//   probe_lds_read: every workgroup fills 16 KiB of LDS, then each lane
//     reads 16 bytes per instruction (ds_read_b128, lanes on consecutive
//     16-byte words: no bank conflicts) `iters` x 16 times; the XOR of what
//     it read goes to out[] so that no read can be dropped.  LDS bytes read:
//     blocks x threads x iters x 16 x 16.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void hbm_copy_kernel(const uint4 *__restrict__ src,
                                                       uint4 *__restrict__ dst, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

constexpr int kLdsBytes = 16 * 1024;
constexpr int kLdsThreads = 256;

__global__ __launch_bounds__(kLdsThreads) void lds_read_kernel(int iters, uint32_t *__restrict__ out) {
    __shared__ __align__(16) uint4 buf[kLdsBytes / 16];
    const int tid = threadIdx.x;
    for (int i = tid; i < kLdsBytes / 16; i += kLdsThreads)
        buf[i] = make_uint4(i, i * 3u + 1u, i * 5u + 2u, i * 7u + blockIdx.x);
    __syncthreads();
    uint4 acc = make_uint4(0, 0, 0, 0);
    // the 16 unrolled reads of a lane are 64 words (1 KiB) apart, so no two
    // of them read the same word (16 x 64 = 1024 words, the buffer); each
    // iteration starts 16 words further on; the mask keeps every address
    // inside the buffer
    int idx = tid;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint4 u = buf[(idx + j * 64) & (kLdsBytes / 16 - 1)];
            acc.x ^= u.x;
            acc.y ^= u.y;
            acc.z ^= u.z;
            acc.w ^= u.w;
        }
        idx = (idx + 16) & (kLdsBytes / 16 - 1);
    }
    out[static_cast<int64_t>(blockIdx.x) * kLdsThreads + tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" {

// n16: number of 16-byte words; src and dst 16-byte aligned device buffers.
int probe_hbm_copy(const void *src, void *dst, int64_t n16, int blocks, void *stream) {
    if (!src || !dst || n16 <= 0 || blocks <= 0) return -1;
    hipLaunchKernelGGL(hbm_copy_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), n16);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

// out: blocks * 256 uint32 words of device memory.
int probe_lds_read(int blocks, int iters, uint32_t *out, void *stream) {
    if (!out || blocks <= 0 || iters <= 0) return -1;
    hipLaunchKernelGGL(lds_read_kernel, dim3(blocks), dim3(kLdsThreads), 0,
                       static_cast<hipStream_t>(stream), iters, out);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int probe_threads_per_lds_block(void) { return kLdsThreads; }

}  // extern "C"
