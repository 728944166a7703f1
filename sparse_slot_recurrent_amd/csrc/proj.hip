// Dense steps either side of the RAM-Net layer (RAM-Net project page, the
// layer outline: the token is projected to key, query, value and the GSU's
// gamma; the gated read is projected out).
//
//   temper_kernel   the re-parameterised address weights W = e^alpha W' of
//                   the paper digest's stability note: the q and k columns of
//                   head h are scaled by t_h = fp32(e^alpha_h) and rounded to
//                   bf16 once, from the exact product (a bf16 times an fp32
//                   has at most 32 significant bits, so fp64 holds it).
//   gemm_bf16       row-major C[m,n] = A[m,k] B[k,n], bf16 operands, fp32
//                   accumulation, C rounded to bf16: hipBLASLt on the matrix
//                   cores, one handle per device and one cached algorithm
//                   per shape.
//   to_bf16_kernel  fp32 layer output -> bf16, when the scan could not write
//                   bf16 itself.
#include <hipblaslt/hipblaslt.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <tuple>

#include "device_common.h"
#include "launch.h"

namespace ramnet {
namespace {

// Nearest bf16, ties to even, of a finite fp64 value in fp32's normal
// range: clear the 45 low mantissa bits with rounding, after which the value
// has 8 significant bits and converts to fp32 exactly.
__device__ __forceinline__ bf16_t bf16_of_double(double d) {
    uint64_t u = static_cast<uint64_t>(__double_as_longlong(d));
    const uint64_t lsb = (u >> 45) & 1;
    u += (uint64_t(1) << 44) - 1 + lsb;
    u &= ~((uint64_t(1) << 45) - 1);
    const float f = static_cast<float>(__longlong_as_double(static_cast<long long>(u)));
    return bf16_t{static_cast<uint16_t>(__float_as_uint(f) >> 16)};
}

__global__ __launch_bounds__(256) void temper_kernel(const bf16_t *__restrict__ wp,
                                                     const float *__restrict__ alpha,
                                                     bf16_t *__restrict__ w, int64_t n,
                                                     int cols, int L) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += stride) {
        const int h = static_cast<int>(i % cols) / L;
        const float t = static_cast<float>(exp(static_cast<double>(alpha[h])));
        w[i] = bf16_of_double(static_cast<double>(to_f32(wp[i])) * static_cast<double>(t));
    }
}

struct Quad4 {
    float e[4];
};
struct Bf4 {
    bf16_t e[4];
};

__global__ __launch_bounds__(256) void to_bf16_kernel(const float *__restrict__ in,
                                                      bf16_t *__restrict__ out, int64_t n4) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4;
         i += stride) {
        const Quad4 x = reinterpret_cast<const Quad4 *>(in)[i];
        Bf4 y;
#pragma unroll
        for (int j = 0; j < 4; ++j) y.e[j] = bf16_rne(x.e[j]);
        reinterpret_cast<Bf4 *>(out)[i] = y;
    }
}

unsigned grid_for(int64_t n) {
    return static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 8192));
}

// ---------------------------------------------------------------- hipBLASLt

struct GemmPlan {
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
    hipblasLtMatmulAlgo_t algo{};
    size_t ws = 0;
};

std::mutex g_mu;
std::map<int, hipblasLtHandle_t> g_handles;
std::map<std::tuple<int, int64_t, int64_t, int64_t>, GemmPlan> g_plans;

std::string blas_err(const char *what, hipblasStatus_t s) {
    return std::string(what) + " failed (hipBLASLt status " + std::to_string(static_cast<int>(s)) + ")";
}

// Plan for row-major C[m,n] = A[m,k] B[k,n].  hipBLASLt is column-major, so
// the call computes C^T[n,m] = B^T[n,k] A^T[k,m]: its first operand is B
// (n x k, leading dimension n), its second A (k x m, leading dimension k).
bool gemm_plan(int dev, int64_t m, int64_t n, int64_t k, hipblasLtHandle_t &h, GemmPlan &out,
               std::string &err) {
    std::lock_guard<std::mutex> lock(g_mu);
    auto hi = g_handles.find(dev);
    if (hi == g_handles.end()) {
        hipblasLtHandle_t nh = nullptr;
        const hipblasStatus_t s = hipblasLtCreate(&nh);
        if (s != HIPBLAS_STATUS_SUCCESS) {
            err = blas_err("hipblasLtCreate", s);
            return false;
        }
        hi = g_handles.emplace(dev, nh).first;
    }
    h = hi->second;
    const auto key = std::make_tuple(dev, m, n, k);
    auto pi = g_plans.find(key);
    if (pi != g_plans.end()) {
        out = pi->second;
        return true;
    }
    GemmPlan p;
    hipblasStatus_t s = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F);
    const hipblasOperation_t op = HIPBLAS_OP_N;
    if (s == HIPBLAS_STATUS_SUCCESS)
        s = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &op, sizeof(op));
    if (s == HIPBLAS_STATUS_SUCCESS)
        s = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &op, sizeof(op));
    if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, n, k, n);
    if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, k, m, k);
    if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatrixLayoutCreate(&p.lc, HIP_R_16BF, n, m, n);
    if (s != HIPBLAS_STATUS_SUCCESS) {
        err = blas_err("hipBLASLt descriptor setup", s);
        return false;
    }
    hipblasLtMatmulPreference_t pref = nullptr;
    s = hipblasLtMatmulPreferenceCreate(&pref);
    uint64_t max_ws = kGemmWorkspace;
    if (s == HIPBLAS_STATUS_SUCCESS)
        s = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                  &max_ws, sizeof(max_ws));
    hipblasLtMatmulHeuristicResult_t res[1];
    int got = 0;
    if (s == HIPBLAS_STATUS_SUCCESS)
        s = hipblasLtMatmulAlgoGetHeuristic(h, p.desc, p.la, p.lb, p.lc, p.lc, pref, 1, res, &got);
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (s != HIPBLAS_STATUS_SUCCESS || got < 1 || res[0].state != HIPBLAS_STATUS_SUCCESS) {
        err = s != HIPBLAS_STATUS_SUCCESS ? blas_err("hipblasLtMatmulAlgoGetHeuristic", s)
                                          : std::string("hipBLASLt has no algorithm for a bf16 GEMM of ") +
                                                std::to_string(m) + "x" + std::to_string(n) + "x" +
                                                std::to_string(k);
        return false;
    }
    p.algo = res[0].algo;
    p.ws = res[0].workspaceSize;
    g_plans.emplace(key, p);
    out = p;
    return true;
}

}  // namespace

bool gemm_bf16(const void *A, const void *B, void *Cm, int64_t m, int64_t n, int64_t k,
               void *ws, hipStream_t st, std::string &err) {
    if (m == 0 || n == 0) return true;
    int dev = 0;
    const hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) {
        err = std::string("hipGetDevice: ") + hipGetErrorString(he);
        return false;
    }
    hipblasLtHandle_t h;
    GemmPlan p;
    if (!gemm_plan(dev, m, n, k, h, p, err)) return false;
    const float one = 1.0f, zero = 0.0f;
    const hipblasStatus_t s = hipblasLtMatmul(h, p.desc, &one, B, p.la, A, p.lb, &zero, Cm, p.lc,
                                              Cm, p.lc, &p.algo, ws, p.ws, st);
    if (s != HIPBLAS_STATUS_SUCCESS) {
        err = blas_err("hipblasLtMatmul", s);
        return false;
    }
    return true;
}

bool gemm_prepare(int64_t m, int64_t n, int64_t k, std::string &err) {
    if (m == 0 || n == 0) return true;
    int dev = 0;
    const hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) {
        err = std::string("hipGetDevice: ") + hipGetErrorString(he);
        return false;
    }
    hipblasLtHandle_t h;
    GemmPlan p;
    return gemm_plan(dev, m, n, k, h, p, err);
}

hipError_t launch_temper(const void *wp, const float *alpha, void *w, int64_t rows, int cols,
                         int L, hipStream_t st) {
    const int64_t n = rows * cols;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(temper_kernel, dim3(grid_for(n)), dim3(256), 0, st,
                       static_cast<const bf16_t *>(wp), alpha, static_cast<bf16_t *>(w), n, cols, L);
    return hipGetLastError();
}

hipError_t launch_to_bf16(const float *in, void *out, int64_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    if (n % 4) return hipErrorInvalidValue;
    hipLaunchKernelGGL(to_bf16_kernel, dim3(grid_for(n / 4)), dim3(256), 0, st, in,
                       static_cast<bf16_t *>(out), n / 4);
    return hipGetLastError();
}

}  // namespace ramnet
