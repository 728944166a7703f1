// Dense steps either side of the RAM-Net layer (RAM-Net project page, the
// layer outline: the token is projected to key, query, value and the GSU's
// gamma; the gated read is projected out).
//
//   pack_kernel     the five input weights stacked in one [N, D] bf16
//                   matrix, so that one GEMM projects a token to all of q, k,
//                   v, g and gamma; the q and k columns carry the
//                   re-parameterised address weights W = e^alpha W' of the
//                   AI Radio page's stability remark: head h's columns are
//                   scaled by t_h = fp32(e^alpha_h) and rounded to bf16 once,
//                   from the exact product (a bf16 times an fp32 has at most
//                   32 significant bits, so fp64 holds it).
//   split_kernel    the packed projections back into five contiguous
//                   tensors (for ramnet_project_inputs).
//   gemm_bf16       row-major C[m,n] = A[m,k] W[n,k]^T, bf16 operands, fp32
//                   accumulation, C rounded to bf16: hipBLASLt on the matrix
//                   cores, one handle per device, with the library's first
//                   heuristic choice of algorithm (the same in every
//                   process).  Opt-in (RAMNET_GEMM_TUNE=1 in the
//                   environment): the first call of a shape outside graph
//                   capture times hipBLASLt's candidates on the call's own
//                   operands, synchronising the host, and keeps the fastest
//                   for the process.
//   to_bf16_kernel  fp32 layer output -> bf16, when the scan could not write
//                   bf16 itself.
#include <hipblaslt/hipblaslt.h>

#include <algorithm>
#include <stdlib.h>

#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

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

__device__ __forceinline__ bf16_t temper(bf16_t w, const float *alpha, int h) {
    if (!alpha) return w;
    const float t = static_cast<float>(exp(static_cast<double>(alpha[h])));
    return bf16_of_double(static_cast<double>(to_f32(w)) * static_cast<double>(t));
}

// Weights are [out, in] row-major (each output's weights contiguous over
// the D inputs), so the packed matrix is the five weight matrices' rows one
// after another, [N, D].
__global__ __launch_bounds__(256) void pack_kernel(const bf16_t *__restrict__ wq,
                                                   const bf16_t *__restrict__ wk,
                                                   const bf16_t *__restrict__ wv,
                                                   const bf16_t *__restrict__ wg,
                                                   const bf16_t *__restrict__ wgam,
                                                   const float *__restrict__ alpha,
                                                   bf16_t *__restrict__ out, PackLayout pl) {
    const int64_t n = pl.D * pl.N;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += stride) {
        const int r = static_cast<int>(i / pl.D);  // packed row = output column
        const int64_t c = i - static_cast<int64_t>(r) * pl.D;
        bf16_t val{0};
        if (r < pl.o_k) {
            if (r < pl.HL) val = temper(wq[static_cast<int64_t>(r) * pl.D + c], alpha, r / pl.L);
        } else if (r < pl.o_v) {
            const int j = r - pl.o_k;
            if (j < pl.HL) val = temper(wk[static_cast<int64_t>(j) * pl.D + c], alpha, j / pl.L);
        } else if (r < pl.o_g) {
            val = wv[static_cast<int64_t>(r - pl.o_v) * pl.D + c];
        } else if (r < pl.o_gamma) {
            val = wg[static_cast<int64_t>(r - pl.o_g) * pl.D + c];
        } else {
            const int j = r - pl.o_gamma;
            if (j < pl.H) val = wgam[static_cast<int64_t>(j) * pl.D + c];
        }
        out[i] = val;
    }
}

__global__ __launch_bounds__(256) void split_kernel(const bf16_t *__restrict__ in,
                                                    bf16_t *__restrict__ q, bf16_t *__restrict__ k,
                                                    bf16_t *__restrict__ v, bf16_t *__restrict__ g,
                                                    bf16_t *__restrict__ gam, int64_t rows,
                                                    PackLayout pl) {
    const int64_t n = rows * pl.N;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += stride) {
        const int64_t r = i / pl.N;
        const int c = static_cast<int>(i - r * pl.N);
        const bf16_t x = in[i];
        if (c < pl.o_k) {
            if (c < pl.HL) q[r * pl.HL + c] = x;
        } else if (c < pl.o_v) {
            if (c - pl.o_k < pl.HL) k[r * pl.HL + (c - pl.o_k)] = x;
        } else if (c < pl.o_g) {
            v[r * pl.HV + (c - pl.o_v)] = x;
        } else if (c < pl.o_gamma) {
            g[r * pl.HV + (c - pl.o_g)] = x;
        } else if (c - pl.o_gamma < pl.H) {
            gam[r * pl.H + (c - pl.o_gamma)] = x;
        }
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
    std::vector<hipblasLtMatmulHeuristicResult_t> cands;  // library order
    bool tuned = false;
};

constexpr int kCandidates = 24;

// Timing hipBLASLt's candidates is opt-in: it blocks the host, and the pick
// (hence the rounding of the sums) can differ between processes.
bool tuning_enabled() {
    const char *e = getenv("RAMNET_GEMM_TUNE");
    return e && e[0] == '1';
}

std::mutex g_mu;
std::map<int, hipblasLtHandle_t> g_handles;
std::map<std::tuple<int, int64_t, int64_t, int64_t>, GemmPlan> g_plans;

std::string blas_err(const char *what, hipblasStatus_t s) {
    return std::string(what) + " failed (hipBLASLt status " + std::to_string(static_cast<int>(s)) + ")";
}

// Plan for row-major C[m,n] = A[m,k] W[n,k]^T.  hipBLASLt is column-major,
// so the call computes C^T[n,m] = W[n,k] A^T[k,m]: its first operand is W
// stored k x n (leading dimension k) and transposed, its second A stored
// k x m (leading dimension k).  Both operands run contiguously along k.
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
    const hipblasOperation_t opa = HIPBLAS_OP_T, opb = HIPBLAS_OP_N;
    if (s == HIPBLAS_STATUS_SUCCESS)
        s = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opa, sizeof(opa));
    if (s == HIPBLAS_STATUS_SUCCESS)
        s = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opb, sizeof(opb));
    if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, k, n, k);
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
    hipblasLtMatmulHeuristicResult_t res[kCandidates];
    int got = 0;
    if (s == HIPBLAS_STATUS_SUCCESS)
        s = hipblasLtMatmulAlgoGetHeuristic(h, p.desc, p.la, p.lb, p.lc, p.lc, pref,
                                            tuning_enabled() ? kCandidates : 1, res, &got);
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
    for (int i = 0; i < got; ++i)
        if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize <= kGemmWorkspace)
            p.cands.push_back(res[i]);
    p.tuned = p.cands.size() <= 1;
    g_plans.emplace(key, p);
    out = p;
    return true;
}

// Times every candidate on the call's operands (one warm-up and three timed
// runs each, on the call's stream) and returns the fastest; C is written by
// every run, the last write being the caller's own GEMM that follows.
bool tune(hipblasLtHandle_t h, GemmPlan &p, const void *A, const void *B, void *Cm, void *ws,
          hipStream_t st, std::string &err) {
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        err = "hipEventCreate failed";
        return false;
    }
    const float one = 1.0f, zero = 0.0f;
    float best = 0.f;
    int best_i = -1;
    for (size_t i = 0; i < p.cands.size(); ++i) {
        const hipblasLtMatmulHeuristicResult_t &c = p.cands[i];
        hipblasStatus_t s = HIPBLAS_STATUS_SUCCESS;
        for (int r = 0; r < 4 && s == HIPBLAS_STATUS_SUCCESS; ++r) {
            if (r == 1 && hipEventRecord(e0, st) != hipSuccess) s = HIPBLAS_STATUS_INTERNAL_ERROR;
            s = hipblasLtMatmul(h, p.desc, &one, B, p.la, A, p.lb, &zero, Cm, p.lc, Cm, p.lc,
                                &c.algo, ws, c.workspaceSize, st);
        }
        if (hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) {
            err = "hipEventSynchronize failed while timing GEMM algorithms";
            (void)hipEventDestroy(e0);
            (void)hipEventDestroy(e1);
            return false;
        }
        float ms = 0.f;
        if (s != HIPBLAS_STATUS_SUCCESS || hipEventElapsedTime(&ms, e0, e1) != hipSuccess) continue;
        if (best_i < 0 || ms < best) {
            best = ms;
            best_i = static_cast<int>(i);
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (best_i >= 0) {
        p.algo = p.cands[best_i].algo;
        p.ws = p.cands[best_i].workspaceSize;
    }
    p.tuned = true;
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
    if (!p.tuned) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(st, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone) {
            if (!tune(h, p, A, B, Cm, ws, st, err)) return false;
            std::lock_guard<std::mutex> lock(g_mu);
            GemmPlan &q = g_plans[std::make_tuple(dev, m, n, k)];
            q.algo = p.algo;
            q.ws = p.ws;
            q.tuned = true;
        }
    }
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

PackLayout pack_layout(int H, int L, int d_v, int64_t D) {
    auto pad8 = [](int x) { return (x + 7) & ~7; };
    PackLayout pl{};
    pl.D = D;
    pl.H = H;
    pl.L = L;
    pl.HL = H * L;
    pl.HV = H * d_v;
    pl.o_k = pad8(pl.HL);
    pl.o_v = pl.o_k + pad8(pl.HL);
    pl.o_g = pl.o_v + pl.HV;
    pl.o_gamma = pl.o_g + pl.HV;
    pl.N = pad8(pl.o_gamma + H);
    return pl;
}

hipError_t launch_pack(const void *wq, const void *wk, const void *wv, const void *wg,
                       const void *wgam, const float *alpha, void *out, const PackLayout &pl,
                       hipStream_t st) {
    const int64_t n = pl.D * pl.N;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_kernel, dim3(grid_for(n)), dim3(256), 0, st,
                       static_cast<const bf16_t *>(wq), static_cast<const bf16_t *>(wk),
                       static_cast<const bf16_t *>(wv), static_cast<const bf16_t *>(wg),
                       static_cast<const bf16_t *>(wgam), alpha, static_cast<bf16_t *>(out), pl);
    return hipGetLastError();
}

hipError_t launch_split(const void *in, void *q, void *k, void *v, void *g, void *gam,
                        int64_t rows, const PackLayout &pl, hipStream_t st) {
    const int64_t n = rows * pl.N;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(split_kernel, dim3(grid_for(n)), dim3(256), 0, st,
                       static_cast<const bf16_t *>(in), static_cast<bf16_t *>(q),
                       static_cast<bf16_t *>(k), static_cast<bf16_t *>(v),
                       static_cast<bf16_t *>(g), static_cast<bf16_t *>(gam), rows, pl);
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
