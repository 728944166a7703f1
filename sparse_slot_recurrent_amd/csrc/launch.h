// Internal launcher interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

namespace ramnet {

// Address Decoder over n = B*T*H addresses of both q (read) and k (write).
struct DecodeArgs {
    const void *q, *k;
    int64_t n;
    int T, H, U, K, d_p;
    const int32_t *pos0;  // position of token t of sequence b: pos0[b] + t
    int cape;               // 0 off, 1..3 the CAPE reading
    uint64_t content_heads;  // bit h: head h is content-only (bit 63 for h >= 63)
    int64_t M;
    bool in_bf16;
    bool unit_major;  // write addresses as [B,H,T,K] (else [B,T,H,K])
    int64_t ld;       // elements between tokens (b, t) of q and k; 0: H*U*d_p
    int32_t *w_idx, *r_idx;
    float *w_wt, *r_wt;
    // NULL: every address is searched in fp64.  Else (bf16 logits, K <= 32)
    // scratch of decode_fails_bytes(n): the search runs in fixed point,
    // exact, and the few addresses whose logits span too many binary orders
    // for 32-bit drops are marked there and searched in fp64; the slots are
    // the same either way.
    unsigned long long *fails;
};
// Scratch of the fixed-point search for n addresses (of each of q and k):
// one failure word per wave.
size_t decode_fails_bytes(int64_t n);
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
    bool addr_unit_major;  // addresses are [B,H,T,K] (else [B,T,H,K])
    void *S;
    float *mass;
    void *out;
    void *out_bf16;  // chunked path: if set, the normalised output goes here as
                     // bf16 instead of to out (out still holds r meanwhile)
    float eps_gsu, eps_norm;
    // elements between tokens (b, t) of v, g and gamma; 0: contiguous
    // (H*d_v, H*d_v, H).  Head h of a token starts at h*d_v (h for gamma).
    int64_t ld_v, ld_g, ld_gamma;
};
// LDS bytes the serial scan needs to keep one head's state on chip, and
// whether that fits a workgroup.
size_t scan_state_lds_bytes(int64_t M, int d_v, bool state_bf16);
bool scan_state_fits_lds(int64_t M, int d_v, bool state_bf16);
hipError_t launch_scan_serial(const ScanArgs &a, hipStream_t st);

// Slot-grouped chunked recurrence, in three kernels: a plan kernel groups
// every chunk's events by slot (all chunks at once, they do not depend on
// the state), the scan kernel replays the plans chunk after chunk, and an
// epilogue applies RMSNorm and the gate.  Rows on chip (M <= 1024,
// scan_chunked.hip): one workgroup per (unit, channel slice); r (fp32
// [B,T,H,d_v]) and per-slice square sums ([B,T,H,d_v/CG]) pass through
// global memory between the last two.
// Rows in HBM (M > 1024): the slot-range path (scan_ranges.hip).  The slots
// of a unit are split into kRanges ranges (slot mod kRanges); one workgroup
// per (unit, range) gathers, updates and writes back whole rows of its
// range and sums its part of every token's read, the partial sums of the
// ranges are added by an epilogue that applies RMSNorm and the gate.
constexpr int kRanges = 8;

struct ChunkPlan {
    bool ok;
    bool resident;      // slot rows live in registers (M <= 1024); else in HBM (slot ranges)
    int CG;             // channels per slice
    int C;              // tokens per chunk
    int EV;             // C * K: events of one kind per chunk
    int ENT;            // most slots one chunk touches
    int ENTA;           // ENT rounded up to 64 (stride of the entry arrays)
    int HT;             // rows in HBM: plan hash table size, 0: the slot is its own index
    int ncg;            // d_v / CG
    int RG;             // lanes per token in the read reduction
    bool raw_values;    // values kept in LDS as the bf16 input (else fp32)
    // Resident mode: a slot with more than n0 writes in a chunk may be handed
    // off after its first n0 writes to one of at most HMAX helper threads
    // (busiest slots first), so that no wave waits on its busiest slot.
    int n0;
    int HMAX;
    int64_t n_chunks;
    // rows in HBM: per range, the write and read lists staged in LDS (longer
    // lists are read from the record), and the version rows held in LDS
    // (later ones go to a spill area in the workspace)
    int CAPW, CAPR, VCAP;
    int MSL;  // > 0: the masses of a range's slots (M / kRanges) live in LDS for the whole scan
    // one (unit, chunk) plan record and its sections (byte offsets)
    size_t rec_bytes, o_ent, o_map, o_hl, o_wtv, o_ww, o_wa, o_rv, o_rr, o_rt;
    size_t lds_plan, lds_scan;
    size_t ws_rbuf, ws_sumsq, ws_mass, ws_plan;  // workspace section sizes
    size_t ws_partial, ws_spill;                 // rows in HBM: partial reads, spilled versions
};

struct ChunkArgs : ScanArgs {
    ChunkPlan p;
    float *rbuf;     // may alias out when the output is fp32
    float *sumsq;
    float *mass_ws;  // rows on chip: final mass [units][M]
    unsigned char *plan;
    float *partial;  // rows in HBM: [B,T,H][kRanges][d_v] partial reads (fp16 for a bf16 state)
    void *spill;     // rows in HBM: [units][kRanges][EV][d_v] version rows beyond VCAP
};

constexpr size_t kChunkLdsLimit = 160 * 1024;
// Token groups of the backward's output/read kernel: each (unit, group)
// leaves one partial of d omega in the workspace.
constexpr int kBwdOutBlocks = 16;

ChunkPlan plan_chunked(int64_t M, int K, int d_v, int B, int T, int H, bool in_bf16,
                       bool state_bf16);
// The rows-in-HBM plan (M > 1024) and launch (scan_ranges.hip).
ChunkPlan plan_ranges(int64_t M, int K, int d_v, int B, int T, int H, bool in_bf16,
                      bool state_bf16);
hipError_t launch_scan_ranges(const ChunkArgs &a, hipStream_t st);
// Workspace bytes of the chunked path beyond the addresses.
size_t chunk_workspace_bytes(const ChunkPlan &p);
hipError_t launch_scan_chunked(const ChunkArgs &a, hipStream_t st);

// One fused decoding step (decode + CAPE + GSU + read + norm + gate).
struct StepArgs {
    int B, H;
    int64_t M;
    int K, d_v, U, d_p, cape;
    uint64_t content_heads;
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
    // elements between sequences b of q and k, v, g, gamma; 0: contiguous
    int64_t ld_qk, ld_v, ld_g, ld_gamma;
    // tiered state (cache != NULL): S is the host copy, cached slots' rows
    // live in cache [units][C][d_v] at line slot_line[unit][slot]; hits
    // counts each accessed slot
    void *cache;
    const int32_t *slot_line;
    uint32_t *hits;
    int C;
};
bool step_fused_supported(int K, int d_p, int U, int d_v, bool state_bf16);
hipError_t launch_step_fused(const StepArgs &a, hipStream_t st);

// Tiered state maintenance (tier.hip).
struct TierArgs {
    int units, C, d_v;
    int64_t M;
    bool state_bf16;
    void *S_host, *cache;
    int32_t *line_slot, *slot_line;
    uint32_t *hits;
};
hipError_t launch_tier_reset(const TierArgs &a, hipStream_t st);
hipError_t launch_tier_rebalance(const TierArgs &a, hipStream_t st);
hipError_t launch_tier_flush(const TierArgs &a, hipStream_t st);

// Backward pass of the recurrence (backward.hip), given the forward's
// addresses; gradients in fp32.  d_v = 64 with M <= 1024 takes the
// slot-owner kernels (state on chip); every other shape the per-token walk
// with the state in HBM.
struct BwdArgs {
    int B, T, H;
    int64_t M;
    int K, U, d_p, cape, d_v;
    uint64_t content_heads;
    bool in_bf16, state_bf16;
    float eps_gsu, eps_norm;
    const void *q, *k, *v, *gamma, *g;
    const float *norm_w;
    const int32_t *pos0;
    const void *S0;  // state dtype
    const float *mass0;
    const int32_t *w_idx, *r_idx;
    const float *w_wt, *r_wt;
    const float *dout, *dS_final, *dmass_final;
    float *dq, *dk, *dv, *dgamma, *dg, *dnorm_w, *dS0, *dmass0;
    // workspace: per token-head records and weight gradients, per unit d omega
    float *rec_w, *rec_r, *rec_m, *dw, *drho, *dom_part, *dr, *dvk, *dgk;
    // per-token walk only: the replayed state [units][M][d_v] (state dtype)
    // and mass [units][M]
    void *Sw;
    float *mw;
};
bool backward_supported(int64_t M, int d_v, int U, int d_p, bool state_bf16);
// Whether the slot-owner kernels serve this shape (else the per-token walk).
bool backward_slot_owner(int64_t M, int d_v);
size_t backward_workspace_bytes(int B, int T, int H, int K, int64_t M, int d_v, bool state_bf16);
hipError_t launch_backward(const BwdArgs &a, hipStream_t st);

// Dense projections around the layer (proj.hip).
constexpr size_t kGemmWorkspace = size_t(32) << 20;  // hipBLASLt scratch per call
// Row-major C[m,n] = A[m,k] W[n,k]^T (W as [out, in]): bf16 in and out,
// fp32 accumulation.
// Returns false with a message in err.
bool gemm_bf16(const void *A, const void *B, void *C, int64_t m, int64_t n, int64_t k,
               void *ws, hipStream_t st, std::string &err);
// Creates the device's handle and picks the algorithm for a shape, so that
// a sequence of GEMMs can be validated before any of it is enqueued.
bool gemm_prepare(int64_t m, int64_t n, int64_t k, std::string &err);
// Row layout of the packed input weights [N, D] (= column layout of the
// packed projections [rows, N]): q at 0, k at o_k, v at o_v, g at o_g, gamma
// at o_gamma; every block starts at a multiple of 8, padding is zero.
struct PackLayout {
    int64_t D;
    int H, L, HL, HV;
    int o_k, o_v, o_g, o_gamma, N;
};
PackLayout pack_layout(int H, int L, int d_v, int64_t D);
// Packs w_q, w_k (tempered by e^alpha, if alpha is set), w_v, w_g, w_gamma.
hipError_t launch_pack(const void *wq, const void *wk, const void *wv, const void *wg,
                       const void *wgam, const float *alpha, void *out, const PackLayout &pl,
                       hipStream_t st);
// Packed projections [rows, N] -> contiguous q, k, v, g, gamma.
hipError_t launch_split(const void *in, void *q, void *k, void *v, void *g, void *gam,
                        int64_t rows, const PackLayout &pl, hipStream_t st);
hipError_t launch_to_bf16(const float *in, void *out, int64_t n, hipStream_t st);

}  // namespace ramnet
