// Internal declarations shared by the host API (pw_api.cpp) and the gfx950
// kernels (pw_kernels.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pw {

// One entry of the device page table: the pages of one (expert, linear) block
// at its planned bitwidth. 80 bytes, read with scalar loads by the kernels.
struct DevBlock {
    uint64_t planes[8];  // device addresses of planes 0..bits-1 (rest 0)
    uint64_t lut;        // device address of LUT_bits, R * 2^bits fp16
    int32_t bits;        // 1..8
    int32_t pad;
};
static_assert(sizeof(DevBlock) == 80, "DevBlock layout");

// Workspace carved out of one device allocation per layer.
struct Workspace {
    int64_t* logits;     // [max_T][E]   exact logits, units of 2^-48
    int32_t* ids;        // [max_T][k]
    float* w;            // [max_T][k]
    int32_t* counts;     // [E]
    int32_t* offsets;    // [E+1]
    int32_t* sorted;     // [max_T*k]    assignment t*k+j, grouped by expert
    uint16_t* xperm;     // [max_T][d]   x with columns permuted inside 32-groups
    uint16_t* act;       // [max_T*k + max_T*has_shared][F_max]  SwiGLU output, permuted
    uint32_t* tok_cnt;   // [max_T]      per-token arrival counters (last-block pattern)
    uint32_t* glob_cnt;  // [1]          per-call arrival counter
    uint32_t* status;    // [1]          PW_STATUS_* bits
};

struct RouteParams {
    const uint16_t* x;
    const uint16_t* wr;
    const uint16_t* bias;  // may be null
    int T, d, E, k;
    int n_eg;              // expert groups (grid.x)
    int epb;               // experts per group
    Workspace ws;
    float* y;              // zeroed here
    // optional caller copies of the routing outputs
    int32_t* o_ids;
    float* o_w;
    int32_t* o_counts;
    int32_t* o_offsets;
    int32_t* o_sorted;
};

// Dequantising GEMM over (expert, row tile, token group) work items.
// gate_up: set 0 = gate rows [f0, f0+32), set 1 = up rows [f0, f0+32), K = d,
//          B = xperm rows (tokens), epilogue SwiGLU -> act.
// down:    set 0 = down rows [r0, r0+32), set 1 = rows [r0+32, r0+64), K = F,
//          B = act rows (slots), epilogue w * o atomically added to y.
struct GemmParams {
    const DevBlock* blocks;   // [n_total*3]
    int E, k, T, d;
    int F, Fs;                // routed / shared ffn (Fs = 0: none)
    int tiles_r, tiles_s;     // row tiles per routed expert / for the shared expert
    int n_work;               // E*tiles_r + tiles_s (grid.x may be padded above it)
    Workspace ws;
    int ld_act;               // row stride of act (F_max)
    int shared_base;          // first act row of the shared expert (max_T*k)
    int lds_stripe;           // LDS bytes reserved for the LUT stripe / reduction
    int min_count;            // work items with fewer tokens than this exit
    int max_count;            // work items with more tokens than this exit
    float* y;
};

hipError_t launch_init_ws(const Workspace& ws, int max_T, hipStream_t s);
hipError_t launch_route(const RouteParams& p, hipStream_t s);
// tile_tokens: 32 (one MFMA token tile per work item) or 128 (four tiles).
hipError_t launch_gemm(int mode, int tile_tokens, const GemmParams& p, int lds_bytes,
                       int n_zgroups, hipStream_t s);
hipError_t launch_residual(const uint16_t* x, const float* y, uint16_t* x_next, long n,
                           hipStream_t s);
hipError_t launch_debug(const uint64_t* planes8, int b, const uint16_t* lut, int R, int K,
                        uint8_t* idx_out, uint16_t* w_out, hipStream_t s);

// LDS bytes of the gemm kernels for a largest bitwidth bmax.
int gemm_lds_bytes(int bmax);

constexpr int kTokInfoBytes = 128 * 12;   // per-work-item token rows / outputs / weights

}  // namespace pw
