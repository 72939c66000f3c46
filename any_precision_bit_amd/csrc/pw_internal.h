// Internal declarations shared by the host API (pw_api.cpp) and the gfx950
// kernels (pw_kernels.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pw {

// One entry of the device page table: the pages of one (expert, linear) block
// at its planned bitwidth. 80 bytes, read with scalar loads by the kernels.
struct DevBlock {
    uint64_t planes[8];  // slot s: device address of plane s - (8 - bits); slots below 8 - bits are 0
    uint64_t lut;        // device address of LUT_bits, R * 2^bits fp16
    int32_t bits;        // 1..8
    int32_t pad;
};
static_assert(sizeof(DevBlock) == 80, "DevBlock layout");

// Work lists of the gemm kernels: for list position p (p = 0 is the shared
// expert when there is one, then routed experts 0..E-1), items
// [prefix[p], prefix[p+1]) belong to that expert; item i of an expert is
// (row tile i % tiles, token group i / tiles).
enum { LIST_GU_SMALL = 0, LIST_GU_LARGE = 1, LIST_DN_SMALL = 2, LIST_DN_LARGE = 3, N_LISTS = 4 };

// Workspace carved out of one device allocation per layer.
struct Workspace {
    int32_t* ids;        // [max_T][k]
    float* w;            // [max_T][k]
    int32_t* counts;     // [E]
    int32_t* offsets;    // [E+1]
    int32_t* sorted;     // [max_T*k]    assignment t*k+j, grouped by expert
    int32_t* slot_tok;   // [max_T*k]    token t of each sorted slot
    float* slot_w;       // [max_T*k]    routing weight of each sorted slot
    int32_t* prefix;     // [N_LISTS][E+2]
    uint16_t* act;       // [max_T*k + max_T*has_shared][F_max]  SwiGLU output, permuted
    uint32_t* status;    // [1]          PW_STATUS_* bits
    uint32_t* wait_limit;// [1]          polls of a down item's dependency counter before
                         //              PW_STATUS_DEP_TIMEOUT (host-written, read-only in kernels)
    long long* lg;       // [max_T][E]   exact router logits, units of 2^-48 (route kernel, between work-groups)
    // counters, contiguous and zeroed once; every launch leaves them at zero
    uint32_t* dep;       // [(E+1)*dep_stride + 1]  gate_up items done per (list position, down
                         //              K-piece); last word: work-groups finished (expert kernel)
    uint32_t* tok_cnt;   // [max_T]      route work-groups finished per token
    uint32_t* route_done;// [1]          tokens finished (route kernel)
    int dep_stride;      // down K-pieces of the widest expert
};

struct RouteParams {
    const uint16_t* x;
    const uint16_t* wr;
    const uint16_t* bias;  // may be null
    int T, d, E, k;
    int has_shared;
    int tiles_gu_r, tiles_gu_s, tiles_dn;   // row tiles per item list
    int pieces_dn_r, pieces_dn_s;           // K-pieces of a routed / the shared down item
    Workspace ws;
    float* y;              // zeroed here
    int32_t* o_ids;        // optional caller copies of the routing outputs
    float* o_w;
    int32_t* o_counts;
    int32_t* o_offsets;
    int32_t* o_sorted;
};

// Dequantising GEMM over (expert, row tile, K-piece, token group) items of one
// list (the expert kernel runs a gate_up list, then a down list). An item covers 32 rows of each of two row-sets over its K range; wave w
// of the work-group owns rows 16*(w >> 1) .. +15 and half-line w & 1 of every
// 128-byte plane line.
// gate_up: set 0 = gate rows [f0, f0+32), set 1 = up rows [f0, f0+32), K = d,
//          B = x rows (tokens), epilogue SwiGLU -> act (fp16).
// down:    set 0 = rows [r0, r0+32), set 1 = rows [r0+32, r0+64), K = F (in
//          pieces of kDownPiece columns), B = act rows (slots), epilogue
//          w * o atomically added to y (fp32).
struct GemmParams {
    const DevBlock* blocks;   // [n_total*3]
    int E, k, T, d;
    int F, Fs;                // routed / shared ffn (Fs = 0: none)
    int has_shared;
    int tiles_r, tiles_s;     // row tiles per routed expert / for the shared expert
    int pieces_r, pieces_s;   // K-pieces per row tile (down only; gate_up: 1)
    int list;                 // LIST_*
    Workspace ws;
    int ld_act;               // row stride of act (F_max)
    int shared_base;          // first act row of the shared expert (max_T*k)
    const uint16_t* x;        // layer input (gate_up B operand)
    uint32_t b_bytes;         // size of the B-operand buffer (x or act)
    float* y;
};

// One launch of the expert kernel: a gate_up list and the down list of the same
// token-tile size (gu.list, dn.list); down items wait on gate_up items of their
// expert through ws.dep.
struct ExpertParams {
    GemmParams gu;
    GemmParams dn;
};

hipError_t launch_init_ws(const Workspace& ws, int n_counters, uint32_t wait_limit, hipStream_t s);
hipError_t launch_route(const RouteParams& p, hipStream_t s);
// tile_tokens: kSmallTokens (one MFMA token tile per item) or kLargeTokens (four).
// The grid is every work-group the device can hold at once (per-CU occupancy x n_cu).
hipError_t launch_experts(int tile_tokens, const ExpertParams& p, int n_cu, hipStream_t s);
hipError_t launch_residual(const uint16_t* x, const float* y, uint16_t* x_next, long n,
                           hipStream_t s);
hipError_t launch_debug(const uint64_t* planes8, int b, const uint16_t* lut, int R, int K,
                        uint8_t* idx_out, uint16_t* w_out, hipStream_t s);

// LDS bytes of the expert kernel for items of tile_tokens tokens.
int expert_lds_bytes(int tile_tokens);

constexpr int kSmallTokens = 16;          // token group of the one-tile kernel (one 16-token MFMA tile)
constexpr int kSmallMax = 32;             // experts with 1..32 tokens: groups of 16 in the one-tile kernel
constexpr int kLargeTokens = 64;          // larger experts: groups of 64 tokens (four tiles)
constexpr int kDownPiece = 2048;          // K columns of one down item (partial sums add into y)
constexpr int kRouteThreads = 256;          // route kernel: 4 waves
constexpr int kRouteExpertsPerWave = 2;     // router rows per wave
constexpr int kMaxModel = 8192;           // d_model limit (x row staged in LDS)

}  // namespace pw
