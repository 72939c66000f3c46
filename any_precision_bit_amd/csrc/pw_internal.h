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
// Three kernels take an expert by its token count (small: one-tile kernel,
// four: four-tile kernel, big: dequantise-once kernel), each over a gate_up
// and a down list.
enum {
    LIST_GU_SMALL = 0, LIST_GU_FOUR = 1, LIST_GU_BIG = 2,
    LIST_DN_SMALL = 3, LIST_DN_FOUR = 4, LIST_DN_BIG = 5, N_LISTS = 6
};

// Workspace carved out of one device allocation per layer.
struct Workspace {
    int32_t* ids;        // [max_T][k]
    float* w;            // [max_T][k]
    int32_t* counts;     // [E]
    int32_t* offsets;    // [E+1]
    int32_t* sorted;     // [max_T*k]    assignment t*k+j, grouped by expert
    int32_t* slot_of;    // [max_T*k]    sorted position of assignment t*k+j (inverse of sorted)
    float* part;         // [max_T*k*pieces_r + max_T*pieces_s][d]  deterministic mode only (else null):
                         //              each down item's weighted output rows, summed by reduce_kernel
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
    int exact_all;         // 1: exact logits of every expert in the first pass (small T); 0: fp32
                           // bounds first, exact logits of the candidates only
    int small_tokens;      // token group of the small lists: 16 (one-tile kernel) or 32 (two-tile)
    int small_max;         // experts with 1..small_max tokens: small lists
    int four_max;          // small_max+1..four_max tokens: four-tile lists (64-token groups);
                           // more: dequantise-once lists (128-token groups)
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
    int det;                  // deterministic accumulation: down items write ws.part rows
    int part_shared;          // first ws.part row of the shared expert (T*k*pieces_r)
    int lut_tiled;            // LUT pages in the 32-row tiled order (else row-major)
    int rb_lg;                // log2 of the rows per linear-block (0: whole linears); blocks
                              // are numbered expert, linear, row-block
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

// Planner problem: one entry per block (expert, linear), host arrays.
struct PlanProblem {
    int n_blocks;
    const int32_t* rows;      // R of each block
    const int32_t* cols;      // K of each block
    const uint8_t* min_bits;  // floor of a downgrade
    const uint8_t* max_bits;  // ceiling of an upgrade
    const float* sens;        // offline sensitivity
    const float* resid;       // prompt residual (may be null)
    const double* mass;       // routing mass of the block's expert
};
// Resident bytes of an [R x K] block at bitwidth b: planes R*K*b/8 + LUT R*2^b*2.
double block_bytes(int64_t R, int64_t K, int b);
// Greedy plan change (see pw_plan.cpp); bits is updated in place. Returns the
// number of actions; *moved = bytes released (> 0) or added (< 0).
int plan_greedy(const PlanProblem& P, double bytes_to_free, uint8_t* bits, double* moved, double* damage);

hipError_t launch_init_ws(const Workspace& ws, int n_counters, uint32_t wait_limit, hipStream_t s);
hipError_t launch_route(const RouteParams& p, hipStream_t s);
// tile_tokens: kSmallTokens (one MFMA token tile per item), kTwoTokens (two) or
// kLargeTokens (four).
// The grid is every work-group the device can hold at once (per-CU occupancy x n_cu).
hipError_t launch_experts(int tile_tokens, const ExpertParams& p, int n_cu, hipStream_t s);
// The dequantise-once kernel over the large lists (groups of kBigTokens tokens).
hipError_t launch_experts_big(const ExpertParams& p, int n_cu, hipStream_t s);
// Sets the expert kernels' attributes and caches their per-CU occupancy; the
// forward calls it before enqueueing anything, so a launch precondition that
// cannot be met fails the call with nothing enqueued.
hipError_t prepare_experts(bool det);
hipError_t launch_residual(const uint16_t* x, const float* y, uint16_t* x_next, long n,
                           hipStream_t s);
// Deterministic mode: y[t] = sum over j < k, piece < pr of part[slot_of[t*k+j]*pr + piece]
// + sum over piece < ps of part[part_shared + t*ps + piece], in that order.
hipError_t launch_reduce(const Workspace& ws, float* y, int T, int k, int d, int pr, int ps, int part_shared,
                         hipStream_t s);
hipError_t launch_debug(const uint64_t* planes8, int b, const uint16_t* lut, int lut_tiled, int R, int K,
                        uint8_t* idx_out, uint16_t* w_out, hipStream_t s);

// Device scratch of the no-allocation forward: the device address of the
// static array on device dev (which must be current) and its size.
constexpr size_t kScratchBytes = 32u << 20;
hipError_t scratch_memory(int dev, void** ptr, size_t* bytes);

// LDS bytes of the expert kernel for items of tile_tokens tokens.
int expert_lds_bytes(int tile_tokens);

constexpr int kSmallTokens = 16;          // token group of the one-tile kernel (one 16-token MFMA tile)
constexpr int kTwoTokens = 32;            // token group of the two-tile kernel
constexpr int kSmallMax = 32;             // experts with 1..32 tokens: the small lists, in groups of 16,
                                          // or of 32 when T k > 16 E (each weight dequantised once)
constexpr int kLargeTokens = 64;          // four-tile kernel: groups of 64 tokens
constexpr int kBigTokens = 128;           // dequantise-once kernel: groups of 128 tokens
// Experts with 33..kFourMax tokens go to the four-tile kernel (one or two
// 64-token groups). The dequantise-once kernel has the higher cost per item and
// pays off once a forward brings it many items: from kBigBatch tokens on, the
// bound drops to kFourMaxBig = kSmallMax, so every expert above 32 tokens takes
// the dequantise-once kernel and the four-tile kernel is not launched (measured
// crossover on the qwen and fine-grained layers at T = 128 and T = 1024).
constexpr int kFourMax = 128;
constexpr int kFourMaxBig = 32;
constexpr int kBigBatch = 512;
// Which kernel takes which experts (PW_FORCE_PATH, pw_debug_set_path):
//   AUTO  1..kSmallMax tokens: two-tile kernel when T k > 16 E, else one-tile kernel;
//         up to kFourMax (kFourMaxBig when T >= kBigBatch): four-tile kernel;
//         more: dequantise-once kernel
//   SMALL every expert in the one-tile kernel (16-token groups)
//   FOUR  1..kSmallMax: as AUTO; more: four-tile kernel (64-token groups)
//   BIG   every expert in the dequantise-once kernel
//   TWO   every expert in the two-tile kernel (32-token groups)
enum { PATH_AUTO = 0, PATH_SMALL = 1, PATH_FOUR = 2, PATH_BIG = 3, PATH_TWO = 4 };
constexpr int kDownPiece = 2048;          // K columns of one down item (partial sums add into y)
// act rows of one K-piece start on a 128-byte line (2-byte elements): a line never holds two pieces
static_assert(kDownPiece % 64 == 0, "K-pieces must start on 128-byte act lines");
constexpr int kRouteThreads = 256;          // route kernel: 4 waves
constexpr int kRouteFilterPerWave = 4;      // router rows per wave in the fp32 pass
constexpr int kRouteExactPerWave = 1;       // router rows per wave when every logit is exact
constexpr int kRouteExactAllWork = 2048;    // T * E up to which every logit is computed exactly in the
                                            // first pass (its T * E / 4 work-groups are all resident at
                                            // once); above it, fp32 bounds and exact candidates
constexpr int kSortBatch = 8;               // bucket sort: chunks of assignments loaded per round trip
constexpr int kMaxModel = 8192;           // d_model limit (x row staged in LDS)

}  // namespace pw
