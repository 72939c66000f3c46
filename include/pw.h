/*
 * pw.h -- C ABI of the fused mixed-precision MoE layer on MI355X (gfx950).
 *
 * The layer follows the PagedWeight pages ("PagedWeight: Efficient MoE LLM
 * Serving with Dynamic Quality-Aware Weight Quantization"):
 *   - a planner chooses a bitwidth per linear-block (legiblepapers "Key
 *     Takeaways" and FAQ Q8)                                -> pw_moe_plan_set
 *   - Any-Precision bit-plane and lookup-table buffers are GPU-resident pages
 *     (arxivlens summary; legiblepapers "Summary & Methodology Analysis")
 *                                                           -> pw_page_table_bind
 *   - one fused mixed-precision MoE kernel path reads those pages directly and
 *     fuses routing, expert activation and output accumulation (legiblepapers
 *     "Key Takeaways" and FAQ Q5)                           -> pw_moe_forward
 *
 * Conventions shared by every entry point
 *   - Every function returns pw_status; nothing throws across the ABI. Every
 *     argument, shape and launch precondition is checked before anything is
 *     enqueued: on a non-OK status from a check nothing is enqueued on any
 *     stream and the layer's state is unchanged. The one exception is
 *     PW_E_HIP from pw_moe_forward when the HIP runtime rejects a kernel
 *     launch itself (after the checks passed): kernels enqueued before the
 *     failing launch stay enqueued, y is then undefined, and the device
 *     tables are uploaded again by the next forward. pw_last_error()
 *     (thread-local) describes every failure.
 *   - "device pointer" means memory of the GPU the layer runs on. The caller
 *     owns every device buffer (pages, LUTs, x, y, router weights, route
 *     outputs); the library owns only the handle, its device tables and its
 *     workspace.
 *   - A handle is not thread-safe, and forwards of one handle must not overlap
 *     in time on different streams. Several handles may share one stream.
 *
 * Data format of one linear-block (expert e, linear l), an [R x K] matrix
 * (gate and up: R = d_ffn, K = d_model; down: R = d_model, K = d_ffn; the
 * shared expert uses d_ffn_shared for d_ffn):
 *   - 8-bit parent index q per weight; plane p (p = 0 is the most significant
 *     bit of q) is R * K/8 bytes, row-major with row stride K/8 bytes; column c
 *     of a row is bit (c & 7) of byte (c >> 3).
 *   - at bitwidth b the weight is LUT_b[r][q >> (8-b)], read from planes 0..b-1;
 *     LUT_b has one table of 2^b fp16 entries per output row r (R * 2^b values),
 *     row-major: entry i of row r at element r * 2^b + i.
 *   - alternative LUT page order, selected per layer with PW_FLAG_LUT_TILED in
 *     pw_moe_desc.flags: 32-row tiles; with E = min(8, 2^b) and G = 2^b / E,
 *     entry i of row r sits at element ((t*G + g)*32 + rr)*E + j, where
 *     t = r / 32, rr = r % 32, g = i / E, j = i % E. It holds the same values in
 *     the same bytes; a work-group then stages a tile's tables with contiguous
 *     loads. (For b < 3 both orders are the same array.)
 *   - R (every block's row count: d_model and the ffn sizes) is a multiple of
 *     32 and K a multiple of 128, which the size limits below imply.
 */
#ifndef PW_H
#define PW_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PW_ABI_VERSION 2
#define PW_MAX_BITS 8
#define PW_MAX_TOP_K 16
#define PW_MAX_EXPERTS 256

typedef enum {
    PW_OK = 0,
    PW_E_ARG = 1,      /* null / negative / inconsistent argument */
    PW_E_SHAPE = 2,    /* unsupported dimension (see pw_layer_create) */
    PW_E_BITS = 3,     /* bitwidth outside 1..8 */
    PW_E_UNBOUND = 4,  /* a block's pages do not cover its planned bitwidth */
    PW_E_ALIGN = 5,    /* pointer not 16-byte aligned */
    PW_E_RANGE = 6,    /* T outside 0..max_tokens */
    PW_E_STATE = 7,    /* call out of order (e.g. forward before plan_set), or
                          pw_layer_status found the device range flag set */
    PW_E_NOMEM = 8,    /* device or pinned host allocation failed */
    PW_E_HIP = 9       /* a HIP runtime call failed; text in pw_last_error() */
} pw_status;

enum { PW_GATE = 0, PW_UP = 1, PW_DOWN = 2 };

/* bits of the device status word read by pw_layer_status */
#define PW_STATUS_ROUTER_RANGE 1u  /* a token/expert left the exact-router range */
#define PW_STATUS_DEP_TIMEOUT 2u   /* a down item stopped waiting for its gate_up rows
                                      (work-groups not all resident); y is undefined */

typedef struct pw_layer_s* pw_layer;  /* opaque; one MoE layer */

typedef struct {
    int32_t abi_version;   /* PW_ABI_VERSION */
    int32_t d_model;       /* d: hidden size, multiple of 128, at most 8192 */
    int32_t n_experts;     /* E routed experts, 1..PW_MAX_EXPERTS */
    int32_t d_ffn;         /* F: routed expert ffn size, multiple of 128 */
    int32_t top_k;         /* k, 1..min(E, PW_MAX_TOP_K) */
    int32_t d_ffn_shared;  /* F_s: shared expert ffn size, 0 = none, else multiple of 128;
                              the shared expert has expert id E */
    int32_t max_tokens;    /* upper bound on T per forward, 1..65536, with
                              max_tokens*(top_k+1)*max(d_ffn, d_ffn_shared) < 2^31 */
    uint32_t flags;        /* 0 or a combination of PW_FLAG_LUT_TILED (every bound LUT page
                              of this layer is in the 32-row tiled order; default row-major)
                              and PW_FLAG_DETERMINISTIC (see below) */
    int32_t rows_per_block;/* linear-block size: 0 = one block per linear; else a power of
                              two >= 64 dividing d_model, d_ffn and d_ffn_shared, and every
                              linear is cut into row-blocks of that many rows, each a
                              block with its own bitwidth and pages (legiblepapers "Key
                              Takeaways" and FAQ Q5: bitwidths vary per linear-block) */
} pw_moe_desc;

#define PW_FLAG_LUT_TILED 1u
/* Deterministic accumulation: every forward of the same inputs gives the same y
 * bit for bit. Each down-projection work item writes its weighted output rows to
 * a partial buffer of its own (one fp32 row of d_model per routed assignment and
 * K-piece of 2048 ffn columns, and per token and K-piece of the shared expert)
 * instead of adding them into y with fp32 atomics, and a last kernel sums them per
 * token in a fixed order (assignment j = 0..k-1, its pieces in order, then the
 * shared expert's pieces). The layer's workspace grows by
 * max_tokens * (top_k * ceil(d_ffn/2048) + ceil(d_ffn_shared/2048)) * d_model * 4
 * bytes, and pw_moe_forward_noalloc's limit on T shrinks accordingly. */
#define PW_FLAG_DETERMINISTIC 2u

/* Optional routing outputs of a forward, all device pointers; any may be NULL.
 * topk_ids int32 [T][k] (descending logit, ties to the lower expert index),
 * topk_w fp32 [T][k] (softmax over the k selected logits), expert_count int32 [E],
 * expert_offset int32 [E+1] (exclusive prefix sum), sorted_assign int32 [T*k]
 * (assignments t*k + j grouped by expert, ascending (t, j) within an expert). */
typedef struct {
    int32_t* topk_ids;
    float* topk_w;
    int32_t* expert_count;
    int32_t* expert_offset;
    int32_t* sorted_assign;
} pw_route_out;

/* Creates a layer on the current HIP device. Device memory is allocated on the
 * first forward. PW_E_SHAPE for a dimension outside the limits above. */
pw_status pw_layer_create(const pw_moe_desc* desc, pw_layer* out);

/* Frees the handle and its device memory. The caller must have synchronised
 * every stream that ran a forward of this layer. NULL is a no-op. */
pw_status pw_layer_destroy(pw_layer layer);

/* Text of the last error on this thread ("" if none). Valid until the next call. */
const char* pw_last_error(void);

/* Blocks. With rows_per_block = 0 block e*3 + l is linear l in {PW_GATE, PW_UP,
 * PW_DOWN} of expert e in [0, E + has_shared). With rows_per_block = rb > 0 the
 * blocks are numbered expert by expert (routed 0..E-1, then the shared
 * expert), within an expert gate, up, down, and within a linear by row-block j
 * (rows j*rb .. j*rb + rb - 1): expert e (ffn f) owns 2*f/rb + d_model/rb
 * blocks. The planner's arrays (sensitivity, residual, min/max, bits) use the
 * same order.
 *
 * Sets the bitwidth plan: bits[i] for every block i, each in 1..8 (host array,
 * copied before return); n_blocks must equal the layer's block count. The plan takes effect at the next
 * forward, which uploads the tables in stream order before its kernels, so a
 * rewrite between two forwards needs no host synchronisation. */
pw_status pw_moe_plan_set(pw_layer layer, const uint8_t* bits, int32_t n_blocks);

/* Binds the pages of linear (expert, linear): planes[p] for p < n_planes are
 * device pointers to bit-plane p (planes 0..n_planes-1 of the parent, 16-byte
 * aligned, R*K/8 bytes each, the whole linear); lut is a device pointer to
 * LUT_{lut_bits} (R * 2^lut_bits fp16 in the layer's LUT page order above,
 * 16-byte aligned). With row-blocks, every row-block of the linear is bound to
 * its rows of these pages at lut_bits. The host array `planes` is copied
 * before return. The pages must stay alive until every forward enqueued while
 * they were bound has completed on its stream. A forward requires, for every
 * block, n_planes >= b and lut_bits == b for the planned b (else PW_E_UNBOUND). */
pw_status pw_page_table_bind(pw_layer layer, int32_t expert, int32_t linear,
                             const void* const* planes, int32_t n_planes,
                             const void* lut, int32_t lut_bits);

/* Binds the pages of one block: row-block row_block of linear (expert, linear)
 * (0 when the layer's linears are whole). planes[p] are device pointers to the
 * block's rows of bit-plane p (rows x K/8 bytes, 16-byte aligned), lut to the
 * block's rows of LUT_{lut_bits} (rows * 2^lut_bits fp16, layer's page order;
 * in the tiled order the block's rows form whole 32-row tiles). Same
 * lifetime rules as pw_page_table_bind; PW_E_ARG for a row_block outside the
 * linear. */
pw_status pw_page_table_bind_rows(pw_layer layer, int32_t expert, int32_t linear, int32_t row_block,
                                  const void* const* planes, int32_t n_planes,
                                  const void* lut, int32_t lut_bits);

/* One MoE layer on T tokens, enqueued on `stream` (hipStream_t as void*; NULL =
 * the null stream); asynchronous, no host synchronisation.
 *   x        fp16 [T][d] device, 16-byte aligned
 *   router_w fp16 [E][d] device, 16-byte aligned
 *   router_b fp16 [E] device or NULL (added to the logits)
 *   y        fp32 [T][d] device, overwritten with
 *            sum_j w_j * expert_{ids_j}(x_t) (+ shared expert(x_t)); each expert
 *            accumulates in fp32 and rounds its SwiGLU output silu(g) * u to
 *            fp16 (the down projection's matrix-core operand), so outputs are
 *            defined while |silu(g) * u| <= 65504
 *   x_next   fp16 [T][d] device or NULL: fp16 round-to-nearest-even of x + y
 *   route    optional routing outputs (NULL = none)
 * Routing is exact: logits are compared as exact integers in units of 2^-48.
 * Every finite fp16 x, router_w and router_b is accepted; the sum is exact
 * when sum_c |x*w| + |b| < 2^15 per (token, expert) (checked on the device in
 * fp32 with a 2 % margin). A token/expert outside that range, or a non-finite
 * input, sets PW_STATUS_ROUTER_RANGE in the device status word (read with
 * pw_layer_status) and its routing is undefined. The check needs the inputs,
 * which live on the device, so it cannot fail the call itself.
 * T == 0 is a no-op. With the environment variable PW_DEBUG_SYNC set (read once
 * per process) the call synchronises `stream` before returning, so that a
 * kernel fault surfaces here as PW_E_HIP. */
pw_status pw_moe_forward(pw_layer layer, const void* x, int32_t T, const void* router_w,
                         const void* router_b, float* y, void* x_next,
                         const pw_route_out* route, void* stream);

/* For callers that cannot allocate memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation. The same forward as
 * pw_moe_forward (same arguments, kernels and results), but it calls no
 * hipMalloc, hipFree, hipHostMalloc or other allocating routine: the device
 * page table and the forward's workspace live in a static device array of
 * 32 MiB (per GPU, held from library load until the process ends) instead of
 * the layer's own device memory, which is neither allocated nor used.
 *   - T is limited by that array: the page table plus a workspace for T tokens
 *     must fit (about (T*top_k + T*has_shared) * max(d_ffn, d_ffn_shared) * 2
 *     bytes plus T * n_experts * 8); PW_E_RANGE otherwise, with the sizes in
 *     pw_last_error(). The 24-layer qwen shape (T = 256, top-4, ffn 5632)
 *     needs 15 MB.
 *   - Every call on one GPU shares the array, which keeps the last call's
 *     contents; each call zeroes the counters and the status word it uses
 *     before its kernels. Calls that overlap in time on one GPU (on different
 *     streams, or from different threads) race and give undefined results.
 *   - The page table is copied from host memory the layer owns (pageable),
 *     which the copy call consumes before it returns.
 *   - pw_layer_status reports the status word of the last no-alloc call on the
 *     layer's GPU as well as the layer's own; pw_moe_replay and
 *     pw_layer_last_bytes refer to the last pw_moe_forward only. */
pw_status pw_moe_forward_noalloc(pw_layer layer, const void* x, int32_t T, const void* router_w,
                                 const void* router_b, float* y, void* x_next,
                                 const pw_route_out* route, void* stream);

/* Quality-aware runtime planner (legiblepapers "Summary & Methodology Analysis"
 * and FAQ Q8): from the layer's current plan, greedily choose one-bit
 * bitwidth changes per block until bytes_to_free bytes of
 * pages are released, taking at each step the action with the least damage per
 * released byte. bytes_to_free < 0 is a budget to spend instead: upgrades with
 * the most benefit per added byte are taken while they fit. Host-only (no GPU
 * call); the layer's plan is not changed: pass bits_out to pw_moe_plan_set and
 * bind the pages it needs.
 *   A block at bitwidth b holds R*K*b/8 + R*2^b*2 bytes (planes 0..b-1 and
 *   LUT_b). The damage of b -> b-1 on block i of expert e is
 *     (sensitivity[i] + residual[i]) * mass_e * (4^-(b-1) - 4^-b)
 *   (quantisation noise power of a b-bit quantiser scales as 4^-b), with
 *   mass_e = expert_count[e] / n_tokens for a routed expert (how often it is
 *   used) and 1 for the shared expert. Ties go to the lower block index.
 *   A block is a (row-block of a) linear, numbered as for pw_moe_plan_set.
 *   sensitivity  host float [n_blocks], finite, >= 0 (offline sensitivity)
 *   residual     host float [n_blocks], finite, >= 0, or NULL (prompt residuals)
 *   expert_count host int32 [n_experts] >= 0 (e.g. pw_route_out.expert_count of
 *                a forward), n_tokens > 0 the tokens of that forward
 *   min_bits / max_bits  host u8 [n_blocks] in 1..8 or NULL (3 and 8): no
 *                downgrade below min, no upgrade above max; the current plan
 *                must lie within them (PW_E_BITS otherwise)
 *   bits_out     host u8 [n_blocks]: the new plan
 *   result       host double [3]: bytes released (> 0) or added (< 0), damage
 *                added (< 0 for upgrades: damage removed), number of actions
 * A downgrade stops as soon as bytes_to_free is reached (it may overshoot by
 * one action) or no action is left. PW_E_STATE without a plan. */
pw_status pw_plan_greedy(pw_layer layer, const float* sensitivity, const float* residual,
                         const int32_t* expert_count, int32_t n_tokens, const uint8_t* min_bits,
                         const uint8_t* max_bits, double bytes_to_free, uint8_t* bits_out,
                         double* result);

/* Synchronises `stream`, then reads and clears the device status word into
 * *flags (PW_STATUS_* bits). Returns PW_E_STATE if any flag was set. */
pw_status pw_layer_status(pw_layer layer, void* stream, uint32_t* flags);

/* Measurement hook: enqueues again, on `stream`, the kernels of one phase of
 * this layer's last forward with the same arguments: 0 routing (router + bucket
 * sort), 1 experts (one kernel per token-tile size: gate_up + SwiGLU, then down
 * + weighted accumulation), 2 residual. Used to time one phase alone; the
 * buffers of that forward must still be alive. The phase rewrites its outputs
 * (phase 0 zeroes y, phase 1 adds into y again), so y is meaningful only after
 * a full forward. PW_E_STATE before any forward; PW_E_ARG for another phase. */
pw_status pw_moe_replay(pw_layer layer, int32_t phase, void* stream);

/* Algorithmic bytes of the last forward's kernels, computed on the host from
 * the routed counts of that forward (reads them back; synchronises `stream`):
 * bytes[0] route, bytes[1] gate_up, bytes[2] down, bytes[3] residual. Counts
 * planes b/8 B and LUT 2^b*2 B per row of every block of an expert with at
 * least one token (plus the shared expert), and activations read and written. */
pw_status pw_layer_last_bytes(pw_layer layer, void* stream, double* bytes /*[4]*/);

/* Test hooks for one block, same kernels' dequantisation path as the forward:
 * indices u8 [R][K] of bitwidth b (pw_debug_unpack) and weights fp16 [R][K]
 * (pw_debug_dequant; lut row-major, or 32-row tiled when lut_flags has
 * PW_FLAG_LUT_TILED), for an [R x K] block with R % 32 == 0 and K % 128 == 0.
 * All pointers are device pointers; the call is asynchronous on `stream`. */
pw_status pw_debug_unpack(const void* const* planes, int32_t b, int32_t R, int32_t K,
                          uint8_t* idx_out, void* stream);
pw_status pw_debug_dequant(const void* const* planes, int32_t b, const void* lut, uint32_t lut_flags,
                           int32_t R, int32_t K, void* w_out, void* stream);

/* Test hook: how many times a down item polls the counter of its gate_up rows
 * before it gives up, sets PW_STATUS_DEP_TIMEOUT and goes on (later forwards of
 * this layer; default 1 << 20 polls, about a second). The expert kernel's
 * work-groups are all resident at once, so the wait ends unless that fails;
 * the limit turns such a hang into a status flag. PW_E_ARG for a null layer. */
pw_status pw_debug_set_wait_limit(pw_layer layer, uint32_t polls);

/* A/B switch: which expert kernel takes which experts in later forwards of
 * this layer (same results up to fp32 summation order):
 *   PW_PATH_AUTO  experts with 1..32 tokens: the two-tile kernel (one 32-token
 *                 group) when the T*top_k assignments exceed 16 per routed
 *                 expert on average, else the one-tile kernel (16-token
 *                 groups); 33..128 (none when T >= 512): the four-tile
 *                 kernel (64-token groups); more: the dequantise-once kernel
 *                 (128-token groups)
 *   PW_PATH_SMALL every expert in the one-tile kernel (16-token groups)
 *   PW_PATH_FOUR  as PW_PATH_AUTO up to 32 tokens; more: the four-tile kernel
 *                 (64-token groups, every weight dequantised once per group)
 *   PW_PATH_BIG   every expert in the dequantise-once kernel
 *   PW_PATH_TWO   every expert in the two-tile kernel (32-token groups)
 * New layers start from the environment variable PW_FORCE_PATH (auto, small,
 * four, big or two; read once per process), else PW_PATH_AUTO. PW_E_ARG for a
 * null layer or another value. */
#define PW_PATH_AUTO 0
#define PW_PATH_SMALL 1
#define PW_PATH_FOUR 2
#define PW_PATH_BIG 3
#define PW_PATH_TWO 4
pw_status pw_debug_set_path(pw_layer layer, int32_t path);

#ifdef __cplusplus
}
#endif

#endif /* PW_H */
