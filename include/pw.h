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
 *   - Every function returns pw_status; nothing throws across the ABI. On a
 *     non-OK status nothing is enqueued on any stream and the layer's state is
 *     unchanged; pw_last_error() (thread-local) then describes the failure.
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
 *     stored in 32-row tiles: with E = min(8, 2^b) and G = 2^b / E, entry i of
 *     row r sits at element ((t*G + g)*32 + rr)*E + j, where t = r / 32,
 *     rr = r % 32, g = i / E, j = i % E (R must be a multiple of 32).
 */
#ifndef PW_H
#define PW_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PW_ABI_VERSION 1
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
    uint32_t flags;        /* must be 0 */
} pw_moe_desc;

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

/* Sets the bitwidth plan: bits[e*3 + l] for e in [0, E + has_shared), l in
 * {PW_GATE, PW_UP, PW_DOWN}, each in 1..8 (host array, copied before return).
 * n_blocks must equal 3*(E + has_shared). The plan takes effect at the next
 * forward, which uploads the tables in stream order before its kernels, so a
 * rewrite between two forwards needs no host synchronisation. */
pw_status pw_moe_plan_set(pw_layer layer, const uint8_t* bits, int32_t n_blocks);

/* Binds the pages of block (expert, linear): planes[p] for p < n_planes are
 * device pointers to bit-plane p (planes 0..n_planes-1 of the parent, 16-byte
 * aligned, R*K/8 bytes each); lut is a device pointer to LUT_{lut_bits}
 * (R * 2^lut_bits fp16 in the tiled order above, 16-byte aligned). The host
 * array `planes` is copied before return. The pages must stay alive until every forward enqueued while
 * they were bound has completed on its stream. A forward requires, for every
 * block, n_planes >= b and lut_bits == b for the planned b (else PW_E_UNBOUND). */
pw_status pw_page_table_bind(pw_layer layer, int32_t expert, int32_t linear,
                             const void* const* planes, int32_t n_planes,
                             const void* lut, int32_t lut_bits);

/* One MoE layer on T tokens, enqueued on `stream` (hipStream_t as void*; NULL =
 * the null stream); asynchronous, no host synchronisation.
 *   x        fp16 [T][d] device, 16-byte aligned
 *   router_w fp16 [E][d] device, 16-byte aligned
 *   router_b fp16 [E] device or NULL (added to the logits)
 *   y        fp32 [T][d] device, overwritten with
 *            sum_j w_j * expert_{ids_j}(x_t) (+ shared expert(x_t))
 *   x_next   fp16 [T][d] device or NULL: fp16 round-to-nearest-even of x + y
 *   route    optional routing outputs (NULL = none)
 * Routing is exact: logits are compared as exact integers in units of 2^-48.
 * That needs |x|, |router_w| < 128 and sum_c |x*w| + |b| < 2^15 per (token,
 * expert); a token/expert outside that range sets PW_STATUS_ROUTER_RANGE in the
 * device status word (read with pw_layer_status) and its routing is undefined.
 * T == 0 is a no-op. With the environment variable PW_DEBUG_SYNC set (read once
 * per process) the call synchronises `stream` before returning, so that a
 * kernel fault surfaces here as PW_E_HIP. */
pw_status pw_moe_forward(pw_layer layer, const void* x, int32_t T, const void* router_w,
                         const void* router_b, float* y, void* x_next,
                         const pw_route_out* route, void* stream);

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
 * (pw_debug_dequant, lut in the tiled order above), for an [R x K] block with
 * R % 32 == 0 and K % 128 == 0.
 * All pointers are device pointers; the call is asynchronous on `stream`. */
pw_status pw_debug_unpack(const void* const* planes, int32_t b, int32_t R, int32_t K,
                          uint8_t* idx_out, void* stream);
pw_status pw_debug_dequant(const void* const* planes, int32_t b, const void* lut, int32_t R,
                           int32_t K, void* w_out, void* stream);

/* Test hook: how many times a down item polls the counter of its gate_up rows
 * before it gives up, sets PW_STATUS_DEP_TIMEOUT and goes on (later forwards of
 * this layer; default 1 << 20 polls, about a second). The expert kernel's
 * work-groups are all resident at once, so the wait ends unless that fails;
 * the limit turns such a hang into a status flag. PW_E_ARG for a null layer. */
pw_status pw_debug_set_wait_limit(pw_layer layer, uint32_t polls);

#ifdef __cplusplus
}
#endif

#endif /* PW_H */
