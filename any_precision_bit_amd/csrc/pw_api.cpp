// Host side of the C ABI declared in pw.h: argument validation, the host shadow
// of the bitwidth plan and the page table, the device tables uploaded in stream
// order, the per-layer workspace and the kernel launch sequence.
//
// The three calls follow the PagedWeight pages' statement of the problem: the
// planner picks a bitwidth per linear-block (legiblepapers "Key Takeaways", FAQ
// Q8), the Any-Precision bit-plane and LUT buffers are GPU-resident pages
// (arxivlens summary; legiblepapers "Summary & Methodology Analysis"), and the
// fused kernel reads them directly (legiblepapers FAQ Q5).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "pw.h"
#include "pw_internal.h"

using pw::DevBlock;

namespace {

thread_local std::string g_err;

pw_status fail(pw_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

pw_status hip_fail(hipError_t e, const char* what) {
    return fail(PW_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kStageSlots = 4;

struct Page {
    const void* planes[8] = {};
    int n_planes = 0;
    const void* lut = nullptr;
    int lut_bits = 0;
};

// Restores the caller's current device on scope exit.
struct DeviceGuard {
    int prev = -1;
    bool ok = true;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) {
            ok = false;
            return;
        }
        if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

}  // namespace

struct pw_layer_s {
    pw_moe_desc desc{};
    int n_total = 0;       // E + has_shared
    int device = 0;
    std::vector<uint8_t> bits;   // empty until plan_set
    std::vector<Page> pages;
    bool dirty = true;

    // device state (allocated on the first forward)
    bool dev_ready = false;
    DevBlock* d_blocks = nullptr;
    char* d_ws = nullptr;
    pw::Workspace ws{};
    int f_max = 0;
    int n_cu = 256;

    // pinned staging ring for table uploads
    DevBlock* h_stage[kStageSlots] = {};
    hipEvent_t stage_ev[kStageSlots] = {};
    bool stage_used[kStageSlots] = {};
    int stage_i = 0;

    // launch record of the last forward (for pw_layer_last_bytes and pw_moe_replay)
    int last_T = 0;
    uint32_t wait_limit = 1u << 20;   // polls of a down item's dependency counter
    pw::RouteParams rp{};
    pw::GemmParams gp_gu{}, gp_dn{};
    const uint16_t* res_x = nullptr;
    const float* res_y = nullptr;
    uint16_t* res_out = nullptr;
};

namespace {

int n_blocks(const pw_layer_s* L) { return L->n_total * 3; }

int block_rows(const pw_layer_s* L, int e, int lin) {
    const int f = (e == L->desc.n_experts) ? L->desc.d_ffn_shared : L->desc.d_ffn;
    return lin == PW_DOWN ? L->desc.d_model : f;
}
int block_cols(const pw_layer_s* L, int e, int lin) {
    const int f = (e == L->desc.n_experts) ? L->desc.d_ffn_shared : L->desc.d_ffn;
    return lin == PW_DOWN ? f : L->desc.d_model;
}

// Checks that every block's pages cover its planned bitwidth.
pw_status validate_tables(const pw_layer_s* L) {
    if (L->bits.empty()) return fail(PW_E_STATE, "pw_moe_forward: no plan set (call pw_moe_plan_set)");
    for (int i = 0; i < n_blocks(L); ++i) {
        const int b = L->bits[i];
        const Page& pg = L->pages[i];
        if (pg.n_planes < b || pg.lut_bits != b || pg.lut == nullptr)
            return fail(PW_E_UNBOUND,
                        "block (expert %d, linear %d): planned b=%d but bound %d planes and LUT bits %d",
                        i / 3, i % 3, b, pg.n_planes, pg.lut_bits);
    }
    return PW_OK;
}

// Frees every device and pinned resource of the layer and clears the pointers,
// so that a failed set-up leaves nothing behind and a later forward retries
// from scratch. The caller has selected the layer's device.
void release_device(pw_layer_s* L) {
    for (int i = 0; i < kStageSlots; ++i) {
        if (L->stage_ev[i]) (void)hipEventDestroy(L->stage_ev[i]);
        if (L->h_stage[i]) (void)hipHostFree(L->h_stage[i]);
        L->stage_ev[i] = nullptr;
        L->h_stage[i] = nullptr;
        L->stage_used[i] = false;
    }
    if (L->d_ws) (void)hipFree(L->d_ws);
    if (L->d_blocks) (void)hipFree(L->d_blocks);
    L->d_ws = nullptr;
    L->d_blocks = nullptr;
    L->dev_ready = false;
}

pw_status ensure_device(pw_layer_s* L, hipStream_t s) {
    if (L->dev_ready) return PW_OK;
    const pw_moe_desc& D = L->desc;
    const int T = D.max_tokens, E = D.n_experts, k = D.top_k, d = D.d_model;
    const int has_shared = D.d_ffn_shared > 0;
    L->f_max = std::max(D.d_ffn, D.d_ffn_shared);
    const size_t act_rows = (size_t)T * k + (size_t)T * has_shared;
    auto al = [](size_t n) { return (n + 255) & ~(size_t)255; };
    size_t off = 0;
    const size_t o_ids = off;    off += al(sizeof(int32_t) * (size_t)T * k);
    const size_t o_w = off;      off += al(sizeof(float) * (size_t)T * k);
    const size_t o_cnt = off;    off += al(sizeof(int32_t) * (size_t)E);
    const size_t o_off = off;    off += al(sizeof(int32_t) * ((size_t)E + 1));
    const size_t o_srt = off;    off += al(sizeof(int32_t) * (size_t)T * k);
    const size_t o_stk = off;    off += al(sizeof(int32_t) * (size_t)T * k);
    const size_t o_sw = off;     off += al(sizeof(float) * (size_t)T * k);
    const size_t o_pre = off;    off += al(sizeof(int32_t) * (size_t)pw::N_LISTS * (E + 2));
    const size_t o_act = off;    off += al(sizeof(uint16_t) * act_rows * (size_t)L->f_max);
    const size_t o_st = off;     off += al(2 * sizeof(uint32_t));   // status, wait limit
    const size_t o_lg = off;     off += al(sizeof(long long) * (size_t)T * E);
    const int dep_stride = (L->f_max + pw::kDownPiece - 1) / pw::kDownPiece;
    const int n_dep = (E + 1) * dep_stride + 1;
    const int n_counters = n_dep + T + 1;   // dep, tok_cnt, route_done
    const size_t o_dep = off;    off += al(sizeof(uint32_t) * (size_t)n_counters);
    hipError_t e;
    int cus = 0;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, L->device)) != hipSuccess)
        return hip_fail(e, "device attribute");
    L->n_cu = cus > 0 ? cus : 256;
    if ((e = hipMalloc((void**)&L->d_ws, off)) != hipSuccess) {
        L->d_ws = nullptr;
        return fail(PW_E_NOMEM, "workspace (%zu bytes): %s", off, hipGetErrorString(e));
    }
    if ((e = hipMalloc((void**)&L->d_blocks, sizeof(DevBlock) * n_blocks(L))) != hipSuccess) {
        L->d_blocks = nullptr;
        release_device(L);
        return fail(PW_E_NOMEM, "page table: %s", hipGetErrorString(e));
    }
    char* b = L->d_ws;
    L->ws.ids = (int32_t*)(b + o_ids);
    L->ws.w = (float*)(b + o_w);
    L->ws.counts = (int32_t*)(b + o_cnt);
    L->ws.offsets = (int32_t*)(b + o_off);
    L->ws.sorted = (int32_t*)(b + o_srt);
    L->ws.slot_tok = (int32_t*)(b + o_stk);
    L->ws.slot_w = (float*)(b + o_sw);
    L->ws.prefix = (int32_t*)(b + o_pre);
    L->ws.act = (uint16_t*)(b + o_act);
    L->ws.status = (uint32_t*)(b + o_st);
    L->ws.wait_limit = L->ws.status + 1;
    L->ws.lg = (long long*)(b + o_lg);
    L->ws.dep = (uint32_t*)(b + o_dep);
    L->ws.tok_cnt = L->ws.dep + n_dep;
    L->ws.route_done = L->ws.tok_cnt + T;
    L->ws.dep_stride = dep_stride;
    for (int i = 0; i < kStageSlots; ++i) {
        if ((e = hipHostMalloc((void**)&L->h_stage[i], sizeof(DevBlock) * n_blocks(L), hipHostMallocDefault)) !=
            hipSuccess) {
            L->h_stage[i] = nullptr;
            release_device(L);
            return fail(PW_E_NOMEM, "pinned staging: %s", hipGetErrorString(e));
        }
        if ((e = hipEventCreateWithFlags(&L->stage_ev[i], hipEventDisableTiming)) != hipSuccess) {
            L->stage_ev[i] = nullptr;
            release_device(L);
            return hip_fail(e, "hipEventCreate");
        }
    }
    if ((e = pw::launch_init_ws(L->ws, n_counters, L->wait_limit, s)) != hipSuccess) {
        release_device(L);
        return hip_fail(e, "init workspace");
    }
    L->dev_ready = true;
    return PW_OK;
}

pw_status upload_tables(pw_layer_s* L, hipStream_t s) {
    if (!L->dirty) return PW_OK;
    const int slot = L->stage_i;
    hipError_t e;
    if (L->stage_used[slot] && (e = hipEventSynchronize(L->stage_ev[slot])) != hipSuccess)
        return hip_fail(e, "staging event");
    DevBlock* h = L->h_stage[slot];
    for (int i = 0; i < n_blocks(L); ++i) {
        const Page& pg = L->pages[i];
        DevBlock& db = h[i];
        std::memset(&db, 0, sizeof db);
        db.bits = L->bits[i];
        // plane p goes to slot p + 8 - b, so slot s always carries bit 7 - s of the index
        for (int p = 0; p < db.bits; ++p) db.planes[p + 8 - db.bits] = (uint64_t)(uintptr_t)pg.planes[p];
        db.lut = (uint64_t)(uintptr_t)pg.lut;
    }
    if ((e = hipMemcpyAsync(L->d_blocks, h, sizeof(DevBlock) * n_blocks(L), hipMemcpyHostToDevice, s)) !=
        hipSuccess)
        return hip_fail(e, "table upload");
    if ((e = hipEventRecord(L->stage_ev[slot], s)) != hipSuccess) return hip_fail(e, "staging event record");
    L->stage_used[slot] = true;
    L->stage_i = (slot + 1) % kStageSlots;
    L->dirty = false;
    return PW_OK;
}


// Enqueues the kernels of one phase of the forward recorded in L:
// 0 routing (router + bucket sort), 1 experts (gate_up + SwiGLU + down +
// accumulation), 2 residual hand-off.
pw_status launch_phase(pw_layer_s* L, int phase, hipStream_t s) {
    const int T = L->last_T;
    hipError_t e = hipSuccess;
    switch (phase) {
        case 0:
            if ((e = pw::launch_route(L->rp, s)) != hipSuccess) return hip_fail(e, "route kernel");
            break;
        case 1: {
            pw::ExpertParams ep{L->gp_gu, L->gp_dn};
            ep.gu.list = pw::LIST_GU_SMALL;
            ep.dn.list = pw::LIST_DN_SMALL;
            if ((e = pw::launch_experts(pw::kSmallTokens, ep, L->n_cu, s)) != hipSuccess)
                return hip_fail(e, "expert kernel");
            if (T > pw::kSmallMax) {
                ep.gu.list = pw::LIST_GU_LARGE;
                ep.dn.list = pw::LIST_DN_LARGE;
                if ((e = pw::launch_experts(pw::kLargeTokens, ep, L->n_cu, s)) != hipSuccess)
                    return hip_fail(e, "expert kernel (large)");
            }
            break;
        }
        case 2:
            if (L->res_out &&
                (e = pw::launch_residual(L->res_x, L->res_y, L->res_out, (long)T * L->desc.d_model, s)) !=
                    hipSuccess)
                return hip_fail(e, "residual kernel");
            break;
        default:
            return fail(PW_E_ARG, "phase %d not in 0..2", phase);
    }
    return PW_OK;
}

}  // namespace

extern "C" {

const char* pw_last_error(void) { return g_err.c_str(); }

pw_status pw_layer_create(const pw_moe_desc* desc, pw_layer* out) {
    g_err.clear();
    if (!desc || !out) return fail(PW_E_ARG, "pw_layer_create: null argument");
    *out = nullptr;
    const pw_moe_desc& D = *desc;
    if (D.abi_version != PW_ABI_VERSION)
        return fail(PW_E_ARG, "abi_version %d, library is %d", D.abi_version, PW_ABI_VERSION);
    if (D.flags != 0) return fail(PW_E_ARG, "flags must be 0");
    if (D.d_model <= 0 || D.d_model % 128 || D.d_model > pw::kMaxModel)
        return fail(PW_E_SHAPE, "d_model %d: must be a positive multiple of 128, at most %d", D.d_model,
                    pw::kMaxModel);
    if (D.n_experts < 1 || D.n_experts > PW_MAX_EXPERTS)
        return fail(PW_E_SHAPE, "n_experts %d: must be in 1..%d", D.n_experts, PW_MAX_EXPERTS);
    if (D.d_ffn <= 0 || D.d_ffn % 128)
        return fail(PW_E_SHAPE, "d_ffn %d: must be a positive multiple of 128", D.d_ffn);
    if (D.d_ffn_shared < 0 || D.d_ffn_shared % 128)
        return fail(PW_E_SHAPE, "d_ffn_shared %d: must be 0 or a multiple of 128", D.d_ffn_shared);
    if (D.top_k < 1 || D.top_k > D.n_experts || D.top_k > PW_MAX_TOP_K)
        return fail(PW_E_SHAPE, "top_k %d: must be in 1..min(n_experts, %d)", D.top_k, PW_MAX_TOP_K);
    if (D.max_tokens < 1 || D.max_tokens > 65536)
        return fail(PW_E_SHAPE, "max_tokens %d: must be in 1..65536", D.max_tokens);
    {
        const double act = ((double)D.max_tokens * (D.top_k + 1)) * std::max(D.d_ffn, D.d_ffn_shared);
        if (act >= 2147483648.0)
            return fail(PW_E_SHAPE, "max_tokens * (top_k + 1) * max(d_ffn, d_ffn_shared) must stay below 2^31");
    }
    pw_layer_s* L = new (std::nothrow) pw_layer_s();
    if (!L) return fail(PW_E_NOMEM, "pw_layer_create: out of host memory");
    L->desc = D;
    L->n_total = D.n_experts + (D.d_ffn_shared > 0 ? 1 : 0);
    L->pages.resize((size_t)n_blocks(L));
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    L->device = dev;
    *out = L;
    return PW_OK;
}

pw_status pw_layer_destroy(pw_layer L) {
    g_err.clear();
    if (!L) return PW_OK;
    if (L->dev_ready || L->d_ws || L->d_blocks) {
        DeviceGuard g(L->device);
        release_device(L);
    }
    delete L;
    return PW_OK;
}

pw_status pw_moe_plan_set(pw_layer L, const uint8_t* bits, int32_t n) {
    g_err.clear();
    if (!L || !bits) return fail(PW_E_ARG, "pw_moe_plan_set: null argument");
    if (n != n_blocks(L))
        return fail(PW_E_ARG, "pw_moe_plan_set: n_blocks %d, layer has %d", n, n_blocks(L));
    for (int i = 0; i < n; ++i)
        if (bits[i] < 1 || bits[i] > PW_MAX_BITS)
            return fail(PW_E_BITS, "block %d (expert %d, linear %d): bits %d not in 1..8", i, i / 3, i % 3,
                        bits[i]);
    L->bits.assign(bits, bits + n);
    L->dirty = true;
    return PW_OK;
}

pw_status pw_page_table_bind(pw_layer L, int32_t expert, int32_t linear, const void* const* planes,
                             int32_t n_planes, const void* lut, int32_t lut_bits) {
    g_err.clear();
    if (!L) return fail(PW_E_ARG, "pw_page_table_bind: null layer");
    if (expert < 0 || expert >= L->n_total)
        return fail(PW_E_ARG, "expert %d not in 0..%d", expert, L->n_total - 1);
    if (linear < PW_GATE || linear > PW_DOWN) return fail(PW_E_ARG, "linear %d not in 0..2", linear);
    if (n_planes < 1 || n_planes > 8) return fail(PW_E_ARG, "n_planes %d not in 1..8", n_planes);
    if (lut_bits < 1 || lut_bits > PW_MAX_BITS) return fail(PW_E_BITS, "lut_bits %d not in 1..8", lut_bits);
    if (!planes || !lut) return fail(PW_E_ARG, "pw_page_table_bind: null planes or lut");
    for (int p = 0; p < n_planes; ++p) {
        if (!planes[p]) return fail(PW_E_ARG, "plane %d is null", p);
        if (!aligned16(planes[p])) return fail(PW_E_ALIGN, "plane %d is not 16-byte aligned", p);
    }
    if (!aligned16(lut)) return fail(PW_E_ALIGN, "lut is not 16-byte aligned");
    Page& pg = L->pages[(size_t)expert * 3 + linear];
    for (int p = 0; p < 8; ++p) pg.planes[p] = p < n_planes ? planes[p] : nullptr;
    pg.n_planes = n_planes;
    pg.lut = lut;
    pg.lut_bits = lut_bits;
    L->dirty = true;
    return PW_OK;
}

pw_status pw_moe_forward(pw_layer L, const void* x, int32_t T, const void* router_w, const void* router_b,
                         float* y, void* x_next, const pw_route_out* route, void* stream) {
    g_err.clear();
    if (!L) return fail(PW_E_ARG, "pw_moe_forward: null layer");
    const pw_moe_desc& D = L->desc;
    if (T < 0 || T > D.max_tokens) return fail(PW_E_RANGE, "T=%d not in 0..max_tokens=%d", T, D.max_tokens);
    pw_status st = validate_tables(L);
    if (st != PW_OK) return st;
    if (T == 0) return PW_OK;
    if (!x || !router_w || !y) return fail(PW_E_ARG, "pw_moe_forward: null x, router_w or y");
    if (!aligned16(x) || !aligned16(router_w) || !aligned16(y) || (x_next && !aligned16(x_next)))
        return fail(PW_E_ALIGN, "x, router_w, y and x_next must be 16-byte aligned");
    if (router_b && (reinterpret_cast<uintptr_t>(router_b) & 1u))
        return fail(PW_E_ALIGN, "router_b must be 2-byte aligned");
    if (route) {
        const void* rp[5] = {route->topk_ids, route->topk_w, route->expert_count, route->expert_offset,
                             route->sorted_assign};
        for (const void* q : rp)
            if (q && (reinterpret_cast<uintptr_t>(q) & 3u))
                return fail(PW_E_ALIGN, "route outputs must be 4-byte aligned");
    }
    DeviceGuard guard(L->device);
    if (!guard.ok) return fail(PW_E_HIP, "cannot select device %d", L->device);
    hipStream_t s = (hipStream_t)stream;
    if ((st = ensure_device(L, s)) != PW_OK) return st;
    if ((st = upload_tables(L, s)) != PW_OK) return st;

    const int E = D.n_experts, k = D.top_k, d = D.d_model;
    const int has_shared = D.d_ffn_shared > 0;
    L->last_T = T;

    pw::RouteParams& rp = L->rp;
    rp = pw::RouteParams{};
    rp.x = (const uint16_t*)x;
    rp.wr = (const uint16_t*)router_w;
    rp.bias = (const uint16_t*)router_b;
    rp.T = T;
    rp.d = d;
    rp.E = E;
    rp.k = k;
    rp.ws = L->ws;
    rp.y = y;
    rp.has_shared = has_shared;
    rp.tiles_gu_r = D.d_ffn / 32;
    rp.tiles_gu_s = D.d_ffn_shared / 32;
    rp.tiles_dn = d / 64;
    rp.pieces_dn_r = (D.d_ffn + pw::kDownPiece - 1) / pw::kDownPiece;
    rp.pieces_dn_s = (D.d_ffn_shared + pw::kDownPiece - 1) / pw::kDownPiece;
    if (route) {
        rp.o_ids = route->topk_ids;
        rp.o_w = route->topk_w;
        rp.o_counts = route->expert_count;
        rp.o_offsets = route->expert_offset;
        rp.o_sorted = route->sorted_assign;
    }
    pw::GemmParams gp{};
    gp.blocks = L->d_blocks;
    gp.E = E;
    gp.k = k;
    gp.T = T;
    gp.d = d;
    gp.F = D.d_ffn;
    gp.Fs = D.d_ffn_shared;
    gp.has_shared = has_shared;
    gp.ws = L->ws;
    gp.ld_act = L->f_max;
    gp.shared_base = D.max_tokens * k;
    gp.y = y;
    // gate_up + SwiGLU: items of 32 rows of F (gate and up)
    L->gp_gu = gp;
    L->gp_gu.tiles_r = D.d_ffn / 32;
    L->gp_gu.tiles_s = D.d_ffn_shared / 32;
    L->gp_gu.pieces_r = L->gp_gu.pieces_s = 1;
    L->gp_gu.x = (const uint16_t*)x;
    L->gp_gu.b_bytes = (uint32_t)((size_t)T * d * 2);
    // down + weighted scatter-accumulate: items of 64 rows of d
    L->gp_dn = gp;
    L->gp_dn.tiles_r = d / 64;
    L->gp_dn.tiles_s = has_shared ? d / 64 : 0;
    L->gp_dn.pieces_r = rp.pieces_dn_r;
    L->gp_dn.pieces_s = has_shared ? rp.pieces_dn_s : 1;
    L->gp_dn.b_bytes = (uint32_t)(((size_t)D.max_tokens * k + (size_t)D.max_tokens * has_shared) * L->f_max * 2);
    L->res_x = (const uint16_t*)x;
    L->res_y = y;
    L->res_out = (uint16_t*)x_next;

    for (int phase = 0; phase < 3; ++phase)
        if ((st = launch_phase(L, phase, s)) != PW_OK) return st;
    static const bool debug_sync = getenv("PW_DEBUG_SYNC") != nullptr;   // read once per process
    if (debug_sync) {
        hipError_t e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail(e, "pw_moe_forward (debug sync)");
    }
    return PW_OK;
}

pw_status pw_moe_replay(pw_layer L, int32_t phase, void* stream) {
    g_err.clear();
    if (!L) return fail(PW_E_ARG, "pw_moe_replay: null layer");
    if (!L->dev_ready || L->last_T == 0) return fail(PW_E_STATE, "pw_moe_replay: no forward has run");
    if (phase < 0 || phase > 2) return fail(PW_E_ARG, "phase %d not in 0..2", phase);
    DeviceGuard guard(L->device);
    if (!guard.ok) return fail(PW_E_HIP, "cannot select device %d", L->device);
    return launch_phase(L, phase, (hipStream_t)stream);
}

pw_status pw_layer_status(pw_layer L, void* stream, uint32_t* flags) {
    g_err.clear();
    if (!L || !flags) return fail(PW_E_ARG, "pw_layer_status: null argument");
    *flags = 0;
    if (!L->dev_ready) return PW_OK;
    DeviceGuard guard(L->device);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    uint32_t v = 0;
    if ((e = hipMemcpyAsync(&v, L->ws.status, sizeof v, hipMemcpyDeviceToHost, s)) != hipSuccess)
        return hip_fail(e, "status read");
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "status sync");
    if (v) {
        const uint32_t zero = 0;
        if ((e = hipMemcpy(L->ws.status, &zero, sizeof zero, hipMemcpyHostToDevice)) != hipSuccess)
            return hip_fail(e, "status clear");
    }
    *flags = v;
    if (v)
        return fail(PW_E_STATE, "device status flags 0x%x (%s%s)", v,
                    (v & PW_STATUS_ROUTER_RANGE) ? "router range " : "",
                    (v & PW_STATUS_DEP_TIMEOUT) ? "dependency wait timed out" : "");
    return PW_OK;
}

pw_status pw_layer_last_bytes(pw_layer L, void* stream, double* bytes) {
    g_err.clear();
    if (!L || !bytes) return fail(PW_E_ARG, "pw_layer_last_bytes: null argument");
    if (!L->dev_ready || L->last_T == 0) return fail(PW_E_STATE, "no forward has run");
    DeviceGuard guard(L->device);
    const pw_moe_desc& D = L->desc;
    const int E = D.n_experts, T = L->last_T, d = D.d_model;
    std::vector<int32_t> cnt((size_t)E);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if ((e = hipMemcpyAsync(cnt.data(), L->ws.counts, sizeof(int32_t) * E, hipMemcpyDeviceToHost, s)) !=
        hipSuccess)
        return hip_fail(e, "counts read");
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "counts sync");
    auto blk_bytes = [&](int ex, int lin) {
        const int b = L->bits[(size_t)ex * 3 + lin];
        const double R = block_rows(L, ex, lin), K = block_cols(L, ex, lin);
        return R * K * b / 8.0 + R * (double)(1 << b) * 2.0;
    };
    double gu = 0, dn = 0;
    for (int ex = 0; ex < L->n_total; ++ex) {
        const bool active = (ex == E) || cnt[ex] > 0;
        if (!active) continue;
        gu += blk_bytes(ex, PW_GATE) + blk_bytes(ex, PW_UP);
        dn += blk_bytes(ex, PW_DOWN);
    }
    bytes[0] = (double)T * d * 2 + (double)E * d * 2;   // x and router weights read
    bytes[1] = gu + (double)T * d * 2;                  // gate/up pages + x
    bytes[2] = dn + (double)T * d * 4;                  // down pages + y
    bytes[3] = (double)T * d * (2 + 4 + 2);             // x, y read; x_next written
    return PW_OK;
}

pw_status pw_debug_unpack(const void* const* planes, int32_t b, int32_t R, int32_t K, uint8_t* idx_out,
                          void* stream) {
    g_err.clear();
    if (!planes || !idx_out) return fail(PW_E_ARG, "pw_debug_unpack: null argument");
    if (b < 1 || b > 8) return fail(PW_E_BITS, "b=%d not in 1..8", b);
    if (R <= 0 || R % 32 || K <= 0 || K % 128) return fail(PW_E_SHAPE, "R %% 32 and K %% 128 must be 0");
    uint64_t p8[8] = {};
    for (int p = 0; p < b; ++p) {
        if (!planes[p] || !aligned16(planes[p])) return fail(PW_E_ALIGN, "plane %d null or misaligned", p);
        p8[p + 8 - b] = (uint64_t)(uintptr_t)planes[p];
    }
    hipError_t e = pw::launch_debug(p8, b, nullptr, R, K, idx_out, nullptr, (hipStream_t)stream);
    return e == hipSuccess ? PW_OK : hip_fail(e, "debug kernel");
}

pw_status pw_debug_dequant(const void* const* planes, int32_t b, const void* lut, int32_t R, int32_t K,
                           void* w_out, void* stream) {
    g_err.clear();
    if (!planes || !lut || !w_out) return fail(PW_E_ARG, "pw_debug_dequant: null argument");
    if (b < 1 || b > 8) return fail(PW_E_BITS, "b=%d not in 1..8", b);
    if (R <= 0 || R % 32 || K <= 0 || K % 128) return fail(PW_E_SHAPE, "R %% 32 and K %% 128 must be 0");
    if (!aligned16(lut) || !aligned16(w_out)) return fail(PW_E_ALIGN, "lut / w_out misaligned");
    uint64_t p8[8] = {};
    for (int p = 0; p < b; ++p) {
        if (!planes[p] || !aligned16(planes[p])) return fail(PW_E_ALIGN, "plane %d null or misaligned", p);
        p8[p + 8 - b] = (uint64_t)(uintptr_t)planes[p];
    }
    hipError_t e = pw::launch_debug(p8, b, (const uint16_t*)lut, R, K, nullptr, (uint16_t*)w_out,
                                    (hipStream_t)stream);
    return e == hipSuccess ? PW_OK : hip_fail(e, "debug kernel");
}

}  // extern "C"

pw_status pw_debug_set_wait_limit(pw_layer L, uint32_t polls) {
    g_err.clear();
    if (!L) return fail(PW_E_ARG, "pw_debug_set_wait_limit: null layer");
    L->wait_limit = polls;
    if (L->dev_ready) {   // later forwards read it from the workspace
        DeviceGuard guard(L->device);
        if (!guard.ok) return fail(PW_E_HIP, "cannot select device %d", L->device);
        const hipError_t e = hipMemcpy(L->ws.wait_limit, &polls, sizeof polls, hipMemcpyHostToDevice);
        if (e != hipSuccess) return hip_fail(e, "wait limit");
    }
    return PW_OK;
}
