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
#include <climits>
#include <cstdlib>
#include <cmath>
#include <array>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "pw.h"
#include "pw_internal.h"

static_assert(PW_PATH_AUTO == pw::PATH_AUTO && PW_PATH_SMALL == pw::PATH_SMALL && PW_PATH_FOUR == pw::PATH_FOUR &&
                  PW_PATH_BIG == pw::PATH_BIG && PW_PATH_TWO == pw::PATH_TWO,
              "path values of the ABI and of the launcher");

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

// Arguments of every kernel of one forward.
struct pw_launch {
    int T = 0;
    int n_cu = 256;
    int path = pw::PATH_AUTO;
    pw::RouteParams rp{};
    pw::GemmParams gu{}, dn{};
    const uint16_t* res_x = nullptr;
    const float* res_y = nullptr;
    uint16_t* res_out = nullptr;
};

// Byte offsets of the workspace arrays for forwards of up to T tokens.
struct WsLayout {
    size_t o_ids, o_w, o_cnt, o_off, o_srt, o_inv, o_stk, o_sw, o_pre, o_act, o_part, o_st, o_lg, o_dep, total;
    bool det;
    int T, n_dep, n_counters, dep_stride;
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

    // launch record of the last pw_moe_forward (for pw_layer_last_bytes and pw_moe_replay)
    pw_launch rec{};
    uint32_t wait_limit = 1u << 20;   // polls of a down item's dependency counter
    int path = pw::PATH_AUTO;          // which expert kernel takes which experts (pw::PATH_*)
    // host copy of the page table for pw_moe_forward_noalloc (sized at create)
    std::vector<DevBlock> shadow;
    uint32_t* noalloc_status = nullptr;   // status word in the device scratch, once used
    // blocks in order (expert, linear, row-block): expert, linear, rows, columns, first block of
    // each (expert, linear)
    std::vector<int32_t> blk_expert, blk_lin, blk_rows, blk_cols, first_block;
};

namespace {

int n_blocks(const pw_layer_s* L) { return (int)L->blk_rows.size(); }

int linear_rows(const pw_layer_s* L, int e, int lin) {
    const int f = (e == L->desc.n_experts) ? L->desc.d_ffn_shared : L->desc.d_ffn;
    return lin == PW_DOWN ? L->desc.d_model : f;
}
int linear_cols(const pw_layer_s* L, int e, int lin) {
    const int f = (e == L->desc.n_experts) ? L->desc.d_ffn_shared : L->desc.d_ffn;
    return lin == PW_DOWN ? f : L->desc.d_model;
}

// The layer's blocks: every linear whole (rows_per_block 0) or cut into row-blocks.
void make_block_list(pw_layer_s* L) {
    const int rb = L->desc.rows_per_block;
    for (int e = 0; e < L->n_total; ++e)
        for (int lin = 0; lin < 3; ++lin) {
            const int R = linear_rows(L, e, lin), rows = rb ? rb : R;
            L->first_block.push_back((int32_t)L->blk_rows.size());
            for (int j = 0; j < R / rows; ++j) {
                L->blk_expert.push_back(e);
                L->blk_lin.push_back(lin);
                L->blk_rows.push_back(rows);
                L->blk_cols.push_back(linear_cols(L, e, lin));
            }
        }
}

// Checks that every block's pages cover its planned bitwidth.
pw_status validate_tables(const pw_layer_s* L) {
    if (L->bits.empty()) return fail(PW_E_STATE, "pw_moe_forward: no plan set (call pw_moe_plan_set)");
    for (int i = 0; i < n_blocks(L); ++i) {
        const int b = L->bits[i];
        const Page& pg = L->pages[i];
        if (pg.n_planes < b || pg.lut_bits != b || pg.lut == nullptr)
            return fail(PW_E_UNBOUND,
                        "block %d (expert %d, linear %d, row-block %d): planned b=%d but bound %d planes and LUT bits %d",
                        i, L->blk_expert[i], L->blk_lin[i], i - L->first_block[L->blk_expert[i] * 3 + L->blk_lin[i]],
                        b, pg.n_planes, pg.lut_bits);
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

// K-pieces of a routed / the shared down projection
int pieces_routed(const pw_moe_desc& D) { return (D.d_ffn + pw::kDownPiece - 1) / pw::kDownPiece; }
int pieces_shared(const pw_moe_desc& D) { return (D.d_ffn_shared + pw::kDownPiece - 1) / pw::kDownPiece; }
size_t part_rows(const pw_moe_desc& D, int T) {
    return (size_t)T * D.top_k * pieces_routed(D) + (size_t)T * pieces_shared(D);
}

WsLayout ws_layout(const pw_moe_desc& D, int T) {
    const int E = D.n_experts, k = D.top_k;
    const int has_shared = D.d_ffn_shared > 0;
    const int f_max = std::max(D.d_ffn, D.d_ffn_shared);
    const size_t act_rows = (size_t)T * k + (size_t)T * has_shared;
    auto al = [](size_t n) { return (n + 255) & ~(size_t)255; };
    WsLayout w{};
    size_t off = 0;
    w.o_ids = off;    off += al(sizeof(int32_t) * (size_t)T * k);
    w.o_w = off;      off += al(sizeof(float) * (size_t)T * k);
    w.o_cnt = off;    off += al(sizeof(int32_t) * (size_t)E);
    w.o_off = off;    off += al(sizeof(int32_t) * ((size_t)E + 1));
    w.o_srt = off;    off += al(sizeof(int32_t) * (size_t)T * k);
    w.o_inv = off;    off += al(sizeof(int32_t) * (size_t)T * k);
    w.o_stk = off;    off += al(sizeof(int32_t) * (size_t)T * k);
    w.o_sw = off;     off += al(sizeof(float) * (size_t)T * k);
    w.o_pre = off;    off += al(sizeof(int32_t) * (size_t)pw::N_LISTS * (E + 2));
    w.o_act = off;    off += al(sizeof(uint16_t) * act_rows * (size_t)f_max);
    // deterministic mode: one fp32 row of d per (routed slot, K-piece) and per (token, shared K-piece)
    w.det = (D.flags & PW_FLAG_DETERMINISTIC) != 0;
    w.o_part = off;
    if (w.det) off += al(sizeof(float) * part_rows(D, T) * (size_t)D.d_model);
    w.o_st = off;     off += al(2 * sizeof(uint32_t));   // status, wait limit
    w.o_lg = off;     off += al(sizeof(long long) * (size_t)T * E);
    w.dep_stride = (f_max + pw::kDownPiece - 1) / pw::kDownPiece;
    w.n_dep = (E + 1) * w.dep_stride + 1;
    w.n_counters = w.n_dep + T + 1;   // dep, tok_cnt, route_done
    w.o_dep = off;    off += al(sizeof(uint32_t) * (size_t)w.n_counters);
    w.total = off;
    w.T = T;
    return w;
}

// The workspace arrays of layout w inside the device buffer at base (256-byte aligned).
pw::Workspace carve(char* b, const WsLayout& w) {
    pw::Workspace ws{};
    ws.ids = (int32_t*)(b + w.o_ids);
    ws.w = (float*)(b + w.o_w);
    ws.counts = (int32_t*)(b + w.o_cnt);
    ws.offsets = (int32_t*)(b + w.o_off);
    ws.sorted = (int32_t*)(b + w.o_srt);
    ws.slot_of = (int32_t*)(b + w.o_inv);
    ws.part = w.det ? (float*)(b + w.o_part) : nullptr;
    ws.slot_tok = (int32_t*)(b + w.o_stk);
    ws.slot_w = (float*)(b + w.o_sw);
    ws.prefix = (int32_t*)(b + w.o_pre);
    ws.act = (uint16_t*)(b + w.o_act);
    ws.status = (uint32_t*)(b + w.o_st);
    ws.wait_limit = ws.status + 1;
    ws.lg = (long long*)(b + w.o_lg);
    ws.dep = (uint32_t*)(b + w.o_dep);
    ws.tok_cnt = ws.dep + w.n_dep;
    ws.route_done = ws.tok_cnt + w.T;
    ws.dep_stride = w.dep_stride;
    return ws;
}

// Compute units of a device, read once per device.
pw_status device_cus(int dev, int* n_cu) {
    static int cached[64] = {};
    if (dev < 0 || dev >= 64) return fail(PW_E_ARG, "device %d", dev);
    if (cached[dev] <= 0) {
        int cus = 0;
        const hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(e, "device attribute");
        cached[dev] = cus > 0 ? cus : 256;
    }
    *n_cu = cached[dev];
    return PW_OK;
}

pw_status ensure_device(pw_layer_s* L, hipStream_t s) {
    if (L->dev_ready) return PW_OK;
    const pw_moe_desc& D = L->desc;
    L->f_max = std::max(D.d_ffn, D.d_ffn_shared);
    const WsLayout lay = ws_layout(D, D.max_tokens);
    hipError_t e;
    pw_status st = device_cus(L->device, &L->n_cu);
    if (st != PW_OK) return st;
    if ((e = hipMalloc((void**)&L->d_ws, lay.total)) != hipSuccess) {
        L->d_ws = nullptr;
        return fail(PW_E_NOMEM, "workspace (%zu bytes): %s", lay.total, hipGetErrorString(e));
    }
    if ((e = hipMalloc((void**)&L->d_blocks, sizeof(DevBlock) * n_blocks(L))) != hipSuccess) {
        L->d_blocks = nullptr;
        release_device(L);
        return fail(PW_E_NOMEM, "page table: %s", hipGetErrorString(e));
    }
    L->ws = carve(L->d_ws, lay);
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
    if ((e = pw::launch_init_ws(L->ws, lay.n_counters, L->wait_limit, s)) != hipSuccess) {
        release_device(L);
        return hip_fail(e, "init workspace");
    }
    L->dev_ready = true;
    return PW_OK;
}

// The device page table entries of every block: plane p goes to slot p + 8 - b,
// so slot s always carries bit 7 - s of the index.
void fill_tables(const pw_layer_s* L, DevBlock* h) {
    for (int i = 0; i < n_blocks(L); ++i) {
        const Page& pg = L->pages[i];
        DevBlock& db = h[i];
        std::memset(&db, 0, sizeof db);
        db.bits = L->bits[i];
        for (int p = 0; p < db.bits; ++p) db.planes[p + 8 - db.bits] = (uint64_t)(uintptr_t)pg.planes[p];
        db.lut = (uint64_t)(uintptr_t)pg.lut;
    }
}

pw_status upload_tables(pw_layer_s* L, hipStream_t s) {
    if (!L->dirty) return PW_OK;
    const int slot = L->stage_i;
    hipError_t e;
    if (L->stage_used[slot] && (e = hipEventSynchronize(L->stage_ev[slot])) != hipSuccess)
        return hip_fail(e, "staging event");
    DevBlock* h = L->h_stage[slot];
    fill_tables(L, h);
    if ((e = hipMemcpyAsync(L->d_blocks, h, sizeof(DevBlock) * n_blocks(L), hipMemcpyHostToDevice, s)) !=
        hipSuccess)
        return hip_fail(e, "table upload");
    if ((e = hipEventRecord(L->stage_ev[slot], s)) != hipSuccess) return hip_fail(e, "staging event record");
    L->stage_used[slot] = true;
    L->stage_i = (slot + 1) % kStageSlots;
    L->dirty = false;
    return PW_OK;
}


// The expert-kernel path of new layers: PW_FORCE_PATH = auto | small | four | big
// (read once per process; anything else is auto).
int default_path() {
    static const int path = [] {
        const char* v = getenv("PW_FORCE_PATH");
        if (!v) return (int)pw::PATH_AUTO;
        if (!strcmp(v, "small")) return (int)pw::PATH_SMALL;
        if (!strcmp(v, "four")) return (int)pw::PATH_FOUR;
        if (!strcmp(v, "big")) return (int)pw::PATH_BIG;
        if (!strcmp(v, "two")) return (int)pw::PATH_TWO;
        return (int)pw::PATH_AUTO;
    }();
    return path;
}

// Kernel arguments of one forward on T tokens with workspace ws, device page
// table blocks and the shared expert's act rows from shared_base on.
pw_launch make_launch(const pw_layer_s* L, const void* x, int T, const void* router_w, const void* router_b,
                      float* y, void* x_next, const pw_route_out* route, const pw::Workspace& ws,
                      const DevBlock* blocks, int shared_base, int n_cu) {
    const pw_moe_desc& D = L->desc;
    const int path = L->path;
    const int E = D.n_experts, k = D.top_k, d = D.d_model;
    const int has_shared = D.d_ffn_shared > 0;
    const int f_max = std::max(D.d_ffn, D.d_ffn_shared);
    pw_launch r{};
    r.T = T;
    r.n_cu = n_cu;
    r.path = path;
    pw::RouteParams& rp = r.rp;
    rp.exact_all = (long)T * E <= pw::kRouteExactAllWork ? 1 : 0;
    // the small lists' token group: 32 when the routed experts average more than
    // one 16-token tile (T k > 16 E), so that an expert of 17..32 tokens is one
    // item per tile (each weight dequantised once) in the two-tile kernel; below
    // that most experts fit one tile, and the one-tile kernel's double-buffered
    // planes run them faster (measured: mixtral_d4096 T = 64, fine_e128 T = 128)
    rp.small_tokens = path == pw::PATH_SMALL ? pw::kSmallTokens : path == pw::PATH_TWO ? pw::kTwoTokens
                    : ((long)T * k > (long)pw::kSmallTokens * E ? pw::kTwoTokens : pw::kSmallTokens);
    rp.small_max = (path == pw::PATH_SMALL || path == pw::PATH_TWO) ? INT_MAX : path == pw::PATH_BIG ? 0 : pw::kSmallMax;
    rp.four_max = (path == pw::PATH_SMALL || path == pw::PATH_TWO || path == pw::PATH_FOUR) ? INT_MAX
                : path == pw::PATH_BIG ? 0 : (T >= pw::kBigBatch ? pw::kFourMaxBig : pw::kFourMax);
    rp.x = (const uint16_t*)x;
    rp.wr = (const uint16_t*)router_w;
    rp.bias = (const uint16_t*)router_b;
    rp.T = T;
    rp.d = d;
    rp.E = E;
    rp.k = k;
    rp.ws = ws;
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
    gp.blocks = blocks;
    gp.E = E;
    gp.k = k;
    gp.T = T;
    gp.d = d;
    gp.F = D.d_ffn;
    gp.Fs = D.d_ffn_shared;
    gp.has_shared = has_shared;
    gp.ws = ws;
    gp.ld_act = f_max;
    gp.shared_base = shared_base;
    gp.lut_tiled = (D.flags & PW_FLAG_LUT_TILED) ? 1 : 0;
    gp.det = (D.flags & PW_FLAG_DETERMINISTIC) ? 1 : 0;
    gp.part_shared = T * k * pieces_routed(D);
    gp.rb_lg = 0;
    while (D.rows_per_block > 0 && (1 << gp.rb_lg) < D.rows_per_block) ++gp.rb_lg;
    gp.y = y;
    // gate_up + SwiGLU: items of 32 rows of F (gate and up)
    r.gu = gp;
    r.gu.tiles_r = D.d_ffn / 32;
    r.gu.tiles_s = D.d_ffn_shared / 32;
    r.gu.pieces_r = r.gu.pieces_s = 1;
    r.gu.x = (const uint16_t*)x;
    r.gu.b_bytes = (uint32_t)((size_t)T * d * 2);
    // down + weighted scatter-accumulate: items of 64 rows of d
    r.dn = gp;
    r.dn.tiles_r = d / 64;
    r.dn.tiles_s = has_shared ? d / 64 : 0;
    r.dn.pieces_r = rp.pieces_dn_r;
    r.dn.pieces_s = has_shared ? rp.pieces_dn_s : 1;
    r.dn.b_bytes = (uint32_t)(((size_t)shared_base + (size_t)T * has_shared) * f_max * 2);
    r.res_x = (const uint16_t*)x;
    r.res_y = y;
    r.res_out = (uint16_t*)x_next;
    return r;
}

// Enqueues the kernels of one phase of a forward: 0 routing (router + bucket
// sort), 1 experts (gate_up + SwiGLU + down + accumulation), 2 residual hand-off.
pw_status launch_phase(const pw_launch& r, int d_model, int phase, hipStream_t s) {
    const int T = r.T;
    hipError_t e = hipSuccess;
    switch (phase) {
        case 0:
            if ((e = pw::launch_route(r.rp, s)) != hipSuccess) return hip_fail(e, "route kernel");
            break;
        case 1: {
            pw::ExpertParams ep{r.gu, r.dn};
            ep.gu.list = pw::LIST_GU_SMALL;
            ep.dn.list = pw::LIST_DN_SMALL;
            // a kernel is launched when some expert can reach its token range
            if (r.rp.small_max > 0 && (e = pw::launch_experts(r.rp.small_tokens, ep, r.n_cu, s)) != hipSuccess)
                return hip_fail(e, "expert kernel");
            if (T > r.rp.small_max && r.rp.four_max > r.rp.small_max) {
                ep.gu.list = pw::LIST_GU_FOUR;
                ep.dn.list = pw::LIST_DN_FOUR;
                if ((e = pw::launch_experts(pw::kLargeTokens, ep, r.n_cu, s)) != hipSuccess)
                    return hip_fail(e, "expert kernel (four-tile)");
            }
            if (T > r.rp.four_max) {
                ep.gu.list = pw::LIST_GU_BIG;
                ep.dn.list = pw::LIST_DN_BIG;
                if ((e = pw::launch_experts_big(ep, r.n_cu, s)) != hipSuccess)
                    return hip_fail(e, "expert kernel (dequantise-once)");
            }
            if (r.dn.det && (e = pw::launch_reduce(r.dn.ws, r.dn.y, T, r.dn.k, r.dn.d, r.dn.pieces_r,
                                                    r.dn.has_shared ? r.dn.pieces_s : 0, r.dn.part_shared, s)) !=
                                hipSuccess)
                return hip_fail(e, "reduce kernel");
            break;
        }
        case 2:
            if (r.res_out && (e = pw::launch_residual(r.res_x, r.res_y, r.res_out, (long)T * d_model, s)) != hipSuccess)
                return hip_fail(e, "residual kernel");
            break;
        default:
            return fail(PW_E_ARG, "phase %d not in 0..2", phase);
    }
    return PW_OK;
}

// Argument checks shared by both forward entry points (no HIP call).
pw_status check_forward(const pw_layer_s* L, const void* x, int32_t T, const void* router_w, const void* router_b,
                        const float* y, const void* x_next, const pw_route_out* route) {
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
    return PW_OK;
}

pw_status enqueue_all(const pw_launch& r, int d_model, hipStream_t s) {
    pw_status st;
    for (int phase = 0; phase < 3; ++phase)
        if ((st = launch_phase(r, d_model, phase, s)) != PW_OK) return st;
    static const bool debug_sync = getenv("PW_DEBUG_SYNC") != nullptr;   // read once per process
    if (debug_sync) {
        hipError_t e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail(e, "pw_moe_forward (debug sync)");
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
    if (D.flags & ~(PW_FLAG_LUT_TILED | PW_FLAG_DETERMINISTIC))
        return fail(PW_E_ARG, "flags 0x%x: only PW_FLAG_LUT_TILED and PW_FLAG_DETERMINISTIC are defined", D.flags);
    if (D.rows_per_block < 0 || D.rows_per_block % 64 || (D.rows_per_block & (D.rows_per_block - 1)) ||
        (D.rows_per_block > 0 && (D.d_model % D.rows_per_block || D.d_ffn % D.rows_per_block ||
                                  D.d_ffn_shared % D.rows_per_block)))
        return fail(PW_E_SHAPE, "rows_per_block %d: must be 0 or a power of two of at least 64 dividing d_model, "
                    "d_ffn and d_ffn_shared", D.rows_per_block);
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
    L->path = default_path();
    L->n_total = D.n_experts + (D.d_ffn_shared > 0 ? 1 : 0);
    make_block_list(L);
    L->pages.resize((size_t)n_blocks(L));
    L->shadow.resize((size_t)n_blocks(L));
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
            return fail(PW_E_BITS, "block %d (expert %d, linear %d): bits %d not in 1..8", i, L->blk_expert[i],
                        L->blk_lin[i], bits[i]);
    L->bits.assign(bits, bits + n);
    L->dirty = true;
    return PW_OK;
}

// Checks the pages of one bind; the caller has checked the layer and the block.
pw_status check_pages(const void* const* planes, int32_t n_planes, const void* lut, int32_t lut_bits) {
    if (n_planes < 1 || n_planes > 8) return fail(PW_E_ARG, "n_planes %d not in 1..8", n_planes);
    if (lut_bits < 1 || lut_bits > PW_MAX_BITS) return fail(PW_E_BITS, "lut_bits %d not in 1..8", lut_bits);
    if (!planes || !lut) return fail(PW_E_ARG, "pw_page_table_bind: null planes or lut");
    for (int p = 0; p < n_planes; ++p) {
        if (!planes[p]) return fail(PW_E_ARG, "plane %d is null", p);
        if (!aligned16(planes[p])) return fail(PW_E_ALIGN, "plane %d is not 16-byte aligned", p);
    }
    if (!aligned16(lut)) return fail(PW_E_ALIGN, "lut is not 16-byte aligned");
    return PW_OK;
}

void set_page(pw_layer_s* L, int block, const void* const* planes, int32_t n_planes, size_t plane_off,
              const void* lut, int32_t lut_bits, size_t lut_off) {
    Page& pg = L->pages[(size_t)block];
    for (int p = 0; p < 8; ++p) pg.planes[p] = p < n_planes ? (const char*)planes[p] + plane_off : nullptr;
    pg.n_planes = n_planes;
    pg.lut = (const char*)lut + lut_off;
    pg.lut_bits = lut_bits;
}

pw_status pw_page_table_bind(pw_layer L, int32_t expert, int32_t linear, const void* const* planes,
                             int32_t n_planes, const void* lut, int32_t lut_bits) {
    g_err.clear();
    if (!L) return fail(PW_E_ARG, "pw_page_table_bind: null layer");
    if (expert < 0 || expert >= L->n_total)
        return fail(PW_E_ARG, "expert %d not in 0..%d", expert, L->n_total - 1);
    if (linear < PW_GATE || linear > PW_DOWN) return fail(PW_E_ARG, "linear %d not in 0..2", linear);
    pw_status st = check_pages(planes, n_planes, lut, lut_bits);
    if (st != PW_OK) return st;
    // every row-block of the linear, from whole-linear pages: row-block j starts j*rows rows in
    const int first = L->first_block[expert * 3 + linear];
    const int R = linear_rows(L, expert, linear), rows = L->blk_rows[first], K = L->blk_cols[first];
    for (int j = 0; j < R / rows; ++j)
        set_page(L, first + j, planes, n_planes, (size_t)j * rows * (K / 8), lut, lut_bits,
                 (size_t)j * rows * ((size_t)1 << lut_bits) * 2);
    L->dirty = true;
    return PW_OK;
}

pw_status pw_page_table_bind_rows(pw_layer L, int32_t expert, int32_t linear, int32_t row_block,
                                  const void* const* planes, int32_t n_planes, const void* lut, int32_t lut_bits) {
    g_err.clear();
    if (!L) return fail(PW_E_ARG, "pw_page_table_bind_rows: null layer");
    if (expert < 0 || expert >= L->n_total)
        return fail(PW_E_ARG, "expert %d not in 0..%d", expert, L->n_total - 1);
    if (linear < PW_GATE || linear > PW_DOWN) return fail(PW_E_ARG, "linear %d not in 0..2", linear);
    const int first = L->first_block[expert * 3 + linear];
    const int n_rb = linear_rows(L, expert, linear) / L->blk_rows[first];
    if (row_block < 0 || row_block >= n_rb)
        return fail(PW_E_ARG, "row_block %d not in 0..%d", row_block, n_rb - 1);
    pw_status st = check_pages(planes, n_planes, lut, lut_bits);
    if (st != PW_OK) return st;
    set_page(L, first + row_block, planes, n_planes, 0, lut, lut_bits, 0);
    L->dirty = true;
    return PW_OK;
}

pw_status pw_moe_forward(pw_layer L, const void* x, int32_t T, const void* router_w, const void* router_b,
                         float* y, void* x_next, const pw_route_out* route, void* stream) {
    g_err.clear();
    if (!L) return fail(PW_E_ARG, "pw_moe_forward: null layer");
    pw_status st = check_forward(L, x, T, router_w, router_b, y, x_next, route);
    if (st != PW_OK || T == 0) return st;
    DeviceGuard guard(L->device);
    if (!guard.ok) return fail(PW_E_HIP, "cannot select device %d", L->device);
    hipStream_t s = (hipStream_t)stream;
    // every launch precondition (kernel attributes, occupancy) before the first enqueue
    {
        const hipError_t e = pw::prepare_experts((L->desc.flags & PW_FLAG_DETERMINISTIC) != 0);
        if (e != hipSuccess) return hip_fail(e, "expert kernel set-up");
    }
    if ((st = ensure_device(L, s)) != PW_OK) return st;
    if ((st = upload_tables(L, s)) != PW_OK) return st;
    L->rec = make_launch(L, x, T, router_w, router_b, y, x_next, route, L->ws, L->d_blocks,
                         L->desc.max_tokens * L->desc.top_k, L->n_cu);
    if ((st = enqueue_all(L->rec, L->desc.d_model, s)) != PW_OK) {
        L->dirty = true;   // the runtime refused a launch: upload the tables again next time
        return st;
    }
    return PW_OK;
}

pw_status pw_moe_forward_noalloc(pw_layer L, const void* x, int32_t T, const void* router_w,
                                 const void* router_b, float* y, void* x_next, const pw_route_out* route,
                                 void* stream) {
    g_err.clear();
    if (!L) return fail(PW_E_ARG, "pw_moe_forward_noalloc: null layer");
    pw_status st = check_forward(L, x, T, router_w, router_b, y, x_next, route);
    if (st != PW_OK || T == 0) return st;
    // scratch = [page table][workspace for T tokens]
    const size_t table_bytes = (sizeof(DevBlock) * (size_t)n_blocks(L) + 255) & ~(size_t)255;
    const WsLayout lay = ws_layout(L->desc, T);
    if (table_bytes + lay.total > pw::kScratchBytes)
        return fail(PW_E_RANGE, "pw_moe_forward_noalloc: T=%d needs %zu bytes of device scratch, the static scratch "
                    "holds %zu", T, table_bytes + lay.total, (size_t)pw::kScratchBytes);
    DeviceGuard guard(L->device);
    if (!guard.ok) return fail(PW_E_HIP, "cannot select device %d", L->device);
    hipStream_t s = (hipStream_t)stream;
    char* scratch = nullptr;
    size_t cap = 0;
    hipError_t e = pw::scratch_memory(L->device, (void**)&scratch, &cap);
    if (e != hipSuccess) return hip_fail(e, "device scratch address");
    if ((e = pw::prepare_experts((L->desc.flags & PW_FLAG_DETERMINISTIC) != 0)) != hipSuccess) return hip_fail(e, "expert kernel set-up");
    int n_cu = 0;
    if ((st = device_cus(L->device, &n_cu)) != PW_OK) return st;
    DevBlock* d_blocks = (DevBlock*)scratch;
    const pw::Workspace ws = carve(scratch + table_bytes, lay);
    // the page table from the layer's host copy (pageable: consumed before the copy call returns)
    fill_tables(L, L->shadow.data());
    if ((e = hipMemcpyAsync(d_blocks, L->shadow.data(), sizeof(DevBlock) * (size_t)n_blocks(L),
                            hipMemcpyHostToDevice, s)) != hipSuccess)
        return hip_fail(e, "table upload");
    // the scratch keeps the last call's contents: counters and status start from zero
    if ((e = pw::launch_init_ws(ws, lay.n_counters, L->wait_limit, s)) != hipSuccess)
        return hip_fail(e, "scratch init");
    L->noalloc_status = ws.status;
    const pw_launch r = make_launch(L, x, T, router_w, router_b, y, x_next, route, ws, d_blocks, T * L->desc.top_k,
                                    n_cu);
    return enqueue_all(r, L->desc.d_model, s);
}

pw_status pw_moe_replay(pw_layer L, int32_t phase, void* stream) {
    g_err.clear();
    if (!L) return fail(PW_E_ARG, "pw_moe_replay: null layer");
    if (!L->dev_ready || L->rec.T == 0) return fail(PW_E_STATE, "pw_moe_replay: no forward has run");
    if (phase < 0 || phase > 2) return fail(PW_E_ARG, "phase %d not in 0..2", phase);
    DeviceGuard guard(L->device);
    if (!guard.ok) return fail(PW_E_HIP, "cannot select device %d", L->device);
    return launch_phase(L->rec, L->desc.d_model, phase, (hipStream_t)stream);
}

pw_status pw_layer_status(pw_layer L, void* stream, uint32_t* flags) {
    g_err.clear();
    if (!L || !flags) return fail(PW_E_ARG, "pw_layer_status: null argument");
    *flags = 0;
    if (!L->dev_ready && !L->noalloc_status) return PW_OK;
    DeviceGuard guard(L->device);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    // the layer's own workspace, and the device scratch if it ran no-alloc forwards
    uint32_t* words[2] = {L->dev_ready ? L->ws.status : nullptr, L->noalloc_status};
    uint32_t v = 0;
    for (uint32_t* w : words) {
        if (!w) continue;
        uint32_t u = 0;
        if ((e = hipMemcpyAsync(&u, w, sizeof u, hipMemcpyDeviceToHost, s)) != hipSuccess)
            return hip_fail(e, "status read");
        if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "status sync");
        if (u) {
            const uint32_t zero = 0;
            if ((e = hipMemcpy(w, &zero, sizeof zero, hipMemcpyHostToDevice)) != hipSuccess)
                return hip_fail(e, "status clear");
        }
        v |= u;
    }
    *flags = v;
    if (v)
        return fail(PW_E_STATE, "device status flags 0x%x (%s%s)", v,
                    (v & PW_STATUS_ROUTER_RANGE) ? "router range " : "",
                    (v & PW_STATUS_DEP_TIMEOUT) ? "dependency wait timed out" : "");
    return PW_OK;
}

pw_status pw_plan_greedy(pw_layer L, const float* sensitivity, const float* residual,
                         const int32_t* expert_count, int32_t n_tokens, const uint8_t* min_bits,
                         const uint8_t* max_bits, double bytes_to_free, uint8_t* bits_out, double* result) {
    g_err.clear();
    if (!L || !sensitivity || !expert_count || !bits_out || !result)
        return fail(PW_E_ARG, "pw_plan_greedy: null argument");
    if (L->bits.empty()) return fail(PW_E_STATE, "pw_plan_greedy: the layer has no plan");
    if (n_tokens <= 0) return fail(PW_E_ARG, "pw_plan_greedy: n_tokens %d", n_tokens);
    if (!std::isfinite(bytes_to_free)) return fail(PW_E_ARG, "pw_plan_greedy: bytes_to_free not finite");
    const pw_moe_desc& D = L->desc;
    const int n = n_blocks(L), E = D.n_experts;
    std::vector<int32_t> rows(n), cols(n);
    std::vector<uint8_t> lo(n), hi(n);
    std::vector<double> mass(n);
    for (int e = 0; e < E; ++e)
        if (expert_count[e] < 0) return fail(PW_E_ARG, "expert_count[%d] = %d", e, expert_count[e]);
    for (int i = 0; i < n; ++i) {
        const int e = L->blk_expert[i];
        if (!(sensitivity[i] >= 0.0f) || !std::isfinite(sensitivity[i]))
            return fail(PW_E_ARG, "sensitivity[%d] must be finite and >= 0", i);
        if (residual && (!(residual[i] >= 0.0f) || !std::isfinite(residual[i])))
            return fail(PW_E_ARG, "residual[%d] must be finite and >= 0", i);
        rows[i] = L->blk_rows[i];
        cols[i] = L->blk_cols[i];
        lo[i] = min_bits ? min_bits[i] : 3;
        hi[i] = max_bits ? max_bits[i] : 8;
        if (lo[i] < 1 || hi[i] > 8 || lo[i] > hi[i] || L->bits[i] < lo[i] || L->bits[i] > hi[i])
            return fail(PW_E_BITS, "block %d: bits %d outside [%d, %d] (min/max in 1..8)", i, L->bits[i], lo[i], hi[i]);
        mass[i] = e == E ? 1.0 : (double)expert_count[e] / (double)n_tokens;
    }
    pw::PlanProblem P{n, rows.data(), cols.data(), lo.data(), hi.data(), sensitivity, residual, mass.data()};
    std::memcpy(bits_out, L->bits.data(), (size_t)n);
    double moved = 0.0, dmg = 0.0;
    const int actions = pw::plan_greedy(P, bytes_to_free, bits_out, &moved, &dmg);
    result[0] = moved;
    result[1] = dmg;
    result[2] = actions;
    return PW_OK;
}

pw_status pw_layer_last_bytes(pw_layer L, void* stream, double* bytes) {
    g_err.clear();
    if (!L || !bytes) return fail(PW_E_ARG, "pw_layer_last_bytes: null argument");
    if (!L->dev_ready || L->rec.T == 0) return fail(PW_E_STATE, "no forward has run");
    DeviceGuard guard(L->device);
    const pw_moe_desc& D = L->desc;
    const int E = D.n_experts, T = L->rec.T, d = D.d_model;
    std::vector<int32_t> cnt((size_t)E);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if ((e = hipMemcpyAsync(cnt.data(), L->ws.counts, sizeof(int32_t) * E, hipMemcpyDeviceToHost, s)) !=
        hipSuccess)
        return hip_fail(e, "counts read");
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "counts sync");
    double gu = 0, dn = 0;
    for (int i = 0; i < n_blocks(L); ++i) {
        const int ex = L->blk_expert[i];
        if (ex != E && cnt[ex] == 0) continue;   // experts without tokens read nothing
        const int b = L->bits[i];
        const double R = L->blk_rows[i], K = L->blk_cols[i];
        const double bytes = R * K * b / 8.0 + R * (double)(1 << b) * 2.0;
        (L->blk_lin[i] == PW_DOWN ? dn : gu) += bytes;
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
    hipError_t e = pw::launch_debug(p8, b, nullptr, 0, R, K, idx_out, nullptr, (hipStream_t)stream);
    return e == hipSuccess ? PW_OK : hip_fail(e, "debug kernel");
}

pw_status pw_debug_dequant(const void* const* planes, int32_t b, const void* lut, uint32_t lut_flags, int32_t R,
                           int32_t K, void* w_out, void* stream) {
    g_err.clear();
    if (!planes || !lut || !w_out) return fail(PW_E_ARG, "pw_debug_dequant: null argument");
    if (lut_flags & ~PW_FLAG_LUT_TILED) return fail(PW_E_ARG, "lut_flags 0x%x", lut_flags);
    if (b < 1 || b > 8) return fail(PW_E_BITS, "b=%d not in 1..8", b);
    if (R <= 0 || R % 32 || K <= 0 || K % 128) return fail(PW_E_SHAPE, "R %% 32 and K %% 128 must be 0");
    if (!aligned16(lut) || !aligned16(w_out)) return fail(PW_E_ALIGN, "lut / w_out misaligned");
    uint64_t p8[8] = {};
    for (int p = 0; p < b; ++p) {
        if (!planes[p] || !aligned16(planes[p])) return fail(PW_E_ALIGN, "plane %d null or misaligned", p);
        p8[p + 8 - b] = (uint64_t)(uintptr_t)planes[p];
    }
    hipError_t e = pw::launch_debug(p8, b, (const uint16_t*)lut, (lut_flags & PW_FLAG_LUT_TILED) ? 1 : 0, R, K,
                                    nullptr, (uint16_t*)w_out, (hipStream_t)stream);
    return e == hipSuccess ? PW_OK : hip_fail(e, "debug kernel");
}

}  // extern "C"

pw_status pw_debug_set_path(pw_layer L, int32_t path) {
    g_err.clear();
    if (!L) return fail(PW_E_ARG, "pw_debug_set_path: null layer");
    if (path < PW_PATH_AUTO || path > PW_PATH_TWO) return fail(PW_E_ARG, "path %d not in 0..4", path);
    L->path = path;
    return PW_OK;
}

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
