// gfx950 (CDNA4) kernels of the fused mixed-precision MoE layer.
//
// The layer (PagedWeight pages: arxivlens summary; legiblepapers "Key Takeaways"
// and FAQ Q5) reads every expert weight straight from Any-Precision bit-planes
// and a per-row lookup table, each (expert, linear) block at its own bitwidth b,
// and fuses routing, SwiGLU expert activation and weighted accumulation.
//
// Kernels, in stream order per forward:
//   route_kernel   exact top-k routing: for T * E <= 2048, T * ceil(E/4) work-groups
//                  compute every exact router logit (int64, units of 2^-48, one
//                  expert per wave); for more, T * ceil(E/16) work-groups
//                  compute fp32 logits with error bounds and the finisher computes
//                  exact logits of the candidates only. Per token, the last
//                  work-group takes the exact top-k and the softmax over the k
//                  selected; the last token's work-group sorts the assignments by
//                  expert (counts, offsets, stable order, each slot's token and
//                  weight) and writes the work lists. Also y = 0.
//   expert_kernel  persistent, one launch per token-tile size: gate and up of
//                  (expert, 32-row tile, token group) items (bit-plane unpack +
//                  LUT dequant into MFMA A fragments, MFMA 16x16x32 fp16 with
//                  fp32 accumulation, SwiGLU -> act fp16), then down of (expert,
//                  64-row tile, K-piece, token group) items scaled by the
//                  routing weight and atomically added into y; a down item waits
//                  on a counter until its expert's act rows are complete.
//   expert_kernel_big  experts with many tokens: producer waves dequantise each
//                  weight once into LDS, consumer waves multiply it with up to 256
//                  tokens.
//   reduce_kernel  deterministic mode only: y from the down items' partial rows.
//   residual_kernel  x_next = fp16_rne(x + y) when requested.
//
// Dequantisation (the hot loop). Lane (r, kg) of a wave owns row r (0..15) of
// its 16-row half of the item and 128 columns (bytes 16*kg of a 64-byte
// half-line) of each plane line. For one 32-column dword of each of the b
// planes, a three-stage bit-matrix transpose (8x8 per byte) turns the plane
// words into eight index words W_i whose byte k is the b-bit index of column
// 8k+i. One v_perm per weight drops that byte into an LDS address, and one
// 16-bit LDS read fetches the fp16 weight from the LUT stripe (dword idx*64 +
// slot holds the two row-sets' entries of one row, low/high half; two copies
// so each half-wave hits 32 distinct banks). Eight looked-up weights form one
// MFMA A operand: step m of a 32-column group takes columns 8m..8m+7, so the B
// operand is the activation row as stored.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdlib>
#include <mutex>

#include "pw.h"
#include "pw_internal.h"

namespace pw {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const _Float16 lds_half;
typedef __attribute__((address_space(3))) unsigned char lds_byte;

// LDS byte address of the dynamic shared segment. The gemm and debug kernels
// declare no static LDS, so it is 0; the lookups only need it 64 KiB-aligned
// (its low 16 bits are replaced by the index and lane slot).
__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
    return (uint32_t)(size_t)(lds_byte*)p;
}

__device__ __forceinline__ float h2f(uint16_t u) {
    return (float)__builtin_bit_cast(_Float16, u);
}
__device__ __forceinline__ uint16_t f2h(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);   // round to nearest even
}

// Raw buffer loads: an offset at or past num_records reads 0 without touching
// memory. Every plane / activation load of the hot loop is issued
// unconditionally this way (absent planes get num_records 0, lanes past K an
// out-of-range offset), so the compiler can count outstanding loads exactly and
// wait only for the chunk it is about to use.
constexpr uint32_t kOOB = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
    // base and size are wave-uniform: keep the descriptor in scalar registers
    const uint64_t b = (uint64_t)(size_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const int n = __builtin_amdgcn_readfirstlane((int)nbytes);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(size_t)(((uint64_t)hi << 32) | lo), (short)0, n, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Loads of wave-uniform addresses from data the kernel does not write (page
// table, routing counts and offsets of an earlier kernel) go through the
// constant address space, so they are scalar loads served by the scalar cache.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* kconst(const T* p) {
    return (const __attribute__((address_space(4))) T*)(size_t)p;
}

// ============================================================================ route

// Waits until every vector-memory operation this wave issued has completed
// (s_waitcnt vmcnt(0); gfx9 encoding, other counters left at their maximum).
__device__ __forceinline__ void vm_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }


// Exact product of two fp16 values in units of 2^-48, added to acc. A finite
// fp16 magnitude is mant * 2^(sh - 24) with mant < 2^11 and sh = max(e, 1) - 1
// (e the biased exponent field; mant carries the implicit bit when e > 0), so
// |x w| * 2^48 = (mant_x * mant_w) << (sh_x + sh_w): a 22-bit integer product
// shifted left, exact whenever |x w| < 2^15. sab accumulates |x w| in fp32 for
// the range check; inf / nan operands set bad.
__device__ __forceinline__ void add_pair(uint32_t xw, uint32_t ww, long long& acc, float& sab,
                                         int& bad) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t hx = (xw >> (16 * h)) & 0xFFFFu, hw = (ww >> (16 * h)) & 0xFFFFu;
        const uint32_t ex = (hx >> 10) & 31u, ew = (hw >> 10) & 31u;
        bad |= (ex == 31u) | (ew == 31u);
        const uint32_t mx = (hx & 1023u) | (ex ? 1024u : 0u);
        const uint32_t mw = (hw & 1023u) | (ew ? 1024u : 0u);
        const uint32_t sh = (ex ? ex - 1u : 0u) + (ew ? ew - 1u : 0u);   // 0..60
        const long long prod = (long long)((unsigned long long)(mx * mw) << sh);
        acc += ((hx ^ hw) & 0x8000u) ? -prod : prod;
        sab = fmaf(fabsf(h2f((uint16_t)hx)), fabsf(h2f((uint16_t)hw)), sab);
    }
}

// Key order of the top-k: larger value first, ties to the lower expert index.
template <typename V>
__device__ __forceinline__ bool key_gt(V va, int ea, V vb, int eb) {
    return va > vb || (va == vb && ea < eb);
}

// Exclusive scan over the kRouteThreads threads; *total gets the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* s_tmp, int* total) {
    constexpr int NW = kRouteThreads / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int inc = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(inc, off);
        if (lane >= off) inc += o;
    }
    if (lane == 63) s_tmp[wave] = inc;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int c = s_tmp[w];
        before += w < wave ? c : 0;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return inc - v + before;
}

// Exclusive scans of N values per thread at once (one pair of barriers for all);
// s_tmp holds N * (kRouteThreads / 64) ints.
template <int N>
__device__ __forceinline__ void block_excl_scan_n(const int (&v)[N], int* s_tmp, int (&ex)[N], int (&total)[N]) {
    constexpr int NW = kRouteThreads / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int inc[N];
#pragma unroll
    for (int l = 0; l < N; ++l) inc[l] = v[l];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
        for (int l = 0; l < N; ++l) {
            const int o = __shfl_up(inc[l], off);
            if (lane >= off) inc[l] += o;
        }
    }
    if (lane == 63) {
#pragma unroll
        for (int l = 0; l < N; ++l) s_tmp[l * NW + wave] = inc[l];
    }
    __syncthreads();
#pragma unroll
    for (int l = 0; l < N; ++l) {
        int before = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int c = s_tmp[l * NW + w];
            before += w < wave ? c : 0;
            tot += c;
        }
        ex[l] = inc[l] - v[l] + before;
        total[l] = tot;
    }
    __syncthreads();
}

template <typename T>
__device__ __forceinline__ T load_agent(const T* a) {
    return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void store_agent(T* a, T v) {
    __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Stable counting sort of the T*k assignments by expert (counts, exclusive
// offsets, assignments in ascending (t, j) order per expert, each slot's token
// and weight) and the per-expert item prefix of each expert-kernel work list.
// One work-group; ids and weights come from other work-groups of this launch.
__device__ void bucket_sort(const RouteParams& p, int* s_cnt, int* s_off, int* s_run, int* s_wc, int* s_tmp) {
    constexpr int NW = kRouteThreads / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = p.E, n = p.T * p.k;
    // ids and weights come from other work-groups through device-coherent loads, a
    // memory round trip each: every loop below issues kSortBatch chunks' loads at once
    // (when every assignment fits one batch, T*k <= kSortBatch*kRouteThreads, the
    // counting pass also loads the weights and the placement reuses both)
    constexpr int B = kSortBatch;
    const bool one_batch = n <= B * kRouteThreads;
    int ev[B];
    float wv[B];
    for (int e = tid; e < E; e += kRouteThreads) s_cnt[e] = 0;
    __syncthreads();
    for (int b0 = 0; b0 < n; b0 += B * kRouteThreads) {
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int i = b0 + u * kRouteThreads + tid;
            ev[u] = i < n ? load_agent(p.ws.ids + i) : -1;
            wv[u] = i < n && one_batch ? load_agent(p.ws.w + i) : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < B; ++u)
            if (ev[u] >= 0) atomicAdd(&s_cnt[ev[u]], 1);
    }
    __syncthreads();
    // exclusive offsets over experts (E <= kRouteThreads)
    {
        int tot;
        const int v = tid < E ? s_cnt[tid] : 0;
        const int ex = block_excl_scan(v, s_tmp, &tot);
        if (tid < E) {
            s_off[tid] = ex;
            s_run[tid] = ex;
            p.ws.counts[tid] = v;
            p.ws.offsets[tid] = ex;
            if (p.o_counts) p.o_counts[tid] = v;
            if (p.o_offsets) p.o_offsets[tid] = ex;
        }
        if (tid == 0) {
            s_off[E] = tot;
            p.ws.offsets[E] = tot;
            if (p.o_offsets) p.o_offsets[E] = tot;
        }
    }
    __syncthreads();
    // stable placement, kRouteThreads assignments at a time: lanes of one wave
    // with the same expert find each other by matching the 8 id bits
    for (int base = 0; base < n; base += kRouteThreads) {
        const int u = (base / kRouteThreads) % B;   // this chunk's entry of the batch
        if (u == 0 && !one_batch) {
#pragma unroll
            for (int v = 0; v < B; ++v) {
                const int i = base + v * kRouteThreads + tid;
                ev[v] = i < n ? load_agent(p.ws.ids + i) : 0;
                wv[v] = i < n ? load_agent(p.ws.w + i) : 0.0f;
            }
        }
        for (int j = tid; j < NW * E; j += kRouteThreads) s_wc[j] = 0;
        __syncthreads();
        const int i = base + tid;
        const bool valid = i < n;
        int e = 0;
        float wi = 0.0f;
#pragma unroll
        for (int v = 0; v < B; ++v)
            if (v == u) {
                e = ev[v];
                wi = wv[v];
            }
        unsigned long long same = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const unsigned long long bb = __ballot(valid && ((e >> bit) & 1));
            same &= ((e >> bit) & 1) ? bb : ~bb;
        }
        const int rank = __popcll(same & __lanemask_lt());
        if (valid && rank == 0) s_wc[wave * E + e] = __popcll(same);
        __syncthreads();
        for (int ee = tid; ee < E; ee += kRouteThreads) {
            int run = s_run[ee];
            for (int w = 0; w < NW; ++w) {
                const int c = s_wc[w * E + ee];
                s_wc[w * E + ee] = run;
                run += c;
            }
            s_run[ee] = run;
        }
        __syncthreads();
        if (valid) {
            const int pos = s_wc[wave * E + e] + rank;
            p.ws.sorted[pos] = i;
            p.ws.slot_of[i] = pos;
            p.ws.slot_tok[pos] = i / p.k;   // token of the slot, and its routing weight
            p.ws.slot_w[pos] = wi;
            if (p.o_sorted) p.o_sorted[pos] = i;
        }
        __syncthreads();
    }

    // ---- work lists: list position 0 is the shared expert (long items first);
    // E + 1 positions can exceed the thread count, so they are scanned in chunks
    const int npos = E + p.has_shared;
    const int stride = E + 2;
    int carry[N_LISTS] = {0, 0, 0, 0, 0, 0};
    for (int p0 = 0; p0 < npos; p0 += kRouteThreads) {
        const int pos = p0 + tid;
        int cnt = 0, tgu = 0, pdn = 1;
        if (pos < npos) {
            const bool sh = p.has_shared && pos == 0;
            const int ex = sh ? E : pos - p.has_shared;
            cnt = sh ? p.T : s_cnt[ex];
            tgu = sh ? p.tiles_gu_s : p.tiles_gu_r;
            pdn = sh ? p.pieces_dn_s : p.pieces_dn_r;
        }
        // up to small_max tokens: groups of small_tokens (16 or 32) in the one- or
        // two-tile kernel (two work-groups per CU: two such items cost less CU time
        // than one item of a large kernel at one work-group per CU); up to
        // four_max: 64-token groups in the four-tile kernel; beyond: 128-token
        // groups in the dequantise-once kernel
        const int small = (cnt >= 1 && cnt <= p.small_max) ? (cnt + p.small_tokens - 1) / p.small_tokens : 0;
        const int four = (cnt > p.small_max && cnt <= p.four_max) ? (cnt + kLargeTokens - 1) / kLargeTokens : 0;
        const int big = cnt > p.four_max ? (cnt + kBigTokens - 1) / kBigTokens : 0;
        const int tdn = p.tiles_dn * pdn;
        const int nitems[N_LISTS] = {small * tgu, four * tgu, big * tgu, small * tdn, four * tdn, big * tdn};
        int ex[N_LISTS], tot[N_LISTS];
        block_excl_scan_n<N_LISTS>(nitems, s_tmp, ex, tot);
#pragma unroll
        for (int l = 0; l < N_LISTS; ++l) {
            if (pos < npos) p.ws.prefix[l * stride + pos] = carry[l] + ex[l];
            carry[l] += tot[l];
        }
    }
    if (tid == 0) {
#pragma unroll
        for (int l = 0; l < N_LISTS; ++l) p.ws.prefix[l * stride + npos] = carry[l];
    }
}

// Exact router logits of the experts ex[0], ex[1] (-1: none) for token t, one
// wave (lane l takes columns l*8 + 512*i, four 512-column blocks per batch, all
// loads of a batch issued first): int64 sums in units of 2^-48, with sum |x w|
// and the out-of-range flag of each.
__device__ __forceinline__ void exact_logits(const RouteParams& p, int t, const int (&ex)[2], int lane,
                                             long long (&acc)[2], float (&sab)[2], int (&bad)[2]) {
    const int d = p.d;
    const uint16_t* xr = p.x + (size_t)t * d;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        acc[j] = 0;
        sab[j] = 0.0f;
        bad[j] = 0;
    }
    for (int c0 = 0; c0 < d; c0 += 2048) {
        uint4 xv[4], wv[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = c0 + lane * 8 + 512 * i;
            const bool ok = c < d;
            xv[i] = ok ? *(const uint4*)(xr + c) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const bool okj = ok && ex[j] >= 0;
                wv[j][i] = okj ? *(const uint4*)(p.wr + (size_t)ex[j] * d + c) : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                add_pair(xv[i].x, wv[j][i].x, acc[j], sab[j], bad[j]);
                add_pair(xv[i].y, wv[j][i].y, acc[j], sab[j], bad[j]);
                add_pair(xv[i].z, wv[j][i].z, acc[j], sab[j], bad[j]);
                add_pair(xv[i].w, wv[j][i].w, acc[j], sab[j], bad[j]);
            }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            acc[j] += __shfl_xor(acc[j], off);
            sab[j] += __shfl_xor(sab[j], off);
            bad[j] |= __shfl_xor(bad[j], off);
        }
    }
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// fp32 logits of kRouteFilterPerWave experts e0, e0 + 1, ... for token t, one wave
// (same column split as exact_logits): l = sum x w and s = sum |x w|, both with
// v_dot2_f32_f16 (each product of two fp16 values is exact in fp32; only the
// additions round). The bias is added by the caller.
__device__ __forceinline__ void filter_logits(const RouteParams& p, int t, int e0, int lane,
                                              float (&l)[kRouteFilterPerWave], float (&sa)[kRouteFilterPerWave]) {
    constexpr int EF = kRouteFilterPerWave;
    const int d = p.d;
    const uint16_t* xr = p.x + (size_t)t * d;
#pragma unroll
    for (int j = 0; j < EF; ++j) l[j] = sa[j] = 0.0f;
    for (int c0 = 0; c0 < d; c0 += 2048) {
        uint4 xv[4], wv[EF][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = c0 + lane * 8 + 512 * i;
            const bool ok = c < d;
            xv[i] = ok ? *(const uint4*)(xr + c) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < EF; ++j) {
                const bool okj = ok && e0 + j < p.E;
                wv[j][i] = okj ? *(const uint4*)(p.wr + (size_t)(e0 + j) * d + c) : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int j = 0; j < EF; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t xw[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
                const uint32_t ww[4] = {wv[j][i].x, wv[j][i].y, wv[j][i].z, wv[j][i].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    l[j] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, xw[q]), __builtin_bit_cast(half2v, ww[q]),
                                                  l[j], false);
                    sa[j] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, xw[q] & 0x7FFF7FFFu),
                                                   __builtin_bit_cast(half2v, ww[q] & 0x7FFF7FFFu), sa[j], false);
                }
            }
    }
#pragma unroll
    for (int j = 0; j < EF; ++j) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            l[j] += __shfl_xor(l[j], off);
            sa[j] += __shfl_xor(sa[j], off);
        }
    }
}

// Routing and bucket sort in one launch of T * ceil(E / (4 * kRouteFilterPerWave))
// work-groups of 4 waves. The selection is exact (ties to the lower expert
// index) without computing every logit exactly:
//   1. work-group (t, eb) computes fp32 logits l_e (with the bias) and the sums
//      s_e = sum |x w| + |bias| of its experts for token t. Every product is
//      exact and at most d/32 + 32 rounded additions lie on the path of any
//      term, so |l_e - L_e| <= err_e = (d/32 + 32) 2^-24 s_e (L_e the exact
//      logit), inflated here by a margin for the rounding of s_e and of l_e -/+
//      err_e themselves;
//   2. the work-group that finishes token t last takes the k-th largest lower
//      bound l_e - err_e; an expert whose upper bound l_e + err_e lies below it
//      is beaten by k experts whatever the exact values, so only the others
//      (candidates, usually k or a few more) get exact int64 logits in units of
//      2^-48 (exponent-aligned integer mantissa products, add_pair), are ranked
//      by exact key, and the top k get the softmax over their exact logits;
//   3. the work-group that finishes the last token does the bucket sort and
//      the work lists.
// The sums are exact for finite fp16 inputs with sum |x w| + |bias| < 2^15
// (checked in fp32 with margin for every expert; outside it, or for non-finite
// inputs, a status flag is raised). Values passed between work-groups are
// device-coherent stores, drained before the counter increment that publishes
// them, and device-coherent loads.
// For small T * E (exact_all) the first pass computes every logit exactly instead
// (one expert per wave, spread over more work-groups), and every expert is a
// candidate of the finisher: the exact work is then parallel rather than on
// the finisher's path.
// Four waves per SIMD (at most 128 VGPRs, no spills): four work-groups per CU
// keep more first-pass and finisher work in flight at large T.
__global__ __launch_bounds__(kRouteThreads) __attribute__((amdgpu_waves_per_eu(4))) void route_kernel(RouteParams p) {
    constexpr int NW = kRouteThreads / 64, EF = kRouteFilterPerWave, EX = kRouteExactPerWave;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int d = p.d, E = p.E, k = p.k;
    const int per_wave = p.exact_all ? EX : EF;
    const int nb = (E + NW * per_wave - 1) / (NW * per_wave);
    const int t = blockIdx.x / nb, eb = blockIdx.x - t * nb;
    __shared__ float s_lo[PW_MAX_EXPERTS];
    __shared__ int s_cand[PW_MAX_EXPERTS + 8];   // candidate experts, + sentinels
    __shared__ long long s_ex[PW_MAX_EXPERTS + 8];   // exact logits (of the candidates), + sentinels
    __shared__ long long s_selv[PW_MAX_TOP_K];
    __shared__ int s_sele[PW_MAX_TOP_K];
    __shared__ int s_wcnt[NW];
    __shared__ float s_kth;
    __shared__ int s_last;
    // bucket sort (last work-group only)
    __shared__ int s_cnt[PW_MAX_EXPERTS];
    __shared__ int s_off[PW_MAX_EXPERTS + 1];
    __shared__ int s_run[PW_MAX_EXPERTS];
    __shared__ int s_wc[NW * PW_MAX_EXPERTS];
    __shared__ int s_tmp[N_LISTS * NW];

    // ---- 1. fp32 logits and bounds of this work-group's experts; y = 0 for the token
    if (eb == 0) {
        for (int c = tid; c < d; c += kRouteThreads) p.y[(size_t)t * d + c] = 0.0f;
    }
    const int e0 = (eb * NW + wave) * per_wave;
    if (p.exact_all) {
        if (e0 < E) {
            const int ex[2] = {e0, EX > 1 && e0 + 1 < E ? e0 + 1 : -1};
            long long acc[2];
            float sab[2];
            int bad[2];
            exact_logits(p, t, ex, lane, acc, sab, bad);
            if (lane == 0) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    if (ex[j] < 0) continue;
                    if (p.bias) {
                        const float bf = h2f(p.bias[ex[j]]);
                        bad[j] |= !(fabsf(bf) < 32768.0f);
                        if (!bad[j]) acc[j] += (long long)((double)bf * 281474976710656.0);  // * 2^48, exact
                        sab[j] += fabsf(bf);
                    }
                    if (bad[j] || !(sab[j] < 32000.0f)) atomicOr(p.ws.status, PW_STATUS_ROUTER_RANGE);
                    store_agent(p.ws.lg + (size_t)t * E + ex[j], acc[j]);
                }
            }
        }
    } else if (e0 < E) {
        float l[EF], sa[EF];
        filter_logits(p, t, e0, lane, l, sa);
        if (lane == 0) {
#pragma unroll
            for (int j = 0; j < EF; ++j) {
                const int e = e0 + j;
                if (e >= E) break;
                if (p.bias) {
                    const float bf = h2f(p.bias[e]);
                    l[j] += bf;
                    sa[j] += fabsf(bf);
                }
                // outside the exact range (or non-finite): flagged, routing undefined
                if (!(sa[j] < 32000.0f) || !(fabsf(l[j]) < 32768.0f)) atomicOr(p.ws.status, PW_STATUS_ROUTER_RANGE);
                const uint64_t pk = (uint64_t)__float_as_uint(l[j]) | ((uint64_t)__float_as_uint(sa[j]) << 32);
                store_agent((unsigned long long*)(p.ws.lg + (size_t)t * E + e), (unsigned long long)pk);
            }
        }
    }
    vm_drain();
    __syncthreads();
    if (tid == 0) s_last = __hip_atomic_fetch_add(p.ws.tok_cnt + t, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(nb - 1);
    __syncthreads();
    if (!s_last) return;

    // ---- 2. token t: candidates by the fp32 bounds, then the exact top-k among them
    if (tid == 0) {
        store_agent(p.ws.tok_cnt + t, 0u);   // every work-group of the token has counted
        s_kth = -INFINITY;                    // replaced below unless the bounds are not finite
    }
    if (tid < k) {   // valid expert ids whatever happens below (non-finite inputs are flagged)
        s_sele[tid] = tid;
        s_selv[tid] = LLONG_MIN;
    }
    // Rank of value v (expert e) among the n exact logits s_ex[0..n) of experts
    // ids(c): the number ahead in key order; eight LDS reads in flight per step
    // (entries n..n+7 are sentinels below every logit).
    auto rank_of = [&](long long v, int e, int n, auto ids) {
        int rank = 0;
        for (int c0 = 0; c0 < n; c0 += 8) {
            long long w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] = s_ex[c0 + j];
#pragma unroll
            for (int j = 0; j < 8; ++j) rank += key_gt(w[j], ids(c0 + j), v, e) ? 1 : 0;
        }
        return rank;
    };
    if (p.exact_all) {
        // every logit already exact: rank all E experts
        for (int i = tid; i < E; i += kRouteThreads) s_ex[i] = load_agent(p.ws.lg + (size_t)t * E + i);
        if (tid < 8) s_ex[E + tid] = LLONG_MIN;   // below every logit (|logit| < 2^63 by the range check)
        __syncthreads();
        if (tid < E) {
            const long long v = s_ex[tid];
            const int rank = rank_of(v, tid, E, [](int c) { return c; });
            if (rank < k) {
                s_selv[rank] = v;
                s_sele[rank] = tid;
            }
        }
    } else {
        const float g = (float)(d / 32 + 32) * 5.9604645e-8f * 1.01f;   // (d/32 + 32) * 2^-24, with margin
        float lo = 0.0f, hi = 0.0f;
        if (tid < E) {
            const unsigned long long pk = load_agent((const unsigned long long*)(p.ws.lg + (size_t)t * E + tid));
            const float l = __uint_as_float((uint32_t)pk), sa = __uint_as_float((uint32_t)(pk >> 32));
            // the bound, widened so that the rounding of l -/+ err keeps it a bound
            const float err = (g * sa + fabsf(l) * 2.4e-7f) * 1.0001f;
            lo = l - err;
            hi = l + err;
            s_lo[tid] = lo;
        }
        __syncthreads();
        if (tid < E) {
            int rank = 0;   // experts ahead of tid by lower bound (ties to the lower index)
#pragma unroll 8
            for (int e = 0; e < E; ++e) {
                const float v = s_lo[e];
                rank += (v > lo || (v == lo && e < tid)) ? 1 : 0;
            }
            if (rank == k - 1) s_kth = lo;
        }
        __syncthreads();
        // candidates in increasing expert order (a non-finite bound makes every expert a candidate)
        const bool cand = tid < E && !(hi < s_kth);
        const unsigned long long bal = __ballot(cand);
        if (lane == 0) s_wcnt[wave] = __popcll(bal);
        __syncthreads();
        int before = 0, C = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            before += w < wave ? s_wcnt[w] : 0;
            C += s_wcnt[w];
        }
        if (cand) s_cand[before + __popcll(bal & __lanemask_lt())] = tid;
        if (tid < 8) {   // sentinels of the candidate ranking
            s_ex[C + tid] = LLONG_MIN;
            s_cand[C + tid] = PW_MAX_EXPERTS;
        }
        __syncthreads();
        // exact logits of the candidates, one per wave and round (two per wave
        // would hold both rows' loads and sums live: 231 VGPRs instead of 106)
        for (int c0 = 0; c0 < C; c0 += NW) {
            const int ca = c0 + wave;
            const int ex[2] = {ca < C ? s_cand[ca] : -1, -1};
            long long acc[2];
            float sab[2];
            int bad[2];
            exact_logits(p, t, ex, lane, acc, sab, bad);
            if (lane == 0) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    if (ex[j] < 0) continue;
                    if (p.bias) {
                        const float bf = h2f(p.bias[ex[j]]);
                        bad[j] |= !(fabsf(bf) < 32768.0f);
                        if (!bad[j]) acc[j] += (long long)((double)bf * 281474976710656.0);  // * 2^48, exact
                        sab[j] += fabsf(bf);
                    }
                    if (bad[j] || !(sab[j] < 32000.0f)) atomicOr(p.ws.status, PW_STATUS_ROUTER_RANGE);
                    s_ex[ca + j] = acc[j];
                }
            }
        }
        __syncthreads();
        if (tid < C) {
            const long long v = s_ex[tid];
            const int e = s_cand[tid];
            // candidates ahead in key order: larger exact logit, ties to the lower index
            const int rank = rank_of(v, e, C, [&](int c) { return s_cand[c]; });
            if (rank < k) {
                s_selv[rank] = v;
                s_sele[rank] = e;
            }
        }
    }
    __syncthreads();
    // softmax over the selected logits (descending order)
    if (tid == 0) {
        float l[PW_MAX_TOP_K], ex[PW_MAX_TOP_K];
        float s = 0.0f;
        for (int j = 0; j < k; ++j) l[j] = ldexpf((float)s_selv[j], -48);
        for (int j = 0; j < k; ++j) {
            ex[j] = expf(l[j] - l[0]);
            s += ex[j];
        }
        for (int j = 0; j < k; ++j) {
            const float wj = ex[j] / s;
            store_agent(p.ws.ids + (size_t)t * k + j, s_sele[j]);
            store_agent(p.ws.w + (size_t)t * k + j, wj);
            if (p.o_ids) p.o_ids[(size_t)t * k + j] = s_sele[j];
            if (p.o_w) p.o_w[(size_t)t * k + j] = wj;
        }
        vm_drain();
        s_last = __hip_atomic_fetch_add(p.ws.route_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 (uint32_t)(p.T - 1);
        if (s_last) store_agent(p.ws.route_done, 0u);   // every token has counted
    }
    __syncthreads();
    if (!s_last) return;

    // ---- 3. the last token: bucket sort and work lists for the expert kernel
    bucket_sort(p, s_cnt, s_off, s_run, s_wc, s_tmp);
}

// ============================================================================ dequant core

// Transposes the plane words of one 32-column group into index words.
// Slot s of `sl` holds plane s - (8 - b) (slots below 8 - b are zero), so slot
// s carries bit 7 - s of the b-bit index for every b: out[i] byte k = index of
// column 8k + i. An 8x8 bit transpose inside every byte: swap the
// off-diagonal 4x4, 2x2 and 1x1 blocks.
__device__ __forceinline__ void slots_to_indices(const uint32_t (&sl)[8], uint32_t (&rw)[8]) {
#pragma unroll
    for (int q = 0; q < 8; ++q) rw[q] = sl[7 - q];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t a = rw[q], b = rw[q + 4];
        rw[q] = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);
        rw[q + 4] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
    }
#pragma unroll
    for (int q0 = 0; q0 < 8; q0 += 4) {
#pragma unroll
        for (int q = q0; q < q0 + 2; ++q) {
            const uint32_t a = rw[q], b = rw[q + 2];
            rw[q] = (a & 0x33333333u) | ((b << 2) & 0xCCCCCCCCu);
            rw[q + 2] = ((a >> 2) & 0x33333333u) | (b & 0xCCCCCCCCu);
        }
    }
#pragma unroll
    for (int q = 0; q < 8; q += 2) {
        const uint32_t a = rw[q], b = rw[q + 1];
        rw[q] = (a & 0x55555555u) | ((b << 1) & 0xAAAAAAAAu);
        rw[q + 1] = ((a >> 1) & 0x55555555u) | (b & 0xAAAAAAAAu);
    }
}

// A fragment of MFMA step m from the index words of one 32-column group:
// half j = LUT[index of column 8m + j], so step m consumes eight consecutive
// columns and the B operand is the activation row as stored. Column 8m + j is
// byte m of index word j. `slot` is the lane's LDS address of stripe entry 0
// (segment base + row slot * 4); byte 1 of it is replaced by the index, i.e.
// entry idx sits idx*256 bytes further. hoff selects the row-set (0: low half,
// 2: high half of the stripe dword).
__device__ __forceinline__ half8 lut_fragment(const uint32_t (&rw)[8], int m, uint32_t slot, int hoff) {
    half8 a;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t addr = __builtin_amdgcn_perm(rw[j], slot, 0x03020400u | (uint32_t)(m << 8));
        a[j] = *(lds_half*)(size_t)(addr + hoff);
    }
    return a;
}

// The A fragments of step m of both row-sets (set 0: low halves of the stripe
// dwords, set 1: high halves), with all 16 lookups issued before the first value
// is packed: the scheduler otherwise waits on each batch of eight, exposing the
// LDS latency at two waves per SIMD.
__device__ __forceinline__ void lut_fragments2(const uint32_t (&rw0)[8], const uint32_t (&rw1)[8], int m,
                                               uint32_t slot, half8& a0, half8& a1) {
    uint32_t ad0[8], ad1[8];
    _Float16 v0[8], v1[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        ad0[j] = __builtin_amdgcn_perm(rw0[j], slot, 0x03020400u | (uint32_t)(m << 8));
        ad1[j] = __builtin_amdgcn_perm(rw1[j], slot, 0x03020400u | (uint32_t)(m << 8)) + 2u;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        v0[j] = *(lds_half*)(size_t)ad0[j];
        v1[j] = *(lds_half*)(size_t)ad1[j];
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);   // scheduling group: the 16 LDS reads,
    __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);   // then VALU
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a0[j] = v0[j];
        a1[j] = v1[j];
    }
}

// 8 LUT entries [c8, c8+8) of one row as four packed fp16 pairs (zeros past 2^b).
// A row of b < 3 is 4 or 8 bytes; it is read whole (c8 is 0 then).
__device__ __forceinline__ uint4 load_lut8(const uint16_t* row, int b, int c8) {
    if (b >= 3) return c8 < (1 << b) ? *(const uint4*)(row + c8) : make_uint4(0, 0, 0, 0);
    if (b == 2) {
        const uint2 v = *(const uint2*)row;
        return make_uint4(v.x, v.y, 0, 0);
    }
    return make_uint4(*(const uint32_t*)row, 0, 0, 0);
}

// Writes 8 consecutive stripe entries (idx = c8..c8+7) of one row slot:
// dword (idx*64 + row) = {set0 LUT[row][idx], set1 LUT[row][idx]}. One base
// address, the entries at fixed offsets of 256 bytes.
__device__ __forceinline__ void write_stripe8(uint32_t* stripe, int c8, int row, int nidx, uint4 a, uint4 b) {
    uint32_t* dst = stripe + c8 * 64 + row;
    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
    if (nidx >= 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dst[(2 * i) * 64] = (av[i] & 0xFFFFu) | (bv[i] << 16);
            dst[(2 * i + 1) * 64] = (av[i] >> 16) | (bv[i] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (2 * i < nidx) dst[(2 * i) * 64] = (av[i] & 0xFFFFu) | (bv[i] << 16);
            if (2 * i + 1 < nidx) dst[(2 * i + 1) * 64] = (av[i] >> 16) | (bv[i] & 0xFFFF0000u);
        }
    }
}

// The LUTs of an item's 32 rows of one row-set are 32 * 2^b contiguous fp16
// values in either page order: row-major (entry i of row r at r * 2^b + i) or,
// with PW_FLAG_LUT_TILED, the 32-row tiled order (entry group g = i / 8 of the
// 32 rows row after row: entry i of row r at (g * 32 + r) * 8 + i % 8). They are
// staged in 16-byte units of 8 entries: thread t takes row t & 31 and entry
// groups g = (t >> 5) + 8 * it, it = 0..3 (4 * 2^b units per set, at most 4 per
// thread at b = 8), so each half-wave covers rows 0..31 and the stripe writes
// hit 32 distinct banks. In the tiled order a wave's loads are contiguous; in
// the row-major order they are 16 bytes per row at a 2^b * 2-byte stride. For
// b < 3 a row is shorter than a unit and both orders are the same row-major
// array (unit u is bytes 16u .. 16u + 15 of it). The loads are issued early
// (lut_stage_load) and written to the stripe later (lut_stage_write).
struct LutStage {
    uint4 v[2][4];
};
__device__ __forceinline__ uint32_t lut_unit_offset(int u, int b, int tiled) {
    if (b < 3 || tiled) return (uint32_t)u * 8u;              // element offset of unit u
    return (uint32_t)(((u & 31) << (b - 3)) + (u >> 5)) * 8u;   // row (u & 31), group u >> 5
}
__device__ __forceinline__ void lut_stage_load(LutStage& st, const uint16_t* lut0, int b0,
                                               const uint16_t* lut1, int b1, int tid, int tiled) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int u = tid + it * 256;
        st.v[0][it] = u < (4 << b0) ? *(const uint4*)(lut0 + lut_unit_offset(u, b0, tiled)) : make_uint4(0, 0, 0, 0);
        st.v[1][it] = u < (4 << b1) ? *(const uint4*)(lut1 + lut_unit_offset(u, b1, tiled)) : make_uint4(0, 0, 0, 0);
    }
}

// The same loads as buffer loads whose instruction count never depends on b or on
// `valid` (units past 2^b, and every unit when !valid, read zeros without touching
// memory), so that a wait issued after them can be counted exactly.
__device__ __forceinline__ void lut_stage_load_buf(LutStage& st, const uint16_t* lut0, int b0,
                                                   const uint16_t* lut1, int b1, int tid, int tiled, bool valid) {
    const __amdgpu_buffer_rsrc_t r0 = make_rsrc(lut0, valid ? (64u << b0) : 0u);
    const __amdgpu_buffer_rsrc_t r1 = make_rsrc(lut1, valid ? (64u << b1) : 0u);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int u = tid + it * 256;
        st.v[0][it] = buf_load16(r0, u < (4 << b0) ? lut_unit_offset(u, b0, tiled) * 2u : kOOB);
        st.v[1][it] = buf_load16(r1, u < (4 << b1) ? lut_unit_offset(u, b1, tiled) * 2u : kOOB);
    }
}

// Debug-kernel stripe (dword idx*64 + row, both halves the same) from the LUTs
// of 32 rows (row-major, or 32-row tiled), one wave, plain loop.
__device__ __forceinline__ void stage_lut32(uint32_t* stripe, const uint16_t* tile, int b, int tiled, int lane) {
    const int nidx = 1 << b;
    for (int e = lane; e < 32 * nidx; e += 64) {
        int row, idx;
        if (b >= 3 && tiled) {
            row = (e >> 3) & 31;
            idx = ((e >> 8) << 3) | (e & 7);
        } else {
            row = e >> b;
            idx = e & (nidx - 1);
        }
        const uint32_t h = tile[e];
        stripe[idx * 64 + row] = h | (h << 16);
    }
}

__device__ __forceinline__ uint32_t word_of(const uint4& q, int dw) {
    return dw == 0 ? q.x : dw == 1 ? q.y : dw == 2 ? q.z : q.w;
}

// ============================================================================ gemm

// One work item of a list, decoded from its index.
struct Item {
    int mode;                 // 0 gate_up, 1 down
    int pos, piece;           // list position (0 = shared expert when present), K-piece
    int ex, tile, grp;        // expert (E = shared), row tile, token group
    int n_tok, tbase, nl;     // tokens of the expert, first token of the group, tokens here
    int K, R;                 // columns / rows of the block
    int kbase, klen;          // K range of this item
    int rows0, rows1;         // first row of set 0 / set 1 within its block's pages (within
                              // the linear: tile * 32 for gate_up, tile * 64 (+ 32) for down)
    const __attribute__((address_space(4))) DevBlock* blk0;   // page-table entries (scalar loads)
    const __attribute__((address_space(4))) DevBlock* blk1;
};

// Token rows of one item for thread tid (tid < nl): B row, output row, weight.
struct TokInfo {
    int brow, orow;
    float w;
};

template <int MODE>
__device__ __forceinline__ TokInfo fetch_tokinfo(const GemmParams& p, const Item& it, int tid) {
    TokInfo tk{0, 0, 0.0f};
    const bool sh = it.ex == p.E;
    const int base = sh ? 0 : kconst(p.ws.offsets)[it.ex];
    if (tid < it.nl) {
        const int tkn = it.tbase + tid;
        const int slot = sh ? (p.shared_base + tkn) : (base + tkn);
        const int tok = sh ? tkn : p.ws.slot_tok[slot];
        if (MODE == 0) {
            tk.brow = tok;    // x row
            tk.orow = slot;   // act row
        } else {
            tk.brow = slot;   // act row
            tk.orow = tok;    // y row
            tk.w = sh ? 1.0f : p.ws.slot_w[slot];
        }
    }
    return tk;
}

// fetch_tokinfo for either list with a fixed instruction count: the slot's token
// and weight are buffer loads (zeros for the shared expert, for threads past the
// group and when !valid), the list's mode picks the fields afterwards.
__device__ __forceinline__ TokInfo fetch_tokinfo_buf(const GemmParams& p, const Item& it, int tid, bool valid) {
    constexpr uint32_t kAny = 0x7FFFFFF0u;   // records: lanes that must not load use kOOB
    const bool sh = it.ex == p.E;
    const int base = kconst(p.ws.offsets)[it.ex];   // offsets has E + 1 entries
    const int tkn = it.tbase + tid;
    const bool in = valid && tid < it.nl;
    const int slot = sh ? (p.shared_base + tkn) : (base + tkn);
    const uint32_t off = (in && !sh) ? (uint32_t)slot * 4u : kOOB;
    const int tokv = __builtin_bit_cast(int, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(p.ws.slot_tok, kAny), (int)off, 0, 0));
    const float wv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(p.ws.slot_w, kAny), (int)off, 0, 0));
    const int tok = sh ? tkn : tokv;
    TokInfo tk;
    tk.brow = it.mode == 0 ? tok : slot;
    tk.orow = it.mode == 0 ? slot : tok;
    tk.w = it.mode == 0 ? 0.0f : (sh ? 1.0f : wv);
    return tk;
}

template <int MODE, int NT>
__device__ __forceinline__ Item decode_item(const GemmParams& p, const int* s_pre, int npos, int item) {
    int lo = 0, hi = npos - 1;   // last position with s_pre[pos] <= item
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pre[mid] <= item) lo = mid; else hi = mid - 1;
    }
    lo = __builtin_amdgcn_readfirstlane(lo);   // uniform: keep the item in scalar registers
    Item it;
    it.mode = MODE;
    it.pos = lo;
    const bool sh = p.has_shared && lo == 0;
    it.ex = sh ? p.E : lo - p.has_shared;
    const int tiles = sh ? p.tiles_s : p.tiles_r;
    const int pieces = sh ? p.pieces_s : p.pieces_r;
    const int local = __builtin_amdgcn_readfirstlane(item - s_pre[lo]);
    it.tile = local % tiles;
    const int piece = (local / tiles) % pieces;
    it.grp = local / tiles / pieces;
    it.piece = piece;
    it.n_tok = sh ? p.T : kconst(p.ws.counts)[it.ex];
    it.tbase = it.grp * 16 * NT;
    it.nl = min(16 * NT, it.n_tok - it.tbase);
    // Blocks are numbered expert by expert, then gate, up, down, then row-block:
    // with 2^rb_lg rows per block (rb_lg = 0: whole linears) expert ex owns
    // 2*f/rb + d/rb blocks (the shared expert, ex = E, follows the routed ones),
    // and the item's rows lie in row-block j of its linear, whose pages start at
    // row j*rb.
    const int f = sh ? p.Fs : p.F;
    const int lg = p.rb_lg;
    const int nF = lg ? f >> lg : 1;
    const int base = it.ex * (lg ? 2 * (p.F >> lg) + (p.d >> lg) : 3);
    const int arow = it.tile * (MODE == 0 ? 32 : 64);
    const int j = lg ? arow >> lg : 0;
    const int rel = arow - (j << lg);
    if (MODE == 0) {
        it.K = p.d;
        it.R = lg ? 1 << lg : f;
        it.rows0 = it.rows1 = rel;
        it.blk0 = kconst(p.blocks) + base + j;
        it.blk1 = kconst(p.blocks) + base + nF + j;
    } else {
        it.K = f;
        it.R = lg ? 1 << lg : p.d;
        it.rows0 = rel;
        it.rows1 = rel + 32;
        it.blk0 = it.blk1 = kconst(p.blocks) + base + 2 * nF + j;
    }
    it.kbase = piece * kDownPiece;
    it.klen = min(it.K - it.kbase, MODE == 0 ? it.K : kDownPiece);
    return it;
}

// LDS of the expert kernel: a 64 KiB LUT stripe whose 256-byte row idx holds, in
// dword 32*h + 16*c + r, the LUT entry idx of item row 16*h + r (low half: set
// 0, high half: set 1), in two copies c so that the 32 lanes of a half-wave
// (rows r, copies kg & 1) hit 32 distinct banks; then the cross-wave partial
// sums, the token rows of two items (double buffer), the work-list prefixes of
// the gate_up and down lists, and one flag.
constexpr int kStripeBytes = 65536;
constexpr int kTokWords = 3 * 64;   // brow, orow, weight bits of up to 64 tokens
constexpr int kPreWords = PW_MAX_EXPERTS + 2;   // work-list prefix of one list

__device__ __forceinline__ int stripe_slot(int row) {   // copy 0 of item row 0..31
    return ((row >> 4) << 5) + (row & 15);
}

// Writes the staged LUT units of both row-sets into the stripe: entry idx of
// item row `row` of set s is the 16-bit half s of dword idx*64 + slot (copy 0)
// and of dword idx*64 + slot + 16 (copy 1). When both sets have b >= 3, unit u
// holds the same (entry group, row) of both, and one dword write stores both
// halves (entries past the smaller set's 2^b are never read); each half-wave
// writes rows 0..31 and the copy order alternates with the row half, so every
// write instruction hits 32 distinct banks. Otherwise each set writes its own
// halves.
__device__ __forceinline__ void lut_stage_write(unsigned char* stripe, const LutStage& st, int b0, int b1, int tid) {
    if (b0 >= 3 && b1 >= 3) {
        const int bmax = b0 > b1 ? b0 : b1;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int u = tid + it * 256;
            if (u >= (4 << bmax)) continue;
            const int row = u & 31, h = (row >> 4) & 1;
            uint32_t* base = (uint32_t*)stripe + ((u >> 5) << 9) + stripe_slot(row);   // idx0 = 8 * (u >> 5)
            const uint32_t a[4] = {st.v[0][it].x, st.v[0][it].y, st.v[0][it].z, st.v[0][it].w};
            const uint32_t c[4] = {st.v[1][it].x, st.v[1][it].y, st.v[1][it].z, st.v[1][it].w};
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t lo = k & 1 ? (a[k >> 1] >> 16) : (a[k >> 1] & 0xFFFFu);
                const uint32_t hi = k & 1 ? (c[k >> 1] & 0xFFFF0000u) : (c[k >> 1] << 16);
                base[k * 64 + 16 * h] = lo | hi;
                base[k * 64 + 16 * (1 - h)] = lo | hi;
            }
        }
        return;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int b = s ? b1 : b0;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int u = tid + it * 256;
            if (u >= (4 << b)) continue;
            const uint4 v = st.v[s][it];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                int row, idx;
                if (b >= 3) {
                    row = u & 31;
                    idx = ((u >> 5) << 3) + k;
                } else {
                    row = (8 * u + k) >> b;
                    idx = (8 * u + k) & ((1 << b) - 1);
                }
                const uint16_t hv = (uint16_t)(w[k >> 1] >> (16 * (k & 1)));
                unsigned char* at = stripe + (idx * 64 + stripe_slot(row)) * 4 + 2 * s;
                *(uint16_t*)at = hv;
                *(uint16_t*)(at + 64) = hv;
            }
        }
    }
}

// Persistent work-group of 4 waves over one gate_up list followed by the down
// list of the same token-tile size, in one launch. An item is 32 rows of each of
// two row-sets over the item's K range, read as 128-byte lines
// (1024 columns of a plane row): wave q owns rows 16*(q >> 1) .. +15 of the
// item and half-line q & 1 of every line, and lane (r, kg) of it loads 16
// bytes (128 columns) of row r. A load instruction so covers 16 rows x 64
// contiguous bytes, and the two waves of a row half read the two halves of each
// line together. MFMA 16x16x32: A = 16 weight rows x 32 columns, B = 32 columns
// x 16 tokens. The two half-line partial sums meet in LDS; wave (h, 0)
// finishes accumulator registers 0, 1 (rows 4*rg + 0, 1) and wave (h, 1)
// registers 2, 3. Items are assigned round-robin, so the next item's metadata
// is known while the current one runs: its first chunk and LUT rows load
// during the current item's last chunk.
//
// Gate_up items come first in the combined order (index i < n_gu), down items
// after them. A down item reads the act rows of its expert's K-piece, so it
// waits until every gate_up item of that (list position, piece) has counted
// itself done. There is no fence on either side; the hand-off rests on these
// invariants:
//   - act is written only with device-coherent (agent-scope, sc1) stores, which
//     write through to memory; each producer wave drains them (vmcnt 0) before
//     the work-group barrier after which thread 0 increments the counter;
//   - the consumer (one wave polls, a barrier releases the others) reads the
//     counter with device-coherent loads and issues no load of act (nor of any
//     line holding act) before its wait ends, so no
//     cache level can hold a stale copy of a piece's act lines: they were last
//     touched by the previous launch, and a kernel boundary writes back and
//     invalidates the non-coherent caches;
//   - K-pieces (kDownPiece columns) and act rows start on 128-byte lines, so a
//     line never mixes act of two pieces.
// A change that loads B rows of a down item before its wait (say, in the
// next-item prefetch) breaks the second invariant. Every dependency points to an
// earlier index of the combined order and each work-group runs its items in
// increasing order, so with all work-groups resident (the launch sizes the grid
// to the occupancy) the earliest unfinished item never waits: no deadlock. The
// last work-group to finish zeroes the counters for the next launch.
// NT: token tiles of 16 per item. NT = 1 and 2 run two work-groups per CU,
// NT = 4 one. NT = 2 keeps a single plane buffer (the registers of the second
// one hold its second token tile's accumulators and B fragments): the next
// chunk's planes load right after the current chunk's last transposes, and
// the lookups and MFMAs of its last 32 columns cover their latency.
// DET: deterministic accumulation (down items write their own partial rows).
template <int NT, bool DET>
__global__ __launch_bounds__(256, NT <= 2 ? 2 : 1) void expert_kernel(ExpertParams p) {
    constexpr bool SB = NT == 2;   // single plane buffer
    extern __shared__ __align__(16) unsigned char smem[];
    // tid, r, kg are re-declared opaque at every item (below) so that the
    // compiler recomputes values derived from them instead of keeping dozens of
    // them live across the persistent loop
    int tid = threadIdx.x;
    const int q = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index: uniform
    const int rh = q >> 1, kh = q & 1;
    int r = tid & 15, kg = (tid >> 4) & 3;
    float* red = (float*)(smem + kStripeBytes);                  // [4 waves][NT][4][64]
    int* s_tok = (int*)(red + 4 * NT * 4 * 64);                  // [2][kTokWords]
    int* s_pre = s_tok + 2 * kTokWords;                          // [2][kPreWords]: gate_up, down
    int* s_flag = s_pre + 2 * kPreWords;
    const GemmParams& g = p.gu;                                  // fields common to both lists
    uint32_t* const dep = g.ws.dep;
    const int dstride = g.ws.dep_stride;
    const int npos = g.E + g.has_shared;
    // A work-group without an item leaves at once and takes no part in the
    // finished-work-group count (a launch whose lists are empty costs little).
    const int n_all = g.ws.prefix[p.gu.list * (g.E + 2) + npos] + g.ws.prefix[p.dn.list * (g.E + 2) + npos];
    if ((int)blockIdx.x >= n_all) return;
    const uint32_t n_working = (uint32_t)min((int)gridDim.x, n_all);
    // Work-group w takes items w, w + G, w + 2G, ... of the combined order (G =
    // grid size): no shared counter, and the next item is always known.
    for (int i = tid; i <= npos; i += 256) {
        s_pre[i] = g.ws.prefix[p.gu.list * (g.E + 2) + i];
        s_pre[kPreWords + i] = g.ws.prefix[p.dn.list * (g.E + 2) + i];
    }
    __syncthreads();
    const int n_gu = __builtin_amdgcn_readfirstlane(s_pre[npos]);
    const int n_items = n_gu + __builtin_amdgcn_readfirstlane(s_pre[kPreWords + npos]);
    int item = blockIdx.x;
    auto decode = [&](int i) -> Item {
        return i < n_gu ? decode_item<0, NT>(p.gu, s_pre, npos, i)
                        : decode_item<1, NT>(p.dn, s_pre + kPreWords, npos, i - n_gu);
    };
    auto tokinfo = [&](const Item& it) -> TokInfo {
        return it.mode == 0 ? fetch_tokinfo<0>(p.gu, it, tid) : fetch_tokinfo<1>(p.dn, it, tid);
    };

    if (item < n_items) {

        uint4 pa0[8], pa1[8], pb0[8], pb1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pa0[i] = pa1[i] = pb0[i] = pb1[i] = make_uint4(0, 0, 0, 0);

        // first column of this lane's 128 columns in chunk ch (relative to the item's K range)
        auto lane_col = [&](int ch) { return ch * 1024 + kh * 512 + kg * 128; };
        // plane loads of chunk ch (line ch of the item's K range) into (c0, c1):
        // slot i holds plane i - (8 - b); absent planes and columns past the range read zeros.
        // Group grp (0..3) is slots 7 - 2 grp and 6 - 2 grp of both sets (the present planes
        // of a small b come first); grp < 0 loads all of them.
        auto load_chunk = [&](const Item& it, int ch, uint4 (&c0)[8], uint4 (&c1)[8], int grp = -1,
                              bool valid = true) {
            const int Kb = it.K >> 3;
            const bool vg = valid && lane_col(ch) < it.klen;
            const uint32_t nrec = (uint32_t)(it.R * Kb);
            const int cb = (it.kbase + lane_col(ch)) >> 3;
            const int row = rh * 16 + r;
            const uint32_t off0 = vg ? (uint32_t)((it.rows0 + row) * Kb + cb) : kOOB;
            const uint32_t off1 = vg ? (uint32_t)((it.rows1 + row) * Kb + cb) : kOOB;
            // the page-table entries are re-read (scalar cache) at every group rather
            // than kept: descriptors of two items' 16 planes do not fit the scalar
            // registers and would be spilled to vector-register lanes
            auto bk0 = it.blk0, bk1 = it.blk1;
            asm volatile("" : "+s"(bk0), "+s"(bk1));
            const int s0 = 8 - bk0->bits, s1 = 8 - bk1->bits;
#pragma unroll
            for (int i = 7; i >= 0; --i) {
                if (grp >= 0 && (7 - i) / 2 != grp) continue;
                c0[i] = buf_load16(make_rsrc((const void*)bk0->planes[i], i >= s0 ? nrec : 0u), off0);
                c1[i] = buf_load16(make_rsrc((const void*)bk1->planes[i], i >= s1 ? nrec : 0u), off1);
            }
        };
        auto n_chunks = [](const Item& it) { return (it.klen + 1023) >> 10; };
        auto lut_load = [&](const Item& it, LutStage& st) {
            const int b0 = it.blk0->bits, b1 = it.blk1->bits;
            lut_stage_load(st, (const uint16_t*)it.blk0->lut + ((size_t)it.rows0 << b0), b0,
                           (const uint16_t*)it.blk1->lut + ((size_t)it.rows1 << b1), b1, tid, g.lut_tiled);
        };
        auto publish_item = [&](const Item& it, const LutStage& st, const TokInfo& tk, int par) {
            if (tid < it.nl) {
                int* tb = s_tok + par * kTokWords;
                tb[tid] = tk.brow;
                tb[64 + tid] = tk.orow;
                tb[128 + tid] = __float_as_int(tk.w);
            }
            lut_stage_write(smem, st, it.blk0->bits, it.blk1->bits, tid);
        };

        Item it = decode(item);
        {
            LutStage st;
            const TokInfo tk = tokinfo(it);
            load_chunk(it, 0, pa0, pa1);
            lut_load(it, st);
            publish_item(it, st, tk, 0);
        }
        __syncthreads();
        int par = 0;
        // The two work-groups sharing a CU (w and w + G/2 in dispatch order)
        // compete for its SIMDs, and at equal priority the older waves win: the
        // later work-group runs its items ~25 % slower. When their item counts
        // are within that ratio, their wave priorities swap every item so that
        // both progress at the same rate; when one has at least 5/4 of the
        // other's items (say 4 against 3), it keeps the higher priority.
        const int half = (int)gridDim.x / 2;
        const int slot = (int)blockIdx.x >= half ? 1 : 0;
        const int partner = slot ? (int)blockIdx.x - half : (int)blockIdx.x + half;
        auto items_of = [&](int w) { return w < (int)gridDim.x && w < n_items ? (n_items - 1 - w) / (int)gridDim.x + 1 : 0; };
        const int mine = items_of((int)blockIdx.x), theirs = items_of(partner);
        const int prio_mode = 4 * mine >= 5 * theirs ? 1 : 4 * theirs >= 5 * mine ? 2 : 0;   // 1 high, 2 low, 0 swap
        int round = 0;

        while (true) {
            asm volatile("" : "+v"(tid), "+v"(r), "+v"(kg));
            const bool high = prio_mode == 0 ? ((round++ ^ slot) & 1) != 0 : prio_mode == 1;
            if (high) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
            const int nch = n_chunks(it);
            const int ntl = (it.nl + 15) >> 4;
            const int* tb = s_tok + par * kTokWords;
            // B operand: x rows (gate_up) or act rows (down)
            const int ldb = it.mode == 0 ? g.d : g.ld_act;
            const __amdgpu_buffer_rsrc_t brsrc =
                it.mode == 0 ? make_rsrc(g.x, p.gu.b_bytes) : make_rsrc(g.ws.act, p.dn.b_bytes);
            if (it.mode == 1) {
                // every gate_up item of this expert's K-piece has released its act rows:
                // wave 0 polls the counter (one poller per work-group keeps the polls off
                // the memory system) and the barrier releases the others; no wave loads
                // act before it
                if (q == 0) {
                    const uint32_t need = (uint32_t)((it.klen >> 5) * ((it.n_tok + 16 * NT - 1) / (16 * NT)));
                    const uint32_t* c = dep + it.pos * dstride + it.piece;
                    uint32_t polls = 0;
                    while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
                        if (polls++ >= kconst(g.ws.wait_limit)[0]) {   // bounded: a missing producer becomes a flag
                            if (tid == 0) atomicOr(g.ws.status, PW_STATUS_DEP_TIMEOUT);
                            break;
                        }
                        __builtin_amdgcn_s_sleep(2);
                    }
                }
                __syncthreads();
            }
            // the next item: its metadata and token rows now
            const int next = item + (int)gridDim.x;
            const bool has_next = next < n_items;
            Item nit = it;
            TokInfo ntk{0, 0, 0.0f};
            if (has_next) nit = decode(next);

            uint32_t boff[NT];
            bool bok[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int i = nt * 16 + r;
                bok[nt] = i < it.nl;
                boff[nt] = bok[nt] ? (uint32_t)(tb[i] * ldb + kh * 512 + kg * 128) : 0u;
            }
            floatx4 acc0[NT], acc1[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                acc0[nt] = (floatx4)0.0f;
                acc1[nt] = (floatx4)0.0f;
            }

            auto load_b = [&](int ch, int dw, half8 (&bf)[NT][4], bool vg) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const uint32_t off =
                        (bok[nt] && vg) ? (boff[nt] + (uint32_t)(it.kbase + ch * 1024 + 32 * dw)) * 2u : kOOB;
#pragma unroll
                    for (int m = 0; m < 4; ++m) bf[nt][m] = __builtin_bit_cast(half8, buf_load16(brsrc, off + 16u * m));
                }
            };

            const uint32_t slot = lds_addr(smem) + (uint32_t)((rh * 32 + (kg & 1) * 16 + r) * 4);
            // One chunk: for each of the lane's four 32-column dwords, transpose the
            // plane words of both sets, look the weights up and feed the MFMAs. The B
            // fragments of a dword (L2-resident activations) load at its start and
            // arrive while the transposes and lookups run. Lanes past K hold zero B
            // fragments, so their A fragments need no masking. A wave whose half of
            // the chunk lies wholly past K skips it.
            // bfr: B fragments of the current dword. Those of dword 0 of a chunk are
            // loaded before the plane prefetch issued at the chunk boundary: loads
            // complete in issue order, so a fragment loaded after a prefetch is
            // waited on only together with it.
            half8 bfr[NT][4];
            // pf(dw) issues group dw of the prefetch into the other plane buffer right
            // after dword dw's B fragments: a wait for those fragments then covers only
            // the groups issued a dword or more before, not the whole next chunk.
            // With a single plane buffer (SB), pf(dw) is called after dword dw's
            // transposes, when the buffer's words have been read.
            auto compute_chunk = [&](int ch, const uint4 (&c0)[8], const uint4 (&c1)[8], auto pf) {
                const bool active = ch * 1024 + kh * 512 < it.klen;   // wave-uniform
                const bool vg = lane_col(ch) < it.klen;
#pragma unroll
                for (int dw = 0; dw < 4; ++dw) {
                    if (dw > 0 && active) load_b(ch, dw, bfr, vg);
                    if (!SB) pf(dw);
                    if (!active) {
                        if (SB) pf(dw);
                        continue;
                    }
                    uint32_t w0[8], w1[8], rw0[8], rw1[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        w0[i] = word_of(c0[i], dw);
                        w1[i] = word_of(c1[i], dw);
                    }
                    slots_to_indices(w0, rw0);
                    slots_to_indices(w1, rw1);
                    if (SB) pf(dw);
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        half8 a0, a1;
                        lut_fragments2(rw0, rw1, m, slot, a0, a1);
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) {
                            // unguarded up to two tiles (a one-tile item always holds a
                            // token; an empty second tile multiplies zero B fragments), so
                            // each step stays one basic block the scheduler can interleave
                            if (NT <= 2 || nt < ntl) {
                                acc0[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bfr[nt][m], acc0[nt], 0, 0, 0);
                                acc1[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bfr[nt][m], acc1[nt], 0, 0, 0);
                            }
                        }
                    }
                }
            };

            // chunks 0, 1, ... alternate between (pa, pb); chunk 0 arrived with the
            // item. The next item's first chunk and LUT rows load into pa / st as soon
            // as pa has been consumed for the last time.
            LutStage st;
            bool fetched = false;
            // The next item's planes, LUT rows and token rows only: never its B rows,
            // which for a down item may only be read after its dependency wait.
            auto fetch_next = [&]() {   // all at once, after the item's last chunk
                if (has_next) {
                    load_chunk(nit, 0, pa0, pa1);
                    lut_load(nit, st);
                    ntk = tokinfo(nit);
                }
                fetched = true;
            };
            auto first_b = [&](int ch) {
                if (ch < nch) load_b(ch, 0, bfr, lane_col(ch) < it.klen);
            };
            first_b(0);
            if constexpr (SB) {
                // one buffer: after the last transposes of chunk ch it receives chunk
                // ch + 1, or the next item's first chunk (loads issued whether or not
                // there is anything to fetch); the next item's LUT and token rows load
                // after the last MFMAs, once the B fragments' registers are free
#pragma unroll 1
                for (int ch = 0; ch < nch; ++ch) {
                    const bool nx = ch + 1 >= nch;
                    compute_chunk(ch, pa0, pa1, [&](int dw) {
                        if (dw == 3) load_chunk(nx ? nit : it, nx ? 0 : ch + 1, pa0, pa1, -1, !nx || has_next);
                    });
                    first_b(ch + 1);
                }
                if (has_next) {
                    lut_load(nit, st);
                    ntk = tokinfo(nit);
                }
                fetched = true;
            }
            // Chunk ch computes from one plane buffer while the other receives the next
            // chunk, or the next item's first chunk (which always goes to pa), one
            // group per dword of ch. Every group issues its loads whether or not there
            // is anything to fetch (then they read zeros), so the waits stay exact;
            // the next item's LUT and token rows follow the last group.
#pragma unroll 1
            for (int ch = 0; ch < (SB ? 0 : nch); ch += 2) {
                compute_chunk(ch, pa0, pa1, [&](int dw) {
                    load_chunk(it, ch + 1, pb0, pb1, dw, ch + 1 < nch);
                });
                first_b(ch + 1);
                if (ch + 1 >= nch) break;
                const bool nx = ch + 2 >= nch;   // the next item's first chunk
                compute_chunk(ch + 1, pb0, pb1, [&](int dw) {
                    load_chunk(nx ? nit : it, nx ? 0 : ch + 2, pa0, pa1, dw, !nx || has_next);
                    if (dw == 3) {
                        const int b0 = nit.blk0->bits, b1 = nit.blk1->bits;
                        lut_stage_load_buf(st, (const uint16_t*)nit.blk0->lut + ((size_t)nit.rows0 << b0), b0,
                                           (const uint16_t*)nit.blk1->lut + ((size_t)nit.rows1 << b1), b1, tid,
                                           g.lut_tiled, nx && has_next);
                        ntk = fetch_tokinfo_buf(nit.mode == 0 ? p.gu : p.dn, nit, tid, nx && has_next);
                    }
                });
                if (nx) fetched = true;
                first_b(ch + 2);
            }
            if (!fetched) fetch_next();

            // partner (other half-line) partial sums of the registers it finishes
            const int pq = q ^ 1;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if (nt < ntl) {
                    float* w = red + ((q * NT + nt) * 4) * 64 + (tid & 63);
                    if (kh == 0) {
                        w[0 * 64] = acc0[nt][2];
                        w[1 * 64] = acc0[nt][3];
                        w[2 * 64] = acc1[nt][2];
                        w[3 * 64] = acc1[nt][3];
                    } else {
                        w[0 * 64] = acc0[nt][0];
                        w[1 * 64] = acc0[nt][1];
                        w[2 * 64] = acc1[nt][0];
                        w[3 * 64] = acc1[nt][1];
                    }
                }
            }
            __syncthreads();   // every wave is done with the LUT stripe; partial sums visible

            // sum of the two half-line partials of registers 2*kh, 2*kh+1 and the epilogue
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                if (nt >= ntl) break;
                const int tok_i = nt * 16 + r;
                const bool tv = tok_i < it.nl;
                const float* pr = red + ((pq * NT + nt) * 4) * 64 + (tid & 63);
                float g0, g1, u0, u1;
                if (kh == 0) {
                    g0 = acc0[nt][0]; g1 = acc0[nt][1]; u0 = acc1[nt][0]; u1 = acc1[nt][1];
                } else {
                    g0 = acc0[nt][2]; g1 = acc0[nt][3]; u0 = acc1[nt][2]; u1 = acc1[nt][3];
                }
                g0 += pr[0 * 64];
                g1 += pr[1 * 64];
                u0 += pr[2 * 64];
                u1 += pr[3 * 64];
                if (tv) {
                    const int row = rh * 16 + kg * 4 + kh * 2;   // rows row, row+1 of the item
                    const int orow = tb[64 + tok_i];
                    if (it.mode == 0) {
                        const float a0 = g0 / (1.0f + expf(-g0)) * u0;
                        const float a1 = g1 / (1.0f + expf(-g1)) * u1;
                        const int f = it.tile * 32 + row;   // even: f, f+1 are adjacent act columns
                        const uint32_t pk = (uint32_t)f2h(a0) | ((uint32_t)f2h(a1) << 16);
                        // device-coherent store: written through to the memory side, so a down
                        // item on another XCD that reads the row after the counter sees it
                        __hip_atomic_store((uint32_t*)(g.ws.act + (size_t)orow * g.ld_act + f), pk,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    } else {
                        const float wv = __int_as_float(tb[128 + tok_i]);
                        float* yr = g.y + (size_t)orow * g.d;
                        float* yo = yr + it.tile * 64 + row;   // set 0 rows; set 1 rows 32 further
                        if (DET) {
                            // this (slot, K-piece)'s own row of the partial buffer: plain stores
                            const int slot = tb[tok_i];
                            const int prow = it.ex == g.E
                                                 ? g.part_shared + (slot - g.shared_base) * p.dn.pieces_s + it.piece
                                                 : slot * p.dn.pieces_r + it.piece;
                            float* po = g.ws.part + (size_t)prow * g.d + it.tile * 64 + row;
                            *(float2*)po = make_float2(wv * g0, wv * g1);
                            *(float2*)(po + 32) = make_float2(wv * u0, wv * u1);
                        } else {
                            unsafeAtomicAdd(yo, wv * g0);
                            unsafeAtomicAdd(yo + 1, wv * g1);
                            unsafeAtomicAdd(yo + 32, wv * u0);
                            unsafeAtomicAdd(yo + 33, wv * u1);
                        }
                    }
                }
            }
            // the next item's LUT rows and token rows (written while the act stores drain)
            if (has_next) publish_item(nit, st, ntk, par ^ 1);
            if (it.mode == 0) vm_drain();   // this wave's act stores are complete
            __syncthreads();   // next item's LUT rows and token rows are in place; partials read
            if (it.mode == 0 && tid == 0)
                __hip_atomic_fetch_add(dep + it.pos * dstride + ((it.tile * 32) / kDownPiece), 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            if (!has_next) break;
            item = next;
            it = nit;
            par ^= 1;
        }
    }

    // the last work-group to finish zeroes the dependency counters
    __syncthreads();
    if (tid == 0) {
        vm_drain();   // this work-group's counter increments (thread 0's) are performed
        const uint32_t prev = __hip_atomic_fetch_add(dep + (size_t)npos * dstride, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = prev == n_working - 1u;
    }
    __syncthreads();
    if (*s_flag) {
        for (int i = tid; i <= npos * dstride; i += 256)
            __hip_atomic_store(dep + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ============================================================================ dequantise-once kernel

// Experts with many tokens: each weight of an item is dequantised once and
// multiplied with up to kBigTokens tokens (legiblepapers FAQ Q5: the fused
// kernel reads the planes and LUTs directly; here the per-weight unpack and
// lookup cost is shared by all of an item's tokens instead of being repeated
// per 64-token group).
//
// Work-group of 8 waves, one per CU. Items are those of the large lists, with
// the same rows and K ranges as in expert_kernel (gate_up: 32 rows of gate and
// of up; down: 64 rows, one K-piece) and up to kBigTokens = 128 tokens each.
//   - Waves 0..3 (producers) unpack and look up exactly as expert_kernel does
//     (wave q: rows 16*(q >> 1) .. +15, half-line q & 1; lane (r, kg)), but
//     write the looked-up weights to LDS instead of multiplying them. One step
//     is one 32-column dword of every lane: 64 rows x 256 columns, 32 KiB, laid
//     out as 32 MFMA A fragments (16 rows x 32 columns, 1 KiB each) whose 32
//     columns are contiguous: fragment (set, row half, kh, kg) holds columns
//     kh*512 + kg*128 + 32*dw + [0, 32) of the chunk, lane (r, kq) of it the
//     eight columns 8*kq .. +7 (the producer's lookup step m = kq).
//   - Waves 4..7 (consumers) take 32 tokens each (two 16-token MFMA tiles)
//     and multiply every fragment of a step with their tokens' activation
//     fragments (x rows or act rows, loaded straight from L2: per token 64
//     contiguous bytes per fragment, 16 rows per load instruction),
//     accumulating the whole item (64 rows x 32 tokens) in registers; the
//     epilogue is expert_kernel's (SwiGLU -> act, or w * o added into y).
// Steps are pipelined through two 32 KiB buffers: in phase f the producers
// write step f into buffer f & 1 while the consumers read step f - 1 from the
// other, and a work-group barrier ends every phase. A producer item starts by
// writing its LUT rows to the stripe, which every producer has stopped reading
// at the previous phase's barrier; a second barrier then publishes them. The
// consumer walks the same item sequence one step behind and executes the same
// barriers. The item order, the dependency counters (one increment per
// consumer wave, after its act stores have drained) and the deadlock argument
// are those of expert_kernel.
constexpr int kBigWaves = 8;
constexpr int kWStepBytes = 32 * 1024;

__device__ __forceinline__ int w_frag(int s, int rh, int kh, int kg) { return ((s * 2 + rh) * 2 + kh) * 4 + kg; }

template <bool DET>
__global__ __launch_bounds__(kBigWaves * 64, 1) void expert_kernel_big(ExpertParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NT = kBigTokens / 16;   // token tiles per item (decode_item's group size)
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    unsigned char* wbuf = smem + kStripeBytes;                    // [2][32 fragments][64 lanes][16 B]
    int* s_pre = (int*)(wbuf + 2 * kWStepBytes);                  // [2][kPreWords]: gate_up, down
    int* s_flag = s_pre + 2 * kPreWords;
    uint32_t* s_ready = (uint32_t*)(s_flag + 1);                  // last down item whose act rows are ready
    const GemmParams& g = p.gu;
    uint32_t* const dep = g.ws.dep;
    const int dstride = g.ws.dep_stride;
    const int npos = g.E + g.has_shared;
    // a work-group without an item leaves at once (as in expert_kernel)
    const int n_all = g.ws.prefix[p.gu.list * (g.E + 2) + npos] + g.ws.prefix[p.dn.list * (g.E + 2) + npos];
    if ((int)blockIdx.x >= n_all) return;
    const uint32_t n_working = (uint32_t)min((int)gridDim.x, n_all);
    for (int i = tid; i <= npos; i += kBigWaves * 64) {
        s_pre[i] = g.ws.prefix[p.gu.list * (g.E + 2) + i];
        s_pre[kPreWords + i] = g.ws.prefix[p.dn.list * (g.E + 2) + i];
    }
    if (tid == 0) *s_ready = 0u;
    __syncthreads();
    const int n_gu = __builtin_amdgcn_readfirstlane(s_pre[npos]);
    const int n_items = n_gu + __builtin_amdgcn_readfirstlane(s_pre[kPreWords + npos]);
    auto decode = [&](int i) -> Item {
        return i < n_gu ? decode_item<0, NT>(p.gu, s_pre, npos, i)
                        : decode_item<1, NT>(p.dn, s_pre + kPreWords, npos, i - n_gu);
    };
    auto n_steps = [](const Item& it) { return 4 * ((it.klen + 1023) >> 10); };

    if (wave < 4 && (int)blockIdx.x < n_items) {
        // ------------------------------------------------------------ producers
        int r = tid & 15, kg = (tid >> 4) & 3;
        const int rh = wave >> 1, kh = wave & 1;
        uint4 pa0[8], pa1[8], pb0[8], pb1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pa0[i] = pa1[i] = pb0[i] = pb1[i] = make_uint4(0, 0, 0, 0);
        auto lane_col = [&](int ch) { return ch * 1024 + kh * 512 + kg * 128; };
        auto load_chunk = [&](const Item& it, int ch, uint4 (&c0)[8], uint4 (&c1)[8]) {
            const int Kb = it.K >> 3;
            const bool vg = lane_col(ch) < it.klen;
            const uint32_t nrec = (uint32_t)(it.R * Kb);
            const int cb = (it.kbase + lane_col(ch)) >> 3;
            const int row = rh * 16 + r;
            const uint32_t off0 = vg ? (uint32_t)((it.rows0 + row) * Kb + cb) : kOOB;
            const uint32_t off1 = vg ? (uint32_t)((it.rows1 + row) * Kb + cb) : kOOB;
            const int s0 = 8 - it.blk0->bits, s1 = 8 - it.blk1->bits;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                c0[i] = buf_load16(make_rsrc((const void*)it.blk0->planes[i], i >= s0 ? nrec : 0u), off0);
                c1[i] = buf_load16(make_rsrc((const void*)it.blk1->planes[i], i >= s1 ? nrec : 0u), off1);
            }
        };
        auto lut_load = [&](const Item& it, LutStage& st) {
            const int b0 = it.blk0->bits, b1 = it.blk1->bits;
            lut_stage_load(st, (const uint16_t*)it.blk0->lut + ((size_t)it.rows0 << b0), b0,
                           (const uint16_t*)it.blk1->lut + ((size_t)it.rows1 << b1), b1, tid, g.lut_tiled);
        };
        int item = blockIdx.x;
        Item it = decode(item);
        LutStage st;
        load_chunk(it, 0, pa0, pa1);
        lut_load(it, st);
        while (true) {
            asm volatile("" : "+v"(r), "+v"(kg));
            lut_stage_write(smem, st, it.blk0->bits, it.blk1->bits, tid);
            __syncthreads();   // the item's LUT rows are in the stripe
            const int nch = (it.klen + 1023) >> 10;
            const int next = item + (int)gridDim.x;
            const bool has_next = next < n_items;
            Item nit = it;
            if (has_next) nit = decode(next);
            const uint32_t slot = lds_addr(smem) + (uint32_t)((rh * 32 + (kg & 1) * 16 + r) * 4);
            // lookup step m of lane (r, kg) is lane (r, kq = m) of fragment kg
            unsigned char* wl = wbuf + r * 16;
            auto produce = [&](int ch, int dw, const uint4 (&c0)[8], const uint4 (&c1)[8], int buf) {
                if (ch * 1024 + kh * 512 >= it.klen) return;   // this wave's half-chunk lies past K
                uint32_t w0[8], w1[8], rw0[8], rw1[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    w0[i] = word_of(c0[i], dw);
                    w1[i] = word_of(c1[i], dw);
                }
                slots_to_indices(w0, rw0);
                slots_to_indices(w1, rw1);
                unsigned char* wb = wl + buf * kWStepBytes;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const half8 a0 = lut_fragment(rw0, m, slot, 0);
                    const half8 a1 = lut_fragment(rw1, m, slot, 2);
                    *(half8*)(wb + w_frag(0, rh, kh, kg) * 1024 + m * 256) = a0;
                    *(half8*)(wb + w_frag(1, rh, kh, kg) * 1024 + m * 256) = a1;
                }
            };
            bool fetched = false;
            auto fetch_next = [&]() {
                if (has_next) {
                    load_chunk(nit, 0, pa0, pa1);
                    lut_load(nit, st);
                }
                fetched = true;
            };
            // global step parity: the consumers read buffer (step & 1) one phase later
            if (1 < nch) load_chunk(it, 1, pb0, pb1);
#pragma unroll 1
            for (int ch = 0; ch < nch; ch += 2) {
#pragma unroll
                for (int dw = 0; dw < 4; ++dw) {
                    produce(ch, dw, pa0, pa1, dw & 1);
                    __syncthreads();   // step published; the other buffer has been read
                }
                if (ch + 2 < nch) load_chunk(it, ch + 2, pa0, pa1);
                else if (ch + 1 < nch) fetch_next();
                if (ch + 1 >= nch) break;
#pragma unroll
                for (int dw = 0; dw < 4; ++dw) {
                    produce(ch + 1, dw, pb0, pb1, dw & 1);
                    __syncthreads();
                }
                if (ch + 3 < nch) load_chunk(it, ch + 3, pb0, pb1);
            }
            if (!fetched) fetch_next();
            if (!has_next) break;
            item = next;
            it = nit;
        }
    } else if (wave >= 4 && (int)blockIdx.x < n_items) {
        // ------------------------------------------------------------ consumers
        constexpr int TPW = kBigTokens / 64;  // 16-token tiles per consumer wave
        const int cw = wave - 4;              // tokens 16*TPW*cw .. +16*TPW-1 of the item
        const int tr = lane & 15, kq = lane >> 4;
        int item = blockIdx.x;
        Item it = decode(item);
        // phase 0: the producers' first step (the first item's stripe write, then the step)
        __syncthreads();
        __syncthreads();
        while (true) {
            const int S = n_steps(it);
            const int next = item + (int)gridDim.x;
            const bool has_next = next < n_items;
            const int ldb = it.mode == 0 ? g.d : g.ld_act;
            const __amdgpu_buffer_rsrc_t brsrc =
                it.mode == 0 ? make_rsrc(g.x, p.gu.b_bytes) : make_rsrc(g.ws.act, p.dn.b_bytes);
            // this wave's tokens: B row, output row and weight of token 16*TPW*cw + 16*t + tr
            const bool sh = it.ex == g.E;
            const int obase = sh ? 0 : kconst(g.ws.offsets)[it.ex];
            int ntl = (it.nl - 16 * TPW * cw + 15) >> 4;
            ntl = ntl < 0 ? 0 : (ntl > TPW ? TPW : ntl);
            uint32_t boff[TPW];
            int orow[TPW], bslot[TPW];
            float wt[TPW];
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int li = 16 * TPW * cw + 16 * t + tr;
                boff[t] = kOOB;
                orow[t] = -1;
                bslot[t] = 0;
                wt[t] = 0.0f;
                if (li < it.nl) {
                    const int tkn = it.tbase + li;
                    const int slotn = sh ? (g.shared_base + tkn) : (obase + tkn);
                    const int tok = sh ? tkn : g.ws.slot_tok[slotn];
                    const int brow = it.mode == 0 ? tok : slotn;
                    orow[t] = it.mode == 0 ? slotn : tok;
                    bslot[t] = slotn;
                    wt[t] = (it.mode == 0 || sh) ? 1.0f : g.ws.slot_w[slotn];
                    boff[t] = (uint32_t)(brow * ldb + kq * 8);
                }
            }
            if (it.mode == 1) {
                // every gate_up item of this expert's K-piece has released its act rows:
                // the first consumer wave polls the counter (one poller per work-group,
                // spaced out, keeps the polls off the memory system) and publishes the
                // item in LDS; the other consumer waves wait for that, and none of them
                // loads act before (the dependency invariants of expert_kernel)
                if (cw == 0) {
                    const uint32_t need =
                        (uint32_t)((it.klen >> 5) * ((it.n_tok + kBigTokens - 1) / kBigTokens) * 4);
                    const uint32_t* c = dep + it.pos * dstride + it.piece;
                    uint32_t polls = 0;
                    while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
                        if (polls++ >= kconst(g.ws.wait_limit)[0]) {
                            if (lane == 0) atomicOr(g.ws.status, PW_STATUS_DEP_TIMEOUT);
                            break;
                        }
                        __builtin_amdgcn_s_sleep(4);
                    }
                    __hip_atomic_store(s_ready, (uint32_t)item + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                } else {
                    // ends once wave 4 has published this item (its own wait is bounded)
                    while (__hip_atomic_load(s_ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != (uint32_t)item + 1u)
                        __builtin_amdgcn_s_sleep(1);
                }
            }
            floatx4 acc[2][2][TPW];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int t = 0; t < TPW; ++t) acc[s][h][t] = (floatx4)0.0f;
            // B fragments of half kh of step sc: tile t, fragment kg (columns
            // kh*512 + kg*128 + 32*dw + [0, 32) of chunk sc >> 2; lane (tok, kq): 8 of them)
            auto kvalid = [&](int sc, int kh, int kg) { return (sc >> 2) * 1024 + kh * 512 + kg * 128 < it.klen; };
            // Every call issues its 16 loads (inactive ones read zeros without touching
            // memory), so the loads in flight are the same on every path and the
            // waits before the MFMAs count exactly: a conditional prefetch would
            // make them wait for it too.
            auto load_b = [&](int sc, int kh, half8 (&bq)[TPW][4], bool on) {
                const int col = (sc >> 2) * 1024 + kh * 512 + (sc & 3) * 32;
#pragma unroll
                for (int t = 0; t < TPW; ++t)
#pragma unroll
                    for (int kg = 0; kg < 4; ++kg) {
                        // a select, not a branch: no short-circuit evaluation
                        const bool ok = on & kvalid(sc, kh, kg) & (t < ntl) & (boff[t] != kOOB);
                        const uint32_t off = ok ? (boff[t] + (uint32_t)(it.kbase + col + kg * 128)) * 2u : kOOB;
                        bq[t][kg] = __builtin_bit_cast(half8, buf_load16(brsrc, off));
                    }
            };
            // All four tiles of a wave with tokens: tiles and lanes without a token
            // hold zero B fragments (per-tile guards would split every MFMA into
            // its own basic block and serialise the fragment reads).
            // The fragments of k-block kg + 1 are read before the MFMAs of kg, so
            // the LDS latency overlaps the matrix work. Fragments past K are never
            // multiplied (their B fragments are zero anyway).
            auto mma = [&](int sc, int kh, const half8 (&bq)[TPW][4]) {
                if (ntl == 0) return;
                const unsigned char* wb = wbuf + (sc & 1) * kWStepBytes + lane * 16;
                half8 a[2][2][2];
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int h = 0; h < 2; ++h) a[0][s][h] = *(const half8*)(wb + w_frag(s, h, kh, 0) * 1024);
#pragma unroll
                for (int kg = 0; kg < 4; ++kg) {
                    if (kg < 3) {
#pragma unroll
                        for (int s = 0; s < 2; ++s)
#pragma unroll
                            for (int h = 0; h < 2; ++h)
                                a[(kg + 1) & 1][s][h] = *(const half8*)(wb + w_frag(s, h, kh, kg + 1) * 1024);
                    }
                    if (!kvalid(sc, kh, kg)) continue;   // columns past K (uniform)
#pragma unroll
                    for (int s = 0; s < 2; ++s)
#pragma unroll
                        for (int h = 0; h < 2; ++h)
#pragma unroll
                            for (int t = 0; t < TPW; ++t)
                                acc[s][h][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[kg & 1][s][h], bq[t][kg], acc[s][h][t], 0, 0, 0);
                }
            };
            half8 bq0[TPW][4], bq1[TPW][4];
            load_b(0, 0, bq0, true);
#pragma unroll 1
            for (int sc = 0; sc < S; ++sc) {
                load_b(sc, 1, bq1, true);
                mma(sc, 0, bq0);
                load_b(sc + 1, 0, bq0, sc + 1 < S);   // the next step's first half (none after the last)
                mma(sc, 1, bq1);
                if (sc + 1 == S) {
                    // epilogue: the item is complete in this wave's registers
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int t = 0; t < TPW; ++t) {
                            if (t >= ntl || orow[t] < 0) continue;
                            const int row = h * 16 + kq * 4;   // rows row .. row+3 of the set
                            if (it.mode == 0) {
                                uint32_t pk[2];
#pragma unroll
                                for (int j = 0; j < 2; ++j) {
                                    const float g0 = acc[0][h][t][2 * j], u0 = acc[1][h][t][2 * j];
                                    const float g1 = acc[0][h][t][2 * j + 1], u1 = acc[1][h][t][2 * j + 1];
                                    const float a0 = g0 / (1.0f + expf(-g0)) * u0;
                                    const float a1 = g1 / (1.0f + expf(-g1)) * u1;
                                    pk[j] = (uint32_t)f2h(a0) | ((uint32_t)f2h(a1) << 16);
                                }
                                const uint64_t v = (uint64_t)pk[0] | ((uint64_t)pk[1] << 32);
                                // device-coherent store (written through), drained before the counter
                                __hip_atomic_store((uint64_t*)(g.ws.act + (size_t)orow[t] * g.ld_act + it.tile * 32 + row),
                                                   v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            } else if (DET) {
                                // this (slot, K-piece)'s own row of the partial buffer: plain stores
                                const int prow = sh ? g.part_shared + (bslot[t] - g.shared_base) * p.dn.pieces_s + it.piece
                                                    : bslot[t] * p.dn.pieces_r + it.piece;
                                float* po = g.ws.part + (size_t)prow * g.d + it.tile * 64 + row;
                                *(float4*)po = make_float4(wt[t] * acc[0][h][t][0], wt[t] * acc[0][h][t][1],
                                                           wt[t] * acc[0][h][t][2], wt[t] * acc[0][h][t][3]);
                                *(float4*)(po + 32) = make_float4(wt[t] * acc[1][h][t][0], wt[t] * acc[1][h][t][1],
                                                                  wt[t] * acc[1][h][t][2], wt[t] * acc[1][h][t][3]);
                            } else {
                                float* yo = g.y + (size_t)orow[t] * g.d + it.tile * 64 + row;
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    unsafeAtomicAdd(yo + i, wt[t] * acc[0][h][t][i]);
                                    unsafeAtomicAdd(yo + 32 + i, wt[t] * acc[1][h][t][i]);
                                }
                            }
                        }
                    if (it.mode == 0) {
                        vm_drain();   // this wave's act stores are complete
                        if (lane == 0)
                            __hip_atomic_fetch_add(dep + it.pos * dstride + ((it.tile * 32) / kDownPiece), 1u,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
                // the producers' step sc + 1 of this item, or the next item's first step
                // (LUT stripe write and its barrier first), in the same phase
                if (sc + 1 < S) {
                    __syncthreads();
                } else if (has_next) {
                    __syncthreads();
                    __syncthreads();
                }
            }
            if (!has_next) break;
            item = next;
            it = decode(item);
        }
    }

    // the last work-group to finish zeroes the dependency counters
    __syncthreads();
    if (tid == 0) {
        vm_drain();
        const uint32_t prev = __hip_atomic_fetch_add(dep + (size_t)npos * dstride, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = prev == n_working - 1u;
    }
    __syncthreads();
    if (*s_flag) {
        for (int i = tid; i <= npos * dstride; i += kBigWaves * 64)
            __hip_atomic_store(dep + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ============================================================================ residual / init / debug

__global__ __launch_bounds__(256) void residual_kernel(const uint16_t* x, const float* y,
                                                       uint16_t* out, long n) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = f2h(h2f(x[i]) + y[i]);
}

// Deterministic mode: each thread sums four columns of one token's partial rows in
// a fixed order (routed assignments j = 0..k-1, each over its K-pieces, then
// the shared expert's pieces), so y does not depend on the order in which the
// down items ran.
__global__ __launch_bounds__(256) void reduce_kernel(Workspace ws, float* y, int T, int k, int d, int pr, int ps,
                                                     int part_shared) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;   // float4 index into y
    const int q = d >> 2;
    if (i >= (long)T * q) return;
    const int t = (int)(i / q), c = (int)(i - (long)t * q) * 4;
    float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    auto add = [&](int row) {
        const float4 v = *(const float4*)(ws.part + (size_t)row * d + c);
        a.x += v.x;
        a.y += v.y;
        a.z += v.z;
        a.w += v.w;
    };
    for (int j = 0; j < k; ++j) {
        const int slot = ws.slot_of[(size_t)t * k + j];
        for (int pc = 0; pc < pr; ++pc) add(slot * pr + pc);
    }
    for (int pc = 0; pc < ps; ++pc) add(part_shared + t * ps + pc);
    *(float4*)(y + (size_t)t * d + c) = a;
}

__global__ __launch_bounds__(64) void init_ws_kernel(Workspace ws, int n_counters, uint32_t wait_limit) {
    if (threadIdx.x == 0) {
        *ws.status = 0u;
        *ws.wait_limit = wait_limit;
    }
    for (int i = threadIdx.x; i < n_counters; i += 64) ws.dep[i] = 0u;   // dep, tok_cnt, route_done
}

struct DebugParams {
    uint64_t planes[8];
    const uint16_t* lut;
    int b, R, K;
    int lut_tiled;
    uint8_t* idx_out;
    uint16_t* w_out;
};

// One wave per 32-row tile; the same index transpose and LDS-stripe lookup as
// the gemm kernels, writing indices and fp16 weights back in row-major order.
__global__ __launch_bounds__(64) void debug_kernel(DebugParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int lane = threadIdx.x, r = lane & 31, g = lane >> 5;
    const int rb = blockIdx.x * 32;
    const int Kb = p.K >> 3;
    if (p.w_out) {
        const uint16_t* lut = p.lut + ((size_t)rb << p.b);
        stage_lut32((uint32_t*)smem, lut, p.b, p.lut_tiled, lane);
    }
    __syncthreads();
    const uint32_t slot = lds_addr(smem) + (uint32_t)(r * 4);
    for (int ch = 0; ch * 256 < p.K; ++ch) {
        const int c0 = ch * 256 + g * 128;
        if (c0 >= p.K) continue;
        uint4 q4[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {   // slot q holds plane q - (8 - b)
            q4[q] = make_uint4(0, 0, 0, 0);
            if (q >= 8 - p.b) q4[q] = *(const uint4*)((const uint8_t*)p.planes[q] + (size_t)(rb + r) * Kb + ch * 32 + g * 16);
        }
#pragma unroll
        for (int dw = 0; dw < 4; ++dw) {
            uint32_t w[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) w[q] = word_of(q4[q], dw);
            const int cg = c0 + 32 * dw;
            const size_t rowoff = (size_t)(rb + r) * p.K;
            uint32_t rw[8];
            slots_to_indices(w, rw);
            if (p.idx_out) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        p.idx_out[rowoff + cg + 8 * kk + i] = (uint8_t)(rw[i] >> (8 * kk));
            }
            if (p.w_out) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const half8 a = lut_fragment(rw, m, slot, 0);
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        p.w_out[rowoff + cg + 8 * m + j] = __builtin_bit_cast(uint16_t, (_Float16)a[j]);
                }
            }
        }
    }
}

// ============================================================================ static scratch

// Device scratch of pw_moe_forward_noalloc: the page table and the workspace of
// one forward live here instead of in memory the library allocates. Each GPU
// holds its own copy from module load until the process ends; every no-alloc
// call on that GPU shares it.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The device address of `scratch` on device dev (the host-side name is only a
// stand-in), looked up once per device with that device current.
hipError_t scratch_memory(int dev, void** ptr, size_t* bytes) {
    static void* addr[64] = {};
    static std::mutex mu;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    *bytes = kScratchBytes;
    return hipSuccess;
}

// ============================================================================ launchers

int expert_lds_bytes(int tile_tokens) {
    const int nt = tile_tokens / 16;
    return kStripeBytes + 4 * nt * 4 * 64 * 4 + 2 * kTokWords * 4 + 2 * kPreWords * 4 + 16;
}

hipError_t launch_init_ws(const Workspace& ws, int n_counters, uint32_t wait_limit, hipStream_t s) {
    hipLaunchKernelGGL(init_ws_kernel, dim3(1), dim3(64), 0, s, ws, n_counters, wait_limit);
    return hipGetLastError();
}

hipError_t launch_route(const RouteParams& p, hipStream_t s) {
    const int per_wg = (kRouteThreads / 64) * (p.exact_all ? kRouteExactPerWave : kRouteFilterPerWave);
    const int nb = (p.E + per_wg - 1) / per_wg;
    hipLaunchKernelGGL(route_kernel, dim3((unsigned)(p.T * nb)), dim3(kRouteThreads), 0, s, p);
    return hipGetLastError();
}

// Resident work-groups per CU of expert_kernel<NT, DET> (0 if it cannot run).
template <int NT, bool DET>
static hipError_t expert_occupancy(int* per_cu) {
    static int cached = -1;
    if (cached < 0) {
        const void* f = (const void*)expert_kernel<NT, DET>;
        hipError_t err = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (err != hipSuccess) return err;
        int n = 0;
        err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, 256, expert_lds_bytes(16 * NT));
        if (err != hipSuccess) return err;
        cached = n < (NT <= 2 ? 2 : 1) ? n : (NT <= 2 ? 2 : 1);
    }
    *per_cu = cached;
    return hipSuccess;
}

// PW_COOPERATIVE=1 (read once per process) launches the expert kernels
// cooperatively: the runtime then guarantees that every work-group is resident
// at once, or fails the launch, instead of the grid being sized to the
// occupancy and trusted to fit.
static bool cooperative_launch() {
    static const bool on = [] {
        const char* v = getenv("PW_COOPERATIVE");
        return v != nullptr && v[0] == '1';
    }();
    return on;
}

template <int NT, bool DET>
static hipError_t launch_experts_t(const ExpertParams& p, int n_cu, hipStream_t s) {
    int per_cu = 0;
    hipError_t err = expert_occupancy<NT, DET>(&per_cu);
    if (err != hipSuccess) return err;
    if (per_cu < 1) return hipErrorLaunchOutOfResources;
    // every work-group resident at once: the dependency waits rely on it
    if (cooperative_launch()) {
        ExpertParams arg = p;
        void* args[] = {(void*)&arg};
        return hipLaunchCooperativeKernel((const void*)expert_kernel<NT, DET>, dim3(per_cu * n_cu), dim3(256), args,
                                          (unsigned)expert_lds_bytes(16 * NT), s);
    }
    hipLaunchKernelGGL((expert_kernel<NT, DET>), dim3(per_cu * n_cu), dim3(256), expert_lds_bytes(16 * NT), s, p);
    return hipGetLastError();
}

static int big_lds_bytes() { return kStripeBytes + 2 * kWStepBytes + 2 * kPreWords * 4 + 16; }   // + flag, ready

// Resident work-groups per CU of the dequantise-once kernel (at most 1).
template <bool DET>
static hipError_t big_occupancy(int* per_cu) {
    static int cached = -1;
    if (cached < 0) {
        const void* f = (const void*)expert_kernel_big<DET>;
        hipError_t err = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (err != hipSuccess) return err;
        int n = 0;
        err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, f, kBigWaves * 64, big_lds_bytes());
        if (err != hipSuccess) return err;
        cached = n < 1 ? n : 1;
    }
    *per_cu = cached;
    return hipSuccess;
}

template <bool DET>
static hipError_t launch_big_t(const ExpertParams& p, int n_cu, hipStream_t s) {
    int per_cu = 0;
    hipError_t err = big_occupancy<DET>(&per_cu);
    if (err != hipSuccess) return err;
    if (per_cu < 1) return hipErrorLaunchOutOfResources;
    if (cooperative_launch()) {
        ExpertParams arg = p;
        void* args[] = {(void*)&arg};
        return hipLaunchCooperativeKernel((const void*)expert_kernel_big<DET>, dim3(per_cu * n_cu),
                                          dim3(kBigWaves * 64), args, (unsigned)big_lds_bytes(), s);
    }
    hipLaunchKernelGGL(expert_kernel_big<DET>, dim3(per_cu * n_cu), dim3(kBigWaves * 64), big_lds_bytes(), s, p);
    return hipGetLastError();
}

hipError_t launch_experts_big(const ExpertParams& p, int n_cu, hipStream_t s) {
    return p.dn.det ? launch_big_t<true>(p, n_cu, s) : launch_big_t<false>(p, n_cu, s);
}

// Every expert-kernel variant the layer's flags can launch.
hipError_t prepare_experts(bool det) {
    int n[4] = {0, 0, 0, 0};
    hipError_t err = det ? expert_occupancy<1, true>(&n[0]) : expert_occupancy<1, false>(&n[0]);
    if (err == hipSuccess) err = det ? expert_occupancy<2, true>(&n[1]) : expert_occupancy<2, false>(&n[1]);
    if (err == hipSuccess) err = det ? expert_occupancy<4, true>(&n[2]) : expert_occupancy<4, false>(&n[2]);
    if (err == hipSuccess) err = det ? big_occupancy<true>(&n[3]) : big_occupancy<false>(&n[3]);
    if (err != hipSuccess) return err;
    return (n[0] < 1 || n[1] < 1 || n[2] < 1 || n[3] < 1) ? hipErrorLaunchOutOfResources : hipSuccess;
}

template <bool DET>
static hipError_t launch_experts_d(int tile_tokens, const ExpertParams& p, int n_cu, hipStream_t s) {
    if (tile_tokens == kSmallTokens) return launch_experts_t<1, DET>(p, n_cu, s);
    if (tile_tokens == kTwoTokens) return launch_experts_t<2, DET>(p, n_cu, s);
    return launch_experts_t<4, DET>(p, n_cu, s);
}

hipError_t launch_experts(int tile_tokens, const ExpertParams& p, int n_cu, hipStream_t s) {
    return p.dn.det ? launch_experts_d<true>(tile_tokens, p, n_cu, s) : launch_experts_d<false>(tile_tokens, p, n_cu, s);
}

hipError_t launch_reduce(const Workspace& ws, float* y, int T, int k, int d, int pr, int ps, int part_shared,
                         hipStream_t s) {
    const long n = (long)T * (d / 4);
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ws, y, T, k, d, pr, ps,
                       part_shared);
    return hipGetLastError();
}

hipError_t launch_residual(const uint16_t* x, const float* y, uint16_t* x_next, long n,
                           hipStream_t s) {
    const long blocks = (n + 255) / 256;
    hipLaunchKernelGGL(residual_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, y, x_next, n);
    return hipGetLastError();
}

hipError_t launch_debug(const uint64_t* planes8, int b, const uint16_t* lut, int lut_tiled, int R, int K,
                        uint8_t* idx_out, uint16_t* w_out, hipStream_t s) {
    DebugParams p;
    for (int q = 0; q < 8; ++q) p.planes[q] = planes8[q];
    p.lut = lut;
    p.lut_tiled = lut_tiled;
    p.b = b;
    p.R = R;
    p.K = K;
    p.idx_out = idx_out;
    p.w_out = w_out;
    const int lds = 256 << b;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t err = hipFuncSetAttribute((const void*)debug_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (err != hipSuccess) return err;
        attr_set = true;
    }
    hipLaunchKernelGGL(debug_kernel, dim3(R / 32), dim3(64), lds, s, p);
    return hipGetLastError();
}

}  // namespace pw
