// gfx950 (CDNA4) kernels of the fused mixed-precision MoE layer.
//
// The layer (PagedWeight pages: arxivlens summary; legiblepapers "Key Takeaways"
// and FAQ Q5) reads every expert weight straight from Any-Precision bit-planes
// and a per-row lookup table, each (expert, linear) block at its own bitwidth b,
// and fuses routing, SwiGLU expert activation and weighted accumulation.
//
// Kernels, in stream order per forward:
//   route_kernel   exact router logits (int64, units of 2^-48), top-k softmax per
//                  token (last-arriving workgroup of the token), then a stable
//                  token->expert bucket sort (last-arriving workgroup of the call);
//                  also writes the column-permuted copy of x and zeroes y.
//   gemm_kernel<0> gate and up of each (expert, 32-row tile, token group):
//                  bit-plane unpack + LUT dequant into MFMA A fragments, MFMA
//                  32x32x16 fp16 with fp32 accumulation, SwiGLU -> act (fp16).
//   gemm_kernel<1> down of each (expert, 64-row tile, token group), scaled by
//                  the routing weight and atomically added into y (fp32).
//   residual_kernel  x_next = fp16_rne(x + y) when requested.
//
// Dequantisation (the hot loop). Lane (r, g) of a wave owns row r (0..31) of the
// tile and a 128-column half g of each 256-column chunk. For one 32-column dword
// of each of the b planes, a three-stage bit-matrix transpose (8x8 per byte)
// turns the b plane words into eight index words W_i whose byte k is the b-bit
// index of column 8k+i. One v_perm per weight drops that byte into an LDS
// address, and one 16-bit LDS read fetches the fp16 weight from the LUT stripe:
// dword (idx*64 + g*32 + r) holds the two row-sets' LUT entries (low/high half),
// so the 64 lanes of a wave always hit 64 distinct banks. Eight looked-up
// weights form one MFMA A operand; the B operand (activations) is stored with
// the same in-group column permutation, so the contraction is unchanged.
#include <hip/hip_runtime.h>

#include "pw.h"
#include "pw_internal.h"

namespace pw {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
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

// Position of column c (0..31) of a 32-column group in the permuted activation
// layout: column 8k + i goes to 8*(i>>1) + 2k + (i&1). Eight consecutive
// permuted positions 8m..8m+7 are the columns one MFMA step m consumes.
__device__ __forceinline__ int perm32(int c) {
    const int k = c >> 3, i = c & 7;
    return 8 * (i >> 1) + 2 * k + (i & 1);
}

// ============================================================================ route

__device__ __forceinline__ void add_pair(uint32_t xw, uint32_t ww, long long& acc, float& sab,
                                         int& bad) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const float xf = h2f((uint16_t)(xw >> (16 * h)));
        const float wf = h2f((uint16_t)(ww >> (16 * h)));
        bad |= !(fabsf(xf) < 128.0f) | !(fabsf(wf) < 128.0f);
        // exact: |x|,|w| < 128, so x*2^24 and w*2^24 are integers below 2^31
        const int X = (int)(xf * 16777216.0f);
        const int W = (int)(wf * 16777216.0f);
        acc += (long long)X * (long long)W;
        sab = fmaf(fabsf(xf), fabsf(wf), sab);
    }
}

template <typename Tv>
__device__ __forceinline__ Tv load_relaxed(const Tv* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void route_kernel(RouteParams p) {
    const int eg = blockIdx.x, t = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int d = p.d, E = p.E, k = p.k;
    const uint16_t* xr = p.x + (size_t)t * d;
    __shared__ int s_flag;
    __shared__ int s_cnt[PW_MAX_EXPERTS];
    __shared__ int s_off[PW_MAX_EXPERTS + 1];

    // ---- exact logits of this group's experts: one wave per expert
    const int e_begin = eg * p.epb;
    const int e_end = min(E, e_begin + p.epb);
    for (int e = e_begin + wave; e < e_end; e += 4) {
        const uint16_t* wrow = p.wr + (size_t)e * d;
        long long acc = 0;
        float sab = 0.0f;
        int bad = 0;
        for (int c = lane * 8; c < d; c += 512) {
            const uint4 xv = *(const uint4*)(xr + c);
            const uint4 wv = *(const uint4*)(wrow + c);
            add_pair(xv.x, wv.x, acc, sab, bad);
            add_pair(xv.y, wv.y, acc, sab, bad);
            add_pair(xv.z, wv.z, acc, sab, bad);
            add_pair(xv.w, wv.w, acc, sab, bad);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            acc += __shfl_xor(acc, off);
            sab += __shfl_xor(sab, off);
            bad |= __shfl_xor(bad, off);
        }
        if (lane == 0) {
            if (p.bias) {
                const float bf = h2f(p.bias[e]);
                bad |= !(fabsf(bf) < 32768.0f);
                if (!bad) acc += (long long)((double)bf * 281474976710656.0);  // * 2^48, exact
                sab += fabsf(bf);
            }
            // the fp32 bound has relative error below d*2^-24, far inside the margin
            if (bad || !(sab < 32000.0f)) atomicOr(p.ws.status, PW_STATUS_ROUTER_RANGE);
            p.ws.logits[(size_t)t * E + e] = acc;
        }
    }

    // ---- permuted copy of x (MFMA B-operand layout) and zeroed y, once per token
    if (eg == 0) {
        for (int c = tid; c < d; c += 256) {
            p.ws.xperm[(size_t)t * d + (c & ~31) + perm32(c & 31)] = xr[c];
            p.y[(size_t)t * d + c] = 0.0f;
        }
    }

    // ---- last workgroup of this token selects its experts
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = atomicAdd(&p.ws.tok_cnt[t], 1u);
        s_flag = (prev == (unsigned)(p.n_eg - 1));
    }
    __syncthreads();
    if (!s_flag) return;
    __threadfence();

    if (wave == 0) {
        long long v[PW_MAX_EXPERTS / 64];
        bool taken[PW_MAX_EXPERTS / 64];
#pragma unroll
        for (int j = 0; j < PW_MAX_EXPERTS / 64; ++j) {
            const int e = lane + 64 * j;
            v[j] = (e < E) ? load_relaxed(&p.ws.logits[(size_t)t * E + e]) : 0;
            taken[j] = (e >= E);
        }
        long long selv[PW_MAX_TOP_K];
        int sele[PW_MAX_TOP_K];
        for (int j = 0; j < k; ++j) {
            long long bv = LLONG_MIN;
            int be = 0x7fffffff;
#pragma unroll
            for (int q = 0; q < PW_MAX_EXPERTS / 64; ++q) {
                const int e = lane + 64 * q;
                if (!taken[q] && (v[q] > bv || (v[q] == bv && e < be))) {
                    bv = v[q];
                    be = e;
                }
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                const long long ov = __shfl_xor(bv, off);
                const int oe = __shfl_xor(be, off);
                if (ov > bv || (ov == bv && oe < be)) {
                    bv = ov;
                    be = oe;
                }
            }
            selv[j] = bv;
            sele[j] = be;
#pragma unroll
            for (int q = 0; q < PW_MAX_EXPERTS / 64; ++q)
                if (be == lane + 64 * q) taken[q] = true;
        }
        if (lane == 0) {
            float l[PW_MAX_TOP_K], ex[PW_MAX_TOP_K];
            float s = 0.0f;
            for (int j = 0; j < k; ++j) l[j] = ldexpf((float)selv[j], -48);
            for (int j = 0; j < k; ++j) {
                ex[j] = expf(l[j] - l[0]);
                s += ex[j];
            }
            for (int j = 0; j < k; ++j) {
                const float wj = ex[j] / s;
                p.ws.ids[(size_t)t * k + j] = sele[j];
                p.ws.w[(size_t)t * k + j] = wj;
                if (p.o_ids) p.o_ids[(size_t)t * k + j] = sele[j];
                if (p.o_w) p.o_w[(size_t)t * k + j] = wj;
            }
            p.ws.tok_cnt[t] = 0u;   // ready for the next call
        }
    }

    // ---- last workgroup of the call: stable bucket sort of the T*k assignments
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = atomicAdd(p.ws.glob_cnt, 1u);
        s_flag = (prev == (unsigned)(p.T - 1));
    }
    __syncthreads();
    if (!s_flag) return;
    __threadfence();

    const int n = p.T * k;
    for (int e = tid; e < E; e += 256) s_cnt[e] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += 256) atomicAdd(&s_cnt[load_relaxed(&p.ws.ids[i])], 1);
    __syncthreads();
    if (wave == 0) {
        // exclusive scan over E <= 256 counts: 4 consecutive experts per lane
        int c4[4], loc = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane * 4 + j;
            c4[j] = (e < E) ? s_cnt[e] : 0;
            loc += c4[j];
        }
        int inc = loc;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(inc, off);
            if (lane >= off) inc += o;
        }
        int run = inc - loc;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane * 4 + j;
            if (e < E) s_off[e] = run;
            run += c4[j];
        }
        if (lane == 63) s_off[E] = inc;
    }
    __syncthreads();
    for (int e = tid; e <= E; e += 256) {
        p.ws.offsets[e] = s_off[e];
        if (p.o_offsets) p.o_offsets[e] = s_off[e];
        if (e < E) {
            p.ws.counts[e] = s_cnt[e];
            if (p.o_counts) p.o_counts[e] = s_cnt[e];
        }
    }
    __syncthreads();
    if (wave == 0) {
        // s_cnt becomes the running insert position of each expert
        for (int e = lane; e < E; e += 64) s_cnt[e] = s_off[e];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        for (int base = 0; base < n; base += 64) {
            const int i = base + lane;
            const bool valid = i < n;
            const int e = valid ? load_relaxed(&p.ws.ids[i]) : 0;
            unsigned long long same = __ballot(valid);
#pragma unroll
            for (int bit = 0; bit < 8; ++bit) {
                const unsigned long long bb = __ballot(valid && ((e >> bit) & 1));
                same &= ((e >> bit) & 1) ? bb : ~bb;
            }
            const int rank = __popcll(same & __lanemask_lt());
            const int pos = s_cnt[e] + rank;
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
            __builtin_amdgcn_wave_barrier();
            if (valid) {
                p.ws.sorted[pos] = i;
                if (p.o_sorted) p.o_sorted[pos] = i;
                if ((same >> lane) == 1ull) s_cnt[e] += __popcll(same);   // highest lane of its group
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
            __builtin_amdgcn_wave_barrier();
        }
        if (lane == 0) *p.ws.glob_cnt = 0u;
    }
}

// ============================================================================ dequant core

// Transposes the b plane words of one 32-column group into index words:
// out[i] byte k = index of column 8k+i (plane p is bit b-1-p of the index).
template <int B>
__device__ __forceinline__ void planes_to_indices(const uint32_t (&pl)[8], uint32_t (&rw)[8]) {
#pragma unroll
    for (int q = 0; q < 8; ++q) rw[q] = (q < B) ? pl[B - 1 - q] : 0u;
    // 8x8 bit transpose inside every byte: swap the off-diagonal 4x4, 2x2, 1x1 blocks
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

// A fragments of four MFMA steps from one 32-column dword per plane:
// a[m] half 2k+e = LUT[index of column 8k + 2m + e]. `slot` is the lane's LDS
// address of stripe entry 0 (segment base + (g*32 + r)*4); byte 1 of it is
// replaced by the index, i.e. entry idx sits idx*256 bytes further.
template <int B>
__device__ __forceinline__ void dq_dword(const uint32_t (&pl)[8], uint32_t slot, int hoff,
                                         half8 (&a)[4]) {
    uint32_t rw[8];
    planes_to_indices<B>(pl, rw);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint32_t addr =
                    __builtin_amdgcn_perm(rw[2 * m + e], slot, 0x03020400u | (uint32_t)(kk << 8));
                a[m][2 * kk + e] = *(lds_half*)(size_t)(addr + hoff);
            }
        }
    }
}

__device__ __forceinline__ void dq_dword_rt(int b, const uint32_t (&pl)[8], uint32_t slot, int hoff,
                                            half8 (&a)[4]) {
    switch (b) {
        case 1: dq_dword<1>(pl, slot, hoff, a); break;
        case 2: dq_dword<2>(pl, slot, hoff, a); break;
        case 3: dq_dword<3>(pl, slot, hoff, a); break;
        case 4: dq_dword<4>(pl, slot, hoff, a); break;
        case 5: dq_dword<5>(pl, slot, hoff, a); break;
        case 6: dq_dword<6>(pl, slot, hoff, a); break;
        case 7: dq_dword<7>(pl, slot, hoff, a); break;
        default: dq_dword<8>(pl, slot, hoff, a); break;
    }
}

// 8 LUT entries [c8, c8+8) of one row (zeros past 2^b).
__device__ __forceinline__ void load_lut8(const uint16_t* row, int b, int c8, uint32_t (&v)[8]) {
    const int n = 1 << b;
    if (b >= 3) {
        uint4 q = make_uint4(0, 0, 0, 0);
        if (c8 < n) q = *(const uint4*)(row + c8);
        v[0] = q.x & 0xFFFF; v[1] = q.x >> 16; v[2] = q.y & 0xFFFF; v[3] = q.y >> 16;
        v[4] = q.z & 0xFFFF; v[5] = q.z >> 16; v[6] = q.w & 0xFFFF; v[7] = q.w >> 16;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (c8 + i < n) ? row[c8 + i] : 0u;
    }
}

// Stages the LUT rows of both row-sets into the LDS stripe (two copies, one per
// lane half g), cooperatively over nthreads threads.
__device__ __forceinline__ void stage_luts(uint32_t* stripe, const uint16_t* lut0, int b0,
                                           const uint16_t* lut1, int b1, int tid, int nthreads) {
    const int bmax = b0 > b1 ? b0 : b1;
    const int nc8 = (1 << bmax) >= 8 ? (1 << bmax) / 8 : 1;
    for (int j = tid; j < nc8 * 32; j += nthreads) {
        const int r = j & 31, c = j >> 5;
        uint32_t v0[8], v1[8];
        load_lut8(lut0 + ((size_t)r << b0), b0, c * 8, v0);
        load_lut8(lut1 + ((size_t)r << b1), b1, c * 8, v1);
        const int first = (j >> 5) & 1;   // alternate copies so a wave's halves hit different banks
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int idx = c * 8 + i;
            if (idx < (1 << bmax)) {
                const uint32_t dw = v0[i] | (v1[i] << 16);
                stripe[idx * 64 + first * 32 + r] = dw;
                stripe[idx * 64 + (1 - first) * 32 + r] = dw;
            }
        }
    }
}

__device__ __forceinline__ uint32_t word_of(const uint4& q, int dw) {
    return dw == 0 ? q.x : dw == 1 ? q.y : dw == 2 ? q.z : q.w;
}

// ============================================================================ gemm

// MODE 0: gate_up, MODE 1: down. NT: MFMA token tiles of 32 per work item.
template <int MODE, int NT>
__global__ __launch_bounds__(256, NT == 1 ? 2 : 1) void gemm_kernel(GemmParams p) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bid = blockIdx.x;
    if (bid >= p.n_work) return;
    int e, tile;
    if (bid < p.E * p.tiles_r) {
        e = bid / p.tiles_r;
        tile = bid - e * p.tiles_r;
    } else {
        e = p.E;
        tile = bid - p.E * p.tiles_r;
    }
    const bool shared = (e == p.E);
    const int n_tok = shared ? p.T : p.ws.counts[e];
    if (n_tok < p.min_count || n_tok > p.max_count) return;
    const int tbase = blockIdx.y * (32 * NT);
    if (tbase >= n_tok) return;
    const int nl = min(32 * NT, n_tok - tbase);
    const int ntl = (nl + 31) >> 5;

    const DevBlock* blk0 = &p.blocks[e * 3 + (MODE == 0 ? 0 : 2)];
    const DevBlock* blk1 = &p.blocks[e * 3 + (MODE == 0 ? 1 : 2)];
    const int rb0 = MODE == 0 ? tile * 32 : tile * 64;
    const int rb1 = MODE == 0 ? tile * 32 : tile * 64 + 32;
    const int K = MODE == 0 ? p.d : (shared ? p.Fs : p.F);
    const int b0 = blk0->bits, b1 = blk1->bits;
    const int Kb = K >> 3;

    // ---- token rows of this work item
    int* s_brow = (int*)(smem + p.lds_stripe);
    int* s_orow = s_brow + 128;
    float* s_ow = (float*)(s_orow + 128);
    for (int i = tid; i < nl; i += 256) {
        const int slot = shared ? (p.shared_base + tbase + i) : (p.ws.offsets[e] + tbase + i);
        if (MODE == 0) {
            s_brow[i] = shared ? (tbase + i) : p.ws.sorted[slot] / p.k;   // token (xperm row)
            s_orow[i] = slot;                                              // act row
        } else {
            const int asg = shared ? 0 : p.ws.sorted[slot];
            s_brow[i] = slot;                                              // act row
            s_orow[i] = shared ? (tbase + i) : asg / p.k;                  // token (y row)
            s_ow[i] = shared ? 1.0f : p.ws.w[asg];
        }
    }

    // ---- plane bases are uniform (SGPRs); each lane adds one 32-bit offset per set
    const int r = lane & 31, g = lane >> 5;
    const uint32_t slot = lds_addr(smem) + (uint32_t)((g * 32 + r) * 4);
    const int nch = (K + 255) >> 8;
    const uint8_t* base0[8];
    const uint8_t* base1[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        base0[q] = (const uint8_t*)blk0->planes[q];
        base1[q] = (const uint8_t*)blk1->planes[q];
    }
    const uint32_t off0 = (uint32_t)((rb0 + r) * Kb + g * 16);
    const uint32_t off1 = (uint32_t)((rb1 + r) * Kb + g * 16);
    auto load_chunk = [&](int ch, uint4 (&c0)[8], uint4 (&c1)[8]) {
        const bool vg = (ch * 256 + g * 128) < K;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (q < b0 && vg) c0[q] = *(const uint4*)(base0[q] + (off0 + (uint32_t)ch * 32u));
            if (q < b1 && vg) c1[q] = *(const uint4*)(base1[q] + (off1 + (uint32_t)ch * 32u));
        }
    };
    // ping-pong plane buffers: chunk ch in A while chunk ch+4 loads into B
    uint4 pa0[8], pa1[8], pb0[8], pb1[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        pa0[q] = pa1[q] = pb0[q] = pb1[q] = make_uint4(0, 0, 0, 0);
    }
    if (wave < nch) load_chunk(wave, pa0, pa1);

    stage_luts((uint32_t*)smem, (const uint16_t*)blk0->lut + ((size_t)rb0 << b0), b0,
               (const uint16_t*)blk1->lut + ((size_t)rb1 << b1), b1, tid, 256);
    __syncthreads();

    const uint16_t* Bbase = MODE == 0 ? p.ws.xperm : p.ws.act;
    const int ldb = MODE == 0 ? p.d : p.ld_act;
    uint32_t boff[NT];
    bool bok[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int i = nt * 32 + r;
        bok[nt] = i < nl;
        boff[nt] = bok[nt] ? (uint32_t)(s_brow[i] * ldb + g * 128) : 0u;
    }

    floatx16 acc0[NT], acc1[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        acc0[nt] = (floatx16)0.0f;
        acc1[nt] = (floatx16)0.0f;
    }
    auto compute_chunk = [&](int ch, const uint4 (&c0)[8], const uint4 (&c1)[8]) {
        const bool vg = (ch * 256 + g * 128) < K;
#pragma unroll
        for (int dw = 0; dw < 4; ++dw) {
            half8 bf[NT][4];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
                for (int m = 0; m < 4; ++m) bf[nt][m] = (half8)(_Float16)0.0f;
                if (nt < ntl && bok[nt] && vg) {
                    const half8* src = (const half8*)(Bbase + (boff[nt] + (uint32_t)(ch * 256 + 32 * dw)));
#pragma unroll
                    for (int m = 0; m < 4; ++m) bf[nt][m] = src[m];
                }
            }
            uint32_t w0[8], w1[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                w0[q] = word_of(c0[q], dw);
                w1[q] = word_of(c1[q], dw);
            }
            half8 a0[4], a1[4];
            dq_dword_rt(b0, w0, slot, 0, a0);
            dq_dword_rt(b1, w1, slot, 2, a1);
            if (!vg) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    a0[m] = (half8)(_Float16)0.0f;
                    a1[m] = (half8)(_Float16)0.0f;
                }
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    if (nt < ntl) {
                        acc0[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[m], bf[nt][m], acc0[nt], 0, 0, 0);
                        acc1[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[m], bf[nt][m], acc1[nt], 0, 0, 0);
                    }
                }
            }
        }
    };

    for (int ch = wave; ch < nch; ch += 8) {
        if (ch + 4 < nch) load_chunk(ch + 4, pb0, pb1);
        compute_chunk(ch, pa0, pa1);
        if (ch + 4 >= nch) break;
        if (ch + 8 < nch) load_chunk(ch + 8, pa0, pa1);
        compute_chunk(ch + 4, pb0, pb1);
    }

    // ---- cross-wave K reduction through LDS, then the epilogue
    float* red = (float*)smem;   // [4 waves][64 lanes][16]
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        if (nt >= ntl) break;
        float s0[4], s1[4];
#pragma unroll
        for (int set = 0; set < 2; ++set) {
            const floatx16& a = set == 0 ? acc0[nt] : acc1[nt];
#pragma unroll
            for (int v = 0; v < 16; ++v) red[wave * 1024 + lane * 16 + v] = a[v];
            __syncthreads();
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = tid + 256 * q;
                const float sum = red[j] + red[1024 + j] + red[2048 + j] + red[3072 + j];
                if (set == 0) s0[q] = sum; else s1[q] = sum;
            }
            __syncthreads();
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int j = tid + 256 * q;
            const int ln = j >> 4, reg = j & 15;
            const int tok_i = nt * 32 + (ln & 31);
            const int row = (reg >> 2) * 8 + (ln >> 5) * 4 + (reg & 3);
            if (tok_i < nl) {
                if (MODE == 0) {
                    const float gv = s0[q], uv = s1[q];
                    const float av = gv / (1.0f + expf(-gv)) * uv;
                    p.ws.act[(size_t)s_orow[tok_i] * p.ld_act + rb0 + perm32(row)] = f2h(av);
                } else {
                    const float wv = s_ow[tok_i];
                    float* yr = p.y + (size_t)s_orow[tok_i] * p.d;
                    unsafeAtomicAdd(yr + rb0 + row, wv * s0[q]);
                    unsafeAtomicAdd(yr + rb1 + row, wv * s1[q]);
                }
            }
        }
    }
}

// ============================================================================ residual / init / debug

__global__ __launch_bounds__(256) void residual_kernel(const uint16_t* x, const float* y,
                                                       uint16_t* out, long n) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = f2h(h2f(x[i]) + y[i]);
}

__global__ __launch_bounds__(256) void init_ws_kernel(Workspace ws, int max_T) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < max_T) ws.tok_cnt[i] = 0u;
    if (i == 0) {
        *ws.glob_cnt = 0u;
        *ws.status = 0u;
    }
}

struct DebugParams {
    uint64_t planes[8];
    const uint16_t* lut;
    int b, R, K;
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
    const uint16_t* lut = p.lut + ((size_t)rb << p.b);
    if (p.w_out) stage_luts((uint32_t*)smem, lut, p.b, lut, p.b, lane, 64);
    __syncthreads();
    const uint32_t slot = lds_addr(smem) + (uint32_t)((g * 32 + r) * 4);
    for (int ch = 0; ch * 256 < p.K; ++ch) {
        const int c0 = ch * 256 + g * 128;
        if (c0 >= p.K) continue;
        uint4 q4[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            q4[q] = make_uint4(0, 0, 0, 0);
            if (q < p.b) q4[q] = *(const uint4*)((const uint8_t*)p.planes[q] + (size_t)(rb + r) * Kb + ch * 32 + g * 16);
        }
#pragma unroll
        for (int dw = 0; dw < 4; ++dw) {
            uint32_t w[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) w[q] = word_of(q4[q], dw);
            const int cg = c0 + 32 * dw;
            const size_t rowoff = (size_t)(rb + r) * p.K;
            if (p.idx_out) {
                uint32_t rw[8];
                switch (p.b) {
                    case 1: planes_to_indices<1>(w, rw); break;
                    case 2: planes_to_indices<2>(w, rw); break;
                    case 3: planes_to_indices<3>(w, rw); break;
                    case 4: planes_to_indices<4>(w, rw); break;
                    case 5: planes_to_indices<5>(w, rw); break;
                    case 6: planes_to_indices<6>(w, rw); break;
                    case 7: planes_to_indices<7>(w, rw); break;
                    default: planes_to_indices<8>(w, rw); break;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        p.idx_out[rowoff + cg + 8 * kk + i] = (uint8_t)(rw[i] >> (8 * kk));
            }
            if (p.w_out) {
                half8 a[4];
                dq_dword_rt(p.b, w, slot, 0, a);
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                        for (int e = 0; e < 2; ++e)
                            p.w_out[rowoff + cg + 8 * kk + 2 * m + e] =
                                __builtin_bit_cast(uint16_t, (_Float16)a[m][2 * kk + e]);
            }
        }
    }
}

// ============================================================================ launchers

int gemm_lds_bytes(int bmax) {
    const int stripe = 256 << bmax;
    const int red = 4 * 64 * 16 * 4;
    return (stripe > red ? stripe : red) + kTokInfoBytes;
}

hipError_t launch_init_ws(const Workspace& ws, int max_T, hipStream_t s) {
    const int blocks = (max_T + 255) / 256 > 0 ? (max_T + 255) / 256 : 1;
    hipLaunchKernelGGL(init_ws_kernel, dim3(blocks), dim3(256), 0, s, ws, max_T);
    return hipGetLastError();
}

hipError_t launch_route(const RouteParams& p, hipStream_t s) {
    hipLaunchKernelGGL(route_kernel, dim3(p.n_eg, p.T), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int MODE, int NT>
static hipError_t launch_gemm_t(const GemmParams& p, int lds_bytes, int nz, hipStream_t s) {
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t err = hipFuncSetAttribute((const void*)gemm_kernel<MODE, NT>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (err != hipSuccess) return err;
        attr_set = true;
    }
    const int gx = (p.n_work + 7) / 8 * 8;   // multiple of 8: token groups of one tile share an XCD
    hipLaunchKernelGGL((gemm_kernel<MODE, NT>), dim3(gx, nz), dim3(256), lds_bytes, s, p);
    return hipGetLastError();
}

hipError_t launch_gemm(int mode, int tile_tokens, const GemmParams& p, int lds_bytes, int nz,
                       hipStream_t s) {
    if (mode == 0) {
        return tile_tokens == 32 ? launch_gemm_t<0, 1>(p, lds_bytes, nz, s)
                                 : launch_gemm_t<0, 4>(p, lds_bytes, nz, s);
    }
    return tile_tokens == 32 ? launch_gemm_t<1, 1>(p, lds_bytes, nz, s)
                             : launch_gemm_t<1, 4>(p, lds_bytes, nz, s);
}

hipError_t launch_residual(const uint16_t* x, const float* y, uint16_t* x_next, long n,
                           hipStream_t s) {
    const long blocks = (n + 255) / 256;
    hipLaunchKernelGGL(residual_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, y, x_next, n);
    return hipGetLastError();
}

hipError_t launch_debug(const uint64_t* planes8, int b, const uint16_t* lut, int R, int K,
                        uint8_t* idx_out, uint16_t* w_out, hipStream_t s) {
    DebugParams p;
    for (int q = 0; q < 8; ++q) p.planes[q] = planes8[q];
    p.lut = lut;
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
