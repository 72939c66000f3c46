/*
 * CPU oracle for the fused mixed-precision MoE layer -- TEST INFRASTRUCTURE.
 *
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
 * load this library. The product path never calls it, and it shares no code
 * with the GPU library.
 *
 * What it computes (PagedWeight pages: arxivlens summary, legiblepapers
 * "Key Takeaways" and FAQ Q5): one MoE layer whose expert weights are read
 * straight from Any-Precision bit-planes and per-row lookup tables, each
 * (expert, linear) block at its own bitwidth b, with routing, SwiGLU expert
 * activation and weighted output accumulation. The pages print no formula,
 * so each step below follows the plainest reading:
 *
 *   O1 router logits  L[t][e] = sum_c x[t][c] * Wr[e][c] + bias[e], computed
 *      exactly as an integer in units of 2^-48 (every fp16 value is an integer
 *      multiple of 2^-24, so every product is a multiple of 2^-48).
 *   O2 top-k          the k largest L[t][.], ties to the lower expert index,
 *      emitted in descending order.
 *   O3 weights        softmax over the k selected logits in fp32:
 *      l_j = float(L) * 2^-48, w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0).
 *   O4 bucket sort    for each expert ascending, the assignments t*k + j that
 *      chose it, in ascending (t, j); counts and exclusive offsets.
 *   O5 index assembly idx = sum_{p<b} bit_p(r, c) << (b-1-p), bit_p read from
 *      plane p (plane 0 = most significant bit of the 8-bit parent), byte c>>3,
 *      bit c&7 of row r; weight = LUT_b[r][idx] (fp16 -> fp32).
 *   O6 expert         g = Wg x, u = Wu x (fp32, c ascending),
 *      a = silu(g) * u with silu(z) = z / (1 + exp(-z)), o = Wd a (r ascending).
 *   O7 combine        y[t] = sum_j w_j o_{t,j} (j ascending), then + the shared
 *      expert's output (weight 1) when the layer has one.
 *
 * All floating point is fp32 with no contraction into FMA (compile with
 * -ffp-contract=off); the logits are exact integers (__int128 accumulation).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_E_RANGE 1
#define ORC_E_ARG 2

/* ---------------------------------------------------------------- fp16 helpers */

/* fp16 bit pattern -> fp32 value (exact: every fp16 value is an fp32 value). */
static float h2f(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024 + m), e - 25);
    return s ? -v : v;
}

/* fp16 bit pattern -> exact integer value * 2^24. Sets *bad for inf/nan. */
static __int128 h2i24(uint16_t h, int* bad) {
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    __int128 v;
    if (e == 31) {
        *bad = 1;
        return 0;
    }
    if (e == 0)
        v = m;                                       /* m * 2^-24 */
    else
        v = (__int128)(1024 + m) << (e - 1);         /* (1024+m) * 2^(e-25) * 2^24 */
    return s ? -v : v;
}

/* ---------------------------------------------------------------- O1..O4 routing */

/* O1: L[t*E + e] in units of 2^-48. Returns ORC_E_RANGE when a logit does not fit
 * in int64 or an input is not finite; the value is then clamped. */
int orc_router_logits(const uint16_t* x, int T, int d, const uint16_t* wr, int E,
                      const uint16_t* bias, int64_t* L) {
    int status = ORC_OK;
#pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            int bad = 0;
            __int128 acc = 0;
            for (int c = 0; c < d; ++c)
                acc += h2i24(x[(size_t)t * d + c], &bad) * h2i24(wr[(size_t)e * d + c], &bad);
            if (bias) acc += h2i24(bias[e], &bad) * ((__int128)1 << 24);
            const __int128 lim = ((__int128)1) << 63;
            if (acc >= lim || acc < -lim || bad) {
#pragma omp atomic write
                status = ORC_E_RANGE;
                acc = acc >= lim ? lim - 1 : (acc < -lim ? -lim : acc);
            }
            L[(size_t)t * E + e] = (int64_t)acc;
        }
    }
    return status;
}

/* O2 + O3: ids[t*k + j] (descending logit, ties to lower index), w[t*k + j]. */
void orc_topk_softmax(const int64_t* L, int T, int E, int k, int32_t* ids, float* w) {
    if (k <= 0 || k > 64 || k > E) return;
    for (int t = 0; t < T; ++t) {
        const int64_t* row = L + (size_t)t * E;
        int32_t* id = ids + (size_t)t * k;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                int taken = 0;
                for (int i = 0; i < j; ++i) taken |= (id[i] == e);
                if (taken) continue;
                /* strictly greater keeps the lower index on ties */
                if (best < 0 || row[e] > row[best]) best = e;
            }
            id[j] = best;
        }
        float l[64], ex[64];
        for (int j = 0; j < k; ++j) l[j] = ldexpf((float)row[id[j]], -48);
        float s = 0.0f;
        for (int j = 0; j < k; ++j) {
            ex[j] = expf(l[j] - l[0]);
            s += ex[j];
        }
        for (int j = 0; j < k; ++j) w[(size_t)t * k + j] = ex[j] / s;
    }
}

/* O4: counts[E], offsets[E+1] (exclusive prefix sum), sorted[T*k]. */
void orc_bucket_sort(const int32_t* ids, int T, int E, int k, int32_t* counts,
                     int32_t* offsets, int32_t* sorted) {
    int pos = 0;
    for (int e = 0; e < E; ++e) {
        offsets[e] = pos;
        int n = 0;
        for (int t = 0; t < T; ++t)
            for (int j = 0; j < k; ++j)
                if (ids[(size_t)t * k + j] == e) {
                    sorted[pos++] = t * k + j;
                    ++n;
                }
        counts[e] = n;
    }
    offsets[E] = pos;
}

/* ---------------------------------------------------------------- O5 index assembly */

/* planes: array of b plane pointers, each [R][K/8] bytes. */
static inline int idx_at(const uint8_t* const* planes, int b, int K, int r, int c) {
    int idx = 0;
    size_t byte = (size_t)r * (K / 8) + (c >> 3);
    for (int p = 0; p < b; ++p) {
        int bit = (planes[p][byte] >> (c & 7)) & 1;
        idx |= bit << (b - 1 - p);
    }
    return idx;
}

/* indices u8 [R][K] of one block at bitwidth b */
void orc_unpack_indices(const uint8_t* const* planes, int b, int R, int K, uint8_t* out) {
    for (int r = 0; r < R; ++r)
        for (int c = 0; c < K; ++c) out[(size_t)r * K + c] = (uint8_t)idx_at(planes, b, K, r, c);
}

/* dequantized weights fp32 [R][K]: LUT_b[r][idx] (lut: fp16 [R][2^b]) */
void orc_dequant(const uint8_t* const* planes, int b, const uint16_t* lut, int R, int K,
                 float* out) {
    for (int r = 0; r < R; ++r)
        for (int c = 0; c < K; ++c)
            out[(size_t)r * K + c] = h2f(lut[((size_t)r << b) + idx_at(planes, b, K, r, c)]);
}

/* out[r] = sum_c W[r][c] * v[c], c ascending, fp32, weights read bit by bit. */
static void linear_f32(const uint8_t* const* planes, int b, const uint16_t* lut, int R, int K,
                       const float* v, float* out) {
    for (int r = 0; r < R; ++r) {
        float acc = 0.0f;
        for (int c = 0; c < K; ++c) {
            float wv = h2f(lut[((size_t)r << b) + idx_at(planes, b, K, r, c)]);
            acc += wv * v[c];
        }
        out[r] = acc;
    }
}

/* one linear on an fp16 input vector (test hook for the addressing pin) */
void orc_linear(const uint8_t* const* planes, int b, const uint16_t* lut, int R, int K,
                const uint16_t* x, float* out) {
    float* v = (float*)malloc(sizeof(float) * (size_t)K);
    for (int c = 0; c < K; ++c) v[c] = h2f(x[c]);
    linear_f32(planes, b, lut, R, K, v, out);
    free(v);
}

/* ---------------------------------------------------------------- O6 expert */

/* Linear-blocks. A linear-block is a whole linear (rb = 0), or, with rb > 0, a
 * block of rb consecutive rows of a linear (legiblepapers "Key Takeaways" and
 * FAQ Q5: variable bitwidths per linear-block; the pages do not say how large a
 * block is, so both readings are served). Blocks are numbered expert by expert
 * (routed 0..E-1, then the shared expert), within an expert gate, up, down, and
 * within a linear by row-block. Each block has its own bitwidth, planes (its
 * rows only, row-major) and LUT (its rows only). */
typedef struct {
    int d, E, F, Fs, k;
    int rb;                         /* rows per linear-block; 0 = whole linears */
    const uint8_t* bits;            /* [n_blocks] */
    const uint8_t* const* planes;   /* [n_blocks * 8], NULL beyond b */
    const uint16_t* const* luts;    /* [n_blocks], LUT for that block's b */
} orc_layer;

/* row-blocks of a linear with R rows */
static int n_rowblocks(const orc_layer* L, int R) { return L->rb ? R / L->rb : 1; }

/* index of the first block of expert e (the shared expert, e = E, follows the routed ones) */
static size_t expert_base(const orc_layer* L, int e) {
    return (size_t)e * (size_t)(2 * n_rowblocks(L, L->F) + n_rowblocks(L, L->d));
}

/* out[r] = sum_c W[r][c] * v[c] for a linear of R rows whose row-blocks are blocks
 * base, base+1, ...: row r is row r - j*rows of block base + j, j = r / rows,
 * read at that block's bitwidth (rows = rb, or R for a whole linear). */
static void linear_blocks_f32(const orc_layer* L, size_t base, int R, int K, const float* v, float* out) {
    int rows = L->rb ? L->rb : R;
    for (int j = 0; j * rows < R; ++j) {
        size_t bi = base + (size_t)j;
        linear_f32(L->planes + bi * 8, L->bits[bi], L->luts[bi], rows, K, v, out + (size_t)j * rows);
    }
}

static float silu(float z) { return z / (1.0f + expf(-z)); }

/* o[d] = expert e applied to the fp32 token vector xv[d] */
static void expert_forward(const orc_layer* L, int e, const float* xv, float* o) {
    int f = (e == L->E) ? L->Fs : L->F;
    int d = L->d;
    size_t base = expert_base(L, e);
    int nf = n_rowblocks(L, f);
    float* g = (float*)malloc(sizeof(float) * (size_t)f);
    float* u = (float*)malloc(sizeof(float) * (size_t)f);
    linear_blocks_f32(L, base, f, d, xv, g);              /* gate */
    linear_blocks_f32(L, base + nf, f, d, xv, u);         /* up */
    for (int r = 0; r < f; ++r) g[r] = silu(g[r]) * u[r];
    linear_blocks_f32(L, base + 2 * nf, d, f, g, o);      /* down */
    free(g);
    free(u);
}

/* ---------------------------------------------------------------- whole layer */

/*
 * Full layer on T tokens, linear-blocks of rb rows (0: whole linears; bits,
 * planes and luts then hold one entry per block in the order above). Routing
 * (logits, ids, w, counts, offsets, sorted) is
 * computed for all tokens; the expert outputs y[t][:] only for the tokens listed
 * in `subset` (all tokens when subset == NULL). y is [T][d], fp32; rows outside
 * the subset are left untouched. Any routing output pointer may be NULL.
 * Returns ORC_OK or ORC_E_RANGE (logit out of int64 range / non-finite input).
 */
int orc_moe_forward(int d, int E, int F, int Fs, int k, int rb, const uint8_t* bits,
                    const uint8_t* const* planes, const uint16_t* const* luts,
                    const uint16_t* x, int T, const uint16_t* router_w, const uint16_t* router_b,
                    const int32_t* subset, int n_subset, float* y, int64_t* logits_out,
                    int32_t* ids_out, float* w_out, int32_t* counts_out, int32_t* offsets_out,
                    int32_t* sorted_out, int nthreads) {
    if (T < 0 || d <= 0 || E <= 0 || k <= 0 || k > E || k > 64 || rb < 0) return ORC_E_ARG;
    if (rb && (d % rb || F % rb || (Fs > 0 && Fs % rb))) return ORC_E_ARG;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
    orc_layer Ly = {d, E, F, Fs, k, rb, bits, planes, luts};
    int64_t* Lg = (int64_t*)malloc(sizeof(int64_t) * ((size_t)T * E + 1));
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * ((size_t)T * k + 1));
    float* w = (float*)malloc(sizeof(float) * ((size_t)T * k + 1));
    int status = orc_router_logits(x, T, d, router_w, E, router_b, Lg);
    orc_topk_softmax(Lg, T, E, k, ids, w);
    if (counts_out || offsets_out || sorted_out) {
        int32_t* cnt = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
        int32_t* off = (int32_t*)malloc(sizeof(int32_t) * ((size_t)E + 1));
        int32_t* srt = (int32_t*)malloc(sizeof(int32_t) * ((size_t)T * k + 1));
        orc_bucket_sort(ids, T, E, k, cnt, off, srt);
        if (counts_out) memcpy(counts_out, cnt, sizeof(int32_t) * (size_t)E);
        if (offsets_out) memcpy(offsets_out, off, sizeof(int32_t) * ((size_t)E + 1));
        if (sorted_out) memcpy(sorted_out, srt, sizeof(int32_t) * (size_t)T * k);
        free(cnt);
        free(off);
        free(srt);
    }
    if (logits_out) memcpy(logits_out, Lg, sizeof(int64_t) * (size_t)T * E);
    if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * (size_t)T * k);
    if (w_out) memcpy(w_out, w, sizeof(float) * (size_t)T * k);

    int n = subset ? n_subset : T;
    int has_shared = Fs > 0;
    int per_tok = k + has_shared;
    /* expert outputs for every (token, slot); slot k is the shared expert */
    float* o = (float*)malloc(sizeof(float) * ((size_t)n * per_tok * d + 1));
#pragma omp parallel for schedule(dynamic, 1)
    for (int ij = 0; ij < n * per_tok; ++ij) {
        int i = ij / per_tok, j = ij % per_tok;
        int t = subset ? subset[i] : i;
        float* xv = (float*)malloc(sizeof(float) * (size_t)d);
        for (int c = 0; c < d; ++c) xv[c] = h2f(x[(size_t)t * d + c]);
        int e = (j < k) ? ids[(size_t)t * k + j] : E;
        expert_forward(&Ly, e, xv, o + ((size_t)i * per_tok + j) * d);
        free(xv);
    }
    for (int i = 0; i < n; ++i) {
        int t = subset ? subset[i] : i;
        for (int c = 0; c < d; ++c) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j)
                acc += w[(size_t)t * k + j] * o[((size_t)i * per_tok + j) * d + c];
            if (has_shared) acc += o[((size_t)i * per_tok + k) * d + c];
            y[(size_t)t * d + c] = acc;
        }
    }
    free(o);
    free(Lg);
    free(ids);
    free(w);
    return status;
}

/* O9 residual hand-off: x_next = fp16_rne(float(x) + y). Returns fp16 bit patterns. */
static uint16_t f2h_rne(float f) {
    /* round an fp32 value to the nearest fp16 (ties to even), with overflow to inf */
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t s = (u >> 16) & 0x8000u;
    float a = fabsf(f);
    if (isnan(f)) return (uint16_t)(s | 0x7e00u);
    if (a >= 65520.0f) return (uint16_t)(s | 0x7c00u);      /* rounds to inf */
    if (a < ldexpf(1.0f, -14)) {
        /* subnormal range: value = m * 2^-24, m = rne(a * 2^24) */
        float m = rintf(ldexpf(a, 24));                     /* rintf: ties to even */
        return (uint16_t)(s | (uint32_t)m);
    }
    int ex;
    float fr = frexpf(a, &ex);                              /* a = fr * 2^ex, fr in [0.5,1) */
    float m = rintf(ldexpf(fr, 11));                        /* 11 significant bits */
    if (m >= 2048.0f) {
        m = 1024.0f;
        ex += 1;
    }
    int e16 = ex - 1 + 15;                                  /* a = (m/1024) * 2^(ex-1) */
    if (e16 >= 31) return (uint16_t)(s | 0x7c00u);
    return (uint16_t)(s | ((uint32_t)e16 << 10) | ((uint32_t)m - 1024u));
}

void orc_residual(const uint16_t* x, const float* y, size_t n, uint16_t* out) {
    for (size_t i = 0; i < n; ++i) out[i] = f2h_rne(h2f(x[i]) + y[i]);
}
