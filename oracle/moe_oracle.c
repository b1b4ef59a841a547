/*
 * CPU oracle for the 4-bit group-affine MoE FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP path; it is plain, single-threaded,
 * unvectorised C built without fast-math or FP contraction.
 *
 * Sources (the "Optimizing on-device inference for Apple Silicon" page unless
 * said otherwise):
 *   - layer shape: a router scores E experts and keeps the top k, plus one
 *     shared expert that every token passes through (section "Qwen creates
 *     three different workload shapes");
 *   - weight format: every weight is a 4-bit integer code, every group of 64
 *     weights shares one bf16 scale and one bf16 bias that rebuild the weight
 *     (section "Dequantise weights during matrix multiplication");
 *   - routing metadata: histogram of assignments per expert, prefix scan into
 *     start offsets, scatter of rows into expert groups, map of fixed-size
 *     blocks (section "Keep expert routing on the GPU");
 *   - fused chains: gate and up projections with their gated activation; the
 *     output projection with the routing score and the shared-expert result
 *     (section "Reduce intermediate and state traffic").
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - dequant: w = s*q + b, q unsigned 0..15, groups of 64 along K, the even
 *     k in the low nibble of byte k/2;
 *   - router logit: the products x*Wr accumulated in float64 in increasing h,
 *     rounded once to float32, then the float32 logit bias added in float32;
 *   - top-k on the float32 logits, larger logit first, equal logits broken
 *     towards the lower expert index; weights = softmax over the k selected
 *     logits (= the full softmax renormalised over the selected experts),
 *     computed in float64 and rounded to float32;
 *   - scatter stable in flat assignment id t*k+j inside each expert segment;
 *   - block map: tiles of BM rows per expert in increasing expert then row
 *     order, experts without rows get no tile, the last tile of an expert may
 *     be partial; the shared expert's tiles follow as expert index E over the
 *     chunk's tokens in token order;
 *   - activation SiLU(g)*u with SiLU(z) = z/(1+exp(-z)); the shared expert
 *     has weight 1 and no gate of its own;
 *   - the expert FFN and the combine are evaluated in float64 (the exact
 *     definition; the GPU's float32 accumulation and bf16 intermediates are
 *     judged against it within tolerance).
 *
 * Pins: every function here is checked by the CPU tests against values the
 * pages or the mathematics fix (hand-computed groups, library sorts and
 * counts, a dense all-experts brute force written independently in numpy,
 * special cases that reduce to a textbook gated MLP).  No function is left
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const uint8_t *codes;    /* [N][K/2] */
    const uint16_t *scales;  /* [N][K/64] bf16 bits */
    const uint16_t *biases;  /* [N][K/64] bf16 bits */
} oq_matrix;

typedef struct {
    int32_t H, E, k, I, Is;
    oq_matrix gate, up, down;          /* routed experts: leading dim E */
    oq_matrix sh_gate, sh_up, sh_down; /* shared expert (unused if Is == 0) */
} oq_layer;

#define OQ_GROUP 64

static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Weight (n, k) of matrix number `e` of a stack of [N][K] matrices. */
static double oq_weight(const oq_matrix *m, int64_t e, int N, int K, int n, int k)
{
    int64_t row = e * N + n;
    uint8_t byte = m->codes[row * (K / 2) + k / 2];
    int q = (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
    int64_t gi = row * (K / OQ_GROUP) + k / OQ_GROUP;
    return bf16_value(m->scales[gi]) * (double)q + bf16_value(m->biases[gi]);
}

/* Dequantise a whole [N][K] matrix to float64 (used by the pin tests). */
void oracle_dequant(const uint8_t *codes, const uint16_t *scales, const uint16_t *biases,
                    int N, int K, double *out)
{
    oq_matrix m = {codes, scales, biases};
    for (int n = 0; n < N; n++)
        for (int k = 0; k < K; k++)
            out[(int64_t)n * K + k] = oq_weight(&m, 0, N, K, n, k);
}

/* Router logits: float64 accumulation, one rounding to float32, float32 bias. */
void oracle_router_logits(const uint16_t *x, int T, int H, const float *router_w,
                          const float *logit_bias, int E, float *logits)
{
    for (int t = 0; t < T; t++) {
        for (int e = 0; e < E; e++) {
            double acc = 0.0;
            for (int h = 0; h < H; h++)
                acc += bf16_value(x[(int64_t)t * H + h]) * (double)router_w[(int64_t)e * H + h];
            float l = (float)acc;
            if (logit_bias)
                l = l + logit_bias[e];
            logits[(int64_t)t * E + e] = l;
        }
    }
}

/* Top-k selection and renormalised softmax weights. */
void oracle_topk(const float *logits, int T, int E, int k, int32_t *ids, float *weights)
{
    char *taken = (char *)malloc((size_t)E);
    for (int t = 0; t < T; t++) {
        const float *l = logits + (int64_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int e = 0; e < E; e++) {
                if (taken[e])
                    continue;
                if (best < 0 || l[e] > l[best])
                    best = e;
            }
            taken[best] = 1;
            ids[(int64_t)t * k + j] = best;
        }
        double lmax = (double)l[ids[(int64_t)t * k]];
        double denom = 0.0;
        for (int j = 0; j < k; j++)
            denom += exp((double)l[ids[(int64_t)t * k + j]] - lmax);
        for (int j = 0; j < k; j++)
            weights[(int64_t)t * k + j] =
                (float)(exp((double)l[ids[(int64_t)t * k + j]] - lmax) / denom);
    }
    free(taken);
}

/*
 * Routing metadata for one chunk of T tokens: histogram, exclusive prefix
 * scan, stable scatter and the block map of BM-row tiles.  tiles holds
 * (expert, first row inside the expert's segment, rows) triples.
 */
void oracle_route_meta(const int32_t *ids, int T, int k, int E, int BM, int with_shared,
                       int32_t *counts, int32_t *offsets, int32_t *sorted_assign,
                       int32_t *tiles, int32_t *n_tiles)
{
    int64_t n_assign = (int64_t)T * k;
    for (int e = 0; e < E; e++)
        counts[e] = 0;
    for (int64_t a = 0; a < n_assign; a++)
        counts[ids[a]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; e++)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    for (int e = 0; e < E; e++)
        fill[e] = offsets[e];
    for (int64_t a = 0; a < n_assign; a++)
        sorted_assign[fill[ids[a]]++] = (int32_t)a;
    free(fill);
    int32_t n = 0;
    for (int e = 0; e < E; e++) {
        for (int r0 = 0; r0 < counts[e]; r0 += BM) {
            int rows = counts[e] - r0 < BM ? counts[e] - r0 : BM;
            tiles[3 * n + 0] = e;
            tiles[3 * n + 1] = r0;
            tiles[3 * n + 2] = rows;
            n++;
        }
    }
    if (with_shared) {
        for (int r0 = 0; r0 < T; r0 += BM) {
            int rows = T - r0 < BM ? T - r0 : BM;
            tiles[3 * n + 0] = E;
            tiles[3 * n + 1] = r0;
            tiles[3 * n + 2] = rows;
            n++;
        }
    }
    *n_tiles = n;
}

/* One SwiGLU expert on one token, float64: out[H] = Wd (silu(Wg x) * (Wu x)). */
static void oq_expert(const oq_matrix *gate, const oq_matrix *up, const oq_matrix *down,
                      int64_t e, int H, int I, const double *x, double *hbuf, double *out)
{
    for (int n = 0; n < I; n++) {
        double g = 0.0, u = 0.0;
        for (int k = 0; k < H; k++) {
            g += oq_weight(gate, e, I, H, n, k) * x[k];
            u += oq_weight(up, e, I, H, n, k) * x[k];
        }
        hbuf[n] = g / (1.0 + exp(-g)) * u;
    }
    for (int c = 0; c < H; c++) {
        double o = 0.0;
        for (int n = 0; n < I; n++)
            o += oq_weight(down, e, H, I, c, n) * hbuf[n];
        out[c] = o;
    }
}

/*
 * Layer output for a list of tokens, given the routing (ids, weights) of all
 * T tokens: y = sum_j w_j * expert_{id_j}(x) in top-k order, then + shared.
 */
void oracle_ffn_tokens(const oq_layer *L, const uint16_t *x, const int32_t *ids,
                       const float *weights, const int32_t *tokens, int n_tokens, double *y)
{
    int H = L->H, I = L->I, Is = L->Is, k = L->k;
    int hmax = I > Is ? I : Is;
    double *xv = (double *)malloc(sizeof(double) * (size_t)H);
    double *o = (double *)malloc(sizeof(double) * (size_t)H);
    double *hb = (double *)malloc(sizeof(double) * (size_t)(hmax > 0 ? hmax : 1));
    for (int i = 0; i < n_tokens; i++) {
        int64_t t = tokens[i];
        double *yt = y + (int64_t)i * H;
        for (int c = 0; c < H; c++) {
            xv[c] = bf16_value(x[t * H + c]);
            yt[c] = 0.0;
        }
        for (int j = 0; j < k; j++) {
            int32_t e = ids[t * k + j];
            double wj = (double)weights[t * k + j];
            oq_expert(&L->gate, &L->up, &L->down, e, H, I, xv, hb, o);
            for (int c = 0; c < H; c++)
                yt[c] += wj * o[c];
        }
        if (Is > 0) {
            oq_expert(&L->sh_gate, &L->sh_up, &L->sh_down, 0, H, Is, xv, hb, o);
            for (int c = 0; c < H; c++)
                yt[c] += o[c];
        }
    }
    free(xv);
    free(o);
    free(hb);
}
