/*
 * moe.h - C ABI of the MI355X (gfx950) 4-bit group-affine MoE FFN layer.
 *
 * The layer (the "Optimizing on-device inference for Apple Silicon" page):
 *   - a router scores E experts per token and keeps the top k; one shared
 *     expert processes every token (section "Qwen creates three different
 *     workload shapes");
 *   - each expert is a SwiGLU FFN whose weights are 4-bit integer codes, every
 *     64 consecutive weights along the input dimension sharing one bf16 scale
 *     and one bf16 bias that rebuild the weight as w = s*q + b (section
 *     "Dequantise weights during matrix multiplication");
 *   - routing runs on the GPU as top-k, histogram, prefix scan, scatter and a
 *     block map, with no CPU round trip inside the layer (section "Keep
 *     expert routing on the GPU");
 *   - prefill uses a grouped matrix-matrix product over the routed rows;
 *     single-row decode uses a row-parallel matrix-vector product (sections
 *     "Apple silicon provides different paths for different workloads" and
 *     "Optimise the one-row weight path");
 *   - long prompts are processed in bounded chunks (section "Bound temporary
 *     memory with prompt chunking").
 *
 * Conventions shared by every entry point
 *   - All data pointers are DEVICE pointers unless stated otherwise, and are
 *     owned by the caller.  The library allocates no memory in any call and
 *     never reads device memory on the host.
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on `stream` and returns; no call synchronises.
 *   - Argument and shape errors are reported before anything is enqueued, so a
 *     failed call leaves no partial work.  A failed kernel launch returns
 *     MOE_ERR_HIP; faults during execution surface at the caller's next
 *     synchronisation.  moe_last_error() gives a thread-local message for the
 *     last failure.
 *   - T = 0 is a valid no-op returning MOE_OK.
 *   - Calls on different streams are safe given distinct workspaces and
 *     outputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad count, k > E, ... */
    MOE_ERR_UNSUPPORTED_SHAPE = 2,  /* H or I not a multiple of 64, group != 64, sizes over limits */
    MOE_ERR_WORKSPACE_TOO_SMALL = 3,/* ws_bytes or packed_bytes below the required size */
    MOE_ERR_HIP = 4,                /* a HIP runtime call or kernel launch failed */
    MOE_ERR_DEVICE_UNSUPPORTED = 5  /* the current device is not gfx950 */
} moe_status;

/*
 * Supported activation range.  The grouped-GEMM path feeds its MFMAs fp16(x /
 * 256) and fp16(h / 256) (h = silu(gate) * up) and stores each routed expert
 * output as fp16(o / 256): exact scalings, in range while |x|, |h| and |o|
 * stay below 65504 * 256 (about 1.7e7).  h grows with the square of the
 * activations' scale; for this layer's weights that is activations up to a
 * few hundred times N(0, 1).  Beyond that the path gives inf or NaN in y
 * (with MOE_OK); the decode GEMV path keeps h in bf16 hi/lo parts and reaches
 * further.  Inputs must be finite.
 */

/*
 * Layer description.  Limits: hidden and inter multiples of 64 (the group
 * size; the pages' format cannot quantise a width that is not a multiple of
 * the group, cf. the Laya page's quantisation section), hidden <= 8192,
 * inter <= 4096, shared_inter a multiple of 64 or 0, 1 <= top_k <= 16,
 * top_k <= n_experts <= 512.
 */
typedef struct {
    int32_t hidden;        /* H: model width, the input of gate/up and the output of down */
    int32_t n_experts;     /* E: routed experts */
    int32_t top_k;         /* k: experts kept per token */
    int32_t inter;         /* I: routed expert intermediate width */
    int32_t shared_inter;  /* Is: shared expert intermediate width, 0 = no shared expert */
    int32_t group_size;    /* must be 64 */
    int32_t gemv_max_rows; /* R*: moe_forward_decode uses the row-parallel GEMV path for
                              T <= R* and the grouped GEMM path above; -1 = library default
                              (8, or 4 with batch_invariant = 1); 0 = always GEMM; at most 8 */
    int32_t max_chunk;     /* tokens per prefill chunk (1..8192); routing metadata is per chunk */
    int32_t tile_rows;     /* BM: rows per tile of the block map; 0 = library default (128);
                              one of 16, 32, 64, 128 */
    int32_t host_sync_routing; /* 0 (the normal path): routing never returns to the host.  1: a
                              measurement of the alternative the pages argue against ("Keep expert
                              routing on the GPU"): after each chunk's routing, the grouped-GEMM path
                              copies the schedule's entry count to the host, synchronises the stream
                              and sizes the GEMM launches from it.  Same kernels and results; the
                              call then blocks and cannot be captured in a graph. */
    int32_t dequant_pass;  /* 0 (the normal path): weights are rebuilt inside the grouped GEMMs.  1: a
                              measurement of the alternative the pages compare against ("Dequantise
                              weights during matrix multiplication"): each chunk's active experts and
                              the shared expert are first rebuilt as fp16 into the workspace (a
                              separate pass), then the grouped GEMMs read fp16 weights.  Same rounding,
                              same results; the workspace grows by 4096/1152 x the packed size. */
    int32_t batch_invariant; /* 0: the decode GEMV path folds scale and bias per group and splits the
                              down projection (its own rounding).  1: the GEMV path computes every
                              output element with the grouped-GEMM path's operations in the same order
                              (fp16 weights rebuilt as s*q + b, fp16(x / 256), one MFMA chain over K,
                              fp16(h / 256) and fp16(o / 256) intermediates, ranked routing weights,
                              combine in rank order), so a row's output does not depend on the row
                              threshold or on the other rows of the call (the dothoosh page on Candle,
                              its section on outputs that change with the kernel chosen by row count).
                              Costs time: the chain over K runs in order, so one row takes about 26 us
                              instead of 20; the default R* is then 4, above which the grouped GEMM
                              path (same bits) is faster. */
} moe_layer_desc;

/*
 * One quantised matrix stack in the canonical format (device pointers):
 *   codes  [M][N][K/2]  uint8, two codes per byte, the even k in the low nibble
 *   scales [M][N][K/64] bf16 bits
 *   biases [M][N][K/64] bf16 bits
 * with M = E for routed matrices and M = 1 for the shared expert; gate and up
 * have N = inter (or shared_inter), K = hidden; down has N = hidden, K = inter.
 */
typedef struct {
    const uint8_t *codes;
    const uint16_t *scales;
    const uint16_t *biases;
} moe_qmatrix;

/*
 * Routing outputs for one chunk of T tokens (device pointers, caller-owned):
 *   topk_ids       [T][k]  int32, experts in order of decreasing logit
 *   topk_weights   [T][k]  float, softmax over the k selected logits
 *   expert_counts  [E]     int32, assignments per expert (histogram)
 *   expert_offsets [E+1]   int32, exclusive prefix scan of the counts
 *   sorted_assign  [T*k]   int32, flat assignment ids t*k+j grouped by expert,
 *                          increasing inside each expert (stable scatter)
 *   tile_map       [moe_max_tiles][3] int32, (expert, first row inside the
 *                          expert's segment, rows) per BM-row tile, experts in
 *                          increasing order, then the shared expert's tiles as
 *                          expert E over the tokens
 *   n_tiles        [1]     int32, the number of valid tile_map entries
 */
typedef struct {
    int32_t *topk_ids;
    float *topk_weights;
    int32_t *expert_counts;
    int32_t *expert_offsets;
    int32_t *sorted_assign;
    int32_t *tile_map;
    int32_t *n_tiles;
} moe_routing;

/*
 * Size in bytes of the packed weight blob for `desc` (host output): the
 * canonical 4-bit codes plus one bf16 scale and one bf16 bias per 64 weights,
 * 0.5625 bytes per parameter (the Laya page's quantisation section gives this
 * storage cost of the group-64 4-bit format), plus a 256-byte trailer (a flag
 * the packer writes for the kernels).  Host-only; no device access.
 */
moe_status moe_packed_bytes(const moe_layer_desc *desc, size_t *bytes);

/*
 * Workspace bytes needed by moe_route / moe_forward_* for up to max_tokens per
 * call (host output).  The workspace holds one chunk's routing metadata and
 * intermediates; prefill reuses it chunk after chunk, so its size is bounded
 * by max_chunk whatever T is ("Optimizing on-device inference for Apple
 * Silicon", section "Bound temporary memory with prompt chunking").  For
 * max_tokens > max_chunk the size includes a second routing area (about 18 MB
 * at H=2048, E=256, k=8 and 2048-token chunks), with which the forward calls
 * route the next chunk while the current one's GEMMs run; a workspace of the
 * one-chunk size (moe_workspace_bytes(desc, min(T, max_chunk))) is still
 * valid for any T and runs the chunks one after the other.
 * Host-only; no device access.
 */
moe_status moe_workspace_bytes(const moe_layer_desc *desc, int32_t max_tokens, size_t *bytes);

/*
 * Upper bound of the tile_map entries moe_route writes for a chunk of T tokens
 * (host output): the block map of fixed-size tiles per expert (section "Keep
 * expert routing on the GPU" of the same page).  Host-only.
 */
moe_status moe_max_tiles(const moe_layer_desc *desc, int32_t T, int32_t *n);

/*
 * Repack canonical quantised weights into the library's blob (device, size
 * moe_packed_bytes).  The format is the page's: 4-bit codes, every 64 weights
 * along the input dimension sharing one bf16 scale and one bf16 bias, w = s*q
 * + b ("Optimizing on-device inference for Apple Silicon", section
 * "Dequantise weights during matrix multiplication").  The blob is opaque and valid only for the desc that
 * made it.  It stores exactly the canonical codes (0.5625 bytes per parameter
 * with the scales and biases), rearranged so that one 64-lane wave reads a
 * 32-row x 64-column group with one 16-byte load per lane; the scales and
 * biases are stored converted to fp16 (round to nearest even), the type the
 * kernels rebuild weights in.  The conversion is exact for magnitudes in
 * [2^-14, 65504]; smaller values lose bits as fp16 subnormals and larger
 * ones become infinity, so the supported scale and bias range is fp16's.  The
 * blob's last 256 bytes are a trailer whose first int32 the packer sets to 1
 * when every scale is below 2^-4 in magnitude (0 otherwise); the grouped GEMM
 * then rebuilds weights with fewer instructions, to the same bits.  sh_* are ignored when
 * shared_inter == 0.  One-time preparation; not part of the forward path.
 */
moe_status moe_pack_weights(const moe_layer_desc *desc, moe_qmatrix gate, moe_qmatrix up,
                            moe_qmatrix down, moe_qmatrix sh_gate, moe_qmatrix sh_up,
                            moe_qmatrix sh_down, void *packed, size_t packed_bytes, void *stream);

/*
 * Route one chunk of T <= max_chunk tokens on the GPU, with no return to the
 * host ("Optimizing on-device inference for Apple Silicon", section "Keep
 * expert routing on the GPU": top-k, histogram, prefix scan, scatter, block
 * map; section "Qwen creates three different workload shapes": top-8 of 256
 * routed experts plus one shared expert): router logits
 * fp32(sum_h x[t,h]*Wr[e,h] accumulated in float64) + logit_bias[e], top-k,
 * softmax weights, then histogram, prefix scan, stable scatter and block map,
 * all on the GPU.
 *   x          [T][H] bf16
 *   router_w   [E][H] float
 *   logit_bias [E] float or NULL
 *   ws         workspace of at least moe_workspace_bytes(desc, T) bytes
 */
moe_status moe_route(const moe_layer_desc *desc, const uint16_t *x, int32_t T,
                     const float *router_w, const float *logit_bias, const moe_routing *out,
                     void *ws, size_t ws_bytes, void *stream);

/*
 * Full layer over T tokens with the grouped dequantising GEMM path, chunk by
 * chunk (max_chunk tokens each; "Optimizing on-device inference for Apple
 * Silicon", sections "Dequantise weights during matrix multiplication", "Match
 * tile size to expert load", "Reduce intermediate and state traffic" and
 * "Bound temporary memory with prompt chunking"):
 *   y[t] = sum_j topk_weights[t,j] * FFN_{topk_ids[t,j]}(x[t]) + FFN_shared(x[t])
 * with FFN(x) = Wd (silu(Wg x) * (Wu x)).
 *   packed  blob from moe_pack_weights
 *   y       [T][H] float (written, not accumulated)
 *   ws      at least moe_workspace_bytes(desc, min(T, max_chunk)) bytes
 * With more than one chunk and a workspace of moe_workspace_bytes(desc, T)
 * bytes, two chunks are in flight at once: even chunks run on `stream` and odd
 * chunks on a second stream of the library's (one per device, created on first
 * use, default priority), except that the combine of a last odd chunk runs on
 * `stream`.  Events order the two streams, and the call returns with all of its
 * work joined to `stream`, so stream order holds for the caller as with one
 * stream (also under graph capture of `stream`).  The result is the same bits
 * either way.  The second stream and its events are created by the first such
 * call on a device; make that call outside graph capture, as HIP may refuse to
 * create a stream while one is being captured.
 */
moe_status moe_forward_prefill(const moe_layer_desc *desc, const void *packed,
                               const float *router_w, const float *logit_bias,
                               const uint16_t *x, int32_t T, float *y,
                               void *ws, size_t ws_bytes, void *stream);

/*
 * Same layer for a few rows: the row-parallel GEMV path when T <=
 * gemv_max_rows (at most 8), otherwise the grouped GEMM path of
 * moe_forward_prefill (any T, chunked the same way).  The pages' one-row
 * weight path ("Optimizing on-device inference for Apple Silicon", section
 * "Optimise the one-row weight path") and the choice of kernel by row count
 * (the dothoosh page on Candle's Metal kernels, its kernel-selection and
 * crossover sections).
 * The GEMV path is three launches: exact router logits; top-k, gate/up +
 * SwiGLU and the down projection of each workgroup's 32 intermediate columns
 * (partial output rows in the workspace); the sum of each token's partials in
 * a fixed order.  y is written once per element, with no atomics, so repeated
 * calls give identical bits.  With batch_invariant = 1 the GEMV path is
 * instead: exact router logits; top-k, gate/up + SwiGLU into fp16 rows of h;
 * down projection and combine, with the grouped GEMM path's operations, so
 * its output equals that path's bit for bit at every T.
 */
moe_status moe_forward_decode(const moe_layer_desc *desc, const void *packed,
                              const float *router_w, const float *logit_bias,
                              const uint16_t *x, int32_t T, float *y,
                              void *ws, size_t ws_bytes, void *stream);

/*
 * moe_forward_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, kernels and results as
 * moe_forward_decode, whose workspace is here a fixed device array of
 * MOE_STATIC_SCRATCH_BYTES inside the library; each GPU the library runs on
 * holds its own copy until the process ends.  The call allocates and frees
 * nothing (its first call on a device looks the array's address up once).
 * Limits and errors:
 *   - MOE_ERR_WORKSPACE_TOO_SMALL when the layer's decode workspace at this T
 *     exceeds MOE_STATIC_SCRATCH_BYTES (moe_workspace_bytes(desc, T) tells);
 *     16 MiB hold T <= 8 at H=2048, E=256, k=8, I=Is=512 (9.2 MiB);
 *   - MOE_ERR_INVALID_ARGUMENT for host_sync_routing or dequant_pass set.
 * Every call on one GPU uses the same array: calls that overlap in time on
 * one GPU (other streams, other threads) race and give undefined results;
 * serialise them.  Stream-ordered calls on one stream are safe.
 */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
moe_status moe_forward_decode_static(const moe_layer_desc *desc, const void *packed,
                                     const float *router_w, const float *logit_bias,
                                     const uint16_t *x, int32_t T, float *y, void *stream);

/* Default R* of the library with batch_invariant = 0 (host output); with
 * batch_invariant = 1 the default is 4. */
int32_t moe_default_gemv_max_rows(void);

const char *moe_status_str(moe_status s);
const char *moe_last_error(void);

/*
 * Kernel timing for measurement tools.  moe_profile_enable(mask) makes every
 * launch of the kernels whose bit is set in `mask` (bit i = kernel id i; 0
 * turns timing off) stamp a HIP event pair on the launch stream: the first
 * kernel of the step stamps its own start and the last its own end
 * (hipExtLaunchKernel).  A stamped launch costs a few microseconds more than
 * a plain one, so time whole steps with timing off.  moe_profile_read
 * synchronises on those events and returns the summed duration (ms) and
 * launch count of kernel `kernel_id` since the last reset.  Never needed on
 * the forward path.  Not thread-safe.
 *   0 = router logits (screen, or exact for T <= 8), 1 = exact top-k
 *   selection (T > 8), 2 = routing metadata (with top-k for T <= 8 outside
 *   the decode GEMV path), 3 = gate/up grouped GEMM, 4 = down grouped GEMM,
 *   5 = top-k + gate/up GEMV + split down GEMV (decode GEMV path), 6 = sum of
 *   the decode path's partial outputs, 7 = per-token combine of the
 *   grouped-GEMM path, 8 = separate dequant pass (dequant_pass = 1)
 */
moe_status moe_profile_enable(int32_t mask);
moe_status moe_profile_reset(void);
moe_status moe_profile_read(int32_t kernel_id, double *total_ms, int32_t *launches);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
