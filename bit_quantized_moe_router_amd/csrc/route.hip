// GPU-resident routing ("Optimizing on-device inference for Apple Silicon",
// section "Keep expert routing on the GPU"): router logits, top-k with
// renormalised softmax weights, then the expert histogram, prefix scan,
// stable scatter and block map.  Everything stays on the device; the host
// never reads any of it.
//
// Precision contract of the logits: every product x[t,h] * Wr[e,h] (bf16 x
// fp32) is exact in float64, the sum is accumulated in float64, rounded once
// to float32, and the float32 logit bias is added in float32.  Top-k compares
// those float32 logits, larger first, equal logits towards the lower expert.
//
// Two routes reach that contract:
//  * few tokens (decode): every logit in float64 directly (k_logits_small);
//  * many tokens (prefill): a bf16 MFMA screen of all logits (k_screen), then
//    per token an exact float64 recomputation of only the experts whose
//    screened logit lies within twice a rigorous error bound of the k-th
//    largest screened logit (k_route_exact).  Any expert of the exact top-k
//    is inside that window, so the selection equals the all-float64 one.
#include "launch.h"
#include "small_route.h"

namespace moe {

constexpr int kMaxTileRows = 128;

// ---------------------------------------------------------------------------
// Few tokens: all T x E logits in float64.  One single-wave workgroup per
// expert (the router rows spread over every compute unit), lanes split h in
// 16-byte slices of the router row.  When asked (non-null), the grid also
// writes the per-group activation sums and the fp16 activation copy, each
// thread taking a strided share.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_logits_small(const uint16_t* __restrict__ x, int T, int H,
                                                     const float* __restrict__ wr,
                                                     const float* __restrict__ bias, int E,
                                                     float* __restrict__ logits,
                                                     float* __restrict__ xsum,
                                                     uint16_t* __restrict__ x16) {
  const int e = blockIdx.x;
  const int gt = blockIdx.x * 64 + threadIdx.x, gn = gridDim.x * 64;
  if (xsum) group_sums(x, T, H, xsum, gt, gn);
  if (x16) {
    for (int i = gt; i < T * H; i += gn) x16[i] = f32_to_f16_scaled(x[i]);
  }
  if (e < E) logits_one_expert(x, T, H, wr, bias, E, e, logits);
}

// ---------------------------------------------------------------------------
// Many tokens, step 1: screened logits.  Each router weight w (fp32) is split
// into hi = bf16(w) and lo = bf16(w - hi) (w - hi is exact in fp32, and
// |w - hi - lo| <= 2^-17 |w|); a = sum_h x*hi + x*lo with
// v_mfma_f32_32x32x16_bf16 (bf16 x bf16 products exact in fp32, fp32
// accumulation), split over kScreenSplit slices of h, each slice writing its
// partial sums.  Workgroup tile 64 tokens x 64 experts, four 32x32 waves; per
// 64-wide group the workgroup stages x and the hi/lo weights in LDS (double
// buffered, loads two groups ahead).  The workgroups of the first token tile
// also write the per-slice sums of w^2 (float64) for the error bound.
// ---------------------------------------------------------------------------
constexpr int kScreenSplit = 4;
constexpr int kScrRow = 144;                   // LDS bytes per row of one group: 64 bf16 + pad
constexpr int kScrBuf = 64 * kScrRow;          // one 64-row tile of one group
constexpr int kScrSmem = 2 * 3 * kScrBuf;      // x, hi, lo; double buffered

// LDS bytes of one k_route_exact workgroup: reduction slots, x row (float64),
// screened logits, candidate experts and logits (E each), selected logits (16).
__host__ __device__ constexpr int route_exact_smem_bytes(int H, int E) { return 256 + H * 8 + E * 12 + 64; }


__global__ __launch_bounds__(256) void k_screen(const uint16_t* __restrict__ x, int T, int H,
                                                const float* __restrict__ wr, int E,
                                                float* __restrict__ approx, double* __restrict__ wsq,
                                                int32_t* __restrict__ segcnt, int n_segcnt) {
  __shared__ __attribute__((aligned(16))) uint8_t sm[kScrSmem];
  const int tid = threadIdx.x;
  // The per-segment expert counters that k_route_exact fills start at zero.
  if (segcnt && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int i = tid; i < n_segcnt; i += 256) segcnt[i] = 0;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, c32 = lane & 31;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int G = H / kGroup;
  const int gs = blockIdx.z, g0 = G * gs / kScreenSplit, g1 = G * (gs + 1) / kScreenSplit;
  const bool norms = blockIdx.x == 0;

  // Staging: x pieces (row tid/8 and tid/8 + 32, 16-byte part tid%8); weight
  // float4s (rows tid/16 + 16 i, i < 4, part tid%16).  Rows past T or E
  // reload a valid row whose results are never stored.
  const int xp = tid & 7, xr0 = tid >> 3;
  const uint16_t* xs0 = x + (int64_t)min(t0 + xr0, T - 1) * H + xp * 8;
  const uint16_t* xs1 = x + (int64_t)min(t0 + xr0 + 32, T - 1) * H + xp * 8;
  const int wp = tid & 15, wr0 = tid >> 4;
  const float* ws0 = wr + (int64_t)min(e0 + wr0, E - 1) * H + wp * 4;
  const float* ws1 = wr + (int64_t)min(e0 + wr0 + 16, E - 1) * H + wp * 4;
  const float* ws2 = wr + (int64_t)min(e0 + wr0 + 32, E - 1) * H + wp * 4;
  const float* ws3 = wr + (int64_t)min(e0 + wr0 + 48, E - 1) * H + wp * 4;
  double ss0 = 0.0, ss1 = 0.0, ss2 = 0.0, ss3 = 0.0;

  // One register set of staged data: x pieces X0, X1 and weight float4s W0..W3.
#define MOE_SCR_LOAD(g, S)                                                        \
  do {                                                                            \
    const int gg_ = (g) < g1 ? (g) : g1 - 1;                                      \
    S##x0 = *reinterpret_cast<const uint4*>(xs0 + gg_ * kGroup);                  \
    S##x1 = *reinterpret_cast<const uint4*>(xs1 + gg_ * kGroup);                  \
    S##w0 = *reinterpret_cast<const float4*>(ws0 + gg_ * kGroup);                 \
    S##w1 = *reinterpret_cast<const float4*>(ws1 + gg_ * kGroup);                 \
    S##w2 = *reinterpret_cast<const float4*>(ws2 + gg_ * kGroup);                 \
    S##w3 = *reinterpret_cast<const float4*>(ws3 + gg_ * kGroup);                 \
  } while (0)
  auto stage_w = [&](const float4 w, int row, uint8_t* xb, double& ss) {
    const __bf16 h0 = (__bf16)w.x, h1 = (__bf16)w.y, h2 = (__bf16)w.z, h3 = (__bf16)w.w;
    const __bf16 l0 = (__bf16)(w.x - (float)h0), l1 = (__bf16)(w.y - (float)h1);
    const __bf16 l2 = (__bf16)(w.z - (float)h2), l3 = (__bf16)(w.w - (float)h3);
    const int off = row * kScrRow + wp * 8;
    *reinterpret_cast<uint2*>(xb + kScrBuf + off) =
        make_uint2(__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16),
                   __builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16));
    *reinterpret_cast<uint2*>(xb + 2 * kScrBuf + off) =
        make_uint2(__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16),
                   __builtin_bit_cast(uint16_t, l2) | ((uint32_t)__builtin_bit_cast(uint16_t, l3) << 16));
    if (norms) {
      ss = fma((double)w.x, (double)w.x, ss);
      ss = fma((double)w.y, (double)w.y, ss);
      ss = fma((double)w.z, (double)w.z, ss);
      ss = fma((double)w.w, (double)w.w, ss);
    }
  };
#define MOE_SCR_STAGE(S, buf)                                                     \
  do {                                                                            \
    uint8_t* xb_ = sm + (buf) * 3 * kScrBuf;                                      \
    *reinterpret_cast<uint4*>(xb_ + xr0 * kScrRow + xp * 16) = S##x0;             \
    *reinterpret_cast<uint4*>(xb_ + (xr0 + 32) * kScrRow + xp * 16) = S##x1;      \
    stage_w(S##w0, wr0, xb_, ss0);                                                \
    stage_w(S##w1, wr0 + 16, xb_, ss1);                                           \
    stage_w(S##w2, wr0 + 32, xb_, ss2);                                           \
    stage_w(S##w3, wr0 + 48, xb_, ss3);                                           \
  } while (0)
  f32x16_t acc = {};
  // k-slot j of MFMA c for lane half h carries column 32h + 8c + j of the group (A and B alike).
  const int aoff = (wm * 32 + c32) * kScrRow + h * 64, boff = (wn * 32 + c32) * kScrRow + h * 64;
  auto compute = [&](int buf) {
    const uint8_t* xb = sm + buf * 3 * kScrBuf;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(xb + aoff + c * 16);
      const bf16x8_t bh = *reinterpret_cast<const bf16x8_t*>(xb + kScrBuf + boff + c * 16);
      const bf16x8_t bl = *reinterpret_cast<const bf16x8_t*>(xb + 2 * kScrBuf + boff + c * 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bl, acc, 0, 0, 0);
    }
  };

  const int n = g1 - g0;  // groups of this slice (may be 0 for tiny H)
  if (n > 0) {
    uint4 ax0, ax1, bx0, bx1;
    float4 aw0, aw1, aw2, aw3, bw0, bw1, bw2, bw3;
    MOE_SCR_LOAD(g0, a);
    MOE_SCR_LOAD(g0 + 1, b);
    MOE_SCR_STAGE(a, 0);
    MOE_SCR_LOAD(g0 + 2, a);
    __syncthreads();
    for (int r = 0; r < n; r += 2) {
      compute(0);
      if (r + 1 < n) MOE_SCR_STAGE(b, 1);  // workgroup-uniform condition
      MOE_SCR_LOAD(g0 + r + 3, b);
      __syncthreads();
      if (r + 1 >= n) break;
      compute(1);
      if (r + 2 < n) MOE_SCR_STAGE(a, 0);
      MOE_SCR_LOAD(g0 + r + 4, a);
      __syncthreads();
    }
  }
#undef MOE_SCR_LOAD
#undef MOE_SCR_STAGE

  float* out = approx + (int64_t)gs * T * E;
  const int e = e0 + wn * 32 + c32;
  if (e < E) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int tok = t0 + wm * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
      if (tok < T) out[(int64_t)tok * E + e] = acc[i];
    }
  }
  if (norms) {
    const double sv[4] = {ss0, ss1, ss2, ss3};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const double v = row_sum16(sv[i]);  // the 16 threads of a weight row are one row of lanes
      const int ee = e0 + wr0 + 16 * i;
      if (wp == 0 && ee < E) wsq[gs * E + ee] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Many tokens, step 2: one workgroup per token.  With S = sum_h x w (exact),
// the screened logit a = fp32(sum over slices in float64 + bias) and the
// exact logit l = fp32(fp32(S) + bias) differ by at most
//   B = (2^-17 + (n + 32) 2^-24 + 2^-23) |x|_2 max_e |w_e|_2 + 2^-22 (max|a| + 1),
// taken with a 2^-10 relative margin, where n = 2 x (products of the longest
// slice) = 128 ceil(G / kScreenSplit) (1024 at H = 2048):
//  * |w - hi - lo| <= 2^-17 |w| (bf16 rounding of w, then of the exact rest);
//  * each slice accumulates its hi and lo products, all exact, in fp32: at
//    most n roundings of 2^-24 relative to sum |x||w| over the slice, and by
//    Cauchy-Schwarz the slices together stay below n 2^-24 |x|_2 |w_e|_2 (the
//    32 covers the higher-order terms);
//  * the slices and the bias are summed in float64 (error negligible, covered
//    by the rounding of the result to fp32, 2^-24 |a|);
//  * the exact logit carries two fp32 roundings (2^-24 |S| and 2^-24 |l|).
// Every expert of the exact top-k has a >= a_k - 2 B for any a_k not above
// the k-th largest screened logit (here the k-th largest of the per-lane
// maxima), so only those experts are recomputed in float64 (one per half
// wave) and the exact top-k is taken among them by rank.
// Also writes the fp16 activation copy of the grouped GEMM.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_route_exact(const uint16_t* __restrict__ x, int T, int H,
                                                     const float* __restrict__ wr,
                                                     const float* __restrict__ bias, int E, int k,
                                                     const float* __restrict__ approx,
                                                     const double* __restrict__ wsq,
                                                     int32_t* __restrict__ ids, float* __restrict__ tw,
                                                     uint16_t* __restrict__ x16, int32_t* __restrict__ segcnt) {
  // One workgroup per token.  LDS: reduction slots, x row, screened logits,
  // candidate experts and their exact logits, selected logits.
  extern __shared__ __attribute__((aligned(16))) uint8_t rsm[];
  __shared__ int s_C;
  const int t = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  double* red = reinterpret_cast<double*>(rsm);                 // [4 waves][3]
  double* xl = reinterpret_cast<double*>(rsm + 256);             // x row, widened once for every candidate
  float* av = reinterpret_cast<float*>(rsm + 256 + H * 8);
  int* cand_e = reinterpret_cast<int*>(av + E);
  float* cand_v = reinterpret_cast<float*>(cand_e + E);
  float* sel_v = cand_v + E;
  const uint16_t* xr = x + (int64_t)t * H;

  // ---- x row (LDS copy, fp16 copy, |x|^2) and the screened
  // logits (slices and bias summed in float64, rounded once); all loads are
  // independent of each other ----
  constexpr int kMaxXIter = 4;  // H <= 8192
  uint4 xv[kMaxXIter];
#pragma unroll
  for (int i = 0; i < kMaxXIter; i++) {
    const int h = 8 * tid + 2048 * i;
    if (h < H) xv[i] = *reinterpret_cast<const uint4*>(xr + h);
  }
  float amax = 0.f;
  double w2max = 0.0;
  for (int e = tid; e < E; e += 256) {
    double vd = (double)approx[(int64_t)t * E + e];
    double w2 = wsq[e];
#pragma unroll
    for (int s = 1; s < kScreenSplit; s++) {
      vd += (double)approx[(int64_t)s * T * E + (int64_t)t * E + e];
      w2 += wsq[s * E + e];
    }
    if (bias) vd += (double)bias[e];
    const float v = (float)vd;
    av[e] = v;
    amax = fmaxf(amax, fabsf(v));
    w2max = fmax(w2max, w2);
  }
  double xx = 0.0;
#pragma unroll
  for (int i = 0; i < kMaxXIter; i++) {
    const int h = 8 * tid + 2048 * i;
    if (h < H) {  // H is a multiple of 64: a group of 8 threads is all in or all out
      const uint4 v = xv[i];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t c[4];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        c[j] = f32_to_f16_scaled(w[j] & 0xFFFFu) | ((uint32_t)f32_to_f16_scaled(w[j] >> 16) << 16);
        const double f0 = (double)bf16_bits_to_f32(w[j] & 0xFFFFu), f1 = (double)bf16_bits_to_f32(w[j] >> 16);
        *reinterpret_cast<double2*>(xl + h + 2 * j) = make_double2(f0, f1);
        xx = fma(f0, f0, xx);
        xx = fma(f1, f1, xx);
      }
      *reinterpret_cast<uint4*>(x16 + (int64_t)t * H + h) = make_uint4(c[0], c[1], c[2], c[3]);
    }
  }
  xx = wave_sum_f64(xx);
  amax = wave_max_f32(amax);
  w2max = wave_max_f64(w2max);
  if (lane == 0) {
    red[3 * wave + 0] = xx;
    red[3 * wave + 1] = (double)amax;
    red[3 * wave + 2] = w2max;
  }
  __syncthreads();

  // ---- wave 0: k-th largest screened logit, error bound, candidate list ----
  if (wave == 0) {
    xx = red[0] + red[3] + red[6] + red[9];
    const double amx = fmax(fmax(red[1], red[4]), fmax(red[7], red[10]));
    const double w2m = fmax(fmax(red[2], red[5]), fmax(red[8], red[11]));
    const double xnorm = sqrt(xx) * (1.0 + 1e-6);
    float a[kMaxEPerLane];
    bool alive[kMaxEPerLane];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMaxEPerLane; j++) {
      const int e = lane + 64 * j;
      alive[j] = e < E;
      a[j] = alive[j] ? av[e] : 0.f;
      if (alive[j]) m = fmaxf(m, a[j]);
    }
    // Lower bound of the k-th largest screened logit: the k-th largest of the
    // lanes' maxima (those are k distinct logits, all at least that large).
    const float ak = wave_kth_largest(m, k);
    const int G = H / kGroup;
    const double n_round = 128.0 * (double)((G + kScreenSplit - 1) / kScreenSplit);
    const double c1 = 7.62939453125e-06 + (n_round + 32.0) * 5.9604644775390625e-08 + 1.1920928955078125e-07;
    const double B = (c1 * xnorm * (sqrt(w2m) * (1.0 + 1e-6)) + 2.384185791015625e-07 * (amx + 1.0)) *
                     (1.0 + 0.0009765625);
    const double lo = (double)ak - 2.0 * B;
    // Candidate list in increasing expert order.
    int C = 0;
#pragma unroll
    for (int j = 0; j < kMaxEPerLane; j++) {
      const bool cand = alive[j] && (double)a[j] >= lo;
      const uint64_t m = __ballot(cand);
      if (cand) cand_e[C + __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))))] = lane + 64 * j;
      C += __popcll(m);
    }
    if (lane == 0) s_C = C;
  }
  __syncthreads();

  // ---- exact float64 logits of the candidates, one per half-wave ----
  const int C = s_C;
  const int hw = tid >> 5, l32 = tid & 31;
  for (int c = hw; c < C; c += 8) {
    const int e = cand_e[c];
    const float* wrow = wr + (int64_t)e * H;
    double acc = 0.0;
#pragma unroll 16
    for (int h = 4 * l32; h < H; h += 128) {
      const float4 w4 = *reinterpret_cast<const float4*>(wrow + h);
      const double2 x01 = *reinterpret_cast<const double2*>(xl + h);
      const double2 x23 = *reinterpret_cast<const double2*>(xl + h + 2);
      acc = fma(x01.x, (double)w4.x, acc);
      acc = fma(x01.y, (double)w4.y, acc);
      acc = fma(x23.x, (double)w4.z, acc);
      acc = fma(x23.y, (double)w4.w, acc);
    }
    // Half-wave sum: the two rows of lanes of this half, (row sum) + (row sum).
    // Rows belong to one half whole, so the other half may be inactive here.
    acc = row_sum16(acc);
    const double r0 = lane_value_f64(acc, 0), r1 = lane_value_f64(acc, 16);
    const double r2 = lane_value_f64(acc, 32), r3 = lane_value_f64(acc, 48);
    acc = lane < 32 ? r0 + r1 : r2 + r3;
    float lg = (float)acc;
    if (bias) lg = lg + bias[e];
    if (l32 == 0) cand_v[c] = lg;
  }
  __syncthreads();

  // ---- wave 0: exact top-k by rank (a candidate ranks below every other
  // with a larger logit, or an equal logit and a lower expert index), then
  // the softmax over the selected logits ----
  if (wave != 0) return;
  for (int c = lane; c < C; c += 64) {
    const float vc = cand_v[c];
    const int ec = cand_e[c];
    int rank = 0;
    if (C <= 64) {  // every candidate in a lane: the others broadcast with v_readlane
      for (int c2 = 0; c2 < C; c2++) {
        const float v2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, vc), c2));
        const int e2 = __builtin_amdgcn_readlane(ec, c2);
        rank += (v2 > vc || (v2 == vc && e2 < ec)) ? 1 : 0;
      }
    } else {
      for (int c2 = 0; c2 < C; c2++) {
        const float v2 = cand_v[c2];
        rank += (v2 > vc || (v2 == vc && cand_e[c2] < ec)) ? 1 : 0;
      }
    }
    if (rank < k) {
      ids[(int64_t)t * k + rank] = ec;
      sel_v[rank] = vc;
      // Expert histogram of the assignment's segment (the routing metadata's
      // first step, taken here instead of in a launch of its own).
      if (segcnt) atomicAdd(&segcnt[(((int64_t)t * k + rank) / kSegAssign) * E + ec], 1);
    }
  }
  __builtin_amdgcn_wave_barrier();
  const float myv = lane < k ? sel_v[lane] : 0.f;
  const float vmax = lane_value(myv, 0);
  const float ex = lane < k ? __expf(myv - vmax) : 0.f;
  const float sum = wave_sum_f32(ex);  // the sum topk_small takes, so both give the same weights
  if (lane < k) tw[(int64_t)t * k + lane] = ex / sum;
}

// ---------------------------------------------------------------------------
// Routing metadata for one chunk, one workgroup of 1024 threads (16 waves).
// The flat assignment range [0, T*k) is cut into 16 contiguous segments, one
// per wave, walked 64 assignments (one chunk) at a time.  Inside a chunk the
// lanes holding the same expert find each other with ballots on the expert id
// bits; the lowest such lane (the leader) stands for the group.
//  Phase 1: the leaders add their group sizes to per-(wave, expert) LDS
//           counters.
//  Phase 2: wave-level scans over the experts give counts, offsets, the
//           active list and the tile counts; the per-wave counters become
//           per-wave bases; tiles are written one per thread.
//  Phase 3: per chunk, each leader takes its group's base with one LDS
//           atomic add that returns the old counter (all chunks' atomics of a
//           batch are issued in order before any result is used), and the
//           lanes place their assignments at base + rank in the group.
// The scatter is therefore stable in flat id without any global atomics.
// ---------------------------------------------------------------------------
constexpr int kMetaWaves = 16;
constexpr int kMetaBatch = 8;   // chunks per wave whose ids are loaded together

// Scans over the experts given each expert's assignment count (thread e < E
// holds tot for expert e; every thread of the 1024-thread workgroup calls
// this): counts, offsets, active list, tile map and execution schedule.
// Returns thread e's offset (its expert's first sorted position).
__device__ __forceinline__ int meta_scan_tiles(int tot, int T, int k, int E, int BM, int with_shared, int max_long, bool out,
                               int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                               int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles,
                               int32_t* __restrict__ active, int32_t* __restrict__ n_active,
                               int32_t* __restrict__ sched) {
  __shared__ int s_incl[4][kMaxE];         // inclusive scans: rows, tiles, active, full tiles
  __shared__ int s_wtot[kMaxE / 64][2];    // per-wave totals of the two packed scans
  __shared__ int s_nfull;                  // entries of the full-tile bin
  __shared__ int s_pbin[kMaxTileRows + 1]; // schedule entries per row count, then their next slots
  __shared__ int s_keep[kMaxTileRows + 1]; // long tiles per row count that stay whole
  __shared__ int s_extra[kMaxTileRows + 1];// pieces of cut tiles per row count
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i <= BM; i += blockDim.x) s_pbin[i] = s_keep[i] = s_extra[i] = 0;
  int nt = 0, act = 0, nfull = 0, npart = 0;
  if (tid < E) {
    nt = (tot + BM - 1) / BM;
    act = tot > 0 ? 1 : 0;
    nfull = tot / BM;
    npart = nt - nfull;
  }
  const int nwe = (E + 63) / 64;  // waves that cover the experts
  // Two packed scans carry the four: rows | active << 18 (rows <= 8192 * 16 =
  // 2^17, active <= 512) and tiles | full tiles << 16 (each <= 8192 + 512),
  // so no field's sum reaches the next field.
  int sc[2] = {tot | (act << 18), nt | (nfull << 16)};
  if (wave < nwe) {
#pragma unroll
    for (int q = 0; q < 2; q++) sc[q] = wave_incl_scan(sc[q]);
    if (lane == 63) {
#pragma unroll
      for (int q = 0; q < 2; q++) s_wtot[wave][q] = sc[q];
    }
  }
  __syncthreads();
  if (tid < E) {
    int base0 = 0, base1 = 0;
    for (int w = 0; w < wave; w++) {
      base0 += s_wtot[w][0];
      base1 += s_wtot[w][1];
    }
    const int v0 = sc[0] + base0, v1 = sc[1] + base1;
    s_incl[0][tid] = v0 & ((1 << 18) - 1);
    s_incl[2][tid] = v0 >> 18;
    s_incl[1][tid] = v1 & 0xFFFF;
    s_incl[3][tid] = v1 >> 16;
  }
  __syncthreads();
  const int routed_tiles = s_incl[1][E - 1];
  int my_off = 0;
  if (tid < E) my_off = s_incl[0][tid] - tot;
  if (!out) return my_off;  // workgroup-uniform: offsets only, nothing written
  if (tid < E) {
    const int off_e = my_off;
    counts[tid] = tot;
    offsets[tid] = off_e;
    if (tid == E - 1) offsets[E] = s_incl[0][tid];
    if (act) active[s_incl[2][tid] - 1] = tid;
  }
  // Schedule (execution order of the GEMM workgroups): tiles by row count,
  // largest first, so that the longest work starts first.  A tile of more
  // than BM/2 rows is long; at most max_long of them stay whole (one round of
  // the device's compute units), the others are cut into a BM/2-row piece and
  // the rest, so that no long tile starts after the first round.  Each entry
  // holds (expert, first row, rows, first row in sorted order); entry 0 holds
  // the number of entries.  The GEMMs run entry s on XCD s % 8, so the full
  // tiles that stay whole are placed in expert order as 8 contiguous runs,
  // run x on the entries of XCD x: the row tiles of a large expert then share
  // one XCD's L2 and its weights are fetched there once, not once per XCD.
  // The order among other pieces of equal size is arbitrary; no order changes
  // a result.
  const int sfull = with_shared ? T / BM : 0;
  const int spart = with_shared && T % BM ? T % BM : 0;  // rows of the shared expert's partial tile
  const int half = (sched && max_long > 0 && BM >= 64) ? BM / 2 : 0;
  if (tid < E && nfull) atomicAdd(&s_pbin[BM], nfull);
  if (tid < E && npart) atomicAdd(&s_pbin[tot % BM], 1);
  if (tid == 0 && sfull) atomicAdd(&s_pbin[BM], sfull);
  if (tid == 0 && spart) atomicAdd(&s_pbin[spart], 1);
  __syncthreads();
  if (wave == 0) {
    // Wave 0 over the bins in decreasing row count: lane l has r = BM - l and
    // BM - 64 - l (BM <= 128; r < 1 is no bin).  Long bins keep tiles up to
    // max_long counted from the largest; the cut ones add a BM/2 piece and a
    // rest piece.
    const int ra = BM - lane, rb = BM - 64 - lane;
    const int ca = ra >= 1 ? s_pbin[ra] : 0, cb = rb >= 1 ? s_pbin[rb] : 0;
    int fa = ca, fb = cb;
    if (half) {
      const int la = ra > half ? ca : 0, lb = rb > half ? cb : 0;
      const int ia = wave_incl_scan(la), ib = wave_incl_scan(lb);
      const int ta = lane_value(ia, 63);
      const int ka = ra > half ? min(ca, max(max_long - (ia - la), 0)) : 0;
      const int kb = rb > half ? min(cb, max(max_long - (ta + ib - lb), 0)) : 0;
      if (ra > half) {
        s_keep[ra] = ka;
        fa = ka;
        if (ca > ka) atomicAdd(&s_extra[ra - half], ca - ka);
      }
      if (rb > half) {
        s_keep[rb] = kb;
        fb = kb;
        if (cb > kb) atomicAdd(&s_extra[rb - half], cb - kb);
      }
      const int cut = wave_sum_i32((ra > half ? ca - ka : 0) + (rb > half ? cb - kb : 0));
      if (lane == 0) atomicAdd(&s_extra[half], cut);
      __builtin_amdgcn_wave_barrier();
      fa += ra >= 1 && ra <= half ? s_extra[ra] : 0;
      fb += rb >= 1 && rb <= half ? s_extra[rb] : 0;
    }
    // First entry of each bin: 1 + the entries of all larger bins.
    const int ia = wave_incl_scan(fa), ib = wave_incl_scan(fb);
    const int ta = lane_value(ia, 63), tb = lane_value(ib, 63);
    if (ra >= 1) s_pbin[ra] = 1 + ia - fa;
    if (rb >= 1) s_pbin[rb] = 1 + ta + ib - fb;
    if (lane == 0) s_nfull = fa;  // ra = BM: the full tiles kept whole
    if (lane == 0 && sched) reinterpret_cast<int4*>(sched)[0] = make_int4(ta + tb, 0, 0, 0);
  }
  __syncthreads();
  // Full tiles kept whole: the bin's entries [b0, b0 + n) as 8 runs, run i
  // holding entries b0 + i + 8 j for j < n / 8 + (i < n % 8) (so each run is
  // one XCD's, residue b0 + i mod 8) and, in expert order, the full tiles
  // q = i n/8 + min(i, n%8) + j.  The other tiles go through the bins' LDS
  // counters.
  auto place = [&](int e, int r0, int rows, int rb, int q) {
    int4* sc = reinterpret_cast<int4*>(sched);
    if (rows == BM && q < s_nfull) {
      const int b0 = s_pbin[BM] - 1, n = s_nfull, a = n >> 3, b = n & 7;
      int i = 0;  // the run of q: run x starts at q = x a + min(x, b)
#pragma unroll
      for (int x = 1; x < 8; x++) i += q >= x * a + min(x, b) ? 1 : 0;
      sc[1 + b0 + i + 8 * (q - i * a - min(i, b))] = make_int4(e, r0, rows, rb);
    } else if (half && rows > half && (rows == BM || atomicSub(&s_keep[rows], 1) <= 0)) {
      sc[atomicAdd(&s_pbin[half], 1)] = make_int4(e, r0, half, rb);
      sc[atomicAdd(&s_pbin[rows - half], 1)] = make_int4(e, r0 + half, rows - half, rb + half);
    } else {
      sc[atomicAdd(&s_pbin[rows], 1)] = make_int4(e, r0, rows, rb);
    }
  };
  for (int j = tid; j < routed_tiles; j += blockDim.x) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_incl[1][mid] > j) hi = mid;
      else lo = mid + 1;
    }
    const int e = lo;
    const int nt_e = s_incl[1][e] - (e ? s_incl[1][e - 1] : 0);
    const int tot_e = s_incl[0][e] - (e ? s_incl[0][e - 1] : 0);
    const int off_e = s_incl[0][e] - tot_e;
    const int r = j - (s_incl[1][e] - nt_e);
    const int rows = min(BM, tot_e - r * BM);
    tiles[3 * j + 0] = e;
    tiles[3 * j + 1] = r * BM;
    tiles[3 * j + 2] = rows;
    if (sched) place(e, r * BM, rows, off_e + r * BM, (e ? s_incl[3][e - 1] : 0) + r);
  }
  const int nshared = with_shared ? (T + BM - 1) / BM : 0;
  for (int r = tid; r < nshared; r += blockDim.x) {
    const int rows = min(BM, T - r * BM);
    tiles[3 * (routed_tiles + r) + 0] = E;
    tiles[3 * (routed_tiles + r) + 1] = r * BM;
    tiles[3 * (routed_tiles + r) + 2] = rows;
    if (sched) place(E, r * BM, rows, T * k + r * BM, s_incl[3][E - 1] + r);
  }
  if (tid == 0) {
    n_tiles[0] = routed_tiles + nshared;
    n_active[0] = s_incl[2][E - 1];
  }
  __syncthreads();
  return my_off;
}

// cnt: caller's LDS, kMetaWaves * E ints ([wave][expert]: counts, then bases).
__device__ void meta_body(const int32_t* __restrict__ ids, int T, int k, int E, int BM, int with_shared, int max_long,
                          int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                          int32_t* __restrict__ sorted, int32_t* __restrict__ tiles,
                          int32_t* __restrict__ n_tiles, int32_t* __restrict__ active,
                          int32_t* __restrict__ n_active, int32_t* __restrict__ inv,
                          int32_t* __restrict__ sched, int* __restrict__ cnt) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int N = T * k;
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  for (int i = tid; i < kMetaWaves * E; i += blockDim.x) cnt[i] = 0;
  __syncthreads();

  const int S = (N + kMetaWaves - 1) / kMetaWaves;
  const int seg0 = min(N, wave * S), seg1 = min(N, seg0 + S);
  const int nch = (seg1 - seg0 + 63) / 64;

  // ---- phase 1: per-(wave, expert) counts ----
  for (int c0 = 0; c0 < nch; c0 += kMetaBatch) {
    int ev[kMetaBatch];
#pragma unroll
    for (int i = 0; i < kMetaBatch; i++) {
      const int a = seg0 + 64 * (c0 + i) + lane;
      ev[i] = (c0 + i < nch && a < seg1) ? ids[a] : -1;
    }
#pragma unroll
    for (int i = 0; i < kMetaBatch; i++) {
      if (c0 + i < nch) {  // wave-uniform
        const bool valid = ev[i] >= 0;
        const uint64_t m = match_mask(valid ? ev[i] : 0, valid, nbits);
        if (valid && (m & lt_mask) == 0) atomicAdd(&cnt[wave * E + ev[i]], __popcll(m));
      }
    }
  }
  __syncthreads();

  // ---- phase 2: scans over experts, tiles; per-wave counters -> bases ----
  int tot = 0;
  if (tid < E)
    for (int w = 0; w < kMetaWaves; w++) tot += cnt[w * E + tid];
  const int off_e = meta_scan_tiles(tot, T, k, E, BM, with_shared, max_long, true, counts, offsets, tiles, n_tiles, active,
                                    n_active, sched);
  if (tid < E) {
    int run = off_e;
    for (int w = 0; w < kMetaWaves; w++) {
      const int c = cnt[w * E + tid];
      cnt[w * E + tid] = run;
      run += c;
    }
  }
  __syncthreads();  // cnt now holds the per-wave bases

  // ---- phase 3: stable scatter ----
  for (int c0 = 0; c0 < nch; c0 += kMetaBatch) {
    int ev[kMetaBatch], rk[kMetaBatch], ld[kMetaBatch], bs[kMetaBatch];
#pragma unroll
    for (int i = 0; i < kMetaBatch; i++) {
      const int a = seg0 + 64 * (c0 + i) + lane;
      ev[i] = (c0 + i < nch && a < seg1) ? ids[a] : -1;
    }
#pragma unroll
    for (int i = 0; i < kMetaBatch; i++) {
      rk[i] = 0;
      ld[i] = 0;
      bs[i] = 0;
      if (c0 + i < nch) {  // wave-uniform
        const bool valid = ev[i] >= 0;
        const uint64_t m = match_mask(valid ? ev[i] : 0, valid, nbits);
        rk[i] = __popcll(m & lt_mask);
        ld[i] = m ? __ffsll((unsigned long long)m) - 1 : 0;
        if (valid && rk[i] == 0) bs[i] = atomicAdd(&cnt[wave * E + ev[i]], __popcll(m));
      }
    }
#pragma unroll
    for (int i = 0; i < kMetaBatch; i++) {
      if (c0 + i < nch) {
        const int base = __shfl(bs[i], ld[i]);
        if (ev[i] >= 0) {
          const int a = seg0 + 64 * (c0 + i) + lane;
          const int pos = base + rk[i];
          sorted[pos] = a;
          if (inv) inv[a] = pos;
        }
      }
    }
  }
}

__global__ __launch_bounds__(1024) void k_meta(const int32_t* __restrict__ ids, int T, int k, int E,
                                               int BM, int with_shared, int max_long, int32_t* __restrict__ counts,
                                               int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
                                               int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles,
                                               int32_t* __restrict__ active, int32_t* __restrict__ n_active,
                                               int32_t* __restrict__ inv, int32_t* __restrict__ sched) {
  __shared__ int cnt[kMetaWaves * kMaxE];
  meta_body(ids, T, k, E, BM, with_shared, max_long, counts, offsets, sorted, tiles, n_tiles, active, n_active, inv,
            sched, cnt);
}

// ---------------------------------------------------------------------------
// Routing metadata for many tokens: the same computation spread over
// workgroups.  The flat assignment range is cut into segments of kSegAssign
// ids, one 1024-thread workgroup each (16 waves x one chunk of 64).  The
// per-(segment, expert) counts segcnt[seg][E] are already there (taken by the
// exact top-k).  Every segment workgroup
//  * sums the counts per expert and takes the expert offsets (the scans of
//    meta_scan_tiles);
//  * bases its segment's experts at offset[e] + counts of e in earlier
//    segments, then per wave from the wave counts;
//  * scatters its segment stably with the leader atomics of meta_body.
// One more workgroup (blockIdx.x == nseg) sums the counts and writes counts,
// offsets, the active list, the tile map and the schedule, in parallel with
// the scatter.
// ---------------------------------------------------------------------------
constexpr int kSegWaves = kSegAssign / 64;  // one chunk of 64 per wave

__global__ __launch_bounds__(1024) void k_meta_segments(const int32_t* __restrict__ ids, int T, int k, int E,
                                                        int BM, int with_shared, int max_long, int nseg,
                                                        const int32_t* __restrict__ segcnt,
                                                        int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ sorted, int32_t* __restrict__ inv,
                                                        int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles,
                                                        int32_t* __restrict__ active, int32_t* __restrict__ n_active,
                                                        int32_t* __restrict__ sched) {
  // Segment counts are read kScanBatch at a time (independent loads).
  constexpr int kScanBatch = 16;
  __shared__ int wc[kSegWaves][kMaxE];  // per-wave counts, then per-wave bases
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int seg = blockIdx.x, N = T * k;
  const bool tiles_wg = seg == nseg;  // workgroup-uniform
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // The segment's ids go out first.
  const int a = seg * kSegAssign + tid;
  const int ev = !tiles_wg && a < N ? ids[a] : -1;
  int tot = 0, pre = 0;
  if (tid < E) {
    for (int g0 = 0; g0 < nseg; g0 += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; i++) v[i] = g0 + i < nseg ? segcnt[(int64_t)(g0 + i) * E + tid] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; i++) {
        tot += v[i];
        pre += g0 + i < seg ? v[i] : 0;
      }
    }
  }
  if (tiles_wg) {
    meta_scan_tiles(tot, T, k, E, BM, with_shared, max_long, true, counts, offsets, tiles, n_tiles, active, n_active,
                    sched);
    return;
  }
  for (int i = tid; i < kSegWaves * E; i += blockDim.x) wc[i / E][i % E] = 0;
  const int off_e = meta_scan_tiles(tot, T, k, E, BM, with_shared, max_long, false, counts, offsets, tiles, n_tiles,
                                    active, n_active, sched);
  // (meta_scan_tiles ends with a barrier: wc is cleared.)
  __syncthreads();
  if (ev >= 0) atomicAdd(&wc[wave][ev], 1);
  __syncthreads();
  if (tid < E) {
    int run = off_e + pre;
#pragma unroll
    for (int w = 0; w < kSegWaves; w++) {
      const int c = wc[w][tid];
      wc[w][tid] = run;
      run += c;
    }
  }
  __syncthreads();
  const uint64_t m = match_mask(ev >= 0 ? ev : 0, ev >= 0, nbits);
  const int rk = __popcll(m & lt_mask);
  const int ld = m ? __ffsll((unsigned long long)m) - 1 : 0;
  int bs = 0;
  if (ev >= 0 && rk == 0) bs = atomicAdd(&wc[wave][ev], __popcll(m));
  const int base = __shfl(bs, ld);
  if (ev >= 0) {
    const int pos = base + rk;
    sorted[pos] = a;
    if (inv) inv[a] = pos;
  }
}

// Few tokens: top-k of the exact logits (wave t for token t) and the routing
// metadata in one workgroup, so decode spends one launch on both.  The top-k
// takes the k-th largest of the lanes' maxima as a threshold (at most the
// k-th largest logit), lists the logits at or above it and ranks that short
// list exactly (larger logit first, equal logits towards the lower expert).
constexpr int kTopkLds = kSmallT * (2 * kMaxE + 16);  // per-token lists, then the metadata counters

__global__ __launch_bounds__(1024) void k_topk_meta(const float* __restrict__ logits, int T, int E, int k,
                                                    int32_t* __restrict__ ids, float* __restrict__ tw,
                                                    int BM, int with_shared, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
                                                    int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles,
                                                    int32_t* __restrict__ active, int32_t* __restrict__ n_active,
                                                    int32_t* __restrict__ inv, int32_t* __restrict__ sched) {
  __shared__ int lds[kTopkLds];
  const int wave = threadIdx.x >> 6;
  if (wave < T)
    topk_small(logits + (int64_t)wave * E, E, k, wave, ids, tw, lds + wave * (2 * E + 16));
  __syncthreads();  // ids visible to the workgroup; the lists' LDS is free again
  if (wave == 0)
    meta_small(ids, T, k, E, BM, with_shared, counts, offsets, sorted, tiles, n_tiles, active, n_active, inv,
               sched, lds);
}

// ---------------------------------------------------------------------------
hipError_t launch_route_logits(const uint16_t* x, int T, int H, const float* wr, const float* bias, int E,
                               int k, float* logits, double* wsq, int32_t* ids, float* tw, float* xsum,
                               uint16_t* x16, int32_t* segcnt, hipStream_t s, bool* two_launches,
                               const KTime& kt) {
  if (T == 0) return hipSuccess;
  if (T <= kSmallT) {
    MOE_LAUNCH(k_logits_small, dim3(E), dim3(64), 0, s, kt.start, kt.stop, x, T, H, wr, bias, E, logits, xsum,
               x16);
    *two_launches = false;
    return hipGetLastError();
  }
  const int n_segcnt = segcnt ? (T * k + kSegAssign - 1) / kSegAssign * E : 0;
  MOE_LAUNCH(k_screen, dim3((T + 63) / 64, (E + 63) / 64, kScreenSplit), dim3(256), 0, s, kt.start, kt.stop, x, T,
             H, wr, E, logits, wsq, segcnt, n_segcnt);
  *two_launches = true;
  return hipGetLastError();
}

hipError_t launch_route_select(const uint16_t* x, int T, int H, const float* wr, const float* bias, int E,
                               int k, const float* logits, const double* wsq, int32_t* ids, float* tw,
                               uint16_t* x16, int32_t* segcnt, hipStream_t s, const KTime& kt) {
  if (T <= kSmallT) return hipSuccess;  // few tokens: k_topk_meta selects from the exact logits
  const size_t smem = (size_t)route_exact_smem_bytes(H, E);
  MOE_LAUNCH(k_route_exact, dim3(T), dim3(256), smem, s, kt.start, kt.stop, x, T, H, wr, bias, E, k, logits, wsq, ids,
             tw, x16, segcnt);
  return hipGetLastError();
}

hipError_t launch_meta(const int32_t* ids, int T, int k, int E, int BM, int with_shared, int max_long,
                       int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* tiles,
                       int32_t* n_tiles, int32_t* active, int32_t* n_active, int32_t* inv,
                       int32_t* sched, const int32_t* segcnt, hipStream_t s, const KTime& kt) {
  const int N = T * k;
  const int nseg = (N + kSegAssign - 1) / kSegAssign;
  if (nseg <= 1) {  // one segment: the single-workgroup version (counts its own histogram)
    MOE_LAUNCH(k_meta, dim3(1), dim3(1024), 0, s, kt.start, kt.stop, ids, T, k, E, BM, with_shared, max_long,
               counts, offsets, sorted, tiles, n_tiles, active, n_active, inv, sched);
    return hipGetLastError();
  }
  MOE_LAUNCH(k_meta_segments, dim3(nseg + 1), dim3(kSegAssign), 0, s, kt.start, kt.stop, ids, T, k, E, BM, with_shared,
             max_long, nseg, segcnt, counts, offsets, sorted, inv, tiles, n_tiles, active, n_active, sched);
  return hipGetLastError();
}

hipError_t launch_topk_meta(const float* logits, int T, int E, int k, int32_t* ids, float* tw, int BM,
                            int with_shared, int32_t* counts, int32_t* offsets, int32_t* sorted,
                            int32_t* tiles, int32_t* n_tiles, int32_t* active, int32_t* n_active,
                            int32_t* inv, int32_t* sched, hipStream_t s, const KTime& kt) {
  MOE_LAUNCH(k_topk_meta, dim3(1), dim3(1024), 0, s, kt.start, kt.stop, logits, T, E, k, ids, tw, BM, with_shared,
             counts, offsets, sorted, tiles, n_tiles, active, n_active, inv, sched);
  return hipGetLastError();
}

}  // namespace moe
