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
#include <climits>

#include "launch.h"

namespace moe {

constexpr int kMaxEPerLane = 8;  // E <= 512
constexpr int kSmallT = 8;

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  // Is (va, ia) ranked before (vb, ib)?  ib == INT_MAX marks "none".
  if (ib == INT_MAX) return ia != INT_MAX;
  if (ia == INT_MAX) return false;
  return va > vb || (va == vb && ia < ib);
}

// Wave-wide top-k over per-lane candidate arrays (expert e = lane + 64 j).
// Lane r < k ends with the r-th selected (value, expert).
__device__ __forceinline__ void wave_topk(const float (&v)[kMaxEPerLane], bool (&alive)[kMaxEPerLane],
                                          int k, float& myv, int& myi) {
  const int lane = threadIdx.x & 63;
  myv = 0.f;
  myi = 0;
  for (int r = 0; r < k; r++) {
    float bv = 0.f;
    int bi = INT_MAX;
#pragma unroll
    for (int j = 0; j < kMaxEPerLane; j++) {
      const int e = lane + 64 * j;
      if (alive[j] && better(v[j], e, bv, bi)) {
        bv = v[j];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (bi != INT_MAX && (bi & 63) == lane) {
#pragma unroll
      for (int j = 0; j < kMaxEPerLane; j++)
        if (j == (bi >> 6)) alive[j] = false;
    }
    if (lane == r) {
      myv = bv;
      myi = bi;
    }
  }
}

// Softmax over the k selected logits held by lanes 0..k-1; writes ids and weights.
__device__ __forceinline__ void write_topk(float myv, int myi, int k, int64_t t, int32_t* ids, float* tw) {
  const int lane = threadIdx.x & 63;
  const float vmax = __shfl(myv, 0);
  const float ex = lane < k ? __expf(myv - vmax) : 0.f;
  float sum = ex;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    ids[t * k + lane] = myi;
    tw[t * k + lane] = ex / sum;
  }
}

// bf16 bits -> fp16 bits of value / 256 (exact whenever the result is normal).
__device__ __forceinline__ uint16_t f32_to_f16_scaled(uint16_t b) {
  return __builtin_bit_cast(uint16_t, (_Float16)(bf16_bits_to_f32(b) * 0.00390625f));
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// ---------------------------------------------------------------------------
// Few tokens: all T x E logits in float64.  One wave per expert, lanes split h
// in 16-byte slices of the router row.  Workgroup 0 also writes the per-group
// activation sums used by the expert kernels.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_logits_small(const uint16_t* __restrict__ x, int T, int H,
                                                      const float* __restrict__ wr,
                                                      const float* __restrict__ bias, int E,
                                                      float* __restrict__ logits,
                                                      float* __restrict__ xsum,
                                                      uint16_t* __restrict__ x16) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + wave;
  if (blockIdx.x == 0) {
    const int G = H / kGroup;
    for (int i = threadIdx.x; i < T * G; i += blockDim.x) {
      const int t = i / G, g = i - t * G;
      const uint16_t* p = x + (int64_t)t * H + g * kGroup;
      float s = 0.f;
      for (int j = 0; j < kGroup; j++) s += bf16_bits_to_f32(p[j]);
      xsum[i] = s;
    }
  }
  if (blockIdx.x == (gridDim.x > 1 ? 1 : 0)) {
    for (int i = threadIdx.x; i < T * H; i += blockDim.x) x16[i] = f32_to_f16_scaled(x[i]);
  }
  if (e >= E) return;
  double acc[kSmallT];
#pragma unroll
  for (int t = 0; t < kSmallT; t++) acc[t] = 0.0;
  const float* wrow = wr + (int64_t)e * H;
  for (int h = 4 * lane; h < H; h += 256) {
    const float4 w4 = *reinterpret_cast<const float4*>(wrow + h);
#pragma unroll
    for (int t = 0; t < kSmallT; t++) {
      if (t < T) {
        const uint2 xv = *reinterpret_cast<const uint2*>(x + (int64_t)t * H + h);
        acc[t] = fma((double)bf16_bits_to_f32(xv.x & 0xFFFFu), (double)w4.x, acc[t]);
        acc[t] = fma((double)bf16_bits_to_f32(xv.x >> 16), (double)w4.y, acc[t]);
        acc[t] = fma((double)bf16_bits_to_f32(xv.y & 0xFFFFu), (double)w4.z, acc[t]);
        acc[t] = fma((double)bf16_bits_to_f32(xv.y >> 16), (double)w4.w, acc[t]);
      }
    }
  }
  const float b = bias ? bias[e] : 0.f;
#pragma unroll
  for (int t = 0; t < kSmallT; t++) {
    if (t < T) {
      const double s = wave_sum_f64(acc[t]);
      if (lane == 0) {
        float l = (float)s;
        if (bias) l = l + b;
        logits[(int64_t)t * E + e] = l;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Many tokens, step 1: screened logits a = sum_h x * bf16(Wr) + bias with
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation).  Workgroup tile 64 tokens x
// 64 experts, four 32x32 waves, operands loaded straight from memory.  The
// workgroups of the first token tile also write |Wr_e|_2 (float64 sum,
// rounded up) for the error bound.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_screen(const uint16_t* __restrict__ x, int T, int H,
                                                const float* __restrict__ wr,
                                                const float* __restrict__ bias, int E,
                                                float* __restrict__ approx, float* __restrict__ wnorm) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, c32 = lane & 31;
  const int t = blockIdx.x * 64 + wm * 32 + c32;
  const int e = blockIdx.y * 64 + wn * 32 + c32;
  const bool tv = t < T, ev = e < E;
  const uint16_t* xr = x + (int64_t)(tv ? t : 0) * H + h * 32;
  const float* wrow = wr + (int64_t)(ev ? e : 0) * H + h * 32;
  const bool norms = blockIdx.x == 0 && wm == 0;
  f32x16_t acc = {};
  double ss = 0.0;
  const int G = H / kGroup;
  for (int g = 0; g < G; g++) {
    uint4 a[4];
    float4 w[8];
#pragma unroll
    for (int c = 0; c < 4; c++)
      a[c] = tv ? *reinterpret_cast<const uint4*>(xr + g * kGroup + c * 8) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 8; q++)
      w[q] = ev ? *reinterpret_cast<const float4*>(wrow + g * kGroup + q * 4) : make_float4(0, 0, 0, 0);
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const float4 p = w[2 * c], r = w[2 * c + 1];
      bf16x8_t b = {(__bf16)p.x, (__bf16)p.y, (__bf16)p.z, (__bf16)p.w,
                    (__bf16)r.x, (__bf16)r.y, (__bf16)r.z, (__bf16)r.w};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[c]), b, acc, 0, 0, 0);
    }
    if (norms) {
#pragma unroll
      for (int q = 0; q < 8; q++) {
        ss = fma((double)w[q].x, (double)w[q].x, ss);
        ss = fma((double)w[q].y, (double)w[q].y, ss);
        ss = fma((double)w[q].z, (double)w[q].z, ss);
        ss = fma((double)w[q].w, (double)w[q].w, ss);
      }
    }
  }
  const float b = (ev && bias) ? bias[e] : 0.f;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const int tok = blockIdx.x * 64 + wm * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
    if (tok < T && ev) approx[(int64_t)tok * E + e] = acc[i] + b;
  }
  if (norms) {
    ss += __shfl_xor(ss, 32);
    if (h == 0 && ev) wnorm[e] = (float)(sqrt(ss) * (1.0 + 1e-6));
  }
}

// ---------------------------------------------------------------------------
// Many tokens, step 2: one wave per token.  Error bound of a screened logit
// against the float64-accumulated one (both with the bias added in fp32):
//   |a - l| <= (2^-8 + 2 H 2^-23) * sum_h |x_h||w_h| + 2^-22 (|a| + |l| + 1)
// covering the bf16 rounding of Wr (at most 2^-8 relative, any rounding
// mode), fp32 accumulation of H exact products in any order (2 H 2^-23) and
// the final roundings; sum |x||w| <= |x|_2 max_e |w_e|_2.  Experts with
// a >= a_k - 2 B (a_k the k-th largest screened logit) are recomputed in
// float64 and the exact top-k is taken among them.  Also writes the per-group
// activation sums.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_route_exact(const uint16_t* __restrict__ x, int T, int H,
                                                     const float* __restrict__ wr,
                                                     const float* __restrict__ bias, int E, int k,
                                                     const float* __restrict__ approx,
                                                     const float* __restrict__ wnorm,
                                                     int32_t* __restrict__ ids, float* __restrict__ tw,
                                                     float* __restrict__ xsum, uint16_t* __restrict__ x16) {
  extern __shared__ uint16_t xl_all[];  // [4][H]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  uint16_t* xl = xl_all + wave * H;
  const uint16_t* xr = x + (int64_t)t * H;

  // x row -> LDS, per-group sums, |x|_2^2 in float64.
  double xx = 0.0;
  for (int h0 = 0; h0 < H; h0 += 256) {
    const int h = h0 + 4 * lane;
    float s = 0.f;
    if (h < H) {
      const uint2 v = *reinterpret_cast<const uint2*>(xr + h);
      *reinterpret_cast<uint2*>(xl + h) = v;
      const uint32_t c01 = f32_to_f16_scaled(v.x & 0xFFFFu) | ((uint32_t)f32_to_f16_scaled(v.x >> 16) << 16);
      const uint32_t c23 = f32_to_f16_scaled(v.y & 0xFFFFu) | ((uint32_t)f32_to_f16_scaled(v.y >> 16) << 16);
      *reinterpret_cast<uint2*>(x16 + (int64_t)t * H + h) = make_uint2(c01, c23);
      const float f0 = bf16_bits_to_f32(v.x & 0xFFFFu), f1 = bf16_bits_to_f32(v.x >> 16);
      const float f2 = bf16_bits_to_f32(v.y & 0xFFFFu), f3 = bf16_bits_to_f32(v.y >> 16);
      s = (f0 + f1) + (f2 + f3);
      xx = fma((double)f0, (double)f0, xx);
      xx = fma((double)f1, (double)f1, xx);
      xx = fma((double)f2, (double)f2, xx);
      xx = fma((double)f3, (double)f3, xx);
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) s += __shfl_xor(s, off);
    if ((lane & 15) == 0 && h < H) xsum[(int64_t)t * (H / kGroup) + h / kGroup] = s;
  }
  const double xnorm = sqrt(wave_sum_f64(xx)) * (1.0 + 1e-6);

  float a[kMaxEPerLane];
  bool alive[kMaxEPerLane];
  float wmax = 0.f, amax = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxEPerLane; j++) {
    const int e = lane + 64 * j;
    alive[j] = e < E;
    a[j] = alive[j] ? approx[(int64_t)t * E + e] : 0.f;
    if (alive[j]) {
      wmax = fmaxf(wmax, wnorm[e]);
      amax = fmaxf(amax, fabsf(a[j]));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    wmax = fmaxf(wmax, __shfl_xor(wmax, off));
    amax = fmaxf(amax, __shfl_xor(amax, off));
  }
  // k-th largest screened logit.
  float kv;
  int ki;
  {
    bool al2[kMaxEPerLane];
#pragma unroll
    for (int j = 0; j < kMaxEPerLane; j++) al2[j] = alive[j];
    wave_topk(a, al2, k, kv, ki);
  }
  const float ak = __shfl(kv, k - 1);
  const double c1 = 0.00390625 + 2.0 * H * 1.1920928955078125e-07;
  const double B = c1 * xnorm * (double)wmax + 2.384185791015625e-07 * (2.0 * amax + 1.0) * 2.0;
  const double lo = (double)ak - 2.0 * B;

  // Exact float64 logits of the candidates; everything else drops out.
  float v[kMaxEPerLane];
  const float* bb = bias;
#pragma unroll
  for (int j = 0; j < kMaxEPerLane; j++) {
    const bool cand = alive[j] && (double)a[j] >= lo;
    v[j] = 0.f;
    uint64_t m = __ballot(cand);
    while (m) {
      const int l = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      const int e = l + 64 * j;
      const float* wrow = wr + (int64_t)e * H;
      double acc = 0.0;
      for (int h = 4 * lane; h < H; h += 256) {
        const float4 w4 = *reinterpret_cast<const float4*>(wrow + h);
        const uint2 xv = *reinterpret_cast<const uint2*>(xl + h);
        acc = fma((double)bf16_bits_to_f32(xv.x & 0xFFFFu), (double)w4.x, acc);
        acc = fma((double)bf16_bits_to_f32(xv.x >> 16), (double)w4.y, acc);
        acc = fma((double)bf16_bits_to_f32(xv.y & 0xFFFFu), (double)w4.z, acc);
        acc = fma((double)bf16_bits_to_f32(xv.y >> 16), (double)w4.w, acc);
      }
      const double s = wave_sum_f64(acc);
      float lg = (float)s;
      if (bb) lg = lg + bb[e];
      if (lane == l) v[j] = lg;
    }
    alive[j] = cand;
  }
  float myv;
  int myi;
  wave_topk(v, alive, k, myv, myi);
  write_topk(myv, myi, k, t, ids, tw);
}

// ---------------------------------------------------------------------------
// Routing metadata for one chunk, one workgroup of 1024 threads (16 waves).
// The flat assignment range [0, T*k) is cut into 16 contiguous segments, one
// per wave.  Phase 1 counts per (wave, expert) with LDS atomics (order-free),
// phase 2 scans the per-expert totals (counts -> offsets, tiles, active list)
// and turns the per-wave counts into per-wave bases, phase 3 walks each
// segment in order, 64 assignments at a time, and ranks equal experts inside
// the wave with ballots on the expert id bits.  The scatter is therefore
// stable in flat id without any global atomics.
// ---------------------------------------------------------------------------
constexpr int kMetaWaves = 16;
constexpr int kMaxE = 512;

__device__ void meta_body(const int32_t* __restrict__ ids, int T, int k, int E, int BM, int with_shared,
                          int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                          int32_t* __restrict__ sorted, int32_t* __restrict__ tiles,
                          int32_t* __restrict__ n_tiles, int32_t* __restrict__ active,
                          int32_t* __restrict__ n_active) {
  __shared__ int cnt[kMetaWaves * kMaxE];  // [wave][expert]
  __shared__ int sc0[kMaxE], sc1[kMaxE], sc2[kMaxE];
  __shared__ int s_routed_tiles, s_nact;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int N = T * k;

  for (int i = tid; i < kMetaWaves * E; i += blockDim.x) cnt[i] = 0;
  __syncthreads();

  const int S = (N + kMetaWaves - 1) / kMetaWaves;
  const int seg0 = min(N, wave * S), seg1 = min(N, seg0 + S);
  for (int a = seg0 + lane; a < seg1; a += 64) atomicAdd(&cnt[wave * E + ids[a]], 1);
  __syncthreads();

  int tot = 0, nt = 0, act = 0;
  if (tid < E) {
    for (int w = 0; w < kMetaWaves; w++) tot += cnt[w * E + tid];
    nt = (tot + BM - 1) / BM;
    act = tot > 0 ? 1 : 0;
    sc0[tid] = tot;
    sc1[tid] = nt;
    sc2[tid] = act;
  }
  __syncthreads();
  for (int off = 1; off < E; off <<= 1) {
    int a0 = 0, a1 = 0, a2 = 0;
    if (tid < E && tid >= off) {
      a0 = sc0[tid - off];
      a1 = sc1[tid - off];
      a2 = sc2[tid - off];
    }
    __syncthreads();
    if (tid < E && tid >= off) {
      sc0[tid] += a0;
      sc1[tid] += a1;
      sc2[tid] += a2;
    }
    __syncthreads();
  }
  if (tid < E) {
    const int off_e = sc0[tid] - tot;
    counts[tid] = tot;
    offsets[tid] = off_e;
    if (tid == E - 1) {
      offsets[E] = sc0[tid];
      s_routed_tiles = sc1[tid];
      s_nact = sc2[tid];
    }
    int run = off_e;
    for (int w = 0; w < kMetaWaves; w++) {
      const int c = cnt[w * E + tid];
      cnt[w * E + tid] = run;
      run += c;
    }
    const int ts = sc1[tid] - nt;
    for (int r = 0; r < nt; r++) {
      tiles[3 * (ts + r) + 0] = tid;
      tiles[3 * (ts + r) + 1] = r * BM;
      tiles[3 * (ts + r) + 2] = min(BM, tot - r * BM);
    }
    if (act) active[sc2[tid] - 1] = tid;
  }
  __syncthreads();

  const int rt = s_routed_tiles;
  const int nshared = with_shared ? (T + BM - 1) / BM : 0;
  for (int r = tid; r < nshared; r += blockDim.x) {
    tiles[3 * (rt + r) + 0] = E;
    tiles[3 * (rt + r) + 1] = r * BM;
    tiles[3 * (rt + r) + 2] = min(BM, T - r * BM);
  }
  if (tid == 0) {
    n_tiles[0] = rt + nshared;
    n_active[0] = s_nact;
  }

  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = seg0; base < seg1; base += 64) {
    const int a = base + lane;
    const bool valid = a < seg1;
    const int e = valid ? ids[a] : 0;
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; b++) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(valid && bit);
      m &= bit ? bb : ~bb;
    }
    int rank = 0, pos = 0;
    if (valid) {
      rank = __popcll(m & lt_mask);
      pos = cnt[wave * E + e] + rank;
      sorted[pos] = a;
    }
    __builtin_amdgcn_wave_barrier();
    if (valid && rank == 0) cnt[wave * E + e] += __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
}

__global__ __launch_bounds__(1024) void k_meta(const int32_t* __restrict__ ids, int T, int k, int E,
                                               int BM, int with_shared, int32_t* __restrict__ counts,
                                               int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
                                               int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles,
                                               int32_t* __restrict__ active, int32_t* __restrict__ n_active) {
  meta_body(ids, T, k, E, BM, with_shared, counts, offsets, sorted, tiles, n_tiles, active, n_active);
}

// Few tokens: top-k of the exact logits (wave t for token t) and the routing
// metadata in one workgroup, so decode spends one launch on both.
__global__ __launch_bounds__(1024) void k_topk_meta(const float* __restrict__ logits, int T, int E, int k,
                                                    int32_t* __restrict__ ids, float* __restrict__ tw,
                                                    int BM, int with_shared, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
                                                    int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles,
                                                    int32_t* __restrict__ active, int32_t* __restrict__ n_active) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave < T) {
    const float* l = logits + (int64_t)wave * E;
    float v[kMaxEPerLane];
    bool alive[kMaxEPerLane];
#pragma unroll
    for (int j = 0; j < kMaxEPerLane; j++) {
      const int e = lane + 64 * j;
      alive[j] = e < E;
      v[j] = alive[j] ? l[e] : 0.f;
    }
    float myv;
    int myi;
    wave_topk(v, alive, k, myv, myi);
    write_topk(myv, myi, k, wave, ids, tw);
  }
  __syncthreads();
  meta_body(ids, T, k, E, BM, with_shared, counts, offsets, sorted, tiles, n_tiles, active, n_active);
}

// ---------------------------------------------------------------------------
hipError_t launch_route_logits(const uint16_t* x, int T, int H, const float* wr, const float* bias, int E,
                               int k, float* logits, float* wnorm, int32_t* ids, float* tw, float* xsum,
                               uint16_t* x16, hipStream_t s, bool* two_launches) {
  if (T == 0) return hipSuccess;
  if (T <= kSmallT) {
    k_logits_small<<<dim3((E + 3) / 4), dim3(256), 0, s>>>(x, T, H, wr, bias, E, logits, xsum, x16);
    *two_launches = false;
    return hipGetLastError();
  }
  k_screen<<<dim3((T + 63) / 64, (E + 63) / 64), dim3(256), 0, s>>>(x, T, H, wr, bias, E, logits, wnorm);
  *two_launches = true;
  return hipGetLastError();
}

hipError_t launch_route_select(const uint16_t* x, int T, int H, const float* wr, const float* bias, int E,
                               int k, const float* logits, const float* wnorm, int32_t* ids, float* tw,
                               float* xsum, uint16_t* x16, hipStream_t s) {
  if (T <= kSmallT) return hipSuccess;  // few tokens: k_topk_meta selects from the exact logits
  k_route_exact<<<dim3((T + 3) / 4), dim3(256), (size_t)4 * H * 2, s>>>(x, T, H, wr, bias, E, k, logits,
                                                                        wnorm, ids, tw, xsum, x16);
  return hipGetLastError();
}

hipError_t launch_meta(const int32_t* ids, int T, int k, int E, int BM, int with_shared,
                       int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* tiles,
                       int32_t* n_tiles, int32_t* active, int32_t* n_active, hipStream_t s) {
  k_meta<<<dim3(1), dim3(1024), 0, s>>>(ids, T, k, E, BM, with_shared, counts, offsets, sorted,
                                        tiles, n_tiles, active, n_active);
  return hipGetLastError();
}

hipError_t launch_topk_meta(const float* logits, int T, int E, int k, int32_t* ids, float* tw, int BM,
                            int with_shared, int32_t* counts, int32_t* offsets, int32_t* sorted,
                            int32_t* tiles, int32_t* n_tiles, int32_t* active, int32_t* n_active,
                            hipStream_t s) {
  k_topk_meta<<<dim3(1), dim3(1024), 0, s>>>(logits, T, E, k, ids, tw, BM, with_shared, counts, offsets,
                                             sorted, tiles, n_tiles, active, n_active);
  return hipGetLastError();
}

}  // namespace moe
