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
#include <climits>

#include "launch.h"

namespace moe {

// ---------------------------------------------------------------------------
// Logits for a block of TB tokens x EB experts; also the per-group sums of x
// (used by the expert kernels to undo the +128 code offset).
// ---------------------------------------------------------------------------
constexpr int kMaxTB = 8;

__global__ __launch_bounds__(256) void k_logits(const uint16_t* __restrict__ x, int T, int H,
                                                const float* __restrict__ wr,
                                                const float* __restrict__ bias, int E,
                                                float* __restrict__ logits,
                                                float* __restrict__ xsum, int TB, int EB) {
  extern __shared__ uint16_t xs[];  // [TB][H]
  const int t0 = blockIdx.x * TB;
  const int tb = min(TB, T - t0);
  const int H8 = H / 8;
  for (int i = threadIdx.x; i < tb * H8; i += blockDim.x) {
    const int r = i / H8, c = i - r * H8;
    reinterpret_cast<uint4*>(xs)[i] =
        reinterpret_cast<const uint4*>(x + (int64_t)(t0 + r) * H)[c];
  }
  __syncthreads();

  if (blockIdx.y == 0) {
    const int G = H / kGroup;
    for (int i = threadIdx.x; i < tb * G; i += blockDim.x) {
      const int r = i / G, g = i - r * G;
      float s = 0.f;
      for (int j = 0; j < kGroup; j++) s += bf16_bits_to_f32(xs[r * H + g * kGroup + j]);
      xsum[(int64_t)(t0 + r) * G + g] = s;
    }
  }

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nw = blockDim.x >> 6;
  const int e0 = blockIdx.y * EB;
  const int e1 = min(E, e0 + EB);
  for (int e = e0 + wave; e < e1; e += nw) {
    double acc[kMaxTB];
#pragma unroll
    for (int t = 0; t < kMaxTB; t++) acc[t] = 0.0;
    const float* wrow = wr + (int64_t)e * H;
    for (int h = lane; h < H; h += 64) {
      const double wv = (double)wrow[h];
#pragma unroll
      for (int t = 0; t < kMaxTB; t++)
        if (t < tb) acc[t] = fma((double)bf16_bits_to_f32(xs[t * H + h]), wv, acc[t]);
    }
#pragma unroll
    for (int t = 0; t < kMaxTB; t++) {
      if (t < tb) {
        double v = acc[t];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
        acc[t] = v;
      }
    }
    if (lane == 0) {
      const float b = bias ? bias[e] : 0.f;
#pragma unroll
      for (int t = 0; t < kMaxTB; t++) {
        if (t < tb) {
          float l = (float)acc[t];
          if (bias) l = l + b;
          logits[(int64_t)(t0 + t) * E + e] = l;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k: one wave per token.  Each lane holds the logits of experts
// lane, lane+64, ...; k rounds of a wave-wide (value desc, index asc) argmax.
// ---------------------------------------------------------------------------
constexpr int kMaxEPerLane = 8;  // E <= 512

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  // Is (va, ia) ranked before (vb, ib)?  ib == INT_MAX marks "none".
  if (ib == INT_MAX) return ia != INT_MAX;
  if (ia == INT_MAX) return false;
  return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ tw) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x >> 6) + wave;
  if (t >= T) return;
  const float* l = logits + (int64_t)t * E;
  float v[kMaxEPerLane];
  bool alive[kMaxEPerLane];
#pragma unroll
  for (int j = 0; j < kMaxEPerLane; j++) {
    const int e = lane + 64 * j;
    alive[j] = e < E;
    v[j] = alive[j] ? l[e] : 0.f;
  }
  float myv = 0.f;
  int myi = 0;
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
    if ((bi & 63) == lane) {
#pragma unroll
      for (int j = 0; j < kMaxEPerLane; j++)
        if (j == (bi >> 6)) alive[j] = false;
    }
    if (lane == r) {
      myv = bv;
      myi = bi;
    }
  }
  const float vmax = __shfl(myv, 0);
  const float ex = lane < k ? __expf(myv - vmax) : 0.f;
  float sum = ex;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    ids[(int64_t)t * k + lane] = myi;
    tw[(int64_t)t * k + lane] = ex / sum;
  }
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

__global__ __launch_bounds__(1024) void k_meta(const int32_t* __restrict__ ids, int T, int k, int E,
                                               int BM, int with_shared,
                                               int32_t* __restrict__ counts,
                                               int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ sorted,
                                               int32_t* __restrict__ tiles,
                                               int32_t* __restrict__ n_tiles,
                                               int32_t* __restrict__ active,
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

// ---------------------------------------------------------------------------
hipError_t launch_logits(const uint16_t* x, int T, int H, const float* wr, const float* bias, int E,
                         float* logits, float* xsum, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int TB = min(kMaxTB, T);
  while (TB > 1 && (size_t)TB * H * 2 > 64 * 1024) TB--;
  // Small token counts spread the 2*E*H router bytes over more workgroups.
  const int EB = T <= 8 ? 8 : 64;
  dim3 grid((T + TB - 1) / TB, (E + EB - 1) / EB);
  k_logits<<<grid, dim3(256), (size_t)TB * H * 2, s>>>(x, T, H, wr, bias, E, logits, xsum, TB, EB);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* tw,
                       hipStream_t s) {
  if (T == 0) return hipSuccess;
  k_topk<<<dim3((T + 3) / 4), dim3(256), 0, s>>>(logits, T, E, k, ids, tw);
  return hipGetLastError();
}

hipError_t launch_meta(const int32_t* ids, int T, int k, int E, int BM, int with_shared,
                       int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* tiles,
                       int32_t* n_tiles, int32_t* active, int32_t* n_active, hipStream_t s) {
  k_meta<<<dim3(1), dim3(1024), 0, s>>>(ids, T, k, E, BM, with_shared, counts, offsets, sorted,
                                        tiles, n_tiles, active, n_active);
  return hipGetLastError();
}

}  // namespace moe
