// Routing building blocks for few tokens (T <= 8), shared by the routing
// kernels and the decode GEMV ("Optimizing on-device inference for Apple
// Silicon", section "Keep expert routing on the GPU").
#pragma once

#include "common.h"

namespace moe {

constexpr int kMaxEPerLane = 8;  // E <= 512
constexpr int kSmallT = 8;
constexpr int kMaxE = 512;

// ---- cross-lane sums by DPP (ALU moves within rows of 16 lanes) and
// v_readlane (across rows), instead of LDS permutes.  Fixed order: the same
// inputs give the same bits. ----
template <int kCtrl>
__device__ __forceinline__ int dpp_i32(int v) { return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, false); }
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, dpp_i32<kCtrl>(__builtin_bit_cast(int, v)));
}
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)dpp_i32<kCtrl>((int)(uint32_t)u), hi = (uint32_t)dpp_i32<kCtrl>((int)(uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double lane_value_f64(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over each row of 16 lanes, in every lane of the row: pairs (lane xor
// 1), quads (xor 2), then the row rotated by 4 and by 8.
template <class V>
__device__ __forceinline__ V row_sum16(V v) {
  if constexpr (sizeof(V) == 8) {
    v += dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f64<0x124>(v);  // row_ror:4
    v += dpp_f64<0x128>(v);  // row_ror:8
  } else if constexpr (__is_same(V, float)) {
    v += dpp_f32<0xB1>(v);
    v += dpp_f32<0x4E>(v);
    v += dpp_f32<0x124>(v);
    v += dpp_f32<0x128>(v);
  } else {
    v += dpp_i32<0xB1>(v);
    v += dpp_i32<0x4E>(v);
    v += dpp_i32<0x124>(v);
    v += dpp_i32<0x128>(v);
  }
  return v;
}

// Sum over the wave's 64 lanes: the row sums of lanes 0, 16, 32 and 48 added
// as (r0 + r1) + (r2 + r3); every lane gets that value.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v = row_sum16(v);
  return (lane_value_f64(v, 0) + lane_value_f64(v, 16)) + (lane_value_f64(v, 32) + lane_value_f64(v, 48));
}

// Inclusive prefix sum over the wave's 64 lanes, in ALU cross-lane moves
// (DPP) rather than LDS permutes: shifts by 1, 2, 4 and 8 within each row of
// 16 lanes (lanes shifted in from outside the row read 0), then the total of
// row 0 (lane 15) into row 1 and of row 2 into row 3, then the total of the
// lower half (lane 31) into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31, rows 2 and 3
  return v;
}

// Value of lane l (wave-uniform l) in every lane.
__device__ __forceinline__ int lane_value(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float lane_value(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
  v = row_sum16(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}
__device__ __forceinline__ int wave_sum_i32(int v) {
  v = row_sum16(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// Maximum over the wave's 64 lanes (exact whatever the order).
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x124>(v));
  v = fmaxf(v, dpp_f32<0x128>(v));
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}
__device__ __forceinline__ double wave_max_f64(double v) {
  v = fmax(v, dpp_f64<0xB1>(v));
  v = fmax(v, dpp_f64<0x4E>(v));
  v = fmax(v, dpp_f64<0x124>(v));
  v = fmax(v, dpp_f64<0x128>(v));
  return fmax(fmax(lane_value_f64(v, 0), lane_value_f64(v, 16)), fmax(lane_value_f64(v, 32), lane_value_f64(v, 48)));
}

// k-th largest of the 64 lanes' values m (k <= 64; -inf for lanes without
// one), by a radix select over order-preserving integer keys: from the top
// bit down, keep the bit set if at least k lanes are at or above the prefix
// with it.  One ballot per bit, no cross-lane data movement.
__device__ __forceinline__ float wave_kth_largest(float m, int k) {
  const uint32_t u = __builtin_bit_cast(uint32_t, m);
  const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  uint32_t t = 0;
#pragma unroll
  for (int b = 31; b >= 0; b--) {
    const uint32_t c = t | (1u << b);
    if (__popcll(__ballot(key >= c)) >= k) t = c;
  }
  const uint32_t v = (t & 0x80000000u) ? (t & 0x7FFFFFFFu) : ~t;
  return __builtin_bit_cast(float, v);
}

// A lower bound of the k-th largest of the 64 lanes' values: the same radix
// select, stopped as soon as exactly k lanes lie at or above the prefix (the
// candidates above it are then the lanes holding the k largest values).
__device__ __forceinline__ float wave_kth_lower_bound(float m, int k) {
  const uint32_t u = __builtin_bit_cast(uint32_t, m);
  const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  uint32_t t = 0;
  for (int b = 31; b >= 0; b--) {
    const uint32_t c = t | (1u << b);
    const int n = __popcll(__ballot(key >= c));
    if (n >= k) {
      t = c;
      if (n == k) break;
    }
  }
  const uint32_t v = (t & 0x80000000u) ? (t & 0x7FFFFFFFu) : ~t;
  return __builtin_bit_cast(float, v);
}

// Lanes of this wave that are valid and hold the same expert e.
__device__ __forceinline__ uint64_t match_mask(int e, bool valid, int nbits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; b++) {
    const bool bit = (e >> b) & 1;
    const uint64_t bb = __ballot(valid && bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

// Exact router logits of expert e for T <= 8 tokens, one wave: lanes split h
// in 16-byte slices of the router row (lane l: columns 256 i + 4 l .. +3);
// every product x * Wr is exact in float64, the sums are float64, rounded once
// to fp32, then the fp32 bias.  The loads of 2048 columns of the router row
// and of the rows' matching parts are issued before their sums, so the wave
// waits for memory once per 2048 columns.
__device__ __forceinline__ void logits_one_expert(const uint16_t* __restrict__ x, int T, int H,
                                                  const float* __restrict__ wr, const float* __restrict__ bias,
                                                  int E, int e, float* __restrict__ logits) {
  constexpr int kIt = 8;
  const int lane = threadIdx.x & 63;
  double acc[kSmallT];
#pragma unroll
  for (int t = 0; t < kSmallT; t++) acc[t] = 0.0;
  const float* wrow = wr + (int64_t)e * H;
  for (int h0 = 0; h0 < H; h0 += 256 * kIt) {
    float4 w4[kIt];
#pragma unroll
    for (int i = 0; i < kIt; i++) {
      const int h = h0 + 256 * i + 4 * lane;
      w4[i] = h < H ? *reinterpret_cast<const float4*>(wrow + h) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int t = 0; t < kSmallT; t++) {
      if (t < T) {
        uint2 xv[kIt];
#pragma unroll
        for (int i = 0; i < kIt; i++) {
          const int h = h0 + 256 * i + 4 * lane;
          xv[i] = h < H ? *reinterpret_cast<const uint2*>(x + (int64_t)t * H + h) : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int i = 0; i < kIt; i++) {
          if (h0 + 256 * i + 4 * lane < H) {
            acc[t] = fma((double)bf16_bits_to_f32(xv[i].x & 0xFFFFu), (double)w4[i].x, acc[t]);
            acc[t] = fma((double)bf16_bits_to_f32(xv[i].x >> 16), (double)w4[i].y, acc[t]);
            acc[t] = fma((double)bf16_bits_to_f32(xv[i].y & 0xFFFFu), (double)w4[i].z, acc[t]);
            acc[t] = fma((double)bf16_bits_to_f32(xv[i].y >> 16), (double)w4[i].w, acc[t]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kSmallT; t++) {
    if (t < T) {
      const double sm = wave_sum_f64(acc[t]);
      if (lane == 0) {
        float l = (float)sm;
        if (bias) l = l + bias[e];
        logits[(int64_t)t * E + e] = l;
      }
    }
  }
}

// Per-group sums of the activation rows (sequential within a group), for the
// affine fold of the GEMV path.
__device__ __forceinline__ void group_sums(const uint16_t* __restrict__ x, int T, int H, float* __restrict__ xsum,
                                           int tid, int nthreads) {
  const int G = H / kGroup;
  for (int i = tid; i < T * G; i += nthreads) {
    const int t = i / G, g = i - t * G;
    const uint16_t* p = x + (int64_t)t * H + g * kGroup;
    float sm = 0.f;
    for (int j = 0; j < kGroup; j++) sm += bf16_bits_to_f32(p[j]);
    xsum[i] = sm;
  }
}

// Top-k of one token's exact logits, one wave: a lower bound of the k-th
// largest of the lanes' maxima (k distinct logits lie at or above it) is a
// threshold at most the k-th largest logit; the logits at or above it (float
// comparison, a superset of the key comparison) are listed and ranked exactly
// (larger first, equal logits towards the lower expert), then the softmax
// over the k selected.  lds: 2 E + 16 ints.
//
// ordered = false (a caller that needs the selected set and its weights, not
// their order): when exactly k logits pass the threshold they are all
// selected, and they are written in increasing expert order without the
// ranking (the softmax then sums in that order).
__device__ __forceinline__ void topk_small(const float* __restrict__ l, int E, int k, int t,
                                           int32_t* __restrict__ ids, float* __restrict__ tw, int* lds,
                                           bool ordered = true) {
  const int lane = threadIdx.x & 63;
  int* cand_e = lds;
  float* cand_v = reinterpret_cast<float*>(cand_e + E);
  float* sel_v = cand_v + E;
  float v[kMaxEPerLane];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < kMaxEPerLane; j++) {
    const int e = lane + 64 * j;
    v[j] = e < E ? l[e] : -INFINITY;
    m = fmaxf(m, v[j]);
  }
  const float thr = wave_kth_lower_bound(m, k);
  int C = 0;
#pragma unroll
  for (int j = 0; j < kMaxEPerLane; j++) {
    const int e = lane + 64 * j;
    const bool cand = e < E && v[j] >= thr;
    const uint64_t mk = __ballot(cand);
    if (cand) {
      const int c = C + __popcll(mk & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
      cand_e[c] = e;
      cand_v[c] = v[j];
    }
    C += __popcll(mk);
  }
  __builtin_amdgcn_wave_barrier();
  if (!ordered && C == k) {  // wave-uniform
    const float vc = lane < k ? cand_v[lane] : -INFINITY;
    const float vmax = wave_max_f32(vc);
    const float ex = lane < k ? __expf(vc - vmax) : 0.f;
    const float sum = wave_sum_f32(ex);
    if (lane < k) {
      ids[(int64_t)t * k + lane] = cand_e[lane];
      tw[(int64_t)t * k + lane] = ex / sum;
    }
    return;
  }
  if (C <= 64) {
    // Candidates in lanes; the others are broadcast with v_readlane.
    const float vc = lane < C ? cand_v[lane] : 0.f;
    const int ec = lane < C ? cand_e[lane] : 0;
    int rank = 0;
    for (int c2 = 0; c2 < C; c2++) {
      const float v2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, vc), c2));
      const int e2 = __builtin_amdgcn_readlane(ec, c2);
      rank += (v2 > vc || (v2 == vc && e2 < ec)) ? 1 : 0;
    }
    if (lane < C && rank < k) {
      ids[(int64_t)t * k + rank] = ec;
      sel_v[rank] = vc;
    }
  } else {
    for (int c = lane; c < C; c += 64) {
      const float vc = cand_v[c];
      const int ec = cand_e[c];
      int rank = 0;
      for (int c2 = 0; c2 < C; c2++) {
        const float v2 = cand_v[c2];
        rank += (v2 > vc || (v2 == vc && cand_e[c2] < ec)) ? 1 : 0;
      }
      if (rank < k) {
        ids[(int64_t)t * k + rank] = ec;
        sel_v[rank] = vc;
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  const float myv = lane < k ? sel_v[lane] : 0.f;
  const float vmax = lane_value(myv, 0);
  const float ex = lane < k ? __expf(myv - vmax) : 0.f;
  const float sum = wave_sum_f32(ex);
  if (lane < k) tw[(int64_t)t * k + lane] = ex / sum;
}

// Routing metadata for at most 128 assignments (T <= 8), computed by one
// wave without workgroup barriers; same outputs and order as meta_body.
// Lane l owns experts 8l .. 8l+7 for the scans.  lds: 2 * E ints.
__device__ __forceinline__ void meta_small(const int32_t* __restrict__ ids, int T, int k, int E, int BM, int with_shared,
                           int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                           int32_t* __restrict__ sorted, int32_t* __restrict__ tiles,
                           int32_t* __restrict__ n_tiles, int32_t* __restrict__ active,
                           int32_t* __restrict__ n_active, int32_t* __restrict__ inv,
                           int32_t* __restrict__ sched, int* __restrict__ lds) {
  const int lane = threadIdx.x & 63;
  const int N = T * k;
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int* cnt = lds;      // [E] counts
  int* run = lds + E;  // [E] next free sorted position
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  __builtin_amdgcn_wave_barrier();
  const int e0v = lane < N ? ids[lane] : 0;
  const int e1v = lane + 64 < N ? ids[lane + 64] : 0;
  uint64_t m0 = match_mask(e0v, lane < N, nbits), m1 = match_mask(e1v, lane + 64 < N, nbits);
  if (lane < N && (m0 & lt_mask) == 0) atomicAdd(&cnt[e0v], __popcll(m0));
  if (lane + 64 < N && (m1 & lt_mask) == 0) atomicAdd(&cnt[e1v], __popcll(m1));
  __builtin_amdgcn_wave_barrier();

  // Per lane: its 8 experts' counts, tiles, active flags, full / partial tiles.
  int c[8], sum[5] = {0, 0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int e = 8 * lane + i;
    c[i] = e < E ? cnt[e] : 0;
    sum[0] += c[i];
    sum[1] += (c[i] + BM - 1) / BM;
    sum[2] += c[i] > 0 ? 1 : 0;
    sum[3] += c[i] / BM;
    sum[4] += (c[i] + BM - 1) / BM - c[i] / BM;
  }
  int excl[5], total[5];
#pragma unroll
  for (int q = 0; q < 5; q++) {
    const int inc = wave_incl_scan(sum[q]);
    excl[q] = inc - sum[q];
    total[q] = lane_value(inc, 63);
  }
  const int routed_tiles = total[1], full_total = total[3];
  const int sfull = with_shared ? T / BM : 0;
  int off = excl[0], tl = excl[1], ac = excl[2], fu = excl[3], pa = excl[4];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int e = 8 * lane + i;
    if (e < E) {
      counts[e] = c[i];
      offsets[e] = off;
      run[e] = off;
      if (c[i] > 0) active[ac++] = e;
      const int nt = (c[i] + BM - 1) / BM, nf = c[i] / BM;
      for (int r = 0; r < nt; r++) {
        const int rows = min(BM, c[i] - r * BM);
        tiles[3 * (tl + r) + 0] = e;
        tiles[3 * (tl + r) + 1] = r * BM;
        tiles[3 * (tl + r) + 2] = rows;
        if (sched) {
          const int slot = 1 + (r < nf ? sfull + fu + r : sfull + full_total + pa);
          reinterpret_cast<int4*>(sched)[slot] = make_int4(e, r * BM, rows, off + r * BM);
        }
      }
      tl += nt;
      fu += nf;
      pa += nt - nf;
      off += c[i];
    }
  }
  if (lane == 63) offsets[E] = total[0];
  const int nshared = with_shared ? (T + BM - 1) / BM : 0;
  for (int r = lane; r < nshared; r += 64) {
    tiles[3 * (routed_tiles + r) + 0] = E;
    tiles[3 * (routed_tiles + r) + 1] = r * BM;
    tiles[3 * (routed_tiles + r) + 2] = min(BM, T - r * BM);
    if (sched)
      reinterpret_cast<int4*>(sched)[1 + (r < sfull ? r : routed_tiles + nshared - 1)] =
          make_int4(E, r * BM, min(BM, T - r * BM), T * k + r * BM);
  }
  if (lane == 0) {
    n_tiles[0] = routed_tiles + nshared;
    if (sched) reinterpret_cast<int4*>(sched)[0] = make_int4(routed_tiles + nshared, 0, 0, 0);
    n_active[0] = total[2];
  }
  __builtin_amdgcn_wave_barrier();

  // Stable scatter: chunk 0, then chunk 1; each group's leader takes the base.
  {
    const int rk = __popcll(m0 & lt_mask), ld = m0 ? __ffsll((unsigned long long)m0) - 1 : 0;
    int b = 0;
    if (lane < N && rk == 0) b = atomicAdd(&run[e0v], __popcll(m0));
    b = __shfl(b, ld);
    if (lane < N) {
      sorted[b + rk] = lane;
      if (inv) inv[lane] = b + rk;
    }
  }
  if (N > 64) {
    const int rk = __popcll(m1 & lt_mask), ld = m1 ? __ffsll((unsigned long long)m1) - 1 : 0;
    int b = 0;
    if (lane + 64 < N && rk == 0) b = atomicAdd(&run[e1v], __popcll(m1));
    b = __shfl(b, ld);
    if (lane + 64 < N) {
      sorted[b + rk] = lane + 64;
      if (inv) inv[lane + 64] = b + rk;
    }
  }
}

}  // namespace moe
