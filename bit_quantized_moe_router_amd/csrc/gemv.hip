// Row-parallel GEMV for decode ("Optimizing on-device inference for Apple
// Silicon", section "Optimise the one-row weight path": waves cooperate on the
// outputs while reading different parts of the weight matrix; section
// "Reduce intermediate and state traffic" for the two fused chains).
//
// With one to a few rows the layer is bound by weight bytes, so each expert's
// packed weights are streamed once.  A wave reads one 1152-byte gate or up
// block (32 output rows x one 64-column group) with a single 16-byte load per
// lane, so a lane holds 32 codes of one output row; every wave issues the
// loads of all its blocks before it computes.  Codes expand to bf16 pairs
// (128 + q) and meet the activation pairs in v_dot2_f32_bf16; the per-group
// affine fold is
//   acc += s * dot + (b - 128 s) * sum(x over the group).
// The down projection is split along the intermediate: the workgroup that
// produced 32 columns of h applies the matching 32 columns of the down matrix
// (half of each down block, loaded in the same round as gate/up) and writes a
// partial output row; a second kernel sums the partials of each token in a
// fixed order.  No atomics touch the outputs.
#include "launch.h"
#include "small_route.h"

namespace moe {

constexpr int kGemvMaxRows = 8;
constexpr int kGuPref = 4;     // groups per wave whose gate/up loads are issued together
constexpr int kMaxGroups = 128;              // H / 64 for H <= 8192
constexpr int kMaxAssign = kGemvMaxRows * 16; // T * k on the GEMV path
constexpr int kGuSmemMax = 64 * 1024 + kGemvMaxRows * (2 * 512 + 16) * 4;  // x rows + top-k lists

// ---------------------------------------------------------------------------
// Decode, experts step: top-k, gate/up + SwiGLU, and the down projection
// split along its reduction axis (the intermediate), so that each workgroup
// applies the down matrix to the 32 intermediate columns it has just produced
// and the down weights stream in the same round as gate/up.  grid (1D) =
// n_slots x nbs workgroups (slot: active expert, then the shared expert; nb:
// 32-column block of the intermediate).  For each of its rows (assignment
// a = t*k + j, or T*k + t for the shared expert) a workgroup writes the
// routing-weighted partial output of its 32 columns, part[a][nb][0..H).
// k_gemv_reduce sums them.
// ---------------------------------------------------------------------------
constexpr int kFuWaves = 8;
constexpr int kFuThreads = kFuWaves * 64;
constexpr int kRedCols = 64;                 // output columns per reduce workgroup
constexpr int kRedGroups = kFuThreads / 16;  // term groups of a reduce workgroup (16 float4 columns each)
constexpr int kFuDn = 4;                     // down outputs per thread per load round
constexpr int kFuBatch = 8;                  // partials a reduce thread loads together

// y[t][64 columns] = sum of token t's partials in a fixed order (routed
// assignments j = 0..k-1 with blocks nb ascending, then the shared expert's
// blocks), so y does not depend on the order in which workgroups ran.
// grid = T x H/64.
__global__ __launch_bounds__(kFuThreads) void k_gemv_reduce(LayerArgs L, ChunkArgs C, const float* __restrict__ part,
                                                           int nbs) {
  __shared__ float4 red4[kRedGroups][16];
  const int tid = threadIdx.x;
  const int H = L.H, k = L.k, Tk = C.Tk;
  const int nslice = H / kRedCols;
  const int t = (int)blockIdx.x / nslice, sl = (int)blockIdx.x - t * nslice;
  const int c4 = tid & 15, tg = tid >> 4;
  const int col = sl * kRedCols + c4 * 4;
  const int nI = L.I / 32, nS = L.Is / 32;
  const int nrt = k * nI, nterm = nrt + nS;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i0 = tg; i0 < nterm; i0 += kFuBatch * kRedGroups) {
    float4 v[kFuBatch];
#pragma unroll
    for (int p = 0; p < kFuBatch; p++) {
      const int i = i0 + p * kRedGroups;
      v[p] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < nterm) {
        const int a = i < nrt ? t * k + i / nI : Tk + t;
        const int nb = i < nrt ? i % nI : i - nrt;
        v[p] = *reinterpret_cast<const float4*>(part + ((int64_t)a * nbs + nb) * H + col);
      }
    }
#pragma unroll
    for (int p = 0; p < kFuBatch; p++) {
      acc.x += v[p].x;
      acc.y += v[p].y;
      acc.z += v[p].z;
      acc.w += v[p].w;
    }
  }
  red4[tg][c4] = acc;
  __syncthreads();
  if (tid < 16) {
    float4 sm = red4[0][tid];
    for (int g = 1; g < kRedGroups; g++) {
      const float4 v = red4[g][tid];
      sm.x += v.x;
      sm.y += v.y;
      sm.z += v.z;
      sm.w += v.w;
    }
    *reinterpret_cast<float4*>(C.y + (int64_t)t * H + sl * kRedCols + tid * 4) = sm;
  }
}

__global__ __launch_bounds__(kFuThreads) void k_gemv_experts(LayerArgs L, ChunkArgs C, const float* logits,
                                                            float* __restrict__ part, int nbs) {
  const int slot = (int)blockIdx.x / nbs, nb = (int)blockIdx.x - slot * nbs;
  const int T = C.T, H = L.H, G = H / kGroup, E = L.E, k = L.k, N = T * k;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, col = lane & 31;
  extern __shared__ __attribute__((aligned(16))) uint8_t gsm[];  // [T][H] x rows, then [T][2E+16] top-k lists
  uint16_t* xl = reinterpret_cast<uint16_t*>(gsm);
  int* lists = reinterpret_cast<int*>(gsm + (size_t)T * H * 2);
  __shared__ float xs[kGemvMaxRows * kMaxGroups];
  __shared__ int s_ids[kMaxAssign];
  __shared__ float s_tw[kMaxAssign];
  __shared__ uint32_t s_bm[kMaxE / 32];
  __shared__ int tok[kGemvMaxRows], arow[kGemvMaxRows], s_info[2];
  __shared__ float wgt[kGemvMaxRows], s_hs[kGemvMaxRows];
  __shared__ __attribute__((aligned(16))) uint32_t s_h[kGemvMaxRows][16];  // bf16 h of the 32 columns, as pairs
  __shared__ float red[kFuWaves][kGemvMaxRows][2][32];

  // ---- activation rows into registers (their latency overlaps the top-k) ----
  const int H8 = H / 8, nx = T * H8;
  uint4 xr0 = make_uint4(0u, 0u, 0u, 0u), xr1 = xr0;
  if (tid < nx) xr0 = reinterpret_cast<const uint4*>(C.x)[tid];
  if (tid + kFuThreads < nx) xr1 = reinterpret_cast<const uint4*>(C.x)[tid + kFuThreads];
  // ---- top-k of each row ----
  if (wave < T) topk_small(logits + (int64_t)wave * E, E, k, wave, s_ids, s_tw, lists + wave * (2 * E + 16));
  if (tid < nx) reinterpret_cast<uint4*>(xl)[tid] = xr0;
  if (tid + kFuThreads < nx) reinterpret_cast<uint4*>(xl)[tid + kFuThreads] = xr1;
  for (int i = tid + 2 * kFuThreads; i < nx; i += kFuThreads)
    reinterpret_cast<uint4*>(xl)[i] = reinterpret_cast<const uint4*>(C.x)[i];
  if (tid < kMaxE / 32) s_bm[tid] = 0u;
  __syncthreads();

  // ---- this workgroup's expert (the slot-th smallest selected one, or the
  // shared expert at slot = number of selected experts) and its rows in flat
  // assignment order (wave 0) ----
  if (wave == 0 && T == 1) {
    // One row: its k experts are distinct, the slot-th smallest is found by rank.
    const int id = lane < k ? s_ids[lane] : 0x7fffffff;
    int rank = 0;
    for (int i = 0; i < k; i++) rank += __builtin_amdgcn_readlane(id, i) < id ? 1 : 0;
    if (lane < k && rank == slot) {
      tok[0] = 0;
      arow[0] = lane;
      wgt[0] = s_tw[lane];
      s_info[0] = id;
      s_info[1] = 1;
    }
    if (lane == 0 && slot >= k) {
      const bool sh = slot == k && L.Is > 0;
      tok[0] = 0;
      arow[0] = N;
      wgt[0] = 1.f;
      s_info[0] = slot == k ? L.E : -1;
      s_info[1] = sh ? 1 : 0;
    }
  } else if (wave == 0) {
    const int id0 = lane < N ? s_ids[lane] : -1, id1 = lane + 64 < N ? s_ids[lane + 64] : -1;
    if (id0 >= 0) atomicOr(&s_bm[id0 >> 5], 1u << (id0 & 31));
    if (id1 >= 0) atomicOr(&s_bm[id1 >> 5], 1u << (id1 & 31));
    __builtin_amdgcn_wave_barrier();
    const int nw = (E + 31) / 32;
    const uint32_t word = lane < nw ? s_bm[lane] : 0u;
    const int cnt = __popc(word);
    const int incl = wave_incl_scan(cnt);
    const int nact = __shfl(incl, 63);
    int e = -1;
    if (slot < nact) {
      const bool here = incl > slot && incl - cnt <= slot;
      const uint64_t hm = __ballot(here);
      const int wl = __ffsll((unsigned long long)hm) - 1;
      const uint32_t wv = __shfl(word, wl);
      int r = slot - (__shfl(incl, wl) - __shfl(cnt, wl));
      uint32_t v = wv;
      for (; r > 0; r--) v &= v - 1;
      e = wl * 32 + (__ffs(v) - 1);
    }
    const bool shared = slot == nact;
    int rows = 0;
    if (e >= 0) {
      const uint64_t m0 = __ballot(id0 == e), m1 = __ballot(id1 == e);
      const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      rows = __popcll(m0) + __popcll(m1);
      if (id0 == e) {
        const int r = __popcll(m0 & lt);
        tok[r] = lane / k;
        arow[r] = lane;
        wgt[r] = s_tw[lane];
      }
      if (id1 == e) {
        const int r = __popcll(m0) + __popcll(m1 & lt);
        tok[r] = (lane + 64) / k;
        arow[r] = lane + 64;
        wgt[r] = s_tw[lane + 64];
      }
    } else if (shared && L.Is > 0) {
      rows = T;
      if (lane < T) {
        tok[lane] = lane;
        arow[lane] = N + lane;
        wgt[lane] = 1.f;
      }
    }
    if (lane == 0) {
      s_info[0] = shared ? L.E : e;
      s_info[1] = rows;
    }
  }
  __syncthreads();
  const int e = s_info[0], rows = s_info[1];
  const bool shared = e == L.E;
  const int Iw = shared ? L.Is : L.I;
  if (rows == 0 || nb * 32 >= Iw) return;  // workgroup-uniform
  const uint8_t* ebase = expert_base(L, e);
  const uint8_t* wbase = ebase + (int64_t)nb * G * 2 * kBlockBytes;

  // ---- gate/up codes of the wave's groups, and the first down outputs' codes ----
  uint4 cg[kGuPref], cu[kGuPref];
  uint32_t sbg[kGuPref], sbu[kGuPref];
  auto load = [&](int g0) {
#pragma unroll
    for (int p = 0; p < kGuPref; p++) {
      const int g = g0 + p * kFuWaves;
      if (g < G) {
        const uint8_t* blk = wbase + (int64_t)g * 2 * kBlockBytes;
        cg[p] = *reinterpret_cast<const uint4*>(blk + lane * 16);
        cu[p] = *reinterpret_cast<const uint4*>(blk + kBlockBytes + lane * 16);
        sbg[p] = *reinterpret_cast<const uint32_t*>(blk + kCodeBytes + col * 4);
        sbu[p] = *reinterpret_cast<const uint32_t*>(blk + kBlockBytes + kCodeBytes + col * 4);
      }
    }
  };
  // Down matrix: output row n sits in block (n / 32, nb / 2) as row n % 32;
  // this workgroup's 32 columns are the lane half nb % 2 of that block.
  const int Gd = Iw / kGroup, hh = nb & 1;
  const uint8_t* dbase = ebase + (shared ? L.shared_gateup_bytes : L.gateup_bytes) + (int64_t)(nb >> 1) * kBlockBytes;
  uint4 dq[kFuDn];
  uint32_t dsb[kFuDn];
  auto load_dn = [&](int c) {
#pragma unroll
    for (int p = 0; p < kFuDn; p++) {
      const int n = tid + kFuThreads * (p + kFuDn * c);
      if (n < H) {
        const uint8_t* blk = dbase + (int64_t)(n >> 5) * Gd * kBlockBytes;
        dq[p] = *reinterpret_cast<const uint4*>(blk + (hh * 32 + (n & 31)) * 16);
        dsb[p] = *reinterpret_cast<const uint32_t*>(blk + kCodeBytes + (n & 31) * 4);
      }
    }
  };
  load(wave);
  load_dn(0);

  // Per-group activation sums while the codes are in flight: 8 lanes per
  // group, 8 columns each, then a 3-step shuffle tree.
  for (int i0 = 0; i0 < T * G * 8; i0 += kFuThreads) {
    const int i = i0 + tid, gi = i >> 3, part8 = i & 7;
    float sm = 0.f;
    if (gi < T * G) {
      const int t = gi / G, g = gi - t * G;
      const uint4 v = *reinterpret_cast<const uint4*>(xl + t * H + g * kGroup + part8 * 8);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; j++) sm += bf16_bits_to_f32(w[j] & 0xFFFFu) + bf16_bits_to_f32(w[j] >> 16);
    }
    sm += __shfl_xor(sm, 1);
    sm += __shfl_xor(sm, 2);
    sm += __shfl_xor(sm, 4);
    if (gi < T * G && part8 == 0) xs[gi] = sm;
  }
  __syncthreads();

  // ---- gate/up dot products ----
  float accg[kGemvMaxRows], accu[kGemvMaxRows];
#pragma unroll
  for (int j = 0; j < kGemvMaxRows; j++) accg[j] = accu[j] = 0.f;
  for (int g0 = wave; g0 < G; g0 += kGuPref * kFuWaves) {
    if (g0 != wave) load(g0);
#pragma unroll
    for (int p = 0; p < kGuPref; p++) {
      const int g = g0 + p * kFuWaves;
      if (g >= G) break;
      uint32_t qg[16], qu[16];
      expand_codes(cg[p].x, qg + 0);
      expand_codes(cg[p].y, qg + 4);
      expand_codes(cg[p].z, qg + 8);
      expand_codes(cg[p].w, qg + 12);
      expand_codes(cu[p].x, qu + 0);
      expand_codes(cu[p].y, qu + 4);
      expand_codes(cu[p].z, qu + 8);
      expand_codes(cu[p].w, qu + 12);
      const float sg = bf16_bits_to_f32(sbg[p] & 0xFFFFu), bpg = bf16_bits_to_f32(sbg[p] >> 16) - 128.f * sg;
      const float su = bf16_bits_to_f32(sbu[p] & 0xFFFFu), bpu = bf16_bits_to_f32(sbu[p] >> 16) - 128.f * su;
#pragma unroll
      for (int j = 0; j < kGemvMaxRows; j++) {
        if (j < rows) {
          const int t = tok[j];
          const uint4* xp = reinterpret_cast<const uint4*>(xl + t * H + g * kGroup + h * 32);
          float dg = 0.f, du = 0.f;
#pragma unroll
          for (int c = 0; c < 4; c++) {
            const uint4 xv = xp[c];
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
              dg = dot2_bf16(qg[4 * c + i], xw[i], dg);
              du = dot2_bf16(qu[4 * c + i], xw[i], du);
            }
          }
          const float xsv = h == 0 ? xs[t * G + g] : 0.f;
          accg[j] = fmaf(sg, dg, fmaf(bpg, xsv, accg[j]));
          accu[j] = fmaf(su, du, fmaf(bpu, xsv, accu[j]));
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kGemvMaxRows; j++) {
    if (j < rows) {
      accg[j] += __shfl_xor(accg[j], 32);
      accu[j] += __shfl_xor(accu[j], 32);
      if (h == 0) {
        red[wave][j][0][col] = accg[j];
        red[wave][j][1][col] = accu[j];
      }
    }
  }
  __syncthreads();
  // ---- SwiGLU: thread 32*j + n finishes row j, column n; h is rounded to
  // bf16 and its 32-column sum taken for the down fold ----
  if (tid < kGemvMaxRows * 32) {
    const int j = tid >> 5, n = tid & 31;
    const bool ok = j < rows;
    float gs = 0.f, us = 0.f;
    if (ok) {
#pragma unroll
      for (int w = 0; w < kFuWaves; w++) {
        gs += red[w][j][0][n];
        us += red[w][j][1][n];
      }
    }
    const uint16_t hb = f32_to_bf16_rne(silu_mul(gs, us));
    float hs = ok ? bf16_bits_to_f32(hb) : 0.f;
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) hs += __shfl_xor(hs, off);
    if (ok) {
      reinterpret_cast<uint16_t*>(s_h[j])[n] = hb;
      if (n == 0) s_hs[j] = hs;
    }
  }
  __syncthreads();

  // ---- down projection of the 32 columns: partial outputs, weighted ----
  const int nrounds = (H + kFuThreads * kFuDn - 1) / (kFuThreads * kFuDn);
  for (int c = 0; c < nrounds; c++) {
    if (c != 0) load_dn(c);
#pragma unroll
    for (int p = 0; p < kFuDn; p++) {
      const int n = tid + kFuThreads * (p + kFuDn * c);
      if (n >= H) break;
      uint32_t q[16];
      expand_codes(dq[p].x, q + 0);
      expand_codes(dq[p].y, q + 4);
      expand_codes(dq[p].z, q + 8);
      expand_codes(dq[p].w, q + 12);
      const float s = bf16_bits_to_f32(dsb[p] & 0xFFFFu), bp = bf16_bits_to_f32(dsb[p] >> 16) - 128.f * s;
      for (int j = 0; j < rows; j++) {
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i++) d = dot2_bf16(q[i], s_h[j][i], d);
        part[((int64_t)arow[j] * nbs + nb) * H + n] = wgt[j] * fmaf(s, d, bp * s_hs[j]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_gemv_experts(const LayerArgs& L, const ChunkArgs& C, const float* logits, float* part,
                               hipStream_t s, const KTime& kt) {
  const int Imax = L.I > L.Is ? L.I : L.Is;
  const int n_slots = (L.E < C.Tk ? L.E : C.Tk) + 1;
  const int nbs = Imax / 32;
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = lds_limit_once(reinterpret_cast<const void*>(&k_gemv_experts), kGuSmemMax, lds_set);
  if (e != hipSuccess) return e;
  const size_t smem = (size_t)C.T * L.H * 2 + (size_t)C.T * (2 * L.E + 16) * 4;
  if (smem > (size_t)kGuSmemMax || C.T > kGemvMaxRows || C.Tk > kMaxAssign) return hipErrorInvalidValue;
  MOE_LAUNCH(k_gemv_experts, dim3((unsigned)(n_slots * nbs)), dim3(kFuThreads), smem, s, kt.start, kt.stop, L, C,
             logits, part, nbs);
  return hipGetLastError();
}

hipError_t launch_gemv_reduce(const LayerArgs& L, const ChunkArgs& C, const float* part, hipStream_t s,
                              const KTime& kt) {
  const int Imax = L.I > L.Is ? L.I : L.Is;
  if (L.H % kRedCols != 0) return hipErrorInvalidValue;
  MOE_LAUNCH(k_gemv_reduce, dim3((unsigned)(C.T * (L.H / kRedCols))), dim3(kFuThreads), 0, s, kt.start, kt.stop, L,
             C, part, Imax / 32);
  return hipGetLastError();
}

}  // namespace moe
