// Row-parallel GEMV for decode ("Optimizing on-device inference for Apple
// Silicon", section "Optimise the one-row weight path": waves cooperate on the
// outputs while reading different parts of the weight matrix; section
// "Reduce intermediate and state traffic" for the two fused chains).
//
// With one to a few rows the layer is bound by weight bytes, so each expert's
// packed weights are streamed once.  A wave reads one 1152-byte gate or up
// block (32 output rows x one 64-column group) with a single 16-byte load per
// lane, so a lane holds 32 codes of one output row, in the lane order of the
// MFMA B operand; every wave issues the loads of all its blocks before it
// computes.  Gate/up runs on v_mfma_f32_32x32x16_f16 with the rows (up to 8)
// as the A operand: the expansion of the codes to fp16 is the only per-code
// vector work, and the per-group scale and bias are applied to the group's
// dot products (affine fold) instead of to every weight.  The down projection
// expands codes to bf16 pairs (128 + q) for v_dot2_f32_bf16 with h, carried as
// two bf16 parts hi = bf16(h) and lo = bf16(h - hi) (about 16 significant
// bits), folded as
//   acc += s * (dot(hi) + dot(lo)) + (b - 128 s) * sum(hi + lo over the group).
// The down projection is split along the intermediate: the workgroup that
// produced 32 columns of h applies the matching 32 columns of the down matrix
// (half of each down block, loaded in the same round as gate/up) and writes a
// partial output row; a second kernel sums the partials of each token in a
// fixed order.  No atomics touch the outputs.
#include "launch.h"
#include "small_route.h"

namespace moe {

constexpr int kGemvMaxRows = 8;
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// 8 bf16 activations -> fp16 of value / 256.
__device__ __forceinline__ uint4 to_f16x8_scaled(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; j++) o[j] = f32_to_f16_scaled(w[j] & 0xFFFFu) | ((uint32_t)f32_to_f16_scaled(w[j] >> 16) << 16);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t b) { return (a & mask) | b; }

// The 8 codes of one dword as fp16 pairs for k-slots 0..7 of an MFMA step
// (slot 2i holds nibble i, slot 2i+1 nibble i+4): slots {0,1,4,5} get
// 1024 + q (the nibble in mantissa bits 0-3 of 1024), slots {2,3,6,7} get
// 64 + q (the nibble in bits 4-7, which weigh 1/16 at the exponent of 64).
__device__ __forceinline__ void expand_codes_f16(uint32_t d, uint32_t m1024, uint32_t m64, uint32_t out[4]) {
  const uint32_t d8 = d >> 8;
  out[0] = and_or(d, 0x000F000Fu, m1024);
  out[1] = and_or(d, 0x00F000F0u, m64);
  out[2] = and_or(d8, 0x000F000Fu, m1024);
  out[3] = and_or(d8, 0x00F000F0u, m64);
}
constexpr int kGuPref = 2;     // groups per wave whose gate/up loads are issued together
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
constexpr int kRedThreads = 512;                 // threads of a reduce workgroup
constexpr int kRedCols = 64;                     // output columns per reduce workgroup
constexpr int kRedC4 = kRedCols / 4;             // float4 columns of a reduce workgroup
constexpr int kRedGroups = kRedThreads / kRedC4; // term groups of a reduce workgroup
constexpr int kFuDn = 4;                     // down outputs per thread per load round
constexpr int kFuBatch = 8;                  // partials a reduce thread loads together

// y[t][64 columns] = sum of token t's partials in a fixed order (routed
// assignments j = 0..k-1 with blocks nb ascending, then the shared expert's
// blocks), so y does not depend on the order in which workgroups ran.
// grid = T x H/64.
__global__ __launch_bounds__(kRedThreads) void k_gemv_reduce(LayerArgs L, ChunkArgs C, const float* __restrict__ part,
                                                           int nbs) {
  __shared__ float4 red4[kRedGroups][kRedC4];
  const int tid = threadIdx.x;
  const int H = L.H, k = L.k, Tk = C.Tk;
  const int nslice = H / kRedCols;
  const int t = (int)blockIdx.x / nslice, sl = (int)blockIdx.x - t * nslice;
  const int c4 = tid % kRedC4, tg = tid / kRedC4;
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
  if (tid < kRedC4) {
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

// ---------------------------------------------------------------------------
// Prologue of a decode workgroup (any multiple of 64 threads): the activation rows
// into LDS as fp16(x / 256) (xl, [T][H]), the top-k of each row (wave t for
// row t; `ordered` = false lists a row's experts in expert order when exactly k
// logits pass the threshold, which is all the split-down GEMV needs, while
// true ranks them as the routing outputs do), then this workgroup's expert
// and its rows in flat assignment order: s_info = (expert, rows), tok/arow/wgt
// per row.  Slot i is the i-th smallest selected expert and slot = number of
// selected experts the shared expert, except that with two rows or more the
// shared expert (when there is one) takes slot 0 and the selected experts
// slots 1, 2, ...: it then has the most rows of any expert, and its
// workgroups, which need no routing, skip the top-k and start first (one
// cold decode call of 2, 4 or 8 rows: 26.2 -> 24.5, 34.2 -> 32.0, 55.8 ->
// 50.3 us; with one row no change, so the order there is kept).  Ends with a
// barrier.
__device__ __forceinline__ void decode_prologue(const LayerArgs& L, const ChunkArgs& C, const float* logits, int slot,
                                                bool ordered, uint16_t* xl, int* lists, int* s_ids, float* s_tw,
                                                uint32_t* s_bm, int* tok, int* arow, float* wgt, int* s_info) {
  const int T = C.T, H = L.H, E = L.E, k = L.k, N = T * k;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int wave = tid >> 6, lane = tid & 63;
  const bool sh_first = T > 1 && L.Is > 0;
  const bool sh_slot = sh_first && slot == 0;  // workgroup-uniform
  const int rs = slot - (sh_first ? 1 : 0);    // routed slot index
  // ---- activation rows into registers (their latency overlaps the top-k) ----
  const int H8 = H / 8, nx = T * H8;
  uint4 xr0 = make_uint4(0u, 0u, 0u, 0u), xr1 = xr0;
  if (tid < nx) xr0 = reinterpret_cast<const uint4*>(C.x)[tid];
  if (tid + nthr < nx) xr1 = reinterpret_cast<const uint4*>(C.x)[tid + nthr];
  // ---- top-k of each row ----
  if (!sh_slot && wave < T)
    topk_small(logits + (int64_t)wave * E, E, k, wave, s_ids, s_tw, lists + wave * (2 * E + 16), ordered);
  if (tid < nx) reinterpret_cast<uint4*>(xl)[tid] = to_f16x8_scaled(xr0);
  if (tid + nthr < nx) reinterpret_cast<uint4*>(xl)[tid + nthr] = to_f16x8_scaled(xr1);
  for (int i = tid + 2 * nthr; i < nx; i += nthr)
    reinterpret_cast<uint4*>(xl)[i] = to_f16x8_scaled(reinterpret_cast<const uint4*>(C.x)[i]);
  if (tid < kMaxE / 32) s_bm[tid] = 0u;
  __syncthreads();

  // ---- this workgroup's expert and its rows in flat assignment order (wave 0) ----
  if (sh_slot) {
    if (tid < T) {
      tok[tid] = tid;
      arow[tid] = N + tid;
      wgt[tid] = 1.f;
    }
    if (tid == 0) {
      s_info[0] = L.E;
      s_info[1] = T;
    }
  } else if (wave == 0 && T == 1) {
    // One row: its k experts are distinct, the rs-th smallest is found by rank.
    const int id = lane < k ? s_ids[lane] : 0x7fffffff;
    int rank = 0;
    for (int i = 0; i < k; i++) rank += __builtin_amdgcn_readlane(id, i) < id ? 1 : 0;
    if (lane < k && rank == rs) {
      tok[0] = 0;
      arow[0] = lane;
      wgt[0] = s_tw[lane];
      s_info[0] = id;
      s_info[1] = 1;
    }
    if (lane == 0 && rs >= k) {
      const bool sh = rs == k && L.Is > 0;
      tok[0] = 0;
      arow[0] = N;
      wgt[0] = 1.f;
      s_info[0] = sh ? L.E : -1;
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
    const int nact = lane_value(incl, 63);
    int e = -1;
    if (rs < nact) {
      const bool here = incl > rs && incl - cnt <= rs;
      const uint64_t hm = __ballot(here);
      const int wl = __ffsll((unsigned long long)hm) - 1;
      const uint32_t wv = (uint32_t)lane_value((int)word, wl);
      int r = rs - (lane_value(incl, wl) - lane_value(cnt, wl));
      uint32_t v = wv;
      for (; r > 0; r--) v &= v - 1;
      e = wl * 32 + (__ffs(v) - 1);
    }
    // (Two rows or more: the shared expert, if any, is slot 0, handled above.)
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
    }
    if (lane == 0) {
      s_info[0] = e;
      s_info[1] = rows;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kFuThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_gemv_experts(LayerArgs L, ChunkArgs C, const float* logits,
                                                            float* __restrict__ part, int nbs) {
  const int slot = (int)blockIdx.x / nbs, nb = (int)blockIdx.x - slot * nbs;
  const int T = C.T, H = L.H, G = H / kGroup;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, col = lane & 31;
  // [T][H] x rows as fp16(x / 256), then [T][2E+16] top-k lists
  extern __shared__ __attribute__((aligned(16))) uint8_t gsm[];
  uint16_t* xl = reinterpret_cast<uint16_t*>(gsm);
  int* lists = reinterpret_cast<int*>(gsm + (size_t)T * H * 2);
  // [g][row] sums of the fp16 activations over the slots biased by 1024 (xsa) and by 64 (xsb)
  __shared__ __attribute__((aligned(16))) float xsa[kMaxGroups * kGemvMaxRows];
  __shared__ __attribute__((aligned(16))) float xsb[kMaxGroups * kGemvMaxRows];
  __shared__ int s_ids[kMaxAssign];
  __shared__ float s_tw[kMaxAssign];
  __shared__ uint32_t s_bm[kMaxE / 32];
  __shared__ int tok[kGemvMaxRows], arow[kGemvMaxRows], s_info[2];
  __shared__ float wgt[kGemvMaxRows], s_hs[kGemvMaxRows];
  // h of the 32 columns as two bf16 parts (hi = bf16(h), lo = bf16(h - hi)), as pairs
  __shared__ __attribute__((aligned(16))) uint32_t s_h[kGemvMaxRows][16];
  __shared__ __attribute__((aligned(16))) uint32_t s_hl[kGemvMaxRows][16];
  __shared__ float red[kFuWaves][kGemvMaxRows][2][32];

  decode_prologue(L, C, logits, slot, false, xl, lists, s_ids, s_tw, s_bm, tok, arow, wgt, s_info);
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

  // Per-group activation sums of the workgroup's rows while the codes are in
  // flight, split by the bias of the slots they meet (columns 8i + {0,1,4,5}
  // and 8i + {2,3,6,7}): 8 lanes per (row, group), 8 columns each, then a
  // 3-step shuffle tree.
  for (int i0 = 0; i0 < rows * G * 8; i0 += kFuThreads) {
    const int i = i0 + tid, gj = i >> 3, part8 = i & 7;
    const bool ok = gj < rows * G;
    const int j = ok ? gj / G : 0, g = gj - j * G;
    float sa = 0.f, sb = 0.f;
    if (ok) {
      const uint4 v = *reinterpret_cast<const uint4*>(xl + tok[j] * H + g * kGroup + part8 * 8);
      sa = (f16_bits_to_f32(v.x & 0xFFFFu) + f16_bits_to_f32(v.x >> 16)) +
           (f16_bits_to_f32(v.z & 0xFFFFu) + f16_bits_to_f32(v.z >> 16));
      sb = (f16_bits_to_f32(v.y & 0xFFFFu) + f16_bits_to_f32(v.y >> 16)) +
           (f16_bits_to_f32(v.w & 0xFFFFu) + f16_bits_to_f32(v.w >> 16));
    }
    // 8-lane sums: pairs, quads, then the next quad into lanes 0-3 of the group (row_shl:4).
    sa += dpp_f32<0xB1>(sa);
    sb += dpp_f32<0xB1>(sb);
    sa += dpp_f32<0x4E>(sa);
    sb += dpp_f32<0x4E>(sb);
    sa += dpp_f32<0x104>(sa);
    sb += dpp_f32<0x104>(sb);
    if (ok && part8 == 0) {
      xsa[g * kGemvMaxRows + j] = sa;
      xsb[g * kGemvMaxRows + j] = sb;
    }
  }
  __syncthreads();

  // ---- gate/up: per group, four v_mfma_f32_32x32x16_f16 steps per matrix ----
  // A: lane l supplies row m = l % 32 of the workgroup's rows (rows past the
  // count repeat the last one; their results are never read) with the fp16
  // activations x' = x / 256 of input columns 32h + 8c .. +7 of the group in
  // step c, the k-slots the packer gave the lane's codes.  B: the lane's 8
  // codes of the step as fp16 1024 + q or 64 + q (expand_codes_f16).  Per
  // group D = sum_k x' (q + o_k), o_k the slot's bias, and with s' = 256 s,
  // b' = 256 b the affine fold is
  //   acc += s' D + (b' - 1024 s') Xa + (b' - 64 s') Xb
  // (Xa, Xb: the row's sums of x' over the slots biased by 1024 and by 64).
  // The accumulators hold column n = l % 32 and rows 4h + i in register i.
  uint32_t m1024, m64;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m1024));
  asm volatile("v_mov_b32 %0, 0x54005400" : "=v"(m64));
  const uint16_t* xrow = xl + tok[(lane & 31) < rows ? (lane & 31) : rows - 1] * H + h * 32;
  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  for (int g0 = wave; g0 < G; g0 += kGuPref * kFuWaves) {
    if (g0 != wave) load(g0);
#pragma unroll
    for (int p = 0; p < kGuPref; p++) {
      const int g = g0 + p * kFuWaves;
      if (g >= G) break;
      const uint32_t cgw[4] = {cg[p].x, cg[p].y, cg[p].z, cg[p].w};
      const uint32_t cuw[4] = {cu[p].x, cu[p].y, cu[p].z, cu[p].w};
      f32x16_t dg = {}, du = {};
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const f16x8_t a = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4*>(xrow + g * kGroup + 8 * c));
        uint4 q;
        expand_codes_f16(cgw[c], m1024, m64, reinterpret_cast<uint32_t*>(&q));
        dg = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, __builtin_bit_cast(f16x8_t, q), dg, 0, 0, 0);
        expand_codes_f16(cuw[c], m1024, m64, reinterpret_cast<uint32_t*>(&q));
        du = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, __builtin_bit_cast(f16x8_t, q), du, 0, 0, 0);
      }
      const float sg = 256.f * f16_bits_to_f32(sbg[p] & 0xFFFFu), bg = 256.f * f16_bits_to_f32(sbg[p] >> 16);
      const float su = 256.f * f16_bits_to_f32(sbu[p] & 0xFFFFu), bu = 256.f * f16_bits_to_f32(sbu[p] >> 16);
      const float cga = bg - 1024.f * sg, cgb = bg - 64.f * sg, cua = bu - 1024.f * su, cub = bu - 64.f * su;
      const float4 xav = *reinterpret_cast<const float4*>(&xsa[g * kGemvMaxRows + 4 * h]);
      const float4 xbv = *reinterpret_cast<const float4*>(&xsb[g * kGemvMaxRows + 4 * h]);
      const float xa[4] = {xav.x, xav.y, xav.z, xav.w}, xb[4] = {xbv.x, xbv.y, xbv.z, xbv.w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        accg[i] = fmaf(sg, dg[i], fmaf(cga, xa[i], fmaf(cgb, xb[i], accg[i])));
        accu[i] = fmaf(su, du[i], fmaf(cua, xa[i], fmaf(cub, xb[i], accu[i])));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; i++) {
    if (4 * h + i < rows) {
      red[wave][4 * h + i][0][col] = accg[i];
      red[wave][4 * h + i][1][col] = accu[i];
    }
  }
  __syncthreads();
  // ---- SwiGLU: thread 32*j + n finishes row j, column n; h is split into
  // bf16 hi and lo parts and their 32-column sum taken for the down fold ----
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
    const float hv = silu_mul(gs, us);
    const uint16_t hb = f32_to_bf16_rne(hv);
    const uint16_t hl = f32_to_bf16_rne(hv - bf16_bits_to_f32(hb));  // hv - hi is exact in fp32
    float hs = ok ? bf16_bits_to_f32(hb) + bf16_bits_to_f32(hl) : 0.f;
    // 32-lane sum (two rows of lanes): row sums, then lanes 0 and 32 add rows 1 and 3.
    hs = row_sum16(hs);
    const float r1 = lane_value(hs, 16), r3 = lane_value(hs, 48);
    hs += lane < 32 ? r1 : r3;
    if (ok) {
      reinterpret_cast<uint16_t*>(s_h[j])[n] = hb;
      reinterpret_cast<uint16_t*>(s_hl[j])[n] = hl;
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
      const float s = f16_bits_to_f32(dsb[p] & 0xFFFFu), bp = f16_bits_to_f32(dsb[p] >> 16) - 128.f * s;
      for (int j = 0; j < rows; j++) {
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i++) d = dot2_bf16(q[i], s_h[j][i], d);
#pragma unroll
        for (int i = 0; i < 16; i++) d = dot2_bf16(q[i], s_hl[j][i], d);
        part[((int64_t)arow[j] * nbs + nb) * H + n] = wgt[j] * fmaf(s, d, bp * s_hs[j]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode with the grouped-GEMM path's arithmetic (batch-invariant decode,
// desc.batch_invariant = 1).  The GEMV path above folds scale and bias per
// group and splits the down projection, so its bits differ from the grouped
// GEMM's; these two kernels compute each output element with exactly the
// operations of the grouped-GEMM path, so a row's output is the same at any
// row count and on either side of the row threshold (the dothoosh page on
// Candle's Metal kernels, the section on outputs that change with the kernel
// chosen by row count):
//  * gate/up: the same fp16(x / 256) activations and fp16 weights rebuilt
//    with one rounding of s*q + b (dequant_f16, the grouped GEMM's rebuild),
//    the same v_mfma_f32_32x32x16_f16 steps in the same order over K into one
//    fp32 accumulator per element, starting from zero, with the grouped GEMM's
//    padding of the group count to a multiple of 4 (zero weights, valid A);
//    then silu(256 g) * 256 u rounded to fp16(h / 256);
//  * down: the same chain over the intermediate's groups; routed outputs
//    and the shared expert's output alike rounded to fp16(o / 256);
//  * combine: y = 256 * shared + sum over j in top-k rank order of
//    fma(256 w_tj, o_tj, y), the routing weights from the ranked top-k.
// An MFMA output element depends only on its row of A and its column of B, so
// which other rows share the A operand does not change it.
//
// Gate/up (k_gemv_gateup_bi): one workgroup per (slot, 32 intermediate
// columns), like the GEMV.  The chain over K is sequential, so it is handed
// from wave to wave: each wave loads and rebuilds the weights of four groups
// of one matrix in parallel with the others, then, in step order, continues
// its matrix's accumulators (passed through LDS) over its groups.  Gate and up
// are two chains on different SIMDs; only the MFMAs of each chain are serial,
// the loads and the rebuild are not.
// Down + combine (k_gemv_down_bi): one workgroup per (32 output columns,
// token); each wave runs the chain of one of the token's rows (routed rows in
// rank order, then the shared row), then the workgroup combines them in rank
// order and writes y once.
// ---------------------------------------------------------------------------
constexpr int kBiGroupsPerWave = 4;
constexpr int kBiDnWaves = 16;

__device__ __forceinline__ uint16_t to_f16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

typedef _Float16 f16x2b_t __attribute__((ext_vector_type(2)));

// fp16 weights of one packed dword (8 codes) rebuilt as fp16(s*q + b), the
// k-slot order of the MFMA B operand: the grouped GEMM's rebuild (the
// exponent of 1024 gives nibbles 0-3 unit steps, that of 64 nibbles 4-7;
// the offsets are removed exactly and one fp16 FMA per pair rounds s*q + b).
__device__ __forceinline__ f16x8_t dequant_f16(uint32_t d, f16x2b_t s2, f16x2b_t b2) {
  const f16x2b_t off_lo = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  const f16x2b_t off_hi = {(_Float16)-64.0f, (_Float16)-64.0f};
  const uint32_t d8 = d >> 8;
  const f16x2b_t q0 = __builtin_bit_cast(f16x2b_t, and_or(d, 0x000F000Fu, 0x64006400u)) + off_lo;
  const f16x2b_t q1 = __builtin_bit_cast(f16x2b_t, and_or(d, 0x00F000F0u, 0x54005400u)) + off_hi;
  const f16x2b_t q2 = __builtin_bit_cast(f16x2b_t, and_or(d8, 0x000F000Fu, 0x64006400u)) + off_lo;
  const f16x2b_t q3 = __builtin_bit_cast(f16x2b_t, and_or(d8, 0x00F000F0u, 0x54005400u)) + off_hi;
  return __builtin_bit_cast(
      f16x8_t, make_uint4(__builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q0, s2, b2)),
                          __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q1, s2, b2)),
                          __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q2, s2, b2)),
                          __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q3, s2, b2))));
}

// Scale and bias of a block row (the blob's fp16 pair) broadcast to both
// halves, as the grouped GEMM takes them; zero for padded groups (live = false).
__device__ __forceinline__ void sb_f16(uint32_t sb, bool live, f16x2b_t& s2, f16x2b_t& b2) {
  const f16x2b_t v = __builtin_bit_cast(f16x2b_t, live ? sb : 0u);
  s2 = __builtin_shufflevector(v, v, 0, 0);
  b2 = __builtin_shufflevector(v, v, 1, 1);
}

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int c) { return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w; }

constexpr int kBiUpWaves = 16;  // waves 0-7 carry the gate chain, waves 8-15 the up chain

__global__ __launch_bounds__(kBiUpWaves * 64) __attribute__((amdgpu_waves_per_eu(4, 4)))
void k_gemv_gateup_bi(LayerArgs L, ChunkArgs C, const float* logits, uint16_t* __restrict__ h16,
                      int32_t* __restrict__ ids_out, float* __restrict__ tw_out, int nbs) {
  const int slot = (int)blockIdx.x / nbs, nb = (int)blockIdx.x - slot * nbs;
  const int T = C.T, H = L.H, G = H / kGroup, k = L.k;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, col = lane & 31;
  extern __shared__ __attribute__((aligned(16))) uint8_t gsm[];
  uint16_t* xl = reinterpret_cast<uint16_t*>(gsm);
  int* lists = reinterpret_cast<int*>(gsm + (size_t)T * H * 2);
  __shared__ int s_ids[kMaxAssign];
  __shared__ float s_tw[kMaxAssign];
  __shared__ uint32_t s_bm[kMaxE / 32];
  __shared__ int tok[kGemvMaxRows], arow[kGemvMaxRows], s_info[2];
  __shared__ float wgt[kGemvMaxRows];
  __shared__ f32x16_t hand[2][64];  // the gate and up accumulators handed from wave to wave

  decode_prologue(L, C, logits, slot, true, xl, lists, s_ids, s_tw, s_bm, tok, arow, wgt, s_info);
  // The ranked routing of every row, for the down + combine kernel (the first
  // workgroup of the first routed slot).
  if ((int)blockIdx.x == (T > 1 && L.Is > 0 ? nbs : 0) && tid < T * k) {
    ids_out[tid] = s_ids[tid];
    tw_out[tid] = s_tw[tid];
  }
  const int e = s_info[0], rows = s_info[1];
  const bool shared = e == L.E;
  const int Iw = shared ? L.Is : L.I;
  if (rows == 0 || nb * 32 >= Iw) return;  // workgroup-uniform
  // Chain m (0: gate, 1: up).  Step s of a pass is run by wave s of the gate
  // chain and by wave 8 + (s + 2) % 8 of the up chain, so the two waves of a
  // step sit on different SIMDs (wave w on SIMD w % 4) and their MFMAs overlap.
  const int m = wave >> 3, j = wave & 7;
  const int step = m == 0 ? j : (j + 6) % 8;
  const uint8_t* wbase = expert_base(L, e) + (int64_t)nb * G * 2 * kBlockBytes + m * kBlockBytes;
  // The lane's A row: row col of the workgroup's rows (rows past the count
  // repeat the last one; never stored), input columns 32h + 8c of a group.
  const uint16_t* xrow = xl + tok[col < rows ? col : rows - 1] * H + h * 32;
  const int Gp = (G + 3) & ~3;
  f32x16_t acc = {};
  constexpr int kPass = kFuWaves * kBiGroupsPerWave;
  for (int p0 = 0; p0 < Gp; p0 += kPass) {
    const int g0 = p0 + kBiGroupsPerWave * step;  // this wave's first group in this pass
    f16x8_t bq[kBiGroupsPerWave][4];
    if (g0 < Gp) {
      uint4 cq[kBiGroupsPerWave];
      uint32_t sq[kBiGroupsPerWave];
#pragma unroll
      for (int q = 0; q < kBiGroupsPerWave; q++) {
        const int g = g0 + q, gg = g < G ? g : G - 1;  // padded groups read a valid block, rebuilt as zero
        const uint8_t* blk = wbase + (int64_t)gg * 2 * kBlockBytes;
        cq[q] = *reinterpret_cast<const uint4*>(blk + lane * 16);
        sq[q] = *reinterpret_cast<const uint32_t*>(blk + kCodeBytes + col * 4);
      }
#pragma unroll
      for (int q = 0; q < kBiGroupsPerWave; q++) {
        f16x2b_t s2, b2;
        sb_f16(sq[q], g0 + q < G, s2, b2);
#pragma unroll
        for (int c = 0; c < 4; c++) bq[q][c] = dequant_f16(dword_of(cq[q], c), s2, b2);
      }
    }
    // The chains, in step order: the wave of step s continues its chain's accumulators over its groups.
    for (int st = 0; st < kFuWaves; st++) {
      if (step == st && g0 < Gp) {  // wave-uniform
        if (p0 != 0 || st != 0) acc = hand[m][lane];
#pragma unroll
        for (int q = 0; q < kBiGroupsPerWave; q++) {
          const int g = g0 + q;
          if (g < Gp) {
            const int gg = g < G ? g : G - 1;
#pragma unroll
            for (int c = 0; c < 4; c++) {
              const f16x8_t a = *reinterpret_cast<const f16x8_t*>(xrow + gg * kGroup + 8 * c);
              acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bq[q][c], acc, 0, 0, 0);
            }
          }
        }
        hand[m][lane] = acc;
      }
      __syncthreads();
    }
  }
  // SwiGLU of the grouped GEMM's epilogue, fp16(h / 256) into h16[assignment row].
  if (wave == 0) {
    const f32x16_t accg = hand[0][lane], accu = hand[1][lane];
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int r = 8 * (i >> 2) + 4 * h + (i & 3);
      if (r < rows) {
        const float hv = silu_mul(256.f * accg[i], 256.f * accu[i]);
        h16[(int64_t)arow[r] * C.Imax + nb * 32 + col] = to_f16_bits(hv * (1.f / 256.f));
      }
    }
  }
}

__global__ __launch_bounds__(kBiDnWaves * 64) void k_gemv_down_bi(LayerArgs L, ChunkArgs C, const uint16_t* __restrict__ h16,
                                                                  const int32_t* __restrict__ ids,
                                                                  const float* __restrict__ tw) {
  const int ob = blockIdx.x, t = blockIdx.y;  // 32 output columns of token t
  const int H = L.H, k = L.k, Tk = C.T * k;
  const int nrow = k + (L.Is > 0 ? 1 : 0);  // the token's routed rows in rank order, then its shared row
  const int tid = threadIdx.x, nwave = blockDim.x >> 6;
  const int wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, col = lane & 31;
  __shared__ uint16_t o16[16][32];  // routed outputs, fp16(o / 256)
  __shared__ float ysh[32];         // shared expert's output, 256 * fp16(o / 256)
  for (int j = wave; j < nrow; j += nwave) {  // wave-uniform
    const bool shared = j == k;
    const int a = shared ? Tk + t : t * k + j;  // the row of h
    const int e = shared ? L.E : ids[a];
    const int Iw = shared ? L.Is : L.I, Gd = Iw / kGroup, Gdp = (Gd + 3) & ~3;
    const uint8_t* dbase = expert_base(L, e) + (shared ? L.shared_gateup_bytes : L.gateup_bytes) + (int64_t)ob * Gd * kBlockBytes;
    // Every lane's A row is this assignment's row of h (the one result row read is row 0).
    const uint16_t* hrow = h16 + (int64_t)a * C.Imax + h * 32;
    f32x16_t acc = {};
    // Weight codes of eight groups go out in one round (the cold reads); the
    // rows of h, just written and in L2, four groups at a time.
    for (int g0 = 0; g0 < Gdp; g0 += 8) {
      uint4 cq[8];
      uint32_t sq[8];
#pragma unroll
      for (int q = 0; q < 8; q++) {
        const int g = g0 + q, gg = g < Gd ? g : Gd - 1;
        const uint8_t* blk = dbase + (int64_t)gg * kBlockBytes;
        cq[q] = *reinterpret_cast<const uint4*>(blk + lane * 16);
        sq[q] = *reinterpret_cast<const uint32_t*>(blk + kCodeBytes + col * 4);
      }
#pragma unroll
      for (int q0 = 0; q0 < 8; q0 += 4) {
        if (g0 + q0 >= Gdp) break;  // wave-uniform: Gdp is a multiple of 4
        uint4 av[4][4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int g = g0 + q0 + q, gg = g < Gd ? g : Gd - 1;
#pragma unroll
          for (int c = 0; c < 4; c++) av[q][c] = *reinterpret_cast<const uint4*>(hrow + gg * kGroup + 8 * c);
        }
#pragma unroll
        for (int q = 0; q < 4; q++) {
          f16x2b_t s2, b2;
          sb_f16(sq[q0 + q], g0 + q0 + q < Gd, s2, b2);
#pragma unroll
          for (int c = 0; c < 4; c++)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, av[q][c]),
                                                        dequant_f16(dword_of(cq[q0 + q], c), s2, b2), acc, 0, 0, 0);
        }
      }
    }
    // Row 0 of the result: register 0 of lanes 0..31 (column = lane).
    if (lane < 32) {
      if (shared) ysh[lane] = 256.f * f16_bits_to_f32(to_f16_bits(acc[0]));
      else o16[j][lane] = to_f16_bits(acc[0]);
    }
  }
  __syncthreads();
  // The grouped GEMM's combine: the shared output, then the routed rows in rank order.
  if (tid < 32) {
    float yv = L.Is > 0 ? ysh[tid] : 0.f;
    for (int j = 0; j < k; j++) yv = fmaf(256.f * tw[t * k + j], f16_bits_to_f32(o16[j][tid]), yv);
    C.y[(int64_t)t * H + ob * 32 + tid] = yv;
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

hipError_t launch_gemv_gateup_bi(const LayerArgs& L, const ChunkArgs& C, const float* logits, uint16_t* h16,
                                 int32_t* ids, float* tw, hipStream_t s, const KTime& kt) {
  const int Imax = L.I > L.Is ? L.I : L.Is;
  const int n_slots = (L.E < C.Tk ? L.E : C.Tk) + 1;
  const int nbs = Imax / 32;
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = lds_limit_once(reinterpret_cast<const void*>(&k_gemv_gateup_bi), kGuSmemMax, lds_set);
  if (e != hipSuccess) return e;
  const size_t smem = (size_t)C.T * L.H * 2 + (size_t)C.T * (2 * L.E + 16) * 4;
  if (smem > (size_t)kGuSmemMax || C.T > kGemvMaxRows || C.Tk > kMaxAssign) return hipErrorInvalidValue;
  MOE_LAUNCH(k_gemv_gateup_bi, dim3((unsigned)(n_slots * nbs)), dim3(kBiUpWaves * 64), smem, s, kt.start, kt.stop, L,
             C, logits, h16, ids, tw, nbs);
  return hipGetLastError();
}

hipError_t launch_gemv_down_bi(const LayerArgs& L, const ChunkArgs& C, const uint16_t* h16, const int32_t* ids,
                               const float* tw, hipStream_t s, const KTime& kt) {
  if (L.H % 32 != 0 || C.T > kGemvMaxRows || C.Tk > kMaxAssign || L.k > 16) return hipErrorInvalidValue;
  const int nrow = L.k + (L.Is > 0 ? 1 : 0), nwave = nrow < kBiDnWaves ? nrow : kBiDnWaves;
  MOE_LAUNCH(k_gemv_down_bi, dim3((unsigned)(L.H / 32), (unsigned)C.T), dim3(nwave * 64), 0, s, kt.start, kt.stop, L,
             C, h16, ids, tw);
  return hipGetLastError();
}

hipError_t launch_gemv_reduce(const LayerArgs& L, const ChunkArgs& C, const float* part, hipStream_t s,
                              const KTime& kt) {
  const int Imax = L.I > L.Is ? L.I : L.Is;
  if (L.H % kRedCols != 0) return hipErrorInvalidValue;
  MOE_LAUNCH(k_gemv_reduce, dim3((unsigned)(C.T * (L.H / kRedCols))), dim3(kRedThreads), 0, s, kt.start, kt.stop, L,
             C, part, Imax / 32);
  return hipGetLastError();
}

}  // namespace moe
