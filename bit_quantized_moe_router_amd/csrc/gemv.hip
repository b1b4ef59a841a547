// Row-parallel GEMV for decode ("Optimizing on-device inference for Apple
// Silicon", section "Optimise the one-row weight path": waves cooperate on the
// outputs while reading different parts of the weight matrix; section
// "Reduce intermediate and state traffic" for the two fused chains).
//
// With one to a few rows the layer is bound by weight bytes, so each expert's
// packed weights are streamed once: a wave reads one 1152-byte block (32
// output rows x one 64-column group) with a single 16-byte load per lane, so a
// lane holds 32 codes of one output row.  Every wave issues the loads of
// several blocks before it computes, so most of the working set is in flight
// at once.  Codes expand to bf16 pairs (128 + q) and meet the activation pairs
// in v_dot2_f32_bf16; the per-group affine fold is
//   acc += s * dot + (b - 128 s) * sum(x over the group).
// The two lanes that share an output row are combined with one cross-half
// shuffle, the waves of a workgroup through LDS.  No atomics: every output is
// produced by exactly one workgroup, in a fixed order.
#include "launch.h"

namespace moe {

constexpr int kGemvMaxRows = 8;
constexpr int kGuWaves = 8;    // gate/up workgroup: 8 waves split the H/64 groups
constexpr int kGuPref = 4;     // groups per wave whose loads are issued together
constexpr int kDnWaves = 16;   // down workgroup: 16 waves split the (expert, group) items
constexpr int kDnPref = 4;
constexpr int kMaxGroups = 128;              // H / 64 for H <= 8192
constexpr int kMaxAssign = kGemvMaxRows * 16; // T * k on the GEMV path
constexpr int kMaxSlots = kMaxAssign + 1;     // active experts + the shared expert
constexpr int kDnStageMax = 120 * 1024;       // LDS for staged intermediate rows

// ---------------------------------------------------------------------------
// gate/up + SwiGLU.  grid = (expert slots: active experts, then the shared
// expert; I/32 row blocks).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kGuWaves * 64) void k_gemv_gateup(LayerArgs L, ChunkArgs C) {
  const int slot = blockIdx.x, nb = blockIdx.y;
  const int T = C.T, H = L.H, G = H / kGroup;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, col = lane & 31;
  extern __shared__ uint16_t xl[];  // [T][H]: every row of the chunk
  __shared__ float xs[kGemvMaxRows * kMaxGroups];
  __shared__ int tok[kGemvMaxRows], orow[kGemvMaxRows];
  __shared__ float red[kGuWaves][kGemvMaxRows][2][32];

  // Loads that do not depend on the routing go out first: the chunk's
  // activation rows and their group sums (T <= 8 rows).  The slot's expert
  // is read speculatively (clamped to a valid index) next to n_active.
  const int H8 = H / 8;
  for (int i = tid; i < T * H8; i += blockDim.x) reinterpret_cast<uint4*>(xl)[i] = reinterpret_cast<const uint4*>(C.x)[i];
  for (int i = tid; i < T * G; i += blockDim.x) xs[i] = C.xsum[i];
  const int nact = *C.n_active;
  const int e_spec = C.active[slot < L.E ? slot : L.E - 1];
  const bool shared = slot == nact;
  if (slot > nact || (shared && L.Is == 0)) return;  // workgroup-uniform, before any barrier
  const int e = shared ? L.E : min(max(e_spec, 0), L.E - 1);
  const int Iw = shared ? L.Is : L.I;
  if (nb * 32 >= Iw) return;
  const uint8_t* wbase = expert_base(L, e) + (int64_t)nb * G * 2 * kBlockBytes;

  // This wave's first weight loads.
  uint4 cg[kGuPref], cu[kGuPref];
  uint32_t sbg[kGuPref], sbu[kGuPref];
  auto load = [&](int g0) {
#pragma unroll
    for (int p = 0; p < kGuPref; p++) {
      const int g = g0 + p * kGuWaves;
      if (g < G) {
        const uint8_t* blk = wbase + (int64_t)g * 2 * kBlockBytes;
        cg[p] = *reinterpret_cast<const uint4*>(blk + lane * 16);
        cu[p] = *reinterpret_cast<const uint4*>(blk + kBlockBytes + lane * 16);
        sbg[p] = *reinterpret_cast<const uint32_t*>(blk + kCodeBytes + col * 4);
        sbu[p] = *reinterpret_cast<const uint32_t*>(blk + kBlockBytes + kCodeBytes + col * 4);
      }
    }
  };
  load(wave);

  const int rows = shared ? T : C.counts[e];
  if (tid < rows) {
    tok[tid] = shared ? tid : C.sorted[C.offsets[e] + tid] / L.k;
    orow[tid] = shared ? C.Tk + tid : C.offsets[e] + tid;
  }
  __syncthreads();

  float accg[kGemvMaxRows], accu[kGemvMaxRows];
#pragma unroll
  for (int j = 0; j < kGemvMaxRows; j++) accg[j] = accu[j] = 0.f;

  for (int g0 = wave; g0 < G; g0 += kGuPref * kGuWaves) {
    if (g0 != wave) load(g0);
#pragma unroll
    for (int p = 0; p < kGuPref; p++) {
      const int g = g0 + p * kGuWaves;
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
          // The group's activation sum covers both lane halves: fold it in once.
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
  // Thread 32*j + n finishes row j, column n.
  for (int base = 0; base < kGemvMaxRows * 32; base += blockDim.x) {
    const int j = (base + threadIdx.x) >> 5, n = threadIdx.x & 31;
    const bool ok = j < rows;
    float gs = 0.f, us = 0.f;
    if (ok) {
#pragma unroll
      for (int w = 0; w < kGuWaves; w++) {
        gs += red[w][j][0][n];
        us += red[w][j][1][n];
      }
    }
    const uint16_t hb = f32_to_bf16_rne(silu_mul(gs, us));
    float hs = ok ? bf16_bits_to_f32(hb) : 0.f;
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) hs += __shfl_xor(hs, off);
    if (ok) {
      C.hbuf[(int64_t)orow[j] * C.Imax + nb * 32 + n] = hb;
      if (n == 0) C.hsum[(int64_t)orow[j] * (C.Imax / 32) + nb] = hs;
    }
  }
}

// ---------------------------------------------------------------------------
// down + routing weight + shared add + combine.  grid = H/32 output row
// blocks; the workgroup walks every (expert slot, group) item, waves taking
// items round-robin with their loads issued in batches, and writes y for all
// tokens of the chunk.  The routing tables (slot -> expert, segment, rows;
// sorted position -> token, weight) and, when they fit, all intermediate rows
// and their sums are staged in LDS first, so the item loop only waits for
// the weight codes.  The first batch of codes is issued before the staging,
// from a speculative read of the active list.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kDnWaves * 64) void k_gemv_down(LayerArgs L, ChunkArgs C, int staged) {
  const int nb = blockIdx.x;
  const int H = L.H, T = C.T, Tk = C.Tk;
  const int hsw = C.Imax / 32;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, col = lane & 31;
  const int Gi = L.I / kGroup, Gs = L.Is / kGroup;
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];  // staged h rows, then their sums
  __shared__ int s_e[kMaxSlots], s_seg[kMaxSlots], s_rows[kMaxSlots];
  __shared__ int s_tok[kMaxAssign];
  __shared__ float s_w[kMaxAssign];
  __shared__ float red[kDnWaves][kGemvMaxRows][32];

  const int nact = *C.n_active;
  const int nspec = min(L.E, Tk);  // slots the active list can hold
  // Item it -> (slot, group); the shared expert's items follow the routed ones.
  auto item_expert = [&](int it, int na, int& g) -> int {
    if (it < na * Gi) {
      const int sl = it / Gi;
      g = it - sl * Gi;
      return min(max(C.active[min(sl, nspec - 1)], 0), L.E - 1);
    }
    g = it - na * Gi;
    return L.E;
  };
  const int nitems = nact * Gi + Gs;

  uint4 cd[kDnPref];
  uint32_t sb[kDnPref];
  int pe[kDnPref], pg[kDnPref];
  auto load = [&](int it0) {
#pragma unroll
    for (int p = 0; p < kDnPref; p++) {
      const int it = it0 + p * kDnWaves;
      pe[p] = -1;
      pg[p] = 0;
      if (it < nitems) {
        int g;
        const int e = item_expert(it, nact, g);
        const bool sh = e == L.E;
        const int Gk = sh ? Gs : Gi;
        const uint8_t* blk = expert_base(L, e) + (sh ? L.shared_gateup_bytes : L.gateup_bytes) +
                             (int64_t)(nb * Gk + g) * kBlockBytes;
        cd[p] = *reinterpret_cast<const uint4*>(blk + lane * 16);
        sb[p] = *reinterpret_cast<const uint32_t*>(blk + kCodeBytes + col * 4);
        pe[p] = it < nact * Gi ? it / Gi : nact;  // slot
        pg[p] = g;
      }
    }
  };
  load(wave);

  // ---- staging: routing tables, then (if staged) h rows and their sums ----
  for (int a = tid; a < Tk; a += blockDim.x) {
    const int as = C.sorted[a];
    s_tok[a] = as / L.k;
    s_w[a] = C.tw[as];
  }
  for (int sl = tid; sl <= nact; sl += blockDim.x) {
    if (sl < nact) {
      const int e = C.active[sl];
      s_e[sl] = e;
      s_seg[sl] = C.offsets[e];
      s_rows[sl] = C.counts[e];
    } else {
      s_e[sl] = L.E;
      s_seg[sl] = Tk;
      s_rows[sl] = L.Is > 0 ? T : 0;
    }
  }
  const int nrows = Tk + T;
  uint16_t* hl = reinterpret_cast<uint16_t*>(dsm);
  float* hsl = reinterpret_cast<float*>(dsm + (size_t)nrows * C.Imax * 2);
  if (staged) {
    const int n16 = nrows * C.Imax / 8;
    for (int i = tid; i < n16; i += blockDim.x) reinterpret_cast<uint4*>(hl)[i] = reinterpret_cast<const uint4*>(C.hbuf)[i];
    for (int i = tid; i < nrows * hsw; i += blockDim.x) hsl[i] = C.hsum[i];
  }
  __syncthreads();
  const uint16_t* hb = staged ? hl : C.hbuf;
  const float* hs = staged ? hsl : C.hsum;

  float acc[kGemvMaxRows];
#pragma unroll
  for (int t = 0; t < kGemvMaxRows; t++) acc[t] = 0.f;

  for (int it0 = wave; it0 < nitems; it0 += kDnPref * kDnWaves) {
    if (it0 != wave) load(it0);
#pragma unroll
    for (int p = 0; p < kDnPref; p++) {
      if (pe[p] < 0) break;
      const int sl = pe[p], g = pg[p];
      const bool sh = sl == nact;
      const int rows = s_rows[sl];
      const int seg = s_seg[sl];
      uint32_t q[16];
      expand_codes(cd[p].x, q + 0);
      expand_codes(cd[p].y, q + 4);
      expand_codes(cd[p].z, q + 8);
      expand_codes(cd[p].w, q + 12);
      const float s = bf16_bits_to_f32(sb[p] & 0xFFFFu), bp = bf16_bits_to_f32(sb[p] >> 16) - 128.f * s;
      for (int j = 0; j < rows; j++) {
        const int irow = seg + j;
        const int t = sh ? j : s_tok[irow];
        const float w = sh ? 1.f : s_w[irow];
        const uint4* hp = reinterpret_cast<const uint4*>(hb + (int64_t)irow * C.Imax + g * kGroup + h * 32);
        float d = 0.f;
#pragma unroll
        for (int c = 0; c < 4; c++) {
          const uint4 hv = hp[c];
          d = dot2_bf16(q[4 * c + 0], hv.x, d);
          d = dot2_bf16(q[4 * c + 1], hv.y, d);
          d = dot2_bf16(q[4 * c + 2], hv.z, d);
          d = dot2_bf16(q[4 * c + 3], hv.w, d);
        }
        // hsum holds 32-column sums, so this lane half's own columns.
        const float v = w * fmaf(s, d, bp * hs[(int64_t)irow * hsw + 2 * g + h]);
#pragma unroll
        for (int tt = 0; tt < kGemvMaxRows; tt++)
          if (tt == t) acc[tt] += v;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kGemvMaxRows; t++) {
    if (t < T) {
      acc[t] += __shfl_xor(acc[t], 32);
      if (h == 0) red[wave][t][col] = acc[t];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < T * 32; i += blockDim.x) {
    const int t = i >> 5, n = i & 31;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kDnWaves; w++) v += red[w][t][n];
    C.y[(int64_t)t * H + nb * 32 + n] = v;
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_gemv_gateup(const LayerArgs& L, const ChunkArgs& C, hipStream_t s, const KTime& kt) {
  const int Imax = L.I > L.Is ? L.I : L.Is;
  const int slots = (L.E < C.Tk ? L.E : C.Tk) + 1;
  dim3 grid(slots, Imax / 32);
  static bool attr_set = false;
  if (!attr_set) {  // activation rows: T * H * 2 <= 64 KB on this path, beside ~20 KB of static LDS
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv_gateup),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, 64 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const size_t smem = (size_t)C.T * L.H * 2;
  MOE_LAUNCH(k_gemv_gateup, grid, dim3(kGuWaves * 64), smem, s, kt.start, kt.stop, L, C);
  return hipGetLastError();
}

hipError_t launch_gemv_down(const LayerArgs& L, const ChunkArgs& C, hipStream_t s, const KTime& kt) {
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv_down),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kDnStageMax);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const size_t rows = (size_t)C.Tk + C.T;
  const size_t stage = rows * C.Imax * 2 + rows * (C.Imax / 32) * 4;
  const int staged = stage <= (size_t)kDnStageMax ? 1 : 0;
  MOE_LAUNCH(k_gemv_down, dim3(L.H / 32), dim3(kDnWaves * 64), staged ? stage : 0, s, kt.start, kt.stop, L, C,
             staged);
  return hipGetLastError();
}

}  // namespace moe
