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
#include "small_route.h"

namespace moe {

constexpr int kGemvMaxRows = 8;
constexpr int kGuWaves = 8;    // gate/up workgroup: 8 waves split the H/64 groups
constexpr int kGuPref = 4;     // groups per wave whose loads are issued together
constexpr int kDnWaves = 8;    // down workgroup: 8 waves split the (expert, group) items
constexpr int kDnPref = 4;
constexpr int kMaxGroups = 128;              // H / 64 for H <= 8192
constexpr int kMaxAssign = kGemvMaxRows * 16; // T * k on the GEMV path
constexpr int kMaxSlots = kMaxAssign + 1;     // active experts + the shared expert
constexpr int kDnStageMax = 120 * 1024;       // LDS for staged intermediate rows
constexpr int kGuSmemMax = 64 * 1024 + kGemvMaxRows * (2 * 512 + 16) * 4;  // x rows + top-k lists

// ---------------------------------------------------------------------------
// Top-k + gate/up + SwiGLU.  grid = (expert slots: active experts, then the
// shared expert, then one metadata workgroup; I/32 row blocks).
//
// Routing is folded in, so decode needs no separate top-k launch between the
// logits and the weights: every workgroup takes the top-k of the chunk's rows
// from the exact logits itself (waves t < T, one row each), then wave 0 finds
// the workgroup's expert (the slot-th smallest selected expert: a bitmap of
// the selected experts and prefix popcounts over its words) and the expert's
// rows in flat assignment order.  The last column of workgroups (row block 0
// only) writes the routing tables the down kernel reads (ids, weights,
// counts, offsets, sorted order, active list, ...) with meta_small.  The
// activation rows are staged in LDS first, independent of the routing; their
// per-group sums are taken there.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kGuWaves * 64) void k_gemv_gateup(LayerArgs L, ChunkArgs C, const float* logits,
                                                               int BM, int with_shared) {
  const int slot = blockIdx.x, nb = blockIdx.y;
  const int T = C.T, H = L.H, G = H / kGroup, E = L.E, k = L.k, N = T * k;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, col = lane & 31;
  const bool meta_wg = slot == (int)gridDim.x - 1;
  if (meta_wg && nb != 0) return;  // workgroup-uniform, before any barrier
  extern __shared__ __attribute__((aligned(16))) uint8_t gsm[];  // [T][H] x rows, then [T][2E+16] top-k lists
  uint16_t* xl = reinterpret_cast<uint16_t*>(gsm);
  int* lists = reinterpret_cast<int*>(gsm + (size_t)T * H * 2);
  __shared__ float xs[kGemvMaxRows * kMaxGroups];
  __shared__ int s_ids[kMaxAssign];
  __shared__ float s_tw[kMaxAssign];
  __shared__ uint32_t s_bm[kMaxE / 32];
  __shared__ int tok[kGemvMaxRows], orow[kGemvMaxRows], s_info[3];
  __shared__ float red[kGuWaves][kGemvMaxRows][2][32];

  // ---- loads independent of the routing: the chunk's activation rows, into
  // registers first so that their latency overlaps the top-k's ----
  const int H8 = H / 8, nx = meta_wg ? 0 : T * H8;
  constexpr int kNt = kGuWaves * 64;
  uint4 xr0 = make_uint4(0u, 0u, 0u, 0u), xr1 = xr0;
  if (tid < nx) xr0 = reinterpret_cast<const uint4*>(C.x)[tid];
  if (tid + kNt < nx) xr1 = reinterpret_cast<const uint4*>(C.x)[tid + kNt];
  // ---- top-k of each row ----
  if (wave < T) topk_small(logits + (int64_t)wave * E, E, k, wave, s_ids, s_tw, lists + wave * (2 * E + 16));
  if (tid < nx) reinterpret_cast<uint4*>(xl)[tid] = xr0;
  if (tid + kNt < nx) reinterpret_cast<uint4*>(xl)[tid + kNt] = xr1;
  for (int i = tid + 2 * kNt; i < nx; i += kNt) reinterpret_cast<uint4*>(xl)[i] = reinterpret_cast<const uint4*>(C.x)[i];
  if (tid < kMaxE / 32) s_bm[tid] = 0u;
  __syncthreads();

  if (meta_wg) {
    // Routing tables of the chunk (workspace; the down kernel reads them).
    int32_t* ids = const_cast<int32_t*>(C.ids);
    float* tw = const_cast<float*>(C.tw);
    for (int a = tid; a < N; a += blockDim.x) {
      ids[a] = s_ids[a];
      tw[a] = s_tw[a];
    }
    if (wave == 0)
      meta_small(s_ids, T, k, E, BM, with_shared, const_cast<int32_t*>(C.counts), const_cast<int32_t*>(C.offsets),
                 const_cast<int32_t*>(C.sorted), const_cast<int32_t*>(C.tiles), const_cast<int32_t*>(C.n_tiles),
                 const_cast<int32_t*>(C.active), const_cast<int32_t*>(C.n_active), const_cast<int32_t*>(C.inv),
                 const_cast<int32_t*>(C.sched), lists);
    return;
  }

  // ---- this workgroup's expert and rows (wave 0) ----
  if (wave == 0) {
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
      // The word holding the slot-th set bit, then the bit inside it.
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
      const int off = __popcll(__ballot(id0 >= 0 && id0 < e)) + __popcll(__ballot(id1 >= 0 && id1 < e));
      const uint64_t m0 = __ballot(id0 == e), m1 = __ballot(id1 == e);
      const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      rows = __popcll(m0) + __popcll(m1);
      if (id0 == e) {
        const int r = __popcll(m0 & lt);
        tok[r] = lane / k;
        orow[r] = off + r;
      }
      if (id1 == e) {
        const int r = __popcll(m0) + __popcll(m1 & lt);
        tok[r] = (lane + 64) / k;
        orow[r] = off + r;
      }
    } else if (shared && L.Is > 0) {
      rows = T;
      if (lane < T) {
        tok[lane] = lane;
        orow[lane] = N + lane;
      }
    }
    if (lane == 0) {
      s_info[0] = shared ? L.E : e;
      s_info[1] = rows;
      s_info[2] = nact;
    }
  }
  __syncthreads();
  const int e = s_info[0], rows = s_info[1];
  const bool shared = e == L.E;
  const int Iw = shared ? L.Is : L.I;
  if (rows == 0 || nb * 32 >= Iw) return;  // workgroup-uniform; no barrier before this point is pending
  const uint8_t* wbase = expert_base(L, e) + (int64_t)nb * G * 2 * kBlockBytes;

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
  // Per-group activation sums while the first codes are in flight: 8 lanes
  // per group, 8 columns each, then a 3-step shuffle tree.
  for (int i0 = 0; i0 < T * G * 8; i0 += blockDim.x) {
    const int i = i0 + tid, gi = i >> 3, part = i & 7;
    float sm = 0.f;
    if (gi < T * G) {
      const int t = gi / G, g = gi - t * G;
      const uint4 v = *reinterpret_cast<const uint4*>(xl + t * H + g * kGroup + part * 8);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; j++) sm += bf16_bits_to_f32(w[j] & 0xFFFFu) + bf16_bits_to_f32(w[j] >> 16);
    }
    sm += __shfl_xor(sm, 1);
    sm += __shfl_xor(sm, 2);
    sm += __shfl_xor(sm, 4);
    if (gi < T * G && part == 0) xs[gi] = sm;
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
// down + routing weight + shared add + combine.  grid = H/8 workgroups of 8
// output rows each.  A workgroup walks every (expert slot, group) item; the
// items' 8-row slices of their 1152-byte blocks (two 128-byte runs of codes
// and 32 bytes of scale/bias) are read by 16 lanes each, so a wave covers 4
// items per load: lane l takes item l/16, row l%8 and K half (l/8)%2.  The
// routing tables (slot -> expert, segment, rows; sorted position -> token,
// weight) and, when they fit, all intermediate rows and their sums are staged
// in LDS first; the first item loads go out before the staging, from a
// speculative read of the active list.  Partial sums meet in registers (K
// halves, items of a wave) and LDS (waves); every output has one owner.
// ---------------------------------------------------------------------------
constexpr int kDnRows = 8;                         // output rows per workgroup
constexpr int kDnItemsPerLoad = kDnWaves * 4;      // items one load round covers

__global__ __launch_bounds__(kDnWaves * 64) void k_gemv_down(LayerArgs L, ChunkArgs C, int staged) {
  const int row0 = blockIdx.x * kDnRows;
  const int H = L.H, T = C.T, Tk = C.Tk;
  const int hsw = C.Imax / 32;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int sub = lane >> 4, hh = (lane >> 3) & 1, r = lane & 7;
  const int rr = row0 % 32 + r, nb32 = row0 / 32;  // row inside its 32-row block, block index
  const int Gi = L.I / kGroup, Gs = L.Is / kGroup;
  extern __shared__ __attribute__((aligned(16))) uint8_t dsm[];  // staged h rows, then their sums
  __shared__ int s_e[kMaxSlots], s_seg[kMaxSlots], s_rows[kMaxSlots];
  __shared__ int s_tok[kMaxAssign];
  __shared__ float s_w[kMaxAssign];
  __shared__ float red[kDnWaves][kGemvMaxRows][kDnRows];

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
  auto load = [&](int base) {
#pragma unroll
    for (int p = 0; p < kDnPref; p++) {
      const int it = base + p * kDnItemsPerLoad + wave * 4 + sub;
      pe[p] = -1;
      pg[p] = 0;
      if (it < nitems) {
        int g;
        const int e = item_expert(it, nact, g);
        const bool sh = e == L.E;
        const int Gk = sh ? Gs : Gi;
        const uint8_t* blk = expert_base(L, e) + (sh ? L.shared_gateup_bytes : L.gateup_bytes) +
                             (int64_t)(nb32 * Gk + g) * kBlockBytes;
        cd[p] = *reinterpret_cast<const uint4*>(blk + (hh * 32 + rr) * 16);
        sb[p] = *reinterpret_cast<const uint32_t*>(blk + kCodeBytes + rr * 4);
        pe[p] = it < nact * Gi ? it / Gi : nact;  // slot
        pg[p] = g;
      }
    }
  };
  load(0);

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

  for (int base = 0; base < nitems; base += kDnPref * kDnItemsPerLoad) {
    if (base != 0) load(base);
#pragma unroll
    for (int p = 0; p < kDnPref; p++) {
      if (pe[p] < 0) continue;
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
        const uint4* hp = reinterpret_cast<const uint4*>(hb + (int64_t)irow * C.Imax + g * kGroup + hh * 32);
        float d = 0.f;
#pragma unroll
        for (int c = 0; c < 4; c++) {
          const uint4 hv = hp[c];
          d = dot2_bf16(q[4 * c + 0], hv.x, d);
          d = dot2_bf16(q[4 * c + 1], hv.y, d);
          d = dot2_bf16(q[4 * c + 2], hv.z, d);
          d = dot2_bf16(q[4 * c + 3], hv.w, d);
        }
        // hsum holds 32-column sums, so this lane's K half.
        const float v = w * fmaf(s, d, bp * hs[(int64_t)irow * hsw + 2 * g + hh]);
#pragma unroll
        for (int tt = 0; tt < kGemvMaxRows; tt++)
          if (tt == t) acc[tt] += v;
      }
    }
  }
  // K halves (lane bit 3) and the wave's 4 items (lane bits 4, 5), then waves.
#pragma unroll
  for (int t = 0; t < kGemvMaxRows; t++) {
    if (t < T) {
      acc[t] += __shfl_xor(acc[t], 8);
      acc[t] += __shfl_xor(acc[t], 16);
      acc[t] += __shfl_xor(acc[t], 32);
      if (lane < kDnRows) red[wave][t][lane] = acc[t];
    }
  }
  __syncthreads();
  for (int i = tid; i < T * kDnRows; i += blockDim.x) {
    const int t = i / kDnRows, n = i - t * kDnRows;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kDnWaves; w++) v += red[w][t][n];
    C.y[(int64_t)t * H + row0 + n] = v;
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_gemv_gateup(const LayerArgs& L, const ChunkArgs& C, const float* logits, int BM,
                              int with_shared, hipStream_t s, const KTime& kt) {
  const int Imax = L.I > L.Is ? L.I : L.Is;
  const int slots = (L.E < C.Tk ? L.E : C.Tk) + 1;
  dim3 grid(slots + 1, Imax / 32);  // + the metadata workgroup
  // rows T * H * 2 <= 64 KB on this path, lists <= 8 * 1040 * 4, beside ~22 KB of static LDS
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = lds_limit_once(reinterpret_cast<const void*>(&k_gemv_gateup), kGuSmemMax, lds_set);
  if (e != hipSuccess) return e;
  const size_t smem = (size_t)C.T * L.H * 2 + (size_t)C.T * (2 * L.E + 16) * 4;
  if (smem > (size_t)kGuSmemMax || C.T > kGemvMaxRows || C.Tk > kMaxAssign) return hipErrorInvalidValue;
  MOE_LAUNCH(k_gemv_gateup, grid, dim3(kGuWaves * 64), smem, s, kt.start, kt.stop, L, C, logits, BM, with_shared);
  return hipGetLastError();
}

hipError_t launch_gemv_down(const LayerArgs& L, const ChunkArgs& C, hipStream_t s, const KTime& kt) {
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = lds_limit_once(reinterpret_cast<const void*>(&k_gemv_down), kDnStageMax, lds_set);
  if (e != hipSuccess) return e;
  const size_t rows = (size_t)C.Tk + C.T;
  const size_t stage = rows * C.Imax * 2 + rows * (C.Imax / 32) * 4;
  const int staged = stage <= (size_t)kDnStageMax ? 1 : 0;
  MOE_LAUNCH(k_gemv_down, dim3(L.H / kDnRows), dim3(kDnWaves * 64), staged ? stage : 0, s, kt.start, kt.stop, L,
             C, staged);
  return hipGetLastError();
}

}  // namespace moe
