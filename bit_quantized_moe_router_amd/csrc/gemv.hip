// Row-parallel GEMV for decode ("Optimizing on-device inference for Apple
// Silicon", section "Optimise the one-row weight path": waves cooperate on the
// outputs while reading different parts of the weight matrix; section
// "Reduce intermediate and state traffic" for the two fused chains).
//
// With one to a few rows the layer is bound by weight bytes, so each expert's
// packed weights are streamed once: a wave reads one 1152-byte block (32
// output rows x one 64-column group) with a single 16-byte load per lane, so a
// lane holds 32 codes of one output row.  Codes expand to bf16 pairs
// (128 + q) and meet the activation pairs in v_dot2_f32_bf16; the per-group
// affine fold is acc += s * dot + (b - 128 s) * sum(x over the group).  The
// two lanes that share an output row are combined with one cross-half
// shuffle, the waves of a workgroup through LDS.  No atomics: every output is
// produced by exactly one workgroup, in a fixed order.
#include "launch.h"

namespace moe {

constexpr int kGemvMaxRows = 8;
constexpr int kGemvWaves = 4;

// ---------------------------------------------------------------------------
// gate/up + SwiGLU.  grid = (expert slots: active experts, then the shared
// expert; I/32 row blocks).  Waves split the H/64 groups.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gemv_gateup(LayerArgs L, ChunkArgs C) {
  const int slot = blockIdx.x;
  const int nact = *C.n_active;
  const bool shared = slot == nact;
  if (slot > nact || (shared && L.Is == 0)) return;
  const int e = shared ? L.E : C.active[slot];
  const int Iw = shared ? L.Is : L.I;
  const int nb = blockIdx.y;
  if (nb * 32 >= Iw) return;
  const int rows = shared ? C.T : C.counts[e];
  const int seg = shared ? 0 : C.offsets[e];
  const int H = L.H, G = H / kGroup;
  const uint8_t* wbase = expert_base(L, e);

  extern __shared__ uint16_t xl[];  // [rows][H]
  __shared__ int tok[kGemvMaxRows], orow[kGemvMaxRows];
  __shared__ float red[kGemvWaves][kGemvMaxRows][2][32];
  if (threadIdx.x < rows) {
    const int r = threadIdx.x;
    tok[r] = shared ? r : C.sorted[seg + r] / L.k;
    orow[r] = shared ? C.Tk + r : seg + r;
  }
  __syncthreads();
  const int H8 = H / 8;
  for (int i = threadIdx.x; i < rows * H8; i += blockDim.x) {
    const int r = i / H8, c = i - r * H8;
    reinterpret_cast<uint4*>(xl)[i] = reinterpret_cast<const uint4*>(C.x + (int64_t)tok[r] * H)[c];
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = lane >> 5, col = lane & 31;
  float accg[kGemvMaxRows], accu[kGemvMaxRows];
#pragma unroll
  for (int j = 0; j < kGemvMaxRows; j++) accg[j] = accu[j] = 0.f;

  for (int g = wave; g < G; g += kGemvWaves) {
    const uint8_t* blk = wbase + ((int64_t)(nb * G + g) * 2) * kBlockBytes;
    const uint4 cg = *reinterpret_cast<const uint4*>(blk + lane * 16);
    const uint4 cu = *reinterpret_cast<const uint4*>(blk + kBlockBytes + lane * 16);
    const uint32_t sbg = *reinterpret_cast<const uint32_t*>(blk + kCodeBytes + col * 4);
    const uint32_t sbu = *reinterpret_cast<const uint32_t*>(blk + kBlockBytes + kCodeBytes + col * 4);
    uint32_t qg[16], qu[16];
    expand_codes(cg.x, qg + 0);
    expand_codes(cg.y, qg + 4);
    expand_codes(cg.z, qg + 8);
    expand_codes(cg.w, qg + 12);
    expand_codes(cu.x, qu + 0);
    expand_codes(cu.y, qu + 4);
    expand_codes(cu.z, qu + 8);
    expand_codes(cu.w, qu + 12);
    const float sg = bf16_bits_to_f32(sbg & 0xFFFFu), bpg = bf16_bits_to_f32(sbg >> 16) - 128.f * sg;
    const float su = bf16_bits_to_f32(sbu & 0xFFFFu), bpu = bf16_bits_to_f32(sbu >> 16) - 128.f * su;
#pragma unroll
    for (int j = 0; j < kGemvMaxRows; j++) {
      if (j < rows) {
        const uint4* xp = reinterpret_cast<const uint4*>(xl + j * H + g * kGroup + h * 32);
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
        const float xs = h == 0 ? C.xsum[(int64_t)tok[j] * G + g] : 0.f;
        accg[j] = fmaf(sg, dg, fmaf(bpg, xs, accg[j]));
        accu[j] = fmaf(su, du, fmaf(bpu, xs, accu[j]));
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
  // Thread 32*j + n finishes row j, column n (256 threads = 8 rows x 32 columns).
  const int j = threadIdx.x >> 5, n = threadIdx.x & 31;
  const bool ok = j < rows;
  float gs = 0.f, us = 0.f;
  if (ok) {
#pragma unroll
    for (int w = 0; w < kGemvWaves; w++) {
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

// ---------------------------------------------------------------------------
// down + routing weight + shared add + combine.  grid = H/32 output row
// blocks; the workgroup walks every (expert slot, group) item, waves taking
// items round-robin, and writes y for all tokens of the chunk.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gemv_down(LayerArgs L, ChunkArgs C) {
  const int nb = blockIdx.x;
  const int nact = *C.n_active;
  const int nslots = nact + (L.Is > 0 ? 1 : 0);
  const int H = L.H, T = C.T;
  const int hsw = C.Imax / 32;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = lane >> 5, col = lane & 31;
  __shared__ float red[kGemvWaves][kGemvMaxRows][32];

  float acc[kGemvMaxRows];
#pragma unroll
  for (int t = 0; t < kGemvMaxRows; t++) acc[t] = 0.f;

  int item = 0;
  for (int slot = 0; slot < nslots; slot++) {
    const bool shared = slot == nact;
    const int e = shared ? L.E : C.active[slot];
    const int Kw = shared ? L.Is : L.I;
    const int Gk = Kw / kGroup;
    const int rows = shared ? T : C.counts[e];
    const int seg = shared ? 0 : C.offsets[e];
    const uint8_t* wbase = expert_base(L, e) + (shared ? L.shared_gateup_bytes : L.gateup_bytes);
    for (int g = 0; g < Gk; g++, item++) {
      if ((item % kGemvWaves) != wave) continue;
      const uint8_t* blk = wbase + (int64_t)(nb * Gk + g) * kBlockBytes;
      const uint4 cd = *reinterpret_cast<const uint4*>(blk + lane * 16);
      const uint32_t sb = *reinterpret_cast<const uint32_t*>(blk + kCodeBytes + col * 4);
      uint32_t q[16];
      expand_codes(cd.x, q + 0);
      expand_codes(cd.y, q + 4);
      expand_codes(cd.z, q + 8);
      expand_codes(cd.w, q + 12);
      const float s = bf16_bits_to_f32(sb & 0xFFFFu), bp = bf16_bits_to_f32(sb >> 16) - 128.f * s;
      for (int j = 0; j < rows; j++) {
        const int64_t irow = shared ? C.Tk + j : seg + j;
        int t;
        float w;
        if (shared) {
          t = j;
          w = 1.f;
        } else {
          const int a = C.sorted[seg + j];
          t = a / L.k;
          w = C.tw[a];
        }
        const uint4* hp = reinterpret_cast<const uint4*>(C.hbuf + irow * C.Imax + g * kGroup + h * 32);
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
        const float v = w * fmaf(s, d, bp * C.hsum[irow * hsw + 2 * g + h]);
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
    for (int w = 0; w < kGemvWaves; w++) v += red[w][t][n];
    C.y[(int64_t)t * H + nb * 32 + n] = v;
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_gemv_gateup(const LayerArgs& L, const ChunkArgs& C, hipStream_t s) {
  const int Imax = L.I > L.Is ? L.I : L.Is;
  const int slots = (L.E < C.Tk ? L.E : C.Tk) + 1;
  dim3 grid(slots, Imax / 32);
  const size_t smem = (size_t)C.T * L.H * 2;
  k_gemv_gateup<<<grid, dim3(256), smem, s>>>(L, C);
  return hipGetLastError();
}

hipError_t launch_gemv_down(const LayerArgs& L, const ChunkArgs& C, hipStream_t s) {
  k_gemv_down<<<dim3(L.H / 32), dim3(256), 0, s>>>(L, C);
  return hipGetLastError();
}

}  // namespace moe
