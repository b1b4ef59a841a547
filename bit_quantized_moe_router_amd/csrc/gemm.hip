// Grouped expert GEMMs for prefill ("Optimizing on-device inference for Apple
// Silicon", sections "Dequantise weights during matrix multiplication" and
// "Reduce intermediate and state traffic"):
//   gate/up: per tile of routed rows, h = silu(x Wg^T) * (x Wu^T) -> bf16
//   down:    y[token] += routing weight * (h Wd^T), the shared expert with 1
// Weights stay 4-bit in HBM.  Each wave expands its 16-byte code slice per
// group straight into bf16 MFMA operands (128 + q, exact), multiplies with
// v_mfma_f32_32x32x16_bf16 into a per-group fp32 partial P, and folds the
// group's affine parameters in fp32:  acc += s * P + (b - 128 s) * sum(x).
// The full-precision weights are never materialised, in HBM or in LDS.
//
// Workgroup: 256 threads = 4 waves over a 64-row slab x 64 output columns,
// wave (wm, wn) owning rows 32*wm.. and columns 32*wn.. of the slab.  The tile
// map (expert, first row, rows) comes from the routing kernels; surplus
// workgroups (beyond n_tiles, read on the device) exit at once.
//
// MFMA 32x32x16 operand layout (wave64): lane l supplies row (A) / column (B)
// l % 32 and eight consecutive k-slots 8*(l/32)..+7; the result holds column
// l % 32 and rows 8*(i/4) + 4*(l/32) + i%4 in accumulator i.  The kernels map
// k-slot j of MFMA c for lane half h to input column 32h + 8c + j of the
// group, for A and B alike, which is also the order the packer stores codes
// in; any consistent mapping gives the same product.
#include "launch.h"

namespace moe {

constexpr int kSlab = 64;
constexpr int kAStride = 72;  // bf16 per LDS row of the A slab (64 + 8 pad)

// Stage one 64-row x 64-column bf16 slab of A into LDS; rows with src == null are zero.
__device__ __forceinline__ void stage_a(uint16_t* As, const uint16_t* const* rowsrc, int col0) {
  for (int i = threadIdx.x; i < kSlab * 8; i += 256) {
    const int r = i >> 3, part = i & 7;
    uint4 v = make_uint4(0, 0, 0, 0);
    const uint16_t* p = rowsrc[r];
    if (p) v = *reinterpret_cast<const uint4*>(p + col0 + part * 8);
    *reinterpret_cast<uint4*>(As + r * kAStride + part * 8) = v;
  }
}

__device__ __forceinline__ bf16x8_t a_frag(const uint16_t* As, int row, int h, int c) {
  return *reinterpret_cast<const bf16x8_t*>(As + row * kAStride + h * 32 + c * 8);
}

// One group (64 k) of one 32x32 output block: P = A(32x64) * (128 + Q)(64x32).
__device__ __forceinline__ f32x16_t group_mma(const uint16_t* As, int arow, int h, uint4 codes) {
  f32x16_t p = {};
  const uint32_t cw[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
  for (int c = 0; c < 4; c++) {
    uint32_t b[4];
    expand_codes(cw[c], b);
    p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_frag(As, arow, h, c), as_bf16x8(b[0], b[1], b[2], b[3]),
                                               p, 0, 0, 0);
  }
  return p;
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gateup_gemm(LayerArgs L, ChunkArgs C) {
  const int tile = blockIdx.x;
  if (tile >= *C.n_tiles) return;
  const int e = C.tiles[3 * tile], r0 = C.tiles[3 * tile + 1], rows = C.tiles[3 * tile + 2];
  const bool shared = e == L.E;
  const int Iw = shared ? L.Is : L.I;
  const int ct = blockIdx.y;
  if (ct * 64 >= Iw) return;

  const int H = L.H, G = H / kGroup;
  const uint8_t* wbase = expert_base(L, e);
  const int seg = shared ? 0 : C.offsets[e];
  const int outbase = shared ? C.Tk + r0 : seg + r0;

  extern __shared__ float smem[];
  float* Xs = smem;                                                      // [64][G]
  uint16_t* As = reinterpret_cast<uint16_t*>(Xs + kSlab * G);            // [64][72]
  const uint16_t** rowsrc = reinterpret_cast<const uint16_t**>(As + kSlab * kAStride);  // [64]
  int* tok = reinterpret_cast<int*>(rowsrc + kSlab);                     // [64]

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, col = lane & 31;
  const int nb = ct * 2 + wn;  // 32-row block of gate/up
  const int arow = wm * 32 + col;

  for (int slab = 0; slab < rows; slab += kSlab) {
    const int srows = min(kSlab, rows - slab);
    __syncthreads();
    if (threadIdx.x < kSlab) {
      const int r = threadIdx.x;
      int t = -1;
      if (r < srows) t = shared ? r0 + slab + r : C.sorted[seg + r0 + slab + r] / L.k;
      tok[r] = t;
      rowsrc[r] = t >= 0 ? C.x + (int64_t)t * H : nullptr;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kSlab * G; i += 256) {
      const int r = i / G, g = i - r * G;
      Xs[i] = tok[r] >= 0 ? C.xsum[(int64_t)tok[r] * G + g] : 0.f;
    }

    f32x16_t accg = {}, accu = {};
    for (int g = 0; g < G; g++) {
      const uint8_t* blk = wbase + ((int64_t)(nb * G + g) * 2) * kBlockBytes;
      const uint4 cg = *reinterpret_cast<const uint4*>(blk + lane * 16);
      const uint4 cu = *reinterpret_cast<const uint4*>(blk + kBlockBytes + lane * 16);
      const uint32_t sbg = *reinterpret_cast<const uint32_t*>(blk + kCodeBytes + col * 4);
      const uint32_t sbu = *reinterpret_cast<const uint32_t*>(blk + kBlockBytes + kCodeBytes + col * 4);
      __syncthreads();
      stage_a(As, rowsrc, g * kGroup);
      __syncthreads();
      const f32x16_t pg = group_mma(As, arow, h, cg);
      const f32x16_t pu = group_mma(As, arow, h, cu);
      const float sg = bf16_bits_to_f32(sbg & 0xFFFFu), bg = bf16_bits_to_f32(sbg >> 16);
      const float su = bf16_bits_to_f32(sbu & 0xFFFFu), bu = bf16_bits_to_f32(sbu >> 16);
      const float bpg = bg - 128.f * sg, bpu = bu - 128.f * su;
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int r = wm * 32 + (i >> 2) * 8 + h * 4 + (i & 3);
        const float xsr = Xs[r * G + g];
        accg[i] = fmaf(sg, pg[i], fmaf(bpg, xsr, accg[i]));
        accu[i] = fmaf(su, pu[i], fmaf(bpu, xsr, accu[i]));
      }
    }

    // SwiGLU, bf16 store, and the 32-column sums of bf16(h) for the down GEMM.
    const int hsw = C.Imax / 32;
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int r = wm * 32 + (i >> 2) * 8 + h * 4 + (i & 3);
      const uint16_t hb = f32_to_bf16_rne(silu_mul(accg[i], accu[i]));
      float hs = bf16_bits_to_f32(hb);
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) hs += __shfl_xor(hs, off);
      if (r < srows) {
        const int64_t orow = outbase + slab + r;
        C.hbuf[orow * C.Imax + nb * 32 + col] = hb;
        if (col == 0) C.hsum[orow * hsw + nb] = hs;
      }
    }
  }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_down_gemm(LayerArgs L, ChunkArgs C) {
  const int tile = blockIdx.x;
  if (tile >= *C.n_tiles) return;
  const int e = C.tiles[3 * tile], r0 = C.tiles[3 * tile + 1], rows = C.tiles[3 * tile + 2];
  const bool shared = e == L.E;
  const int Kw = shared ? L.Is : L.I;
  if (Kw == 0) return;
  const int H = L.H;
  const int ct = blockIdx.y;
  const int Gk = Kw / kGroup;
  const uint8_t* wbase = expert_base(L, e) + (shared ? L.shared_gateup_bytes : L.gateup_bytes);
  const int seg = shared ? 0 : C.offsets[e];
  const int inbase = shared ? C.Tk + r0 : seg + r0;
  const int hsw = C.Imax / 32;

  extern __shared__ float smem[];
  float* Hs = smem;                                                      // [64][Gk]
  uint16_t* As = reinterpret_cast<uint16_t*>(Hs + kSlab * Gk);           // [64][72]
  const uint16_t** rowsrc = reinterpret_cast<const uint16_t**>(As + kSlab * kAStride);
  int* tok = reinterpret_cast<int*>(rowsrc + kSlab);
  float* wt = reinterpret_cast<float*>(tok + kSlab);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, col = lane & 31;
  const int nb = ct * 2 + wn;  // 32-row block of down (output columns)
  const int arow = wm * 32 + col;

  for (int slab = 0; slab < rows; slab += kSlab) {
    const int srows = min(kSlab, rows - slab);
    __syncthreads();
    if (threadIdx.x < kSlab) {
      const int r = threadIdx.x;
      int t = -1;
      float w = 0.f;
      const uint16_t* src = nullptr;
      if (r < srows) {
        const int64_t irow = inbase + slab + r;
        if (shared) {
          t = r0 + slab + r;
          w = 1.f;
        } else {
          const int a = C.sorted[irow];
          t = a / L.k;
          w = C.tw[a];
        }
        src = C.hbuf + irow * C.Imax;
      }
      tok[r] = t;
      wt[r] = w;
      rowsrc[r] = src;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kSlab * Gk; i += 256) {
      const int r = i / Gk, g = i - r * Gk;
      float v = 0.f;
      if (r < srows) {
        const float* hp = C.hsum + (int64_t)(inbase + slab + r) * hsw + 2 * g;
        v = hp[0] + hp[1];
      }
      Hs[i] = v;
    }

    f32x16_t acc = {};
    for (int g = 0; g < Gk; g++) {
      const uint8_t* blk = wbase + (int64_t)(nb * Gk + g) * kBlockBytes;
      const uint4 cd = *reinterpret_cast<const uint4*>(blk + lane * 16);
      const uint32_t sb = *reinterpret_cast<const uint32_t*>(blk + kCodeBytes + col * 4);
      __syncthreads();
      stage_a(As, rowsrc, g * kGroup);
      __syncthreads();
      const f32x16_t p = group_mma(As, arow, h, cd);
      const float s = bf16_bits_to_f32(sb & 0xFFFFu), b = bf16_bits_to_f32(sb >> 16);
      const float bp = b - 128.f * s;
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int r = wm * 32 + (i >> 2) * 8 + h * 4 + (i & 3);
        acc[i] = fmaf(s, p[i], fmaf(bp, Hs[r * Gk + g], acc[i]));
      }
    }

#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int r = wm * 32 + (i >> 2) * 8 + h * 4 + (i & 3);
      if (r < srows) atomicAdd(C.y + (int64_t)tok[r] * H + nb * 32 + col, wt[r] * acc[i]);
    }
  }
}

__global__ __launch_bounds__(256) void k_fill_zero(float* __restrict__ p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (; i < n; i += stride) p[i] = 0.f;
}

// ---------------------------------------------------------------------------
hipError_t launch_gateup_gemm(const LayerArgs& L, const ChunkArgs& C, int max_tiles, hipStream_t s) {
  const int G = L.H / kGroup;
  const int Imax = L.I > L.Is ? L.I : L.Is;
  const size_t smem = (size_t)kSlab * G * 4 + (size_t)kSlab * kAStride * 2 + kSlab * 8 + kSlab * 4;
  dim3 grid(max_tiles, Imax / 64);
  k_gateup_gemm<<<grid, dim3(256), smem, s>>>(L, C);
  return hipGetLastError();
}

hipError_t launch_down_gemm(const LayerArgs& L, const ChunkArgs& C, int max_tiles, hipStream_t s) {
  const int Imax = L.I > L.Is ? L.I : L.Is;
  const int Gk = Imax / kGroup;
  const size_t smem = (size_t)kSlab * Gk * 4 + (size_t)kSlab * kAStride * 2 + kSlab * 8 + kSlab * 8;
  dim3 grid(max_tiles, L.H / 64);
  k_down_gemm<<<grid, dim3(256), smem, s>>>(L, C);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  k_fill_zero<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p, n);
  return hipGetLastError();
}

}  // namespace moe
