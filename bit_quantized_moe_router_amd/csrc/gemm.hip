// Grouped expert GEMMs for prefill ("Optimizing on-device inference for Apple
// Silicon", sections "Dequantise weights during matrix multiplication",
// "Match tile size to expert load" and "Reduce intermediate and state
// traffic"):
//   gate/up: per tile of routed rows, h = silu(x Wg^T) * (x Wu^T)
//   down:    y[token] += routing weight * (h Wd^T), the shared expert with 1
//
// Workgroup = 8 waves over a tile of up to 256 rows of one expert x 256 weight
// columns (gate/up: 128 intermediate columns of gate and the same 128 of up;
// down: 256 output columns).  Wave (wm, wn) owns rows 64*wm.. and half the
// columns: 2 x 4 blocks of v_mfma_f32_32x32x16_f16, fp32 accumulation.
//
// Weights stay 4-bit in HBM.  Per 64-wide K group the workgroup reads the
// packed codes of its 8 blocks of 32 columns (one 16-byte load per thread,
// one block per wave), rebuilds w = s*q + b in fp32, rounds it to fp16 and
// writes it to LDS in MFMA operand order (block, k-step, lane), so that every
// wave reads its B operands with conflict-free 16-byte LDS reads.  The LDS
// tile is double buffered: the weights of group g+1 are rebuilt while the
// MFMAs of group g run.  The full-precision weights never reach HBM.
//
// Operand precision: the pages rebuild weights in bf16; here the operands are
// fp16 (11 significant bits instead of 8), which cuts the rounding error of
// the rebuilt weights eightfold.  Activations enter as fp16(x / 256) (written
// by the routing kernels) and the intermediate as fp16(h / 256); the power-of-
// two scale is exact and keeps any bf16-sized value inside the fp16 range, and
// the epilogues multiply it back.
//
// Activations go from memory straight to registers (gathered token rows for
// gate/up, contiguous rows of the expert's segment for down), one group ahead,
// in two register sets that alternate between even and odd groups.  Rows
// beyond the tile's valid count reuse a valid row's address and are never
// stored; a wave whose 64 rows are all beyond the count skips its MFMAs.
// Workgroups beyond n_tiles (read on the device) exit.
//
// MFMA 32x32x16 operand layout (wave64): lane l supplies row (A) / column (B)
// l % 32 and eight consecutive k-slots 8*(l/32)..+7; the result holds column
// l % 32 and rows 8*(i/4) + 4*(l/32) + i%4 in accumulator i.  k-slot j of MFMA
// c for lane half h carries input column 32h + 8c + j of the group, for A and
// B alike, which is the order the packer stores codes in.
//
// Workgroup ids are mapped so that the column tiles of one row tile run on the
// same XCD back to back (dispatch is round-robin over the 8 XCDs), which
// keeps the tile's activation rows in that XCD's L2.
#include "launch.h"

namespace moe {

constexpr int kTileRows = 256;
constexpr int kWaves = 8;
constexpr int kBlocks = 8;                           // 32-column weight blocks per tile
constexpr int kBufBytes = kBlocks * kCodeBytes * 4;  // fp16 tile of one group: 8 x 4 x 64 x 16 B
constexpr int kSmem = 2 * kBufBytes + kTileRows * 8; // + token / weight per row

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// 8 codes of one packed dword -> 8 fp16 weights w = s*q + b (round to nearest
// even), in k order, as four dwords of fp16 pairs.
__device__ __forceinline__ uint4 dequant8(uint32_t d, float s, float b) {
  uint32_t e = d & 0x0F0F0F0Fu;         // bytes: q0 q4 q1 q5
  uint32_t o = (d >> 4) & 0x0F0F0F0Fu;  // bytes: q2 q6 q3 q7
  asm("" : "+v"(e), "+v"(o));            // keep the masks; bytes convert with v_cvt_f32_ubyteN
  const float w0 = fmaf((float)(e & 0xFFu), s, b), w1 = fmaf((float)((e >> 16) & 0xFFu), s, b);
  const float w2 = fmaf((float)(o & 0xFFu), s, b), w3 = fmaf((float)((o >> 16) & 0xFFu), s, b);
  const float w4 = fmaf((float)((e >> 8) & 0xFFu), s, b), w5 = fmaf((float)(e >> 24), s, b);
  const float w6 = fmaf((float)((o >> 8) & 0xFFu), s, b), w7 = fmaf((float)(o >> 24), s, b);
  f16x2_t p0 = {(_Float16)w0, (_Float16)w1}, p1 = {(_Float16)w2, (_Float16)w3};
  f16x2_t p2 = {(_Float16)w4, (_Float16)w5}, p3 = {(_Float16)w6, (_Float16)w7};
  return make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                    __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

template <bool kGateUp>
__global__ __launch_bounds__(kWaves * 64) void k_expert_gemm(LayerArgs L, ChunkArgs C, int n_ct) {
  // ---- workgroup -> (tile, column tile), XCD-aware ----
  const int lin = blockIdx.x;
  const int xcd = lin & 7, m = lin >> 3;
  const int tile = (m / n_ct) * 8 + xcd, ct = m % n_ct;
  if (tile >= *C.n_tiles) return;
  const int e = C.tiles[3 * tile], r0 = C.tiles[3 * tile + 1], rows = C.tiles[3 * tile + 2];
  const bool shared = e == L.E;
  const int Iw = shared ? L.Is : L.I;
  if (Iw == 0) return;
  const int H = L.H;
  // gate/up: columns = intermediate (32-row blocks of gate and up); down: output columns.
  const int ncols = kGateUp ? Iw : H;
  const int K = kGateUp ? H : Iw;
  const int G = K / kGroup;
  const int cb0 = ct * (kGateUp ? 4 : 8);  // first 32-column block of this column tile
  if (cb0 * 32 >= ncols) return;
  const int nvb = min(kGateUp ? 4 : 8, ncols / 32 - cb0);  // valid 32-column blocks (gate/up: per matrix)

  const uint8_t* ebase = expert_base(L, e);
  const uint8_t* wbase = kGateUp ? ebase : ebase + (shared ? L.shared_gateup_bytes : L.gateup_bytes);
  const int seg = shared ? 0 : C.offsets[e];
  const int rowbase = shared ? C.Tk + r0 : seg + r0;  // hbuf row of the tile's first row

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* bt = smem;                                       // [2][blk][c][lane] x 16 B
  int* tok = reinterpret_cast<int*>(smem + 2 * kBufBytes);  // [256]
  float* wt = reinterpret_cast<float*>(tok + kTileRows);    // [256]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, col = lane & 31;

  // Row metadata: token (and routing weight for down).
  if (tid < kTileRows) {
    int t = 0;
    float w = 0.f;
    if (tid < rows) {
      if (shared) {
        t = r0 + tid;
        w = 1.f;
      } else {
        const int a = C.sorted[seg + r0 + tid];
        t = a / L.k;
        w = C.tw[a];
      }
    }
    tok[tid] = t;
    wt[tid] = w;
  }

  // ---- weight block rebuilt by this wave: LDS block `wave`, lane `lane` ----
  // gate/up: LDS blocks 0..3 are gate, 4..7 up, column block cb0 + (wave & 3);
  // down: column block cb0 + wave.
  const int qj = kGateUp ? (wave & 3) : wave;
  const bool qvalid = qj < nvb;  // wave-uniform
  const int qjc = qvalid ? qj : nvb - 1;  // invalid blocks read a valid block and store nothing
  const uint8_t* qsrc = kGateUp ? wbase + ((int64_t)(cb0 + qjc) * G * 2 + (wave >> 2)) * kBlockBytes
                                : wbase + (int64_t)(cb0 + qjc) * G * kBlockBytes;
  const int64_t qstride = kGateUp ? 2 * kBlockBytes : kBlockBytes;
  uint4* qdst0 = reinterpret_cast<uint4*>(bt) + wave * 4 * 64 + lane;

  __syncthreads();  // tok / wt visible

  // ---- A operand pointers: rows 64*wm + 32*f + col, lane half h ----
  const uint16_t* aptr[2];
#pragma unroll
  for (int f = 0; f < 2; f++) {
    const int r = wm * 64 + f * 32 + col;
    const int rr = r < rows ? r : 0;
    if (kGateUp) {
      aptr[f] = C.x16 + (int64_t)tok[rr] * H + h * 32;
    } else {
      aptr[f] = C.hbuf + (int64_t)(rowbase + rr) * C.Imax + h * 32;
    }
  }
  const bool wave_active = __builtin_amdgcn_readfirstlane(wm * 64 < rows ? 1 : 0) != 0;
  // Wave's weight blocks in the LDS tile.
  int wblk[4];
#pragma unroll
  for (int b = 0; b < 4; b++) wblk[b] = kGateUp ? (b >> 1) * 4 + 2 * wn + (b & 1) : 4 * wn + b;

  auto load_a = [&](int g, uint4 (&dst)[2][4]) {
    const int gg = g < G ? g : G - 1;  // past the end: a valid, unused group
#pragma unroll
    for (int f = 0; f < 2; f++)
#pragma unroll
      for (int c = 0; c < 4; c++) dst[f][c] = *reinterpret_cast<const uint4*>(aptr[f] + gg * kGroup + c * 8);
  };
  auto load_q = [&](int g, uint4& code, uint32_t& sb) {
    const int gg = g < G ? g : G - 1;
    const uint8_t* blk = qsrc + gg * qstride;
    code = *reinterpret_cast<const uint4*>(blk + lane * 16);
    sb = *reinterpret_cast<const uint32_t*>(blk + kCodeBytes + col * 4);
  };
  auto dequant_store = [&](int buf, const uint4& code, uint32_t sb) {
    const float s = bf16_bits_to_f32(sb & 0xFFFFu), b = bf16_bits_to_f32(sb >> 16);
    uint4* dst = qdst0 + buf * (kBufBytes / 16);
    dst[0 * 64] = dequant8(code.x, s, b);
    dst[1 * 64] = dequant8(code.y, s, b);
    dst[2 * 64] = dequant8(code.z, s, b);
    dst[3 * 64] = dequant8(code.w, s, b);
  };

  f32x16_t acc[2][4];
#pragma unroll
  for (int f = 0; f < 2; f++)
#pragma unroll
    for (int b = 0; b < 4; b++) acc[f][b] = f32x16_t{};

  auto mma_group = [&](int buf, const uint4 (&a)[2][4]) {
    const uint4* bsrc = reinterpret_cast<const uint4*>(bt + buf * kBufBytes);
#pragma unroll
    for (int c = 0; c < 4; c++) {
      f16x8_t bv[4];
#pragma unroll
      for (int b = 0; b < 4; b++) bv[b] = __builtin_bit_cast(f16x8_t, bsrc[(wblk[b] * 4 + c) * 64 + lane]);
#pragma unroll
      for (int f = 0; f < 2; f++) {
        const f16x8_t av = __builtin_bit_cast(f16x8_t, a[f][c]);
#pragma unroll
        for (int b = 0; b < 4; b++) acc[f][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv[b], acc[f][b], 0, 0, 0);
      }
    }
  };

  // Prologue: group 0 weights into buffer 0; A of group 0; codes of group 1.
  uint4 a0[2][4], a1[2][4];
  uint4 qc0, qc1;
  uint32_t qs0, qs1;
  load_q(0, qc0, qs0);
  load_a(0, a0);
  if (qvalid) dequant_store(0, qc0, qs0);
  load_q(1, qc1, qs1);
  __syncthreads();

  // Two groups per iteration; register sets and LDS buffers alternate.
  for (int g = 0; g < G; g += 2) {
    // even group g: A in a0, weights in buffer 0, codes of g+1 in qc1.
    load_a(g + 1, a1);
    if (qvalid && g + 1 < G) dequant_store(1, qc1, qs1);
    load_q(g + 2, qc0, qs0);
    if (wave_active) mma_group(0, a0);
    __syncthreads();
    if (g + 1 >= G) break;
    // odd group g+1: A in a1, weights in buffer 1, codes of g+2 in qc0.
    load_a(g + 2, a0);
    if (qvalid && g + 2 < G) dequant_store(0, qc0, qs0);
    load_q(g + 3, qc1, qs1);
    if (wave_active) mma_group(1, a1);
    __syncthreads();
  }

  if (!wave_active) return;
  // ---- epilogue: undo the 2^-8 activation scale ----
  if (kGateUp) {
#pragma unroll
    for (int f = 0; f < 2; f++) {
#pragma unroll
      for (int j = 0; j < 2; j++) {
        if (2 * wn + j >= nvb) continue;
        const int icol = (cb0 + 2 * wn + j) * 32 + col;
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const int r = wm * 64 + f * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
          if (r < rows) {
            const float hv = silu_mul(256.f * acc[f][j][i], 256.f * acc[f][j + 2][i]);
            C.hbuf[(int64_t)(rowbase + r) * C.Imax + icol] = f32_to_f16_bits(hv * (1.f / 256.f));
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int f = 0; f < 2; f++) {
#pragma unroll
      for (int b = 0; b < 4; b++) {
        if (4 * wn + b >= nvb) continue;
        const int ocol = (cb0 + 4 * wn + b) * 32 + col;
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const int r = wm * 64 + f * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
          if (r < rows) atomicAdd(C.y + (int64_t)tok[r] * H + ocol, wt[r] * (256.f * acc[f][b][i]));
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_fill_zero(float* __restrict__ p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (; i < n; i += stride) p[i] = 0.f;
}

// ---------------------------------------------------------------------------
template <bool kGateUp>
static hipError_t launch_expert_gemm(const LayerArgs& L, const ChunkArgs& C, int max_tiles, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_expert_gemm<kGateUp>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kSmem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int Imax = L.I > L.Is ? L.I : L.Is;
  const int n_ct = kGateUp ? (Imax + 127) / 128 : (L.H + 255) / 256;
  const int tiles8 = (max_tiles + 7) / 8 * 8;
  k_expert_gemm<kGateUp><<<dim3((unsigned)(tiles8 * n_ct)), dim3(kWaves * 64), kSmem, s>>>(L, C, n_ct);
  return hipGetLastError();
}

hipError_t launch_gateup_gemm(const LayerArgs& L, const ChunkArgs& C, int max_tiles, hipStream_t s) {
  return launch_expert_gemm<true>(L, C, max_tiles, s);
}

hipError_t launch_down_gemm(const LayerArgs& L, const ChunkArgs& C, int max_tiles, hipStream_t s) {
  return launch_expert_gemm<false>(L, C, max_tiles, s);
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  k_fill_zero<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p, n);
  return hipGetLastError();
}

}  // namespace moe
