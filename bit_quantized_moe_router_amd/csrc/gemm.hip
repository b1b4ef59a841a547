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
// keeps the tile's activation rows in that XCD's L2; row tiles run in the
// routing kernel's longest-first order (full tiles before partial ones).
#include "launch.h"

namespace moe {

constexpr int kTileRows = 256;
constexpr int kWaves = 8;
constexpr int kBlocks = 8;                           // 32-column weight blocks per tile
constexpr int kBufBytes = kBlocks * kCodeBytes * 4;  // fp16 tile of one group: 8 x 4 x 64 x 16 B
constexpr int kARow = 144;                           // bytes per A row in LDS: 64 fp16 + 16 B pad
constexpr int kABufBytes = kTileRows * kARow;        // one group of A rows
constexpr int kSmem = 2 * kBufBytes + 2 * kABufBytes + kTileRows * 4;  // + token per row

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

typedef _Float16 f16x2v_t __attribute__((ext_vector_type(2)));

// (a & mask) | magic in one VALU op.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(mask), "v"(magic));
  return r;
}

// 8 codes of one packed dword -> 8 fp16 weights w = s*q + b in k order, as
// four dwords of fp16 pairs.  Pair i of codes sits in nibbles i and 4+i, so
// ((d >> 4i) & 0x000F000F) | 0x64006400 is the fp16 pair (1024 + q, 1024 + q')
// (fp16 0x6400 = 1024 and its 10 mantissa bits step by 1); subtracting 1024 is
// exact, and one packed fp16 FMA per pair rounds s*q + b once.
__device__ __forceinline__ uint4 dequant8(uint32_t d, f16x2v_t s2, f16x2v_t b2, uint32_t mask, uint32_t magic) {
  const f16x2v_t off = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const f16x2v_t q = __builtin_bit_cast(f16x2v_t, and_or(d >> (4 * i), mask, magic)) + off;
    w[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, s2, b2));
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

template <bool kGateUp>
__global__ __launch_bounds__(kWaves * 64) void k_expert_gemm(LayerArgs L, ChunkArgs C, int n_ct) {
  // ---- workgroup -> (tile, column tile), XCD-aware ----
  const int lin = blockIdx.x;
  const int xcd = lin & 7, m = lin >> 3;
  const int slot = (m / n_ct) * 8 + xcd, ct = m % n_ct;
  if (slot >= *C.n_tiles) return;
  const int tile = C.sched[slot];
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
  uint8_t* bt = smem;                                     // B: [2][blk][c][lane] x 16 B
  uint8_t* at = smem + 2 * kBufBytes;                     // A: [2][256 rows][kARow B]
  int* tok = reinterpret_cast<int*>(at + 2 * kABufBytes);  // [256]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, col = lane & 31;

  if (tid < kTileRows) {
    int t = 0;
    if (tid < rows) t = shared ? r0 + tid : C.sorted[seg + r0 + tid] / L.k;
    tok[tid] = t;
  }

  // ---- weight block rebuilt by this wave: LDS block `wave`, lane `lane` ----
  // gate/up: LDS blocks 0..3 are gate, 4..7 up, column block cb0 + (wave & 3);
  // down: column block cb0 + wave.
  const int qj = kGateUp ? (wave & 3) : wave;
  const int qjc = qj < nvb ? qj : nvb - 1;  // columns past the edge rebuild a valid block, never stored
  const uint8_t* qsrc = kGateUp ? wbase + ((int64_t)(cb0 + qjc) * G * 2 + (wave >> 2)) * kBlockBytes
                                : wbase + (int64_t)(cb0 + qjc) * G * kBlockBytes;
  const int64_t qstride = kGateUp ? 2 * kBlockBytes : kBlockBytes;
  uint4* qdst0 = reinterpret_cast<uint4*>(bt) + wave * 4 * 64 + lane;

  __syncthreads();  // tok visible

  // ---- A staging: thread t moves 16-byte parts (row t/8 + 64 i, part t%8), i < 4 ----
  const int apart = tid & 7, arow0 = tid >> 3;
  const uint16_t* asrc0;
  const uint16_t* asrc1;
  const uint16_t* asrc2;
  const uint16_t* asrc3;
  // Every thread stages all four rows each group, without branches, so the
  // number of loads in flight is the same on every path and the compiler can
  // wait for exactly the loads it needs; rows past the tile's end load a
  // valid row (cache hits) and their results are never stored out.
  {
    auto rowptr = [&](int r) {
      const int rr = r < rows ? r : rows - 1;
      return (kGateUp ? C.x16 + (int64_t)tok[rr] * H : C.hbuf + (int64_t)(rowbase + rr) * C.Imax) + apart * 8;
    };
    asrc0 = rowptr(arow0);
    asrc1 = rowptr(arow0 + 64);
    asrc2 = rowptr(arow0 + 128);
    asrc3 = rowptr(arow0 + 192);
  }
  // Two staging register sets: A of even groups in ae*, of odd groups in ao*,
  // loaded two groups before they are written to LDS.
  uint4 ae0 = make_uint4(0, 0, 0, 0), ae1 = ae0, ae2 = ae0, ae3 = ae0;
  uint4 ao0 = ae0, ao1 = ae0, ao2 = ae0, ao3 = ae0;
  uint8_t* const adst = at + apart * 16 + arow0 * kARow;
#define MOE_LOAD_A(g, S)                                                                   \
  do {                                                                                     \
    const int gg_ = (g) < G ? (g) : G - 1; /* past the end: a valid, unused group */       \
    S##0 = *reinterpret_cast<const uint4*>(asrc0 + gg_ * kGroup);                 \
    S##1 = *reinterpret_cast<const uint4*>(asrc1 + gg_ * kGroup);                 \
    S##2 = *reinterpret_cast<const uint4*>(asrc2 + gg_ * kGroup);                 \
    S##3 = *reinterpret_cast<const uint4*>(asrc3 + gg_ * kGroup);                 \
  } while (0)
#define MOE_STORE_A(buf, S)                                                                \
  do {                                                                                     \
    uint8_t* d_ = adst + (buf) * kABufBytes;                                               \
    *reinterpret_cast<uint4*>(d_) = S##0;                                         \
    *reinterpret_cast<uint4*>(d_ + 64 * kARow) = S##1;                            \
    *reinterpret_cast<uint4*>(d_ + 128 * kARow) = S##2;                           \
    *reinterpret_cast<uint4*>(d_ + 192 * kARow) = S##3;                           \
  } while (0)

  // ---- weight codes: a ring of 4 groups in registers (qc0..qc3, qs0..qs3) ----
  uint4 qc0, qc1, qc2, qc3;
  uint32_t qs0, qs1, qs2, qs3;
  auto load_q = [&](int g, uint4& code, uint32_t& sb) {
    const int gg = g < G ? g : G - 1;
    const uint8_t* blk = qsrc + gg * qstride;
    code = *reinterpret_cast<const uint4*>(blk + lane * 16);
    sb = *reinterpret_cast<const uint32_t*>(blk + kCodeBytes + col * 4);
  };
  const uint32_t kMask = 0x000F000Fu, kMagic = 0x64006400u;
  auto dequant_store = [&](int buf, const uint4& code, uint32_t sb) {
    const _Float16 sh = (_Float16)bf16_bits_to_f32(sb & 0xFFFFu), bh = (_Float16)bf16_bits_to_f32(sb >> 16);
    const f16x2v_t s2 = {sh, sh}, b2 = {bh, bh};
    uint4* dst = qdst0 + buf * (kBufBytes / 16);
    dst[0 * 64] = dequant8(code.x, s2, b2, kMask, kMagic);
    dst[1 * 64] = dequant8(code.y, s2, b2, kMask, kMagic);
    dst[2 * 64] = dequant8(code.z, s2, b2, kMask, kMagic);
    dst[3 * 64] = dequant8(code.w, s2, b2, kMask, kMagic);
  };

  const bool wave_active = __builtin_amdgcn_readfirstlane(wm * 64 < rows ? 1 : 0) != 0;
  int wblk[4];
#pragma unroll
  for (int b = 0; b < 4; b++) wblk[b] = kGateUp ? (b >> 1) * 4 + 2 * wn + (b & 1) : 4 * wn + b;
  // A fragment byte offsets inside an A buffer: rows 64 wm + 32 f + col, columns 32 h + 8 c.
  const int aoff0 = (wm * 64 + col) * kARow + h * 64;

  f32x16_t acc[2][4];
#pragma unroll
  for (int f = 0; f < 2; f++)
#pragma unroll
    for (int b = 0; b < 4; b++) acc[f][b] = f32x16_t{};

  // One group of MFMAs on buffers `cur`, fused with the rebuild of the next
  // group's weights (code, sb) into B buffer `nxt`.  The sched_group_barrier
  // sequence pins an interleaved order (each MFMA followed by two VALU ops of
  // the rebuild), so the VALU work runs under the MFMA pipe.
  auto mma_fused = [&](int cur, const uint4& code, uint32_t sb, int nxt) {
    const _Float16 sh = (_Float16)bf16_bits_to_f32(sb & 0xFFFFu), bh = (_Float16)bf16_bits_to_f32(sb >> 16);
    const f16x2v_t s2 = {sh, sh}, b2 = {bh, bh};
    const uint4* bsrc = reinterpret_cast<const uint4*>(bt + cur * kBufBytes);
    const uint8_t* asrc_l = at + cur * kABufBytes + aoff0;
    uint4* dst = qdst0 + nxt * (kBufBytes / 16);
    const uint32_t cw[4] = {code.x, code.y, code.z, code.w};
#pragma unroll
    for (int c = 0; c < 4; c++) {
      f16x8_t bv[4], av[2];
#pragma unroll
      for (int b = 0; b < 4; b++) bv[b] = __builtin_bit_cast(f16x8_t, bsrc[(wblk[b] * 4 + c) * 64 + lane]);
#pragma unroll
      for (int f = 0; f < 2; f++)
        av[f] = *reinterpret_cast<const f16x8_t*>(asrc_l + f * 32 * kARow + c * 16);
      const uint4 dq = dequant8(cw[c], s2, b2, kMask, kMagic);
#pragma unroll
      for (int f = 0; f < 2; f++)
#pragma unroll
        for (int b = 0; b < 4; b++) acc[f][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[f], bv[b], acc[f][b], 0, 0, 0);
      dst[c * 64] = dq;
    }
#pragma unroll
    for (int c = 0; c < 4; c++) {
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // 6 LDS reads (A and B operands of this k-step)
#pragma unroll
      for (int i = 0; i < 8; i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // 2 VALU
      }
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // 1 LDS write (rebuilt weights)
    }
  };

  // One pipeline step for group g, ring slot g % 4 holding (QC, QS) for the
  // codes of g+4 to load and (NC, NS) the codes of g+1 to rebuild; AS is the
  // staging set of group g+1 (its parity): MFMAs of g (buffers g%2) fused with
  // the rebuild of g+1, A of g+1 into LDS, loads for A of g+3 and codes of g+4.
#define MOE_GEMM_STEP(g, CUR, QC, QS, NC, NS, AS)               \
  do {                                                        \
    if (wave_active)                                          \
      mma_fused(CUR, NC, NS, (CUR) ^ 1);                      \
    else                                                      \
      dequant_store((CUR) ^ 1, NC, NS);                       \
    MOE_STORE_A((CUR) ^ 1, AS);                               \
    MOE_LOAD_A((g) + 3, AS);                                  \
    load_q((g) + 4, QC, QS);                                  \
    __syncthreads();                                          \
  } while (0)

  // Prologue: codes of groups 0..3, A and weights of group 0, A loads of groups 1, 2.
  load_q(0, qc0, qs0);
  load_q(1, qc1, qs1);
  load_q(2, qc2, qs2);
  load_q(3, qc3, qs3);
  MOE_LOAD_A(0, ae);
  MOE_STORE_A(0, ae);
  dequant_store(0, qc0, qs0);
  MOE_LOAD_A(1, ao);
  MOE_LOAD_A(2, ae);
  __syncthreads();

  for (int g = 0; g < G; g += 4) {
    MOE_GEMM_STEP(g, 0, qc0, qs0, qc1, qs1, ao);
    if (g + 1 >= G) break;
    MOE_GEMM_STEP(g + 1, 1, qc1, qs1, qc2, qs2, ae);
    if (g + 2 >= G) break;
    MOE_GEMM_STEP(g + 2, 0, qc2, qs2, qc3, qs3, ao);
    if (g + 3 >= G) break;
    MOE_GEMM_STEP(g + 3, 1, qc3, qs3, qc0, qs0, ae);
  }
#undef MOE_GEMM_STEP
#undef MOE_LOAD_A
#undef MOE_STORE_A

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
    // Routed rows: fp16(out / 256) per assignment, combined per token later
    // (k_combine); the shared expert's rows go straight into y in fp32.
#pragma unroll
    for (int f = 0; f < 2; f++) {
#pragma unroll
      for (int b = 0; b < 4; b++) {
        if (4 * wn + b >= nvb) continue;
        const int ocol = (cb0 + 4 * wn + b) * 32 + col;
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const int r = wm * 64 + f * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
          if (r < rows) {
            if (shared)
              C.y[(int64_t)tok[r] * H + ocol] = 256.f * acc[f][b][i];
            else
              C.obuf[(int64_t)(rowbase + r) * H + ocol] = f32_to_f16_bits(acc[f][b][i]);
          }
        }
      }
    }
  }
}

// y[t] = (shared expert's output, already in y) + sum_j w_tj * 256 * obuf[pos(t, j)]
// in top-k order.  One workgroup per token, 8 columns per thread.
__global__ __launch_bounds__(256) void k_combine(LayerArgs L, ChunkArgs C) {
  const int t = blockIdx.x;
  const int H = L.H, k = L.k;
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    float acc[8];
    if (L.Is > 0) {
      const float4 a = *reinterpret_cast<const float4*>(C.y + (int64_t)t * H + c);
      const float4 b = *reinterpret_cast<const float4*>(C.y + (int64_t)t * H + c + 4);
      acc[0] = a.x; acc[1] = a.y; acc[2] = a.z; acc[3] = a.w;
      acc[4] = b.x; acc[5] = b.y; acc[6] = b.z; acc[7] = b.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; i++) acc[i] = 0.f;
    }
    for (int j = 0; j < k; j++) {
      const int a = t * k + j;
      const float w = 256.f * C.tw[a];
      const uint4 o = *reinterpret_cast<const uint4*>(C.obuf + (int64_t)C.inv[a] * H + c);
      const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const f16x2v_t p = __builtin_bit_cast(f16x2v_t, ow[i]);
        acc[2 * i] = fmaf(w, (float)p.x, acc[2 * i]);
        acc[2 * i + 1] = fmaf(w, (float)p.y, acc[2 * i + 1]);
      }
    }
    *reinterpret_cast<float4*>(C.y + (int64_t)t * H + c) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4*>(C.y + (int64_t)t * H + c + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
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

hipError_t launch_combine(const LayerArgs& L, const ChunkArgs& C, hipStream_t s) {
  k_combine<<<dim3(C.T), dim3(256), 0, s>>>(L, C);
  return hipGetLastError();
}

}  // namespace moe
