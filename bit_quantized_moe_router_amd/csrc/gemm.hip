// Grouped expert GEMMs for prefill ("Optimizing on-device inference for Apple
// Silicon", sections "Dequantise weights during matrix multiplication",
// "Match tile size to expert load" and "Reduce intermediate and state
// traffic"):
//   gate/up: per tile of routed rows, h = silu(x Wg^T) * (x Wu^T)
//   down:    y[token] += routing weight * (h Wd^T), the shared expert with 1
//
// Workgroup = 4 waves (one per SIMD) over a tile of up to 128 rows of one
// expert; two workgroups share a compute unit, so one's prologue and
// epilogue run under the other's MFMAs.  Each wave owns 2 weight blocks of 32
// columns (gate/up: one block of gate and the same block of up; down: 2
// output blocks) and all rows of the tile: up to 4 x 2 accumulators of
// v_mfma_f32_32x32x16_f16 (fp32).  The kernel is instantiated per number of
// 32-row fragments the tile needs (1..4), so small tiles issue only the MFMAs
// of their rows.
//
// Weights stay 4-bit in HBM and never pass through LDS: the packed layout puts
// each lane's 16 bytes of codes exactly where the MFMA B operand needs them,
// so a wave loads its blocks with one 16-byte load per block and K group,
// rebuilds w = s*q + b in registers (fp16, one rounding) and feeds them to the
// MFMAs of the same group.  Codes are prefetched four groups ahead, starting
// before the token indices of the tile are known.  When the blob's trailer says
// every scale is below 2^-4 in magnitude, the rebuild takes the subnormal form
// (rebuild16_small), which gives the same bits with fewer instructions.
//
// Activations (gathered token rows for gate/up, the expert's contiguous rows
// of the intermediate for down) are shared by the 4 waves through LDS: per K
// group the workgroup stages up to 128 rows x 64 columns (double buffered,
// one barrier per group); each thread moves up to four 16-byte pieces, loaded
// one group ahead into one register set.  Rows past the tile's count reuse a
// valid row and are never stored.
//
// A second instantiation (kPre) serves the separate-dequant measurement: the
// same kernel reading fp16 weights rebuilt beforehand by k_dequant_active
// instead of rebuilding them from the codes.
//
// Results leave through LDS: the workgroup's output tile is assembled there
// and written back as whole rows with 16-byte stores (the down GEMM writes the
// shared expert's rows into the same fp16 buffer, after the routed rows).
//
// Operand precision: the pages rebuild weights in bf16; here the operands are
// fp16 (11 significant bits instead of 8), which cuts the rounding error of
// the rebuilt weights eightfold.  Activations enter as fp16(x / 256) (written
// by the routing kernels) and the intermediate as fp16(h / 256); the power-of-
// two scale is exact, keeps magnitudes up to 65504 * 256 (about 1.7e7) inside
// the fp16 range (larger ones become infinity; include/moe.h states this as
// the supported activation range), and the epilogues multiply it back.
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

#include <type_traits>

namespace moe {

constexpr int kTileRows = 128;                 // largest tile the kernel takes
constexpr int kWaves = 4;                      // two workgroups per compute unit
constexpr int kARow = 144;                     // bytes per A row in LDS: 64 fp16 + 16 B pad
constexpr int kABufBytes = kTileRows * kARow;  // one K group of A rows
constexpr int kSmemMain = 2 * kABufBytes + kTileRows * 4;  // + token per row
constexpr int kGateUpColsPerWg = kWaves * 32;  // intermediate columns per workgroup
constexpr int kDownColsPerWg = kWaves * 64;    // output columns per workgroup
constexpr int kEpiRowGateUp = kGateUpColsPerWg * 2 + 16;  // LDS bytes per output row (fp16 + pad)
constexpr int kEpiRowDown = kDownColsPerWg * 2 + 16;
constexpr int kSmemGateUp = kTileRows * kEpiRowGateUp > kSmemMain ? kTileRows * kEpiRowGateUp : kSmemMain;
constexpr int kSmemDown = kTileRows * kEpiRowDown > kSmemMain ? kTileRows * kEpiRowDown : kSmemMain;

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2v_t __attribute__((ext_vector_type(2)));

// (a & mask) | magic in one VALU op.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(mask), "v"(magic));
  return r;
}

// 8 codes of one packed dword -> 8 fp16 weights w = s*q + b in k order, as
// four dwords of fp16 pairs.  Pair i of codes sits in nibbles i and 4+i.  An
// fp16 whose exponent is that of 1024 has a mantissa step of 1 in bits 0..3,
// and one with the exponent of 64 has a step of 1 in bits 4..7, so
//   (d & 0x000F000F) | 0x64006400 = (1024 + q0, 1024 + q4)
//   (d & 0x00F000F0) | 0x54005400 = (  64 + q1,   64 + q5)
// and the same on d >> 8 for pairs 2 and 3: one shift for 8 codes.  The
// offset subtraction is exact, and one packed fp16 FMA per pair rounds s*q + b
// once.
__device__ __forceinline__ f16x8_t dequant8(uint32_t d, f16x2v_t s2, f16x2v_t b2) {
  const f16x2v_t off_lo = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  const f16x2v_t off_hi = {(_Float16)-64.0f, (_Float16)-64.0f};
  const uint32_t d8 = d >> 8;
  const f16x2v_t q0 = __builtin_bit_cast(f16x2v_t, and_or(d, 0x000F000Fu, 0x64006400u)) + off_lo;
  const f16x2v_t q1 = __builtin_bit_cast(f16x2v_t, and_or(d, 0x00F000F0u, 0x54005400u)) + off_hi;
  const f16x2v_t q2 = __builtin_bit_cast(f16x2v_t, and_or(d8, 0x000F000Fu, 0x64006400u)) + off_lo;
  const f16x2v_t q3 = __builtin_bit_cast(f16x2v_t, and_or(d8, 0x00F000F0u, 0x54005400u)) + off_hi;
  return __builtin_bit_cast(
      f16x8_t, make_uint4(__builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q0, s2, b2)),
                          __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q1, s2, b2)),
                          __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q2, s2, b2)),
                          __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q3, s2, b2))));
}

// The same rebuild for two dwords of codes d0, d1 (one per weight block),
// valid while |s| < 2^-4.  A nibble in bits 4..7 of an fp16 whose exponent
// field is zero is the subnormal q * 2^-20, exact; with s20 = s * 2^20 (exact
// in fp16 for |s| < 2^-4) one packed FMA forms s20 * (q * 2^-20) + b = s*q + b
// exactly before its single rounding, so the result equals dequant8's bit for
// bit.  Pair i sits in nibbles i and 4+i, so pair 1 is in place and pairs 0, 2
// and 3 need shifts of 4 left, 4 right and 8 right; the shifts run on the two
// dwords as one 64-bit value (a bit that crosses from one dword into the other
// lands outside the mask), so 8 codes cost 1.5 shifts, 4 ANDs and 4 FMAs
// instead of 13 instructions.  It needs fp16 subnormal inputs kept, not
// flushed: the kernels run in the compiler's default fp16/fp64 denormal mode
// (preserve), which a build that flushes fp16 denormals would break.
__device__ __forceinline__ void rebuild16_small(uint32_t d0, uint32_t d1, f16x2v_t s0, f16x2v_t b0, f16x2v_t s1,
                                                f16x2v_t b1, f16x8_t& o0, f16x8_t& o1) {
  constexpr uint32_t m = 0x00F000F0u;
  const uint64_t dd = ((uint64_t)d1 << 32) | d0;
  uint64_t l4, r4, r8;
  // One VALU op each (the compiler would split a 64-bit shift into two 32-bit ones).
  asm("v_lshlrev_b64 %0, 4, %1" : "=v"(l4) : "v"(dd));
  asm("v_lshrrev_b64 %0, 4, %1" : "=v"(r4) : "v"(dd));
  asm("v_lshrrev_b64 %0, 8, %1" : "=v"(r8) : "v"(dd));
  auto w2 = [](uint32_t v, f16x2v_t sc, f16x2v_t bc) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2v_t, v & m), sc, bc));
  };
  o0 = __builtin_bit_cast(f16x8_t, make_uint4(w2((uint32_t)l4, s0, b0), w2(d0, s0, b0), w2((uint32_t)r4, s0, b0),
                                              w2((uint32_t)r8, s0, b0)));
  o1 = __builtin_bit_cast(f16x8_t, make_uint4(w2((uint32_t)(l4 >> 32), s1, b1), w2(d1, s1, b1),
                                              w2((uint32_t)(r4 >> 32), s1, b1), w2((uint32_t)(r8 >> 32), s1, b1)));
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Weight codes of one K group for the wave's 2 blocks.
struct QGroup {
  uint4 c0, c1;
  uint32_t s0, s1;
};

// Pre-dequantised weights of one K group for the wave's 2 blocks (the
// separate-dequant measurement): the fp16 B operands of the group's 4 k-steps.
struct QGroupP {
  uint4 b0[4], b1[4];
};

// Per-workgroup tile description.
struct Tile {
  int e, r0, rows, rowbase, ncols, G, ct;
  bool shared;
};

template <bool kGateUp, int NF, bool kPre, bool kSmall>
__device__ __forceinline__ void gemm_tile(const LayerArgs& L, const ChunkArgs& C, const Tile& T, uint8_t* smem) {
  const int H = L.H;
  const int G = T.G;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, col = lane & 31;
  uint8_t* at = smem;  // A: [2][128 rows][kARow B]
  int* tok = reinterpret_cast<int*>(smem + 2 * kABufBytes);

  // ---- the wave's 2 weight blocks: base of group 0 and stride per group ----
  // gate/up: block nb = 8 ct + wave of gate (b = 0) and of up (b = 1);
  // down: blocks nb = 2 (8 ct + wave) + b.
  const int nb0 = kGateUp ? T.ct * kWaves + wave : (T.ct * kWaves + wave) * 2;
  const int nvb = min(kGateUp ? 1 : 2, T.ncols / 32 - nb0);  // valid blocks of this wave (<= 0: none)
  const bool wave_cols = __builtin_amdgcn_readfirstlane(nvb > 0 ? 1 : 0) != 0;
  const uint8_t* ebase = expert_base(L, T.e);
  const uint8_t* wbase = kGateUp ? ebase : ebase + (T.shared ? L.shared_gateup_bytes : L.gateup_bytes);
  const int64_t qstride = kGateUp ? 2 * kBlockBytes : kBlockBytes;
  const uint8_t *qb0, *qb1;
  if (kGateUp) {
    const int nb = wave_cols ? nb0 : 0;
    qb0 = wbase + (int64_t)nb * G * 2 * kBlockBytes;
    qb1 = qb0 + kBlockBytes;
  } else {
    // A block past the column edge reloads a valid one; its results are never stored.
    const int n0 = wave_cols ? nb0 : 0, n1 = wave_cols && nvb > 1 ? nb0 + 1 : n0;
    qb0 = wbase + (int64_t)n0 * G * kBlockBytes;
    qb1 = wbase + (int64_t)n1 * G * kBlockBytes;
  }
  // Separate-dequant measurement: the same blocks in the fp16 copy.
  const uint8_t* pb0 = kPre ? L.wdq + (qb0 - L.blob) / kBlockBytes * kDqBlockBytes : nullptr;
  const uint8_t* pb1 = kPre ? L.wdq + (qb1 - L.blob) / kBlockBytes * kDqBlockBytes : nullptr;
  const int64_t pstride = qstride / kBlockBytes * kDqBlockBytes;
  using QG = typename std::conditional<kPre, QGroupP, QGroup>::type;
  auto load_q = [&](int g, QG& q) {
    if constexpr (kPre) {
      // Groups padded past G read as zero weights.
      const int64_t off = (int64_t)(g < G ? g : G - 1) * pstride;
#pragma unroll
      for (int c = 0; c < 4; c++) {
        q.b0[c] = g < G ? *reinterpret_cast<const uint4*>(pb0 + off + c * 1024 + lane * 16) : make_uint4(0, 0, 0, 0);
        q.b1[c] = g < G ? *reinterpret_cast<const uint4*>(pb1 + off + c * 1024 + lane * 16) : make_uint4(0, 0, 0, 0);
      }
    } else {
      const int64_t off = (int64_t)(g < G ? g : G - 1) * qstride;
      q.c0 = *reinterpret_cast<const uint4*>(qb0 + off + lane * 16);
      q.c1 = *reinterpret_cast<const uint4*>(qb1 + off + lane * 16);
      q.s0 = *reinterpret_cast<const uint32_t*>(qb0 + off + kCodeBytes + col * 4);
      q.s1 = *reinterpret_cast<const uint32_t*>(qb1 + off + kCodeBytes + col * 4);
    }
  };
  // ---- token of each row (gate/up gathers activation rows by token) ----
  // The index load goes out before the first weight codes so that waiting
  // for it leaves those in flight.
  int my_tok = 0;
  if (kGateUp && tid < kTileRows && tid < T.rows) my_tok = T.shared ? T.r0 + tid : C.sorted[T.rowbase + tid];
  QG q0, q1, q2, q3;
  load_q(0, q0);
  if (kGateUp) {
    if (tid < kTileRows) tok[tid] = T.shared ? my_tok : my_tok / L.k;
    __syncthreads();
  }

  // ---- A staging: thread t moves 16-byte part t%8 of rows t/8 and t/8 + 64 ----
  const int apart = tid & 7, arow0 = tid >> 3;   // rows arow0 + 32 j, j < 4
  const uint16_t *asrc0, *asrc1, *asrc2, *asrc3;
  {
    auto rowptr = [&](int r) {
      const int rr = r < T.rows ? r : T.rows - 1;
      return (kGateUp ? C.x16 + (int64_t)tok[rr] * H : C.hbuf + (int64_t)(T.rowbase + rr) * C.Imax) + apart * 8;
    };
    asrc0 = rowptr(arow0);
    asrc1 = rowptr(arow0 + 32);
    asrc2 = rowptr(arow0 + 64);
    asrc3 = rowptr(arow0 + 96);
  }
  uint8_t* const adst = at + apart * 16 + arow0 * kARow;
  // Rows of fragments the tile does not use are not staged.
#define MOE_LOAD_A(g, S)                                                      \
  do {                                                                        \
    const int gg_ = (g) < G ? (g) : G - 1; /* past the end: a valid, unused group */ \
    S##0 = *reinterpret_cast<const uint4*>(asrc0 + gg_ * kGroup);            \
    if (NF > 1) S##1 = *reinterpret_cast<const uint4*>(asrc1 + gg_ * kGroup); \
    if (NF > 2) S##2 = *reinterpret_cast<const uint4*>(asrc2 + gg_ * kGroup); \
    if (NF > 3) S##3 = *reinterpret_cast<const uint4*>(asrc3 + gg_ * kGroup); \
  } while (0)
#define MOE_STORE_A(buf, S)                                                   \
  do {                                                                        \
    uint8_t* d_ = adst + (buf) * kABufBytes;                                  \
    *reinterpret_cast<uint4*>(d_) = S##0;                                     \
    if (NF > 1) *reinterpret_cast<uint4*>(d_ + 32 * kARow) = S##1;            \
    if (NF > 2) *reinterpret_cast<uint4*>(d_ + 64 * kARow) = S##2;            \
    if (NF > 3) *reinterpret_cast<uint4*>(d_ + 96 * kARow) = S##3;            \
  } while (0)

  f32x16_t acc[NF][2];
#pragma unroll
  for (int f = 0; f < NF; f++) {
    acc[f][0] = f32x16_t{};
    acc[f][1] = f32x16_t{};
  }

  const int aoff0 = col * kARow + h * 64;  // lane's A bytes: row 32 f + col, columns 32 h + 8 c
  // Scale and bias of one block (the blob's fp16 pair) broadcast to both
  // halves, which the packed FMA takes by operand selection; zero (weights
  // rebuild to 0) for groups padded past G.
  // With the subnormal rebuild the scale is taken times 2^20 (exact: |s| < 2^-4).
  auto sbpair = [&](uint32_t sb, bool live, f16x2v_t& s2, f16x2v_t& b2) {
    f16x2v_t v = __builtin_bit_cast(f16x2v_t, live ? sb : 0u);
    if constexpr (kSmall) v.x = __builtin_ldexpf16(v.x, 20);
    s2 = __builtin_shufflevector(v, v, 0, 0);
    b2 = __builtin_shufflevector(v, v, 1, 1);
  };
  auto rebuild2 = [&](uint32_t d0, uint32_t d1, f16x2v_t s0, f16x2v_t b0, f16x2v_t s1, f16x2v_t b1, f16x8_t& o0,
                      f16x8_t& o1) {
    if constexpr (kSmall) {
      rebuild16_small(d0, d1, s0, b0, s1, b1, o0, o1);
    } else {
      o0 = dequant8(d0, s0, b0);
      o1 = dequant8(d1, s1, b1);
    }
  };
  // B operands of k-step 0 of the current group, rebuilt during the last
  // k-step of the previous group.
  f16x8_t bc0, bc1;
  // MFMAs of one K group (codes q, A buffer `cur`), software pipelined: the
  // A fragments and weights of k-step c+1 (for c = 3: k-step 0 of the next
  // group, codes qn) are read and rebuilt while the MFMAs of k-step c run.
  auto compute = [&](int cur, const QG& q, const QG& qn, bool live, bool live_n) {
    f16x2v_t s20, b20, s21, b21, n20, m20, n21, m21;
    uint32_t cw0[4], cw1[4];
    if constexpr (!kPre) {
      sbpair(q.s0, live, s20, b20);
      sbpair(q.s1, live, s21, b21);
      sbpair(qn.s0, live_n, n20, m20);
      sbpair(qn.s1, live_n, n21, m21);
      cw0[0] = q.c0.x; cw0[1] = q.c0.y; cw0[2] = q.c0.z; cw0[3] = q.c0.w;
      cw1[0] = q.c1.x; cw1[1] = q.c1.y; cw1[2] = q.c1.z; cw1[3] = q.c1.w;
    }
    const uint8_t* abase = at + cur * kABufBytes + aoff0;
    f16x8_t av[NF];
#pragma unroll
    for (int f = 0; f < NF; f++) av[f] = *reinterpret_cast<const f16x8_t*>(abase + f * 32 * kARow);
#pragma unroll
    for (int c = 0; c < 4; c++) {
      f16x8_t an[NF], bn0, bn1;
      if (c < 3) {
#pragma unroll
        for (int f = 0; f < NF; f++) an[f] = *reinterpret_cast<const f16x8_t*>(abase + f * 32 * kARow + (c + 1) * 16);
        if constexpr (kPre) {
          bn0 = __builtin_bit_cast(f16x8_t, q.b0[c + 1]);
          bn1 = __builtin_bit_cast(f16x8_t, q.b1[c + 1]);
        } else {
          rebuild2(cw0[c + 1], cw1[c + 1], s20, b20, s21, b21, bn0, bn1);
        }
      } else {
        if constexpr (kPre) {
          bn0 = __builtin_bit_cast(f16x8_t, qn.b0[0]);
          bn1 = __builtin_bit_cast(f16x8_t, qn.b1[0]);
        } else {
          rebuild2(qn.c0.x, qn.c1.x, n20, m20, n21, m21, bn0, bn1);
        }
      }
#pragma unroll
      for (int f = 0; f < NF; f++) {
        acc[f][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[f], bc0, acc[f][0], 0, 0, 0);
        acc[f][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[f], bc1, acc[f][1], 0, 0, 0);
      }
      if (c < 3) {
#pragma unroll
        for (int f = 0; f < NF; f++) av[f] = an[f];
      }
      bc0 = bn0;
      bc1 = bn1;
    }
  };

  // Pipeline step of group g: MFMAs of g (codes Q, A buffer g%2; QN holds
  // the codes of g+1), A of g+1 into the other buffer, loads of A for g+3
  // (register set AS) and of the codes of g+4 (into Q, which g no longer
  // needs).
#define MOE_GEMM_STEP(g, CUR, Q, QN, AS)                     \
  do {                                                       \
    if (wave_cols) compute(CUR, Q, QN, (g) < G, (g) + 1 < G);  \
    MOE_STORE_A((CUR) ^ 1, as);               \
    MOE_LOAD_A((g) + 2, as);                  \
    load_q((g) + (kPre ? 2 : 4), Q);          \
    __syncthreads();                          \
  } while (0)

  uint4 as0 = make_uint4(0, 0, 0, 0), as1 = as0, as2 = as0, as3 = as0;
  // Prologue: A of group 0 into LDS, A of group 1 in registers, codes of
  // groups 1..3 in flight.
  MOE_LOAD_A(0, as);
  load_q(1, q1);
  if constexpr (!kPre) {
    load_q(2, q2);
    load_q(3, q3);
  }
  MOE_STORE_A(0, as);
  MOE_LOAD_A(1, as);
  if (wave_cols) {
    if constexpr (kPre) {
      bc0 = __builtin_bit_cast(f16x8_t, q0.b0[0]);
      bc1 = __builtin_bit_cast(f16x8_t, q0.b1[0]);
    } else {
      f16x2v_t s20, b20, s21, b21;
      sbpair(q0.s0, true, s20, b20);
      sbpair(q0.s1, true, s21, b21);
      rebuild2(q0.c0.x, q0.c1.x, s20, b20, s21, b21, bc0, bc1);
    }
  }
  __syncthreads();

  // G is padded up to a multiple of 4 with groups whose weights read as zero;
  // a loop without early exits lets the compiler count the loads in flight
  // across the back edge instead of draining them at the loop header.
  const int Gp = (G + 3) & ~3;
  for (int g = 0; g < Gp; g += 4) {
    if constexpr (kGateUp) {
      // Issue priority by the work left, in quarters of the K loop.  Of two
      // workgroups on a compute unit the older one otherwise wins every tie
      // and the pair finishes far apart (full tiles: 52 and 67 us per
      // 2048-token chunk); this way the one behind outranks the other, the
      // pair ends closer together and the small tiles that follow start
      // together.  (The down GEMM's loop, 8 groups, is too short for it.)
      const int q = ((Gp - g) * 4 - 1) / Gp;  // 3 .. 0
      if (q >= 3) __builtin_amdgcn_s_setprio(3);
      else if (q == 2) __builtin_amdgcn_s_setprio(2);
      else if (q == 1) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    if constexpr (kPre) {  // two register sets: codes of g+2 into the set g used
      MOE_GEMM_STEP(g, 0, q0, q1, ao);
      MOE_GEMM_STEP(g + 1, 1, q1, q0, ae);
      MOE_GEMM_STEP(g + 2, 0, q0, q1, ao);
      MOE_GEMM_STEP(g + 3, 1, q1, q0, ae);
    } else {
      MOE_GEMM_STEP(g, 0, q0, q1, ao);
      MOE_GEMM_STEP(g + 1, 1, q1, q2, ae);
      MOE_GEMM_STEP(g + 2, 0, q2, q3, ao);
      MOE_GEMM_STEP(g + 3, 1, q3, q0, ae);
    }
  }
#undef MOE_GEMM_STEP
#undef MOE_LOAD_A
#undef MOE_STORE_A

  // ---- epilogue (the last step ended with a barrier: LDS is free) ----
  // gate/up: fp16(silu(256 g) * 256 u / 256) into hbuf; down: fp16(out / 256)
  // into obuf, routed and shared rows alike (the shared expert's rows after the
  // routed ones), combined per token later (k_combine).  The tile is
  // assembled in LDS, then stored row by row in 16-byte pieces.
  constexpr int kRowB = kGateUp ? kEpiRowGateUp : kEpiRowDown;
  if (wave_cols) {
#pragma unroll
    for (int f = 0; f < NF; f++) {
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const int r = f * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        if (kGateUp) {
          const float hv = silu_mul(256.f * acc[f][0][i], 256.f * acc[f][1][i]);
          *reinterpret_cast<uint16_t*>(smem + r * kRowB + (wave * 32 + col) * 2) = f32_to_f16_bits(hv * (1.f / 256.f));
        } else {
          *reinterpret_cast<uint16_t*>(smem + r * kRowB + (wave * 64 + col) * 2) = f32_to_f16_bits(acc[f][0][i]);
          *reinterpret_cast<uint16_t*>(smem + r * kRowB + (wave * 64 + 32 + col) * 2) = f32_to_f16_bits(acc[f][1][i]);
        }
      }
    }
  }
  __syncthreads();
  constexpr int kColsWg = kGateUp ? kGateUpColsPerWg : kDownColsPerWg;
  constexpr int kPieces = kColsWg / 8;           // 16-byte pieces per row
  constexpr int kRowsPerPass = kWaves * 64 / kPieces;
  const int piece = tid % kPieces, prow = tid / kPieces;
  const int c0 = T.ct * kColsWg + piece * 8;      // first column of this thread's piece
  if (c0 < T.ncols) {
    uint16_t* dst = kGateUp ? C.hbuf + (int64_t)T.rowbase * C.Imax + c0 : C.obuf + (int64_t)T.rowbase * H + c0;
    const int64_t rs = kGateUp ? C.Imax : H;
#pragma unroll
    for (int r = prow; r < NF * 32; r += kRowsPerPass)
      if (r < T.rows) *reinterpret_cast<uint4*>(dst + r * rs) = *reinterpret_cast<const uint4*>(smem + r * kRowB + piece * 16);
  }
}

template <bool kGateUp, bool kPre>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_expert_gemm(LayerArgs L, ChunkArgs C, int n_ct) {
  // ---- workgroup -> (tile, column tile), XCD-aware ----
  const int lin = blockIdx.x;
  const int xcd = lin & 7, m = lin >> 3;
  const int slot = (m / n_ct) * 8 + xcd, ct = m % n_ct;
  // The entry count and the slot's descriptor are read together (independent loads).
  const int4* sc = reinterpret_cast<const int4*>(C.sched);
  const int nt = sc[0].x;
  const int4 d = sc[1 + (slot < nt ? slot : 0)];
  const bool small_scales = !kPre && *L.small_scales != 0;
  if (slot >= nt) return;
  Tile T;
  T.e = d.x;
  T.r0 = d.y;
  T.rows = d.z;
  T.rowbase = d.w;  // hbuf / obuf row of the tile's first row
  T.ct = ct;
  T.shared = T.e == L.E;
  const int Iw = T.shared ? L.Is : L.I;
  if (Iw == 0 || T.rows <= 0) return;
  // gate/up: columns = intermediate (32-row blocks of gate and up); down: output columns.
  T.ncols = kGateUp ? Iw : L.H;
  if (ct * (kGateUp ? kGateUpColsPerWg : kDownColsPerWg) >= T.ncols) return;
  T.G = (kGateUp ? L.H : Iw) / kGroup;

  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int nf = (T.rows + 31) >> 5;
  if (kPre || !small_scales) {
    if (nf <= 1)
      gemm_tile<kGateUp, 1, kPre, false>(L, C, T, smem);
    else if (nf == 2)
      gemm_tile<kGateUp, 2, kPre, false>(L, C, T, smem);
    else if (nf == 3)
      gemm_tile<kGateUp, 3, kPre, false>(L, C, T, smem);
    else
      gemm_tile<kGateUp, 4, kPre, false>(L, C, T, smem);
  } else if constexpr (!kPre) {
    if (nf <= 1)
      gemm_tile<kGateUp, 1, false, true>(L, C, T, smem);
    else if (nf == 2)
      gemm_tile<kGateUp, 2, false, true>(L, C, T, smem);
    else if (nf == 3)
      gemm_tile<kGateUp, 3, false, true>(L, C, T, smem);
    else
      gemm_tile<kGateUp, 4, false, true>(L, C, T, smem);
  }
}

// y[t] = 256 * obuf[T k + t] (the shared expert's row) + sum_j w_tj * 256 * obuf[pos(t, j)]
// in top-k order.  One workgroup per token, 8 columns per thread.
__global__ __launch_bounds__(256) void k_combine(LayerArgs L, ChunkArgs C) {
  const int t = blockIdx.x;
  const int H = L.H, k = L.k;
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    float acc[8];
    if (L.Is > 0) {
      const uint4 o = *reinterpret_cast<const uint4*>(C.obuf + ((int64_t)C.Tk + t) * H + c);
      const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const f16x2v_t p = __builtin_bit_cast(f16x2v_t, ow[i]);
        acc[2 * i] = 256.f * (float)p.x;
        acc[2 * i + 1] = 256.f * (float)p.y;
      }
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
int gemm_wgs_per_cu() { return 8 / kWaves; }  // 8 waves, two per SIMD, per compute unit

int gateup_col_tiles(int I, int Is) {
  const int Imax = I > Is ? I : Is;
  return (Imax + kGateUpColsPerWg - 1) / kGateUpColsPerWg;
}

template <bool kGateUp, bool kPre>
static hipError_t launch_expert_gemm(const LayerArgs& L, const ChunkArgs& C, int max_sched, hipStream_t s,
                                     const KTime& kt) {
  constexpr int smem = kGateUp ? kSmemGateUp : kSmemDown;
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = lds_limit_once(reinterpret_cast<const void*>(&k_expert_gemm<kGateUp, kPre>), smem, lds_set);
  if (e != hipSuccess) return e;
  const int n_ct = kGateUp ? gateup_col_tiles(L.I, L.Is) : (L.H + kDownColsPerWg - 1) / kDownColsPerWg;
  const int tiles8 = (max_sched + 7) / 8 * 8;
  MOE_LAUNCH((k_expert_gemm<kGateUp, kPre>), dim3((unsigned)(tiles8 * n_ct)), dim3(kWaves * 64), smem, s, kt.start,
             kt.stop, L, C, n_ct);
  return hipGetLastError();
}

hipError_t launch_gateup_gemm(const LayerArgs& L, const ChunkArgs& C, int max_sched, hipStream_t s,
                              const KTime& kt) {
  return L.wdq ? launch_expert_gemm<true, true>(L, C, max_sched, s, kt)
               : launch_expert_gemm<true, false>(L, C, max_sched, s, kt);
}

hipError_t launch_down_gemm(const LayerArgs& L, const ChunkArgs& C, int max_sched, hipStream_t s,
                            const KTime& kt) {
  return L.wdq ? launch_expert_gemm<false, true>(L, C, max_sched, s, kt)
               : launch_expert_gemm<false, false>(L, C, max_sched, s, kt);
}

// ---------------------------------------------------------------------------
// Separate-dequant measurement ("Optimizing on-device inference for Apple
// Silicon", section "Dequantise weights during matrix multiplication": the
// alternative of rebuilding the weights in a pass of their own): the chunk's
// active experts and the shared expert rebuilt as fp16 into L.wdq, block by
// block, with the same rounding as the fused path (dequant8), so the GEMMs
// that read them give the same bits.  grid = (E + 1 expert slots, kDqSplit).
// ---------------------------------------------------------------------------
constexpr int kDqSplit = 16;

__global__ __launch_bounds__(256) void k_dequant_active(LayerArgs L, ChunkArgs C) {
  const int slot = blockIdx.x;
  const int nact = *C.n_active;
  int e;
  if (slot < nact)
    e = C.active[slot];
  else if (slot == nact && L.Is > 0)
    e = L.E;
  else
    return;
  const int64_t base = e == L.E ? L.shared_base : (int64_t)e * L.expert_bytes;
  const int64_t bytes = e == L.E ? L.shared_gateup_bytes + (int64_t)(L.H / 32) * (L.Is / 64) * kBlockBytes
                                 : L.expert_bytes;
  const int nblk = (int)(bytes / kBlockBytes);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, col = lane & 31;
  for (int b = blockIdx.y * 4 + wave; b < nblk; b += kDqSplit * 4) {
    const uint8_t* blk = L.blob + base + (int64_t)b * kBlockBytes;
    const uint4 q = *reinterpret_cast<const uint4*>(blk + lane * 16);
    const f16x2v_t v = __builtin_bit_cast(f16x2v_t, *reinterpret_cast<const uint32_t*>(blk + kCodeBytes + col * 4));
    const f16x2v_t s2 = __builtin_shufflevector(v, v, 0, 0), b2 = __builtin_shufflevector(v, v, 1, 1);
    uint8_t* dst = L.wdq + (base / kBlockBytes + b) * kDqBlockBytes + lane * 16;
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int c = 0; c < 4; c++) *reinterpret_cast<f16x8_t*>(dst + c * 1024) = dequant8(w[c], s2, b2);
  }
}

hipError_t launch_dequant_active(const LayerArgs& L, const ChunkArgs& C, hipStream_t s, const KTime& kt) {
  MOE_LAUNCH(k_dequant_active, dim3((unsigned)(L.E + 1), kDqSplit), dim3(256), 0, s, kt.start, kt.stop, L, C);
  return hipGetLastError();
}

hipError_t launch_combine(const LayerArgs& L, const ChunkArgs& C, hipStream_t s, const KTime& kt) {
  MOE_LAUNCH(k_combine, dim3(C.T), dim3(256), 0, s, kt.start, kt.stop, L, C);
  return hipGetLastError();
}

}  // namespace moe
