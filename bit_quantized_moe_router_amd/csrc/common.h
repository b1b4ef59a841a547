// Device-side definitions shared by the MoE kernels (gfx950 / CDNA4).
//
// Packed weight blob.  The canonical format is the pages' 4-bit group-affine
// one ("Optimizing on-device inference for Apple Silicon", section
// "Dequantise weights during matrix multiplication": 4-bit codes, one bf16
// scale and one bf16 bias per 64 weights).  The blob holds the same bytes
// (0.5625 B per parameter) rearranged into blocks of 32 output rows x 64
// input columns (one quantisation group):
//
//   block = 1024 B of codes + 128 B of (scale, bias)        = 1152 B
//   codes: 64 lanes x 16 B.  Lane l holds row (l % 32) and the 32 columns
//          [32*(l/32), 32*(l/32)+32) of the group as 4 dwords; dword c covers
//          columns 8c..8c+7 of that range with the even columns' codes in
//          nibbles 0..3 and the odd columns' codes in nibbles 4..7.
//   scale/bias: 32 dwords, dword r = fp16(scale) | fp16(bias) << 16 for row
//          r: the bf16 values rounded to fp16 (to nearest even) by the packer.
//          The conversion is exact for magnitudes in [2^-14, 65504]; smaller
//          ones become fp16 subnormals, larger ones infinity.  The kernels
//          rebuild weights in fp16 and so use these values directly: an fp16
//          pair (s, b) feeds a packed FMA with each half broadcast.
//
// A dword d of codes expands to four bf16 pairs with one AND-OR each:
//   ((d >> 4i) & 0x000F000F) | 0x43004300 = (bf16(128 + q[2i]), bf16(128 + q[2i+1]))
// because bf16 0x4300 is 128.0 and the 7 mantissa bits of [128, 256) step by 1.
// The dot product with the codes then carries an offset 128 * sum(x) that the
// kernels remove with the group's per-row activation sum:
//   sum_k x_k (s q_k + b) = s * sum_k x_k (128 + q_k) + (b - 128 s) * sum_k x_k.
//
// Per expert the blob stores gate and up interleaved per (row block, group),
// then down:
//   gate/up block (nb, g, which) at ((nb * H/64 + g) * 2 + which) * 1152
//   down block (nb, g)           at gateup_bytes + (nb * I/64 + g) * 1152
// Routed experts follow each other with stride expert_bytes; the shared expert
// (width Is) follows the last routed expert.  A trailer of kTrailerBytes ends
// the blob; its first int32 is 1 when every stored scale s has |s| < 2^-4
// (the packer clears it otherwise), which lets the grouped GEMM rebuild
// weights with the subnormal form (gemm.hip), and the rest is zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kGroup = 64;
constexpr int kBlockRows = 32;
constexpr int kCodeBytes = 1024;
constexpr int kBlockBytes = 1152;
constexpr int kTrailerBytes = 256;
// fp16 bits of 2^-4: stored scales below it in magnitude allow the subnormal rebuild.
constexpr uint32_t kSmallScaleBits = 0x2C00u;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Blob geometry and per-chunk pointers passed by value to every kernel.
struct LayerArgs {
  const uint8_t* blob;
  int H, E, k, I, Is;
  int64_t expert_bytes;         // routed expert stride
  int64_t gateup_bytes;         // routed gate/up region
  int64_t shared_base;          // byte offset of the shared expert
  int64_t shared_gateup_bytes;  // shared gate/up region
  const int32_t* small_scales;  // the trailer's flag: 1 = every |s| < 2^-4
  // Separate-dequant measurement only (else null): fp16 weights, each 1152-byte
  // block of the blob expanded to 4096 bytes at the same block index; in a
  // block, the 8 weights of lane l for MFMA k-step c sit at c * 1024 + l * 16.
  uint8_t* wdq;
};

constexpr int kDqBlockBytes = 4096;

struct ChunkArgs {
  const uint16_t* x;      // [T][H] bf16
  const uint16_t* x16;    // [T][H] fp16(x / 256), operand of the grouped GEMM
  int T;                  // tokens in this chunk
  int Tk;                 // T * k: first hbuf row of the shared expert
  const float* xsum;      // [T][H/64] per-group activation sums
  const int32_t* ids;     // [T][k]
  const float* tw;        // [T][k]
  const int32_t* counts;  // [E]
  const int32_t* offsets; // [E+1]
  const int32_t* sorted;  // [T*k]
  const int32_t* inv;     // [T*k] inverse of sorted: position of assignment t*k+j
  const int32_t* tiles;   // [..][3]
  const int32_t* n_tiles; // [1]
  const int32_t* sched;   // [1 + n][4]: entry 0 = (n, 0, 0, 0), then n tiles (or pieces of
                          // tiles) in execution order (longest first): expert, first row,
                          // rows, first row in expert-sorted order
  const int32_t* active;  // [E] experts with rows, increasing
  const int32_t* n_active;// [1]
  uint16_t* hbuf;         // [T*k + T][Imax]: fp16(h / 256), grouped-GEMM path
  uint16_t* obuf;         // [T*k + T][H] GEMM path: fp16(expert output / 256), routed rows per sorted position, then the shared rows
  float* y;               // [T][H]
  int Imax;               // row stride of hbuf
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Four bf16 pairs (128 + code) from one packed dword.
__device__ __forceinline__ void expand_codes(uint32_t d, uint32_t out[4]) {
  out[0] = (d & 0x000F000Fu) | 0x43004300u;
  out[1] = ((d >> 4) & 0x000F000Fu) | 0x43004300u;
  out[2] = ((d >> 8) & 0x000F000Fu) | 0x43004300u;
  out[3] = ((d >> 12) & 0x000F000Fu) | 0x43004300u;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  uint4 v = make_uint4(a, b, c, d);
  return __builtin_bit_cast(bf16x8_t, v);
}

// bf16 bits -> fp16 bits of value / 256 (exact whenever the result is normal).
__device__ __forceinline__ uint16_t f32_to_f16_scaled(uint16_t b) {
  return __builtin_bit_cast(uint16_t, (_Float16)(bf16_bits_to_f32(b) * 0.00390625f));
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// silu(g) * u with the reciprocal instruction (about 1 ulp) in place of an
// IEEE division; g -> -inf gives -0 (1 + e^-g = inf, rcp = 0), as the division does.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Expert weight base pointer and widths.
__device__ __forceinline__ const uint8_t* expert_base(const LayerArgs& L, int e) {
  return L.blob + (e == L.E ? L.shared_base : (int64_t)e * L.expert_bytes);
}

}  // namespace moe
