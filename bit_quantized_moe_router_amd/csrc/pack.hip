// Weight packer: canonical 4-bit codes + bf16 scale/bias -> the blob layout
// described in common.h.  One workgroup of 256 threads writes one 1152-byte
// block: thread j writes code dword j (lane j/4, dword j%4) and, for j < 32,
// the scale/bias dword of row j, both converted from bf16 to fp16 (round to
// nearest even, the conversion every kernel would otherwise make on every
// load).  Reads of the canonical rows are 4-byte aligned because K is a
// multiple of 64.  A scale of magnitude 2^-4 or more clears the trailer's flag
// (common.h), which k_pack_trailer sets before the matrices are packed.
#include "launch.h"

namespace moe {

// Gather the even-column nibbles of a canonical dword into the low half and
// the odd-column nibbles into the high half.
__device__ __forceinline__ uint32_t pack_dword(uint32_t c) {
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    uint32_t byte = (c >> (8 * i)) & 0xFFu;
    out |= (byte & 0xFu) << (4 * i);
    out |= (byte >> 4) << (16 + 4 * i);
  }
  return out;
}

__global__ __launch_bounds__(256) void k_pack(PackArgs P) {
  const int G = P.K / kGroup;
  const int NBn = P.N / kBlockRows;
  int64_t blk = blockIdx.x;
  const int g = (int)(blk % G);
  blk /= G;
  const int nb = (int)(blk % NBn);
  const int m = (int)(blk / NBn);
  uint8_t* out = P.dst + P.dst_base + m * P.stride_m + nb * P.stride_nb + g * P.stride_g;

  const int j = threadIdx.x;
  const int lane = j >> 2, c = j & 3;
  const int row = nb * kBlockRows + (lane & 31);
  const int col = g * kGroup + (lane >> 5) * 32 + c * 8;
  const uint8_t* src = P.codes + ((int64_t)m * P.N + row) * (P.K / 2) + col / 2;
  uint32_t cw = *reinterpret_cast<const uint32_t*>(src);
  reinterpret_cast<uint32_t*>(out)[j] = pack_dword(cw);

  if (j < kBlockRows) {
    const int64_t gi = ((int64_t)m * P.N + nb * kBlockRows + j) * G + g;
    const uint32_t s16 = __builtin_bit_cast(uint16_t, (_Float16)bf16_bits_to_f32(P.scales[gi]));
    const uint32_t sb = s16 | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)bf16_bits_to_f32(P.biases[gi])) << 16);
    reinterpret_cast<uint32_t*>(out + kCodeBytes)[j] = sb;
    // Every writer stores the same 0, so the unordered stores need no atomics.
    if ((s16 & 0x7FFFu) >= kSmallScaleBits) *P.small_scales = 0;
  }
}

__global__ __launch_bounds__(64) void k_pack_trailer(uint8_t* trailer) {
  reinterpret_cast<int32_t*>(trailer)[threadIdx.x] = threadIdx.x == 0 ? 1 : 0;
}

hipError_t launch_pack_trailer(uint8_t* trailer, hipStream_t s) {
  static_assert(kTrailerBytes == 64 * 4, "one int32 per thread");
  k_pack_trailer<<<dim3(1), dim3(64), 0, s>>>(trailer);
  return hipGetLastError();
}

hipError_t launch_pack(const PackArgs& P, hipStream_t s) {
  const int64_t blocks = (int64_t)P.M * (P.N / kBlockRows) * (P.K / kGroup);
  if (blocks == 0) return hipSuccess;
  k_pack<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(P);
  return hipGetLastError();
}

}  // namespace moe
