// Measurement probes: the rates the layer's kernels are judged against on the
// device they run on.  The pages judge their expert kernels against the
// fastest sustained weight-read rate of the access pattern ("Optimizing
// on-device inference for Apple Silicon", section "Limits of further
// optimisation"); these probes measure that rate for this device and the
// MFMA rate the grouped GEMMs can reach at the clock the device holds under
// MFMA load.  Not part of the forward path.
//
//  * k_stream_read: every lane reads 16-byte pieces (the GEMV's and the
//    GEMMs' weight-load width), eight in flight per lane, grid-strided; the
//    values are folded into one word that is stored only if it equals a value
//    the fold cannot produce from the probe's input, so the loads stay live
//    and nothing is written.
//  * k_mfma_rate: eight independent v_mfma_f32_32x32x16_f16 accumulators per
//    wave, two waves per SIMD (the grouped GEMMs' occupancy); wave 0 of each
//    workgroup records the shader-clock counter and the constant-rate counter
//    at its start and end, so the host can derive the clock held under load.
#include "launch.h"

namespace moe {

constexpr int kProbeThreads = 256;
constexpr int kProbeInFlight = 8;  // 16-byte loads in flight per lane

__global__ __launch_bounds__(kProbeThreads) void k_stream_read(const uint4* __restrict__ src, int64_t n16,
                                                               uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i < n16; i += stride * kProbeInFlight) {
    uint4 v[kProbeInFlight];
#pragma unroll
    for (int p = 0; p < kProbeInFlight; p++) {
      const int64_t j = i + p * stride;
      v[p] = j < n16 ? src[j] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int p = 0; p < kProbeInFlight; p++) acc ^= v[p].x ^ v[p].y ^ v[p].z ^ v[p].w;
  }
  // A store that no real fold is expected to trigger keeps the loads live;
  // should it happen, it stays inside sink (one word per workgroup).
  if (acc == 0xA5A5A5A5u) sink[blockIdx.x] = acc;
}

constexpr int kMfmaChains = 8;

__global__ __launch_bounds__(kProbeThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_mfma_rate(int iters, uint64_t* __restrict__ clocks, uint32_t* __restrict__ sink) {
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  const int lane = threadIdx.x & 63;
  f16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    a[j] = (_Float16)(0.001f * (lane + j));
    b[j] = (_Float16)(0.002f * (lane - j));
  }
  f32x16_t acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; c++) acc[c] = f32x16_t{};
  uint64_t t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; c++) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; c++) s += acc[c][0] + acc[c][15];
  if (threadIdx.x == 0) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (clocks) {
      clocks[2 * blockIdx.x] = t1 - t0;
      clocks[2 * blockIdx.x + 1] = r1 - r0;
    }
  }
  if (s == 12345.678f) sink[blockIdx.x] = 1u;
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int max_wgs, hipStream_t s,
                              const KTime& kt) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t per_wg = (int64_t)kProbeThreads * kProbeInFlight;
  int64_t wgs = (n16 + per_wg - 1) / per_wg;
  if (wgs > max_wgs) wgs = max_wgs;
  MOE_LAUNCH(k_stream_read, dim3((unsigned)wgs), dim3(kProbeThreads), 0, s, kt.start, kt.stop,
             reinterpret_cast<const uint4*>(src), n16, sink);
  return hipGetLastError();
}

hipError_t launch_mfma_rate(int iters, int wgs, uint64_t* clocks, uint32_t* sink, hipStream_t s, const KTime& kt) {
  MOE_LAUNCH(k_mfma_rate, dim3((unsigned)wgs), dim3(kProbeThreads), 0, s, kt.start, kt.stop, iters, clocks, sink);
  return hipGetLastError();
}

}  // namespace moe
