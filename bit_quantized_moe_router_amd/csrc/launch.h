// Host-side launchers of the MoE kernels (one per kernel family).
#pragma once

#include <hip/hip_ext.h>

#include <atomic>

#include "common.h"

namespace moe {

// Timing of one launcher call: the first kernel it enqueues stamps `start`
// with its own start and the last one stamps `stop` with its own end
// (hipExtLaunchKernel), so the interval holds the kernels and not the
// dispatch gap before them.  Null events: a plain launch.
// A kernel's dynamic-LDS limit (needed above 64 KB), set once per device on
// the current device; `done` holds one bit per device.
inline hipError_t lds_limit_once(const void* fn, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const uint64_t bit = 1ull << dev;
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  done.fetch_or(bit, std::memory_order_acq_rel);
  return hipSuccess;
}

// Assignments per segment of the many-token routing metadata.
constexpr int kSegAssign = 1024;

struct KTime {
  hipEvent_t start = nullptr, stop = nullptr;
};

#define MOE_LAUNCH(kernel, grid, block, smem, stream, ev0, ev1, ...)                                 \
  do {                                                                                               \
    if ((ev0) != nullptr || (ev1) != nullptr)                                                        \
      hipExtLaunchKernelGGL(kernel, grid, block, smem, stream, ev0, ev1, 0, __VA_ARGS__);            \
    else                                                                                             \
      kernel<<<grid, block, smem, stream>>>(__VA_ARGS__);                                            \
  } while (0)

struct PackArgs {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* biases;
  uint8_t* dst;
  int M, N, K;
  int64_t dst_base;
  int64_t stride_m;
  int64_t stride_nb;
  int64_t stride_g;
  int32_t* small_scales;  // the blob trailer's flag, cleared by a scale with |s| >= 2^-4
};

hipError_t launch_pack(const PackArgs& P, hipStream_t s);
// Writes the blob trailer (flag = 1, rest zero) before the matrices are packed.
hipError_t launch_pack_trailer(uint8_t* trailer, hipStream_t s);
// Router logits: exact float64 ones for T <= 8, otherwise bf16-MFMA screened
// partial sums over 4 slices of h (and partial squared router row norms);
// *two_launches tells which.
hipError_t launch_route_logits(const uint16_t* x, int T, int H, const float* wr, const float* bias, int E,
                               int k, float* logits, double* wsq, int32_t* ids, float* tw, float* xsum,
                               uint16_t* x16, int32_t* segcnt, hipStream_t s, bool* two_launches,
                               const KTime& kt = KTime{});
// Top-k selection (exact recomputation of the screened candidates for T > 8).
hipError_t launch_route_select(const uint16_t* x, int T, int H, const float* wr, const float* bias, int E,
                               int k, const float* logits, const double* wsq, int32_t* ids, float* tw,
                               uint16_t* x16, int32_t* segcnt, hipStream_t s, const KTime& kt = KTime{});
// max_long: tiles of more than BM/2 rows that the schedule keeps whole (the
// rest are cut in two); 0 keeps every tile whole.  segcnt: per-segment expert
// counts of the assignments (kSegAssign ids a segment), taken by the exact
// top-k; used when there is more than one segment.
hipError_t launch_meta(const int32_t* ids, int T, int k, int E, int BM, int with_shared, int max_long,
                       int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* tiles,
                       int32_t* n_tiles, int32_t* active, int32_t* n_active, int32_t* inv,
                       int32_t* sched, const int32_t* segcnt, hipStream_t s, const KTime& kt = KTime{});
// T <= 8: top-k of exact logits and the metadata in one single-workgroup launch.
hipError_t launch_topk_meta(const float* logits, int T, int E, int k, int32_t* ids, float* tw, int BM,
                            int with_shared, int32_t* counts, int32_t* offsets, int32_t* sorted,
                            int32_t* tiles, int32_t* n_tiles, int32_t* active, int32_t* n_active,
                            int32_t* inv, int32_t* sched, hipStream_t s, const KTime& kt = KTime{});
// max_sched: upper bound of the schedule's entry count (sizes the grid).
hipError_t launch_gateup_gemm(const LayerArgs& L, const ChunkArgs& C, int max_sched, hipStream_t s,
                              const KTime& kt = KTime{});
hipError_t launch_down_gemm(const LayerArgs& L, const ChunkArgs& C, int max_sched, hipStream_t s,
                            const KTime& kt = KTime{});
// Separate-dequant measurement: the chunk's active experts (and the shared
// expert) rebuilt as fp16 into L.wdq; the GEMMs then read B from there.
hipError_t launch_dequant_active(const LayerArgs& L, const ChunkArgs& C, hipStream_t s, const KTime& kt = KTime{});
// Gate/up column tiles per row tile (the GEMM grid's second dimension).
int gateup_col_tiles(int I, int Is);
// Grouped-GEMM workgroups resident per compute unit.
int gemm_wgs_per_cu();
// y[t] += sum_j w_tj * routed output of assignment (t, j) (GEMM path).
hipError_t launch_combine(const LayerArgs& L, const ChunkArgs& C, hipStream_t s, const KTime& kt = KTime{});
// Decode GEMV path: top-k, gate/up + SwiGLU and the down projection split
// over the intermediate (partial outputs in `part`), then their fixed-order sum.
hipError_t launch_gemv_experts(const LayerArgs& L, const ChunkArgs& C, const float* logits, float* part,
                               hipStream_t s, const KTime& kt = KTime{});
hipError_t launch_gemv_reduce(const LayerArgs& L, const ChunkArgs& C, const float* part, hipStream_t s,
                              const KTime& kt = KTime{});
// Decode with the grouped-GEMM path's arithmetic: top-k (ranked routing into
// ids/tw), gate/up + SwiGLU into h16 ([T*k + T][Imax] fp16(h / 256)); then the
// down projection of every assignment and the per-token combine into y.
hipError_t launch_gemv_gateup_bi(const LayerArgs& L, const ChunkArgs& C, const float* logits, uint16_t* h16,
                                 int32_t* ids, float* tw, hipStream_t s, const KTime& kt = KTime{});
hipError_t launch_gemv_down_bi(const LayerArgs& L, const ChunkArgs& C, const uint16_t* h16, const int32_t* ids,
                               const float* tw, hipStream_t s, const KTime& kt = KTime{});

// Measurement probes (csrc/probe.hip): a 16-byte-per-lane streaming read of
// `bytes` with at most max_wgs workgroups (sink: max_wgs words), and the
// MFMA-only rate kernel over `wgs` workgroups (clocks: 2 * wgs words or null;
// sink: wgs words).
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int max_wgs, hipStream_t s,
                              const KTime& kt = KTime{});
hipError_t launch_mfma_rate(int iters, int wgs, uint64_t* clocks, uint32_t* sink, hipStream_t s,
                            const KTime& kt = KTime{});

}  // namespace moe
