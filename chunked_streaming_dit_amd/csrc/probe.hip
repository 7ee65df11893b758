// Measured ceilings for the roofline figures: a dense bf16 MFMA loop and a plain copy.
//
// The spec peaks (2.5 PFLOP/s dense bf16 MFMA, 8 TB/s HBM) assume clocks and power that a
// real workload may not get.  These two kernels measure what the board sustains while
// they run, so that a kernel's rate can also be stated as a fraction of a measured
// ceiling: the MFMA loop keeps the matrix pipes busy with operands whose bits change
// from one instruction to the next (as real data does), and the copy streams a buffer
// far larger than the caches.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int PROBE_WAVES = 4;  // waves per workgroup
constexpr int PROBE_ACC = 4;    // independent accumulator chains per wave

// Each wave alternates two operand sets (loaded once from `data`, unrelated bit
// patterns) over PROBE_ACC independent accumulator chains: 2 PROBE_ACC
// v_mfma_f32_32x32x16_bf16 per iteration, no memory traffic in the loop; one float per
// lane is written at the end so the work is kept.
__global__ __launch_bounds__(64 * PROBE_WAVES) void probe_mfma_kernel(const bf16x8* __restrict__ data, int iters,
                                                                      float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const bf16x8 a0 = data[lane], b0 = data[64 + lane], a1 = data[128 + lane], b1 = data[192 + lane];
  f32x16 acc[PROBE_ACC];
#pragma unroll
  for (int j = 0; j < PROBE_ACC; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < PROBE_ACC; ++j) acc[j] = mfma32(a0, b0, acc[j]);
#pragma unroll
    for (int j = 0; j < PROBE_ACC; ++j) acc[j] = mfma32(a1, b1, acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < PROBE_ACC; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// dst[i] = src[i] over n 16-byte chunks: each thread moves COPY_UNROLL chunks per round
// (all loads issued before the stores, so that many requests are in flight), grid-stride
// over rounds; the ragged end is handled one chunk at a time.
constexpr int COPY_UNROLL = 4;
__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         long long n) {
  const long long per_round = (long long)gridDim.x * blockDim.x * COPY_UNROLL;
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long full = n / per_round * per_round;
  for (long long base = 0; base < full; base += per_round) {
    u32x4 v[COPY_UNROLL];
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; ++u) v[u] = src[base + t + (long long)u * gridDim.x * blockDim.x];
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; ++u) dst[base + t + (long long)u * gridDim.x * blockDim.x] = v[u];
  }
  for (long long i = full + t; i < n; i += (long long)gridDim.x * blockDim.x) dst[i] = src[i];
}

}  // namespace

hipError_t probe_mfma(const void* data, int iters, float* sink, double* flop, hipStream_t s) {
  const int wgs = PROBE_SINK_FLOATS / (64 * PROBE_WAVES);
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(wgs), dim3(64 * PROBE_WAVES), 0, s,
                     reinterpret_cast<const bf16x8*>(data), iters, sink);
  *flop = (double)wgs * PROBE_WAVES * iters * 2 * PROBE_ACC * (2.0 * 32 * 32 * 16);
  return hipGetLastError();
}

hipError_t probe_copy(const void* src, void* dst, long long bytes, hipStream_t s) {
  const long long n = bytes / 16;
  const int wgs = device_cus() * 8;
  hipLaunchKernelGGL(probe_copy_kernel, dim3(wgs), dim3(256), 0, s, reinterpret_cast<const u32x4*>(src),
                     reinterpret_cast<u32x4*>(dst), n);
  return hipGetLastError();
}

}  // namespace dit
