// Measurement probe: the bf16 matrix-core rate this chip sustains, and the
// shader clock it runs at meanwhile, with no memory traffic at all.
//
// Every CU runs one workgroup of 8 waves (two per SIMD).  Each wave keeps
// eight independent 32x32x16 bf16 accumulator chains busy for `iters` rounds
// with operands held in registers, either all zero or pseudo-random values
// in [-1, 1).  Lane 0 of every wave records the shader-clock and 100 MHz
// real-time counter deltas around its loop.  The matrix cores draw more power
// on random operands, and the chip lowers its clock to stay within its power
// budget: the published peak assumes the 2.4 GHz clock.
#include "fd_common.h"
#include "flashdec_kernels.h"

namespace fd {
namespace {

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__device__ __forceinline__ bf16x8 operand(uint32_t seed, bool zero) {
  bf16x8 f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t h = mix32(seed * 8u + (uint32_t)i);
    f[i] = (__bf16)(zero ? 0.0f : ((float)(h & 0xFFFFu) - 32768.0f) * (1.0f / 32768.0f));
  }
  return f;
}

constexpr int kProbeWaves = 8;

__global__ __launch_bounds__(kProbeWaves * 64, 1)
void mfma_probe_kernel(int iters, int zero, float* sink, unsigned long long* clocks) {
  const int tid = threadIdx.x, lane = tid & 63;
  const uint32_t seed = (uint32_t)(blockIdx.x * blockDim.x + tid);
  bf16x8 a[4], b[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = operand(seed * 6u + (uint32_t)i, zero != 0);
#pragma unroll
  for (int j = 0; j < 2; ++j) b[j] = operand(seed * 6u + 4u + (uint32_t)j, zero != 0);
  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += acc[i][j][v];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  sink[blockIdx.x * blockDim.x + tid] = s;
  if (lane == 0) {
    const size_t w = (size_t)blockIdx.x * kProbeWaves + (tid >> 6);
    clocks[2 * w] = t1 - t0;
    clocks[2 * w + 1] = r1 - r0;
  }
}

}  // namespace
}  // namespace fd

extern "C" fd_status fdk_mfma_probe(int zero_operands, int iters, float* sink_dev,
                                    uint64_t* clocks_dev, void* stream) {
  if (!sink_dev || !clocks_dev || iters <= 0) return FD_ERR_INVALID_ARG;
  hipLaunchKernelGGL(fd::mfma_probe_kernel, dim3(FDK_PROBE_WORKGROUPS),
                     dim3(fd::kProbeWaves * 64), 0, (hipStream_t)stream, iters,
                     zero_operands, sink_dev, reinterpret_cast<unsigned long long*>(clocks_dev));
  return hipGetLastError() == hipSuccess ? FD_OK : FD_ERR_DEVICE;
}
