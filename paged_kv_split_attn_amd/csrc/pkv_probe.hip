// Read-bandwidth ceiling probe: the achievable HBM read rate of one launch of a
// given size on this machine, with the decode kernel's load shape (one
// workgroup of eight waves per compute unit, 16-byte loads, 1 KiB per wave
// instruction, eight loads in flight per wave).  Diagnostic only; not part of the attention path.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kProbeDepth = 8;

__global__ void __launch_bounds__(kGroupThreads) read_kernel(const uint4* __restrict__ src, size_t n,
                                                             size_t per_wave,
                                                             uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & (kWave - 1);
  const size_t wave = (size_t)blockIdx.x * kWavesPerGroup + threadIdx.x / kWave;
  const size_t begin = wave * per_wave;
  uint32_t x = 0;
  for (size_t i = begin; i < begin + per_wave; i += (size_t)kWave * kProbeDepth) {
    uint4 r[kProbeDepth];
#pragma unroll
    for (int d = 0; d < kProbeDepth; ++d) {
      const size_t idx = i + (size_t)d * kWave + lane;
      r[d] = idx < n ? src[idx] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int d = 0; d < kProbeDepth; ++d) x ^= r[d].x ^ r[d].y ^ r[d].z ^ r[d].w;
  }
  sink[wave * kWave + lane] = x;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int pkv_debug_read_ceiling(const void* src, size_t bytes, uint32_t* sink,
                                      size_t sink_words, void* stream) {
  if (!src || !sink || bytes < 16 || bytes % 16 != 0) return PKV_ERR_INVALID_ARG;
  const int groups = PKV_READ_CEILING_GROUPS;
  if (sink_words < (size_t)groups * kGroupThreads) return PKV_ERR_INVALID_ARG;
  const size_t n = bytes / 16;
  const size_t waves = (size_t)groups * kWavesPerGroup;
  const size_t quantum = (size_t)kWave * kProbeDepth;
  const size_t per_wave = ((n + waves - 1) / waves + quantum - 1) / quantum * quantum;
  hipLaunchKernelGGL(read_kernel, dim3(groups), dim3(kGroupThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), n, per_wave,
                     sink);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}
