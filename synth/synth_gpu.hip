/*
 * synth_gpu.hip - device build of the seeded input generator (see
 * synth_rng.h).  Writes the same values as synth_cpu.c straight into device
 * memory, so the full-size synthetic logits never cross PCIe.  Holds no part
 * of the loss method.
 */
#include <hip/hip_runtime.h>

#include "synth_rng.h"

namespace {

template <int DTYPE>
__global__ void __launch_bounds__(256) k_fill_normal(uint64_t key, uint64_t offset, int64_t n,
                                                     double stdev, void* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float f = synth_normal_f32(key, offset + (uint64_t)i, stdev);
    if (DTYPE == 0)
      static_cast<float*>(out)[i] = f;
    else
      static_cast<uint16_t*>(out)[i] = synth_f32_to_bf16(f);
  }
}

}  // namespace

/* out[i] = element (offset + i) of stream (seed, stream), i in [0, n), on the
 * device, enqueued on `stream_ptr` (a hipStream_t; NULL = default stream).
 * dtype 0 = binary32, 1 = bfloat16.  Returns 0, or -1 on bad arguments, or the
 * HIP error code of the launch. */
extern "C" int synth_gpu_fill_normal(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n,
                                     double stdev, int dtype, void* out, void* stream_ptr) {
  if (n < 0 || out == nullptr || (dtype != 0 && dtype != 1)) return -1;
  if (n == 0) return 0;
  const uint64_t key = synth_key(seed, stream);
  const int64_t blocks_needed = (n + 255) / 256;
  const unsigned blocks = (unsigned)(blocks_needed < 65536 ? blocks_needed : 65536);
  hipStream_t s = static_cast<hipStream_t>(stream_ptr);
  if (dtype == 0)
    hipLaunchKernelGGL(k_fill_normal<0>, dim3(blocks), dim3(256), 0, s, key, offset, n, stdev, out);
  else
    hipLaunchKernelGGL(k_fill_normal<1>, dim3(blocks), dim3(256), 0, s, key, offset, n, stdev, out);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}
