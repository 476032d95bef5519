// Calibration kernel for the benchmark (not part of libexact_attn.so): a streaming read of a
// device buffer, so that the HBM read rate the attention kernels reach can be set beside what
// a plain read of the same size reaches on the same GPU.
//
// Every thread reads 16-byte chunks at a grid stride, four loads in flight, and folds them into
// one word so that the loads cannot be removed; one word per workgroup is written.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16, uint32_t* out) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^
           d[2] ^ d[3];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = p[i];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) at `p` with `blocks` workgroups of 256 threads, writing one
// word per workgroup to `out` (device, `blocks` words).  Returns the hipError_t of the launch.
int calib_stream_read(const void* p, size_t bytes, unsigned* out, int blocks, void* stream) {
  if (p == nullptr || out == nullptr || blocks <= 0 || bytes % 16 != 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)p, bytes / 16, (uint32_t*)out);
  return (int)hipGetLastError();
}

}  // extern "C"
