// Calibration kernels for the benchmark (not part of libexact_attn.so), so that the rates the
// attention kernels reach can be set beside what plain kernels reach on the same GPU:
//   * stream_read_kernel, a streaming read of a device buffer (HBM read rate).  Each workgroup
//     reads one contiguous share of the buffer, every thread eight 16-byte nontemporal loads in
//     flight (the fastest of the plain forms measured: grid-stride loads, four or eight in
//     flight, with and without the hint), folded into one word so that the loads cannot be
//     removed; one word per workgroup is written.
//   * atomic_add_kernel, fp32 atomic adds in 64 x 128 tiles (the atomic rate that a backward
//     summing dQ shares with atomics would depend on).
//   * mfma_loop_kernel, back-to-back v_mfma_f32_32x32x16_bf16 on four independent
//     accumulators per wave (dense bf16 matrix-core rate), which also reads the shader-clock
//     counter (s_memtime) and the 100 MHz reference counter (s_memrealtime) around its loop,
//     so that the clock the matrix cores run at under full load follows from their ratio.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16, uint32_t* out) {
  const size_t chunk = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t base = (size_t)blockIdx.x * chunk;
  const size_t end = base + chunk < n16 ? base + chunk : n16;
  size_t i = base + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * 256 < end; i += 8 * 256) {
    u32x4 v[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) v[f] = __builtin_nontemporal_load(p + i + 256 * f);
#pragma unroll
    for (int f = 0; f < 8; ++f) acc ^= v[f][0] ^ v[f][1] ^ v[f][2] ^ v[f][3];
  }
  for (; i < end; i += 256) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
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

typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* __restrict__ sink,
                                                        unsigned long long* __restrict__ ticks) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (short)(0x3c00 + lane);  // about 2^-7: the sums stay far from overflow
    b[i] = (short)(0x3c00 - i);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  __builtin_amdgcn_sched_barrier(0);
  for (int it = 0; it < iters; it += 2) {  // two rounds per pass: loop overhead under 2%
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  __builtin_amdgcn_sched_barrier(0);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    ticks[2 * (size_t)blockIdx.x] = t1 - t0;
    ticks[2 * (size_t)blockIdx.x + 1] = r1 - r0;
  }
}

// fp32 atomic adds (no return value) into an accumulator of `heads` x N rows of 128 floats, in
// tiles of 64 rows: the traffic a backward would make that summed each key block's dQ share into
// one fp32 dQ with atomics.  Workgroup w adds `reps` tiles of head w % heads; 256 threads add
// 32 floats each per tile.
__global__ __launch_bounds__(256) void atomic_add_kernel(float* __restrict__ acc, int heads, int N, int reps) {
  const int h = blockIdx.x % heads, ntile = N / 64;
  float* base = acc + (size_t)h * N * 128;
  for (int r = 0; r < reps; ++r) {
    float* tp = base + (size_t)((blockIdx.x / heads + 7 * r) % ntile) * (64 * 128);
#pragma unroll 8
    for (int i = 0; i < 32; ++i) atomicAdd(tp + 256 * i + threadIdx.x, 1.0f);
  }
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

// Runs `blocks` workgroups of 256 threads (four waves), each wave issuing 4 * `iters` (`iters`
// even) dense bf16 32x32x16 matrix products (32768 flops each) from registers.  `sink` (device,
// 256 floats per workgroup) receives the folded products; `ticks` (device, 2 words per
// workgroup) the shader-clock cycles and the 100 MHz reference ticks of wave 0's loop.  Returns
// the hipError_t of the launch.
int calib_mfma(int blocks, int iters, float* sink, unsigned long long* ticks, void* stream) {
  if (sink == nullptr || ticks == nullptr || blocks <= 0 || iters <= 0 || iters % 2 != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink, ticks);
  return (int)hipGetLastError();
}

// Runs `blocks` workgroups of atomic_add_kernel on `acc` (device, heads * N * 128 floats; N a
// positive multiple of 64), each adding `reps` tiles of 64 x 128 floats.  Returns the
// hipError_t of the launch.
int calib_atomic_add(float* acc, int heads, int N, int reps, int blocks, void* stream) {
  if (acc == nullptr || heads <= 0 || N < 64 || N % 64 != 0 || reps <= 0 || blocks <= 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(atomic_add_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, acc, heads, N, reps);
  return (int)hipGetLastError();
}

}  // extern "C"
