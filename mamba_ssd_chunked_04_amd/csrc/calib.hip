// Calibration kernels for the benchmark (not part of the SSD library): what
// this GPU actually delivers, measured next to the published peaks.
//   ssd_calib_mfma_f16 : back-to-back v_mfma_f32_16x16x32_f16 on registers
//                        (eight independent accumulators per wave, no memory
//                        traffic) -- the dense fp16 matrix-core rate.  The
//                        MFMAs are written as inline asm on VGPR accumulators:
//                        from the builtins hipcc built a loop that copied
//                        every accumulator between AGPRs and VGPRs on each
//                        iteration, which measured the copies, not the MFMAs;
//   ssd_calib_mfma     : the same loop for another matrix instruction (kind
//                        0: 16x16x32 f16, 1: 32x32x16 f16, 2: 16x16x32 bf16,
//                        3: 16x16x4 fp32), so that each shape's delivered
//                        rate can be set beside the published peak;
//   ssd_calib_read     : a streaming read of a buffer with 16-byte loads (one
//                        float per thread written back) -- the HBM read rate.
// Both enqueue on the given stream and return 0, or a HIP error code.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void mfma_loop_kernel(float *out, int iters) {
  f16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (float)((threadIdx.x + i) & 7));
    b[i] = (_Float16)(0.002f * (float)((threadIdx.x * 3 + i) & 7));
  }
  f32x4 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(acc[k]) : "v"(a), "v"(b));
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// kind 1: 32x32x16 f16, four independent 32x32 accumulators per wave
__global__ __launch_bounds__(256) void mfma32_loop_kernel(float *out, int iters) {
  f16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (float)((threadIdx.x + i) & 7));
    b[i] = (_Float16)(0.002f * (float)((threadIdx.x * 3 + i) & 7));
  }
  f32x16 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[k][r] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc[k]) : "v"(a), "v"(b));
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[k][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// kind 2: 16x16x32 bf16, eight independent accumulators per wave
__global__ __launch_bounds__(256) void mfma_bf16_loop_kernel(float *out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((threadIdx.x + i) & 7));
    b[i] = (__bf16)(0.002f * (float)((threadIdx.x * 3 + i) & 7));
  }
  f32x4 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc[k]) : "v"(a), "v"(b));
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// kind 3: 16x16x4 fp32, eight independent accumulators per wave
__global__ __launch_bounds__(256) void mfma_f32_loop_kernel(float *out, int iters) {
  const float a = 0.001f * (float)(threadIdx.x & 7), b = 0.002f * (float)((threadIdx.x * 3) & 7);
  f32x4 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      asm volatile("v_mfma_f32_16x16x4_f32 %0, %1, %2, %0" : "+v"(acc[k]) : "v"(a), "v"(b));
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void read_kernel(const f32x4 *src, int64_t n4, float *out) {
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += 4 * stride) {
    f32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t j = i + k * stride;
      v[k] = j < n4 ? src[j] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) acc += v[k];
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc[0] + acc[1] + acc[2] + acc[3];
}

}  // namespace

extern "C" {

// `out` holds blocks * 256 floats.  Flops: blocks * 4 waves * iters * 8 * 16384.
int ssd_calib_mfma_f16(float *out, int blocks, int iters, void *stream) {
  if (!out || blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, iters);
  return (int)hipGetLastError();
}

// Flops per call: blocks * 4 waves * iters * (kind 1: 4 * 32768; kinds 0 and
// 2: 8 * 16384; kind 3: 8 * 2048).
int ssd_calib_mfma(float *out, int blocks, int iters, int kind, void *stream) {
  if (!out || blocks < 1 || iters < 1 || kind < 0 || kind > 3) return (int)hipErrorInvalidValue;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (kind == 0) hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)blocks), dim3(256), 0, st, out, iters);
  if (kind == 1) hipLaunchKernelGGL(mfma32_loop_kernel, dim3((unsigned)blocks), dim3(256), 0, st, out, iters);
  if (kind == 2)
    hipLaunchKernelGGL(mfma_bf16_loop_kernel, dim3((unsigned)blocks), dim3(256), 0, st, out, iters);
  if (kind == 3)
    hipLaunchKernelGGL(mfma_f32_loop_kernel, dim3((unsigned)blocks), dim3(256), 0, st, out, iters);
  return (int)hipGetLastError();
}
// Reads `bytes` (a multiple of 16) from the 16-byte aligned `src`; `out`
// holds blocks * 256 floats.
int ssd_calib_read(const void *src, int64_t bytes, float *out, int blocks, void *stream) {
  if (!src || !out || bytes < 16 || (bytes & 15) || ((uintptr_t)src & 15) || blocks < 1)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const f32x4 *>(src), bytes / 16,
                     out);
  return (int)hipGetLastError();
}

}  // extern "C"
