// Sustained matrix-core rates on MI355X (gfx950): a measurement probe for the
// benchmark, not part of the attention path.
//
// Every wave keeps four independent accumulators busy with one instruction type
// (or with the attention forward's mix), operands drawn once per lane from a
// hash of its index and cycled through four fragments, so that the rate and the
// board power under sustained load can be read against the datasheet peaks:
//   mode 0: v_mfma_f32_32x32x16_bf16           (32768 flops per instruction)
//   mode 1: v_mfma_scale_f32_32x32x64_f8f6f4   (E4M3 x E4M3, 131072 flops)
//   mode 2: the forward's mix per 64-key block and 32 query rows at d = 128:
//           16 bf16 logit instructions and 4 FP8 P.V instructions
// One workgroup of 256 threads per compute unit share, two per CU by default;
// the result of every accumulator is folded into one float per thread so the
// work cannot be removed.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;

__device__ inline uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

template <int kMode>
__global__ __launch_bounds__(256, 2) void roof(float* __restrict__ sink, int iters, uint32_t seed) {
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
  // four operand fragments per type: bf16 values in [1, 2) with random mantissas,
  // E4M3 codes with random bits and the NaN pattern cleared
  bf16x8_t a[4], b[4];
  i32x8_t a8[4], b8[4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t h = mix32(seed ^ (tid * 64 + f * 8 + i));
      a[f][i] = __builtin_bit_cast(__bf16, (uint16_t)(0x3F80 | (h & 0x7F)));
      b[f][i] = __builtin_bit_cast(__bf16, (uint16_t)(0x3F80 | ((h >> 7) & 0x7F)));
      a8[f][i] = (int)(h & 0x77777777u);
      b8[f][i] = (int)(mix32(h) & 0x77777777u);
    }
  f32x16_t acc[4] = {};
  f32x16_t acc8[4] = {};
  for (int it = 0; it < iters; ++it) {
    if constexpr (kMode == 0) {
#pragma unroll
      for (int s = 0; s < 16; ++s)
        acc[s % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s % 4], b[(s / 4) % 4], acc[s % 4], 0, 0, 0);
    } else if constexpr (kMode == 1) {
#pragma unroll
      for (int s = 0; s < 16; ++s)
        acc8[s % 4] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8[s % 4], b8[(s / 4) % 4], acc8[s % 4],
                                                                       0, 0, 0, 0, 0, 0);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc8[s] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8[s], b8[s], acc8[s], 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int s = 0; s < 16; ++s)
        acc[s % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s % 4], b[(s / 4) % 4], acc[s % 4], 0, 0, 0);
    }
  }
  float r = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) r += acc[q][i] + acc8[q][i];
  sink[tid] = r;
}

}  // namespace

extern "C" {

// Flops of one launch of pcast_roof_run(mode, iters, blocks, ...), counted as
// 2 * M * N * K per instruction.
double pcast_roof_flops(int mode, int iters, int blocks) {
  const double per_wave = mode == 0 ? 16.0 * 32768 : mode == 1 ? 16.0 * 131072 : 16.0 * 32768 + 4.0 * 131072;
  return per_wave * iters * blocks * 4.0;
}

// Launches the probe: `blocks` workgroups of 256 threads, `iters` iterations each;
// sink holds blocks * 256 floats.  Returns 0, or 1 for a bad argument, or the HIP
// error code of the launch.
int pcast_roof_run(int mode, int iters, int blocks, float* sink, void* stream) {
  if (mode < 0 || mode > 2 || iters < 1 || blocks < 1 || !sink) return 1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (mode == 0) hipLaunchKernelGGL(roof<0>, dim3(blocks), dim3(256), 0, st, sink, iters, 0x9E3779B9u);
  else if (mode == 1) hipLaunchKernelGGL(roof<1>, dim3(blocks), dim3(256), 0, st, sink, iters, 0x9E3779B9u);
  else hipLaunchKernelGGL(roof<2>, dim3(blocks), dim3(256), 0, st, sink, iters, 0x9E3779B9u);
  return (int)hipGetLastError();
}

}  // extern "C"
