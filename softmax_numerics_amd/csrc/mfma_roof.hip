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
//   mode 3: the forward's softmax VALU work per such block and lane, alone: the
//           max of 32 values (16 v_max3), 32 fma + 32 v_exp_f32 + 32 adds, 16
//           P-cast conversions, 8 + 8 counter instructions
//   mode 4: modes 2 and 3 together, interleaved as in the forward's steady step
//           (P.V under the max and the first half's exponentials, the first logit
//           half under the second half's, the second under the counters), on
//           independent registers, so that the time against modes 2 and 3 alone
//           shows how far the SIMD overlaps matrix-core and VALU work
// One workgroup of 256 threads per compute unit share, two per CU by default;
// the result of every accumulator is folded into one float per thread so the
// work cannot be removed.
//
// A second probe (issue_probe) measures issue costs on one SIMD: 512-thread workgroups,
// one per compute unit, so that each SIMD holds two waves (wave w runs on SIMD w % 4);
// waves 0-3 run kind_lo and waves 4-7 kind_hi, where a kind is one instruction type of
// the forward's step, written out in inline assembly so that the count per iteration is
// exact, or the bf16 matrix-core stream, or the forward's softmax VALU work per block.
// With kind_lo == kind_hi the time gives the throughput of that instruction type with two
// waves per SIMD; with the matrix-core stream beside a VALU kind it shows how far the
// SIMD runs the two side by side.
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
  // softmax-like state: 32 values in (0, 1] that each block's exponentials replace
  float x[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) x[j] = 0.5f + (float)(mix32(seed + tid * 32 + j) & 0xFFFF) * 7.6e-6f;
  float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  uint32_t codes[8] = {}, cnt = 0;
  const float c = 0.12752f;  // log2(e)/sqrt(128)
  float mneg = 0.0f;
  auto vmax = [&]() __attribute__((always_inline)) {
    float mx = fmaxf(x[0], x[1]);
#pragma unroll
    for (int j = 2; j < 32; j += 2) mx = fmaxf(fmaxf(mx, x[j]), x[j + 1]);
    mneg = -mx * c;
  };
  auto vexp = [&](int j) __attribute__((always_inline)) {
    x[j] = __builtin_amdgcn_exp2f(fmaf(x[j], c, mneg));
    ps[j % 4] += x[j];
  };
  auto vcast = [&](int w) __attribute__((always_inline)) {
    typedef __attribute__((ext_vector_type(2))) short s16x2;
    s16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(s16x2, codes[w]), x[4 * w], x[4 * w + 1],
                                                         0.00390625f, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, x[4 * w + 2], x[4 * w + 3], 0.00390625f, true);
    codes[w] = __builtin_bit_cast(uint32_t, r);
  };
  auto vcount = [&](int w) __attribute__((always_inline)) {
    cnt = __builtin_amdgcn_msad_u8(codes[w] | 0x80808080u, codes[w], cnt);
  };
  for (int it = 0; it < iters; ++it) {
    if constexpr (kMode == 3) {
      vmax();
#pragma unroll
      for (int j = 0; j < 32; ++j) vexp(j);
#pragma unroll
      for (int w = 0; w < 8; ++w) vcast(w);
#pragma unroll
      for (int w = 0; w < 8; ++w) vcount(w);
    } else if constexpr (kMode == 4) {
      // P.V: 4 FP8 instructions | max, first 16 exponentials, their 4 casts
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        // two operand fragments per type here, so that the softmax state fits beside them
        acc8[s] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8[s % 2], b8[s % 2], acc8[s], 0, 0, 0, 0, 0, 0);
        if (s == 0) vmax();
#pragma unroll
        for (int j = 4 * s; j < 4 * s + 4; ++j) vexp(j);
        vcast(s);
        __builtin_amdgcn_sched_barrier(0);
      }
      // first logit half: 8 bf16 instructions | second 16 exponentials and casts
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        acc[s % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s % 2], b[(s / 4) % 2], acc[s % 4], 0, 0, 0);
        vexp(16 + 2 * s);
        vexp(17 + 2 * s);
        if (s % 2 == 1) vcast(4 + s / 2);
        __builtin_amdgcn_sched_barrier(0);
      }
      // second logit half: 8 bf16 instructions | counters
#pragma unroll
      for (int s = 8; s < 16; ++s) {
        acc[s % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s % 2], b[(s / 4) % 2], acc[s % 4], 0, 0, 0);
        vcount(s - 8);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (kMode == 0) {
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
  float r = (float)cnt + (ps[0] + ps[1]) + (ps[2] + ps[3]);
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) r += acc[q][i] + acc8[q][i];
  sink[tid] = r;
}


// Issue-cost kinds (per wave and iteration):
//   0 idle, 1 sixteen v_mfma_f32_32x32x16_bf16, 2 the softmax VALU work of roof mode 3,
//   3 32 v_exp_f32, 4 64 v_fma_f32, 5 16 v_cvt_scalef32_pk_fp8_f32, 6 16 v_cvt_pk_fp8_f32,
//   7 16 v_max3_f32, 8 32 v_add_f32, 9 8 v_or_b32 + 8 v_msad_u8, 10 32 v_mul_f32
// Every VALU kind keeps 16 or more independent chains, so that with two waves per SIMD
// the time is the issue cost, not the latency.
constexpr int kIssueKinds = 11;
constexpr int kIssueCount[kIssueKinds] = {0, 16, 146, 32, 64, 16, 16, 16, 32, 16, 32};

template <int kKind>
__device__ __attribute__((noinline)) float issue_loop(uint32_t tid, int iters) {
  float x[32], acc[32];
  uint32_t w[16];
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    x[j] = -(float)(mix32(tid * 32 + j) & 0xFF) * 0.01f;
    acc[j] = x[j];
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) w[k] = mix32(tid + k) & 0x7F7F7F7Fu;
  uint32_t cnt = 0;
  const float fa = 0.999f, fb = 0.001f, sc = 0.00390625f;
  for (int it = 0; it < iters; ++it) {
    if constexpr (kKind == 3) {
#pragma unroll
      for (int j = 0; j < 32; ++j) asm volatile("v_exp_f32 %0, %1" : "=v"(acc[j]) : "v"(x[j]));
    } else if constexpr (kKind == 4) {
#pragma unroll
      for (int j = 0; j < 64; ++j) asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(acc[j % 32]) : "v"(fa), "v"(fb));
    } else if constexpr (kKind == 5) {
#pragma unroll
      for (int k = 0; k < 16; ++k)
        asm volatile("v_cvt_scalef32_pk_fp8_f32 %0, %1, %2, %3" : "=v"(w[k]) : "v"(x[2 * k]), "v"(x[2 * k + 1]), "s"(sc));
    } else if constexpr (kKind == 6) {
#pragma unroll
      for (int k = 0; k < 16; ++k) asm volatile("v_cvt_pk_fp8_f32 %0, %1, %2" : "=v"(w[k]) : "v"(x[2 * k]), "v"(x[2 * k + 1]));
    } else if constexpr (kKind == 7) {
#pragma unroll
      for (int k = 0; k < 16; ++k) asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(acc[k]) : "v"(x[k]), "v"(x[16 + k]));
    } else if constexpr (kKind == 8) {
#pragma unroll
      for (int j = 0; j < 32; ++j) asm volatile("v_add_f32 %0, %0, %1" : "+v"(acc[j % 16]) : "v"(x[j]));
    } else if constexpr (kKind == 9) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        asm volatile("v_or_b32 %0, 0x80808080, %1" : "=v"(w[8 + k]) : "v"(w[k]));
        asm volatile("v_msad_u8 %0, %1, %2, %0" : "+v"(acc[k]) : "v"(w[8 + k]), "v"(w[k]));
      }
    } else if constexpr (kKind == 10) {
#pragma unroll
      for (int j = 0; j < 32; ++j) asm volatile("v_mul_f32 %0, %1, %2" : "=v"(acc[j]) : "v"(x[j]), "s"(sc));
    }
  }
  // every asm result above is consumed here, several instructions after the loop
  asm volatile("s_nop 7" ::);
  float r = (float)cnt;
#pragma unroll
  for (int j = 0; j < 32; ++j) r += acc[j];
#pragma unroll
  for (int k = 0; k < 16; ++k) r += (float)w[k];
  return r;
}

__device__ __attribute__((noinline)) float issue_mfma(uint32_t tid, int iters) {
  bf16x8_t a[4], b[4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t h = mix32(tid * 64 + f * 8 + i);
      a[f][i] = __builtin_bit_cast(__bf16, (uint16_t)(0x3F80 | (h & 0x7F)));
      b[f][i] = __builtin_bit_cast(__bf16, (uint16_t)(0x3F80 | ((h >> 7) & 0x7F)));
    }
  f32x16_t acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 16; ++s)
      acc[s % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s % 4], b[(s / 4) % 4], acc[s % 4], 0, 0, 0);
  }
  float r = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) r += acc[q][i];
  return r;
}

__device__ __attribute__((noinline)) float issue_softmax(uint32_t tid, int iters) {
  float x[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) x[j] = 0.5f + (float)(mix32(tid * 32 + j) & 0xFFFF) * 7.6e-6f;
  float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  uint32_t codes[8] = {}, cnt = 0;
  const float c = 0.12752f;
  for (int it = 0; it < iters; ++it) {
    float mx = fmaxf(x[0], x[1]);
#pragma unroll
    for (int j = 2; j < 32; j += 2) mx = fmaxf(fmaxf(mx, x[j]), x[j + 1]);
    const float mneg = -mx * c;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      x[j] = __builtin_amdgcn_exp2f(fmaf(x[j], c, mneg));
      ps[j % 4] += x[j];
    }
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      typedef __attribute__((ext_vector_type(2))) short s16x2;
      s16x2 q = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(s16x2, codes[w]), x[4 * w], x[4 * w + 1],
                                                         0.00390625f, false);
      q = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(q, x[4 * w + 2], x[4 * w + 3], 0.00390625f, true);
      codes[w] = __builtin_bit_cast(uint32_t, q);
    }
#pragma unroll
    for (int w = 0; w < 8; ++w) cnt = __builtin_amdgcn_msad_u8(codes[w] | 0x80808080u, codes[w], cnt);
  }
  return (float)cnt + (ps[0] + ps[1]) + (ps[2] + ps[3]);
}

__global__ __launch_bounds__(512, 1) void issue_probe(float* __restrict__ sink, int iters_lo, int iters_hi,
                                                      int kind_lo, int kind_hi) {
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
  const bool lo = (threadIdx.x / 64) < 4;
  const int kind = lo ? kind_lo : kind_hi, iters = lo ? iters_lo : iters_hi;
  float r = 0.0f;
  switch (kind) {
    case 1: r = issue_mfma(tid, iters); break;
    case 2: r = issue_softmax(tid, iters); break;
    case 3: r = issue_loop<3>(tid, iters); break;
    case 4: r = issue_loop<4>(tid, iters); break;
    case 5: r = issue_loop<5>(tid, iters); break;
    case 6: r = issue_loop<6>(tid, iters); break;
    case 7: r = issue_loop<7>(tid, iters); break;
    case 8: r = issue_loop<8>(tid, iters); break;
    case 9: r = issue_loop<9>(tid, iters); break;
    case 10: r = issue_loop<10>(tid, iters); break;
    default: break;
  }
  sink[tid] = r;
}

}  // namespace

extern "C" {

// Matrix-core flops of one launch of pcast_roof_run(mode, iters, blocks, ...), counted
// as 2 * M * N * K per instruction (0 for the VALU-only mode 3).
double pcast_roof_flops(int mode, int iters, int blocks) {
  const double per_wave = mode == 0 ? 16.0 * 32768
                          : mode == 1 ? 16.0 * 131072
                          : mode == 3 ? 0.0
                                      : 16.0 * 32768 + 4.0 * 131072;
  return per_wave * iters * blocks * 4.0;
}

// Launches the probe: `blocks` workgroups of 256 threads, `iters` iterations each;
// sink holds blocks * 256 floats.  Returns 0, or 1 for a bad argument, or the HIP
// error code of the launch.
int pcast_roof_run(int mode, int iters, int blocks, float* sink, void* stream) {
  if (mode < 0 || mode > 4 || iters < 1 || blocks < 1 || !sink) return 1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (mode == 0) hipLaunchKernelGGL(roof<0>, dim3(blocks), dim3(256), 0, st, sink, iters, 0x9E3779B9u);
  else if (mode == 1) hipLaunchKernelGGL(roof<1>, dim3(blocks), dim3(256), 0, st, sink, iters, 0x9E3779B9u);
  else if (mode == 2) hipLaunchKernelGGL(roof<2>, dim3(blocks), dim3(256), 0, st, sink, iters, 0x9E3779B9u);
  else if (mode == 3) hipLaunchKernelGGL(roof<3>, dim3(blocks), dim3(256), 0, st, sink, iters, 0x9E3779B9u);
  else hipLaunchKernelGGL(roof<4>, dim3(blocks), dim3(256), 0, st, sink, iters, 0x9E3779B9u);
  return (int)hipGetLastError();
}

// Instructions of one kind per wave and iteration of issue_probe (0 for idle, 146 VALU
// instructions for the softmax work, 16 MFMAs for the matrix-core stream); -1 for an
// unknown kind.
int pcast_issue_count(int kind) { return kind >= 0 && kind < kIssueKinds ? kIssueCount[kind] : -1; }

// Launches issue_probe: `blocks` workgroups of 512 threads (one per compute unit gives two
// waves per SIMD); waves 0-3 of each workgroup run kind_lo for iters_lo iterations, waves
// 4-7 kind_hi for iters_hi.  sink holds blocks * 512 floats.  Returns 0, 1 for a bad
// argument, or the HIP error code of the launch.
int pcast_issue_run(int kind_lo, int iters_lo, int kind_hi, int iters_hi, int blocks, float* sink, void* stream) {
  if (kind_lo < 0 || kind_lo >= kIssueKinds || kind_hi < 0 || kind_hi >= kIssueKinds || iters_lo < 1 ||
      iters_hi < 1 || blocks < 1 || !sink)
    return 1;
  hipLaunchKernelGGL(issue_probe, dim3(blocks), dim3(512), 0, static_cast<hipStream_t>(stream), sink, iters_lo,
                     iters_hi, kind_lo, kind_hi);
  return (int)hipGetLastError();
}

}  // extern "C"
