// peak.hip -- a measured compute ceiling for the GEMM roofline: an fp16 MFMA
// loop with no memory traffic, the same instruction the NVFP4 GEMM runs
// (v_mfma_f32_32x32x16_f16, FP32 accumulation).  The datasheet peak assumes
// the top clock; under a sustained MFMA load the card holds a lower clock,
// which also depends on how many operand bits toggle, so the operands here
// are random-looking and change every iteration as the GEMM's do.
#include "nvfp4.h"

#include <hip/hip_runtime.h>

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBlocks = 1024;       // one workgroup per compute unit at a time
constexpr int kPeakThreads = 256;   // 4 waves, one per SIMD

// Like the GEMM's inner loop: 4 A and 4 B fragments, 16 accumulators (all
// AGPRs, one wave per SIMD), 16 MFMAs per iteration, and 4 VALU instructions
// per MFMA that give every fragment fresh random-looking bits (a rotation of
// per-lane random state, masked to finite f16 values with random sign and
// mantissa), since the clock the card holds depends on operand bit toggles.
// `mask` selects the bits that change: 0 keeps every operand constant while
// the same instructions run, 0x87FF87FF toggles sign and mantissa bits.
__global__ __launch_bounds__(kPeakThreads, 1) void mfma_f16_loop_kernel(int iters, uint32_t mask,
                                                                      float* sink) {
  float16_t acc[16];
#pragma unroll
  for (int c = 0; c < 16; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  uint32_t st[8][4];
  uint32_t x = (blockIdx.x * kPeakThreads + threadIdx.x) * 0x9E3779B9u + 0x7F4A7C15u;
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      x ^= x << 13;
      x ^= x >> 17;
      x ^= x << 5;
      st[f][d] = x;
    }
  // operands for iteration it+1 are made while iteration it's MFMAs run
  auto refresh = [&](half8_t (&op)[8]) {
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      u32x4_t v;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        st[f][d] = __builtin_amdgcn_alignbit(st[f][d], st[f][d], 31);  // rotate left 1
        v[d] = (st[f][d] & mask) | 0x30003000u;
      }
      __builtin_memcpy(&op[f], &v, 16);
    }
  };
  half8_t o0[8], o1[8];
  refresh(o0);
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int c = 0; c < 16; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(o0[c >> 2], o0[4 + (c & 3)], acc[c], 0, 0, 0);
    refresh(o1);
#pragma unroll
    for (int c = 0; c < 16; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(o1[c >> 2], o1[4 + (c & 3)], acc[c], 0, 0, 0);
    refresh(o0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 16; ++c) s += acc[c][0];
  if (s == 1234.5f) sink[blockIdx.x] = s;  // keeps the loop; never true in practice
}

// The same MFMAs with no VALU work in the loop: the operands alternate
// between two register sets of random-looking values (bits under `mask`
// random, the rest as above), so every MFMA sees other bits than the one
// before at no instruction cost; mask 0 makes both sets equal (constant
// operands).  This is the fp16 MFMA rate the card holds when nothing else
// competes for issue or power.
__global__ __launch_bounds__(kPeakThreads, 1) void mfma_f16_pure_kernel(int iters, uint32_t mask,
                                                                      float* sink) {
  float16_t acc[16];
#pragma unroll
  for (int c = 0; c < 16; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  uint32_t x = (blockIdx.x * kPeakThreads + threadIdx.x) * 0x9E3779B9u + 0x7F4A7C15u;
  half8_t o[2][8];
#pragma unroll
  for (int set = 0; set < 2; ++set)
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      u32x4_t v;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        x ^= x << 13;
        x ^= x >> 17;
        x ^= x << 5;
        v[d] = ((set == 0 ? x : x ^ 0xFFFFFFFFu) & mask) | 0x30003000u;
      }
      __builtin_memcpy(&o[set][f], &v, 16);
    }
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int set = 0; set < 2; ++set)
#pragma unroll
      for (int c = 0; c < 16; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(o[set][c >> 2], o[set][4 + (c & 3)], acc[c],
                                                        0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 16; ++c) s += acc[c][0];
  if (s == 1234.5f) sink[blockIdx.x] = s;  // keeps the loop; never true in practice
}

// The MXFP4 comparator's instruction, v_mfma_scale_f32_32x32x64_f8f6f4 with
// both operands E2M1 (format 4) and unit E8M0 scales (127), in the same
// VALU-free form: 16 accumulators, operands alternating between two register
// sets that differ in the bits under `mask`.
__global__ __launch_bounds__(kPeakThreads, 1) void mfma_fp4_pure_kernel(int iters, uint32_t mask,
                                                                      float* sink) {
  typedef int v8i __attribute__((ext_vector_type(8)));
  float16_t acc[16];
#pragma unroll
  for (int c = 0; c < 16; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  uint32_t x = (blockIdx.x * kPeakThreads + threadIdx.x) * 0x9E3779B9u + 0x2545F491u;
  v8i o[2][8];
#pragma unroll
  for (int set = 0; set < 2; ++set)
#pragma unroll
    for (int f = 0; f < 8; ++f) {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        x ^= x << 13;
        x ^= x >> 17;
        x ^= x << 5;
        o[set][f][d] = d < 4 ? (int)((set == 0 ? x : x ^ 0xFFFFFFFFu) & mask) : 0;
      }
    }
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int set = 0; set < 2; ++set)
#pragma unroll
      for (int c = 0; c < 16; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(o[set][c >> 2], o[set][4 + (c & 3)],
                                                                 acc[c], 4, 4, 0, 127, 0, 127);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 16; ++c) s += acc[c][0];
  if (s == 1234.5f) sink[blockIdx.x] = s;  // keeps the loop; never true in practice
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_peak_mfma_fp4(int32_t iters, uint32_t toggle_mask, float* sink, double* flops,
                                 void* stream) {
  if (!sink || !flops) return NVFP4_ERR_NULL;
  if (iters <= 0) return NVFP4_ERR_SHAPE;
  hipLaunchKernelGGL(mfma_fp4_pure_kernel, dim3(kBlocks), dim3(kPeakThreads), 0,
                     static_cast<hipStream_t>(stream), iters, toggle_mask, sink);
  if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
  *flops = (double)kBlocks * (kPeakThreads / 64) * ((iters + 1) / 2 * 2) * 16 * (2.0 * 32 * 32 * 64);
  return NVFP4_OK;
}

nvfp4_status nvfp4_peak_mfma_f16(int32_t iters, uint32_t toggle_mask, int32_t valu_per_mfma,
                                 float* sink, double* flops, void* stream) {
  if (!sink || !flops) return NVFP4_ERR_NULL;
  if (iters <= 0) return NVFP4_ERR_SHAPE;
  if (valu_per_mfma != 0 && valu_per_mfma != 4) return NVFP4_ERR_DTYPE;
  if (valu_per_mfma == 4)
    hipLaunchKernelGGL(mfma_f16_loop_kernel, dim3(kBlocks), dim3(kPeakThreads), 0,
                       static_cast<hipStream_t>(stream), iters, toggle_mask & 0x87FF87FFu, sink);
  else
    hipLaunchKernelGGL(mfma_f16_pure_kernel, dim3(kBlocks), dim3(kPeakThreads), 0,
                       static_cast<hipStream_t>(stream), iters, toggle_mask & 0x87FF87FFu, sink);
  if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP;
  *flops = (double)kBlocks * (kPeakThreads / 64) * ((iters + 1) / 2 * 2) * 16 * (2.0 * 32 * 32 * 16);
  return NVFP4_OK;
}

}  // extern "C"
