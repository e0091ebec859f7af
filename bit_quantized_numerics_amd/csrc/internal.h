// internal.h -- launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kDtypeF32 = 0;
constexpr int kDtypeBF16 = 1;

// Tile-quantiser feature flags.
constexpr int kFRow = 1;     // emit the row-wise copy (1x16 along cols, or 16x16)
constexpr int kFCol = 2;     // emit the column-wise copy (operand = x^T)
constexpr int kF2D = 4;      // 16x16 blocks (weights); the column copy is the transpose
constexpr int kFRht = 8;     // RHT16 along rows before the column copy
constexpr int kFSrRow = 16;  // stochastic rounding for the row copy
constexpr int kFSrCol = 32;  // stochastic rounding for the column copy
constexpr int kFRht4 = 64;   // 4-point RHT along rows before the column copy (kFRht unset)

// A tensor amax lives in kAmaxSlots words kAmaxStride words apart (each on
// its own 128-byte line); its value is the max over the slots.
constexpr int kAmaxSlots = 32;
constexpr int kAmaxStride = 32;
constexpr int kAmaxRegionWords = kAmaxSlots * kAmaxStride;  // 4 KB

struct CopyArgs {
  uint8_t* codes = nullptr;
  uint8_t* scales = nullptr;
  float* global = nullptr;
  const uint32_t* amax = nullptr;  // the copy's amax slots (kAmaxSlots words)
  uint64_t seed = 0;
  uint64_t offset = 0;
  uint32_t stream = 0;
};

struct TileArgs {
  const void* x = nullptr;
  int64_t rows = 0, cols = 0, ld = 0;
  CopyArgs row, col;
  uint32_t signs = 0;
  uint32_t* status = nullptr;
};

hipError_t launch_zero_words(uint32_t* p, int n, hipStream_t s);
// rht_d: size of the transform behind out_rht (16, or 4 with out_raw null).
hipError_t launch_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                       uint32_t signs, uint32_t* out_raw, uint32_t* out_rht, hipStream_t s,
                       int rht_d = 16);
hipError_t launch_quant_tile(int dtype, int flags, const TileArgs& a, hipStream_t s);
hipError_t launch_rht_d(const void* x, float* y, int dtype, int64_t rows, int64_t cols, int64_t ld,
                        int axis, int d, const uint32_t* signs, float c, hipStream_t s);
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* global,
                          int64_t rows, int64_t cols, int mode, float* out, int64_t ldo,
                          hipStream_t s);
hipError_t launch_mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                              uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_rht16(const void* x, float* y, int dtype, int64_t rows, int64_t cols, int64_t ld,
                        int axis, uint32_t signs, hipStream_t s);

struct GemmOperand {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* global;
  int64_t rows;
  int scale_shift;  // 0: one scale row per operand row; 4: per 16 rows (16x16)
};

hipError_t launch_gemm(const GemmOperand& a, const GemmOperand& b, int64_t K, void* c,
                       int c_dtype, int64_t ldc, hipStream_t s);
// MXFP4 GEMM (32-element blocks, E8M0 scales [rows][K/32]; global unused).
// Requires K % 128 == 0, K >= 384 and rows * K / 2 < 2^31 for both operands.
hipError_t launch_mx_gemm(const GemmOperand& a, const GemmOperand& b, int64_t K, void* c,
                          int c_dtype, int64_t ldc, hipStream_t s);
// Plain BF16 GEMM C = A B^T, A [M, K] and B [N, K] dense bf16 (row stride K),
// FP32 accumulation.  Requires K % 32 == 0, K >= 96, rows * K * 2 < 2^31.
hipError_t launch_bf16_gemm(const void* a, int64_t M, const void* b, int64_t N, int64_t K, void* c,
                            int c_dtype, int64_t ldc, hipStream_t s);
// Two independent GEMMs in one launch where the kernel allows it (so that the
// tail of one fills with the tiles of the other), else two launches.  With
// `scratch` (>= split_scratch_bytes(), 16-byte aligned) the second GEMM's last
// tiles may run as two K halves added by a combine pass (shorter last round).
hipError_t launch_gemm_pair(const GemmOperand& a0, const GemmOperand& b0, int64_t K0, void* c0,
                            int c0_dtype, int64_t ldc0, const GemmOperand& a1,
                            const GemmOperand& b1, int64_t K1, void* c1, int c1_dtype,
                            int64_t ldc1, float* scratch, size_t scratch_bytes, hipStream_t s);
size_t split_scratch_bytes();

}  // namespace nvfp4
