// gemm.hip -- NVFP4 x NVFP4 GEMM with FP32 accumulation on gfx950 MFMA.
//
// Citations: [Review] = web page "NVFP4 4-bit Pretraining, Made Practical: 12B
// up to 10T Tokens, Effectively On Par with FP8" (review of arXiv 2509.25149),
// by numbered section; [Captions] = that paper's figure-caption list.
//
// C[m][n] = g_A g_B sum_k (q_A d_A)[m][k] (q_B d_B)[n][k]   [Review s6; Captions Fig. 5]
// with q an E2M1 value and d the E4M3 scale of its 16-element block.
//
// Dtype choice.  gfx950's scaled FP4 MFMA takes one power-of-two (E8M0)
// scale per 32 elements, so it cannot apply NVFP4's E4M3 scale per 16
// elements without masking 3/4 of every instruction.  Instead each element is
// dequantised exactly to fp16: q has 2 significant bits and d 4, so q*d has at
// most 5 and lies in [2^-10, 2688], which fp16 represents exactly.  The
// products then run on the dense fp16 MFMA (v_mfma_f32_32x32x16_f16, FP32
// accumulate) and the epilogue multiplies by g_A g_B.
//
// Dequantisation: v_cvt_scalef32_pk_f16_fp4 with unit scale turns two codes
// into two exact fp16 values (the instruction honours only the exponent of a
// non-unit scale), then v_pk_mul_f16 applies the block scale d, also exactly.
#include "device_common.h"
#include "internal.h"

namespace nvfp4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kGemmThreads = 256;

// E4M3 code -> its value as fp16 (exact: E4M3 values lie in [2^-9, 448]).
__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t code) {
  const float d = code >= 8u ? __uint_as_float((code + 960u) << 20) : (float)code * 0x1p-9f;
  return (_Float16)d;
}

// Eight packed codes (one dword) -> eight fp16 values times d, as 4 dwords.
__device__ __forceinline__ void dequant8(uint32_t w, half2_t d2, uint32_t* out) {
  half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  h0 = h0 * d2;
  h1 = h1 * d2;
  h2 = h2 * d2;
  h3 = h3 * d2;
  __builtin_memcpy(&out[0], &h0, 4);
  __builtin_memcpy(&out[1], &h1, 4);
  __builtin_memcpy(&out[2], &h2, 4);
  __builtin_memcpy(&out[3], &h3, 4);
}

// One thread's share of a 128 x 64 operand tile: row (t >> 1), k-half (t & 1)
// = 32 codes (16 bytes) and their two block scales.
struct TileLoad {
  uint4 codes;
  uint32_t s0, s1;
};

__device__ __forceinline__ TileLoad load_tile_part(const GemmOperand& op, int64_t K, int64_t row0,
                                                   int64_t k0, int t) {
  TileLoad L;
  L.codes = make_uint4(0, 0, 0, 0);
  L.s0 = 0;
  L.s1 = 0;
  const int64_t row = row0 + (t >> 1);
  const int64_t kk = k0 + 32 * (t & 1);
  if (row < op.rows && kk < K) {
    const uint8_t* p = op.codes + row * (K / 2) + kk / 2;
    const uint8_t* sp = op.scales + (row >> op.scale_shift) * (K / 16) + kk / 16;
    if (kk + 32 <= K) {
      if ((K & 31) == 0) {
        L.codes = *reinterpret_cast<const uint4*>(p);
      } else {
        const uint2 a = *reinterpret_cast<const uint2*>(p);
        const uint2 b = *reinterpret_cast<const uint2*>(p + 8);
        L.codes = make_uint4(a.x, a.y, b.x, b.y);
      }
      L.s0 = sp[0];
      L.s1 = sp[1];
    } else {  // K tail: only the first 16 elements exist
      const uint2 a = *reinterpret_cast<const uint2*>(p);
      L.codes = make_uint4(a.x, a.y, 0, 0);
      L.s0 = sp[0];
    }
  }
  return L;
}

// Dequantise and store one thread's 32 values into the LDS tile [128][64]
// (fp16, rows of 128 bytes = 8 chunks of 16 bytes, chunk index XOR (row & 7)).
__device__ __forceinline__ void store_tile_part(_Float16* lds, const TileLoad& L, int t) {
  const int row = t >> 1, half = t & 1;
  const _Float16 d0 = e4m3_to_f16(L.s0), d1 = e4m3_to_f16(L.s1);
  const half2_t d0v = {d0, d0}, d1v = {d1, d1};
  uint32_t o[16];
  dequant8(L.codes.x, d0v, o + 0);
  dequant8(L.codes.y, d0v, o + 4);
  dequant8(L.codes.z, d1v, o + 8);
  dequant8(L.codes.w, d1v, o + 12);
  uint8_t* base = reinterpret_cast<uint8_t*>(lds) + row * 128;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int chunk = half * 4 + c;
    const int phys = chunk ^ (row & 7);
    *reinterpret_cast<uint4*>(base + phys * 16) = make_uint4(o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
  }
}

__device__ __forceinline__ half8_t read_frag(const _Float16* lds, int row, int chunk) {
  const int phys = chunk ^ (row & 7);
  const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(lds) + row * 128 + phys * 16);
  half8_t h;
  __builtin_memcpy(&h, &v, 16);
  return h;
}

template <bool OUT_BF16>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemmOperand a, GemmOperand b, int64_t K,
                                                            void* __restrict__ c, int64_t ldc) {
  __shared__ __align__(16) _Float16 lds_a[2][kBM * kBK];
  __shared__ __align__(16) _Float16 lds_b[2][kBN * kBK];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;
  const int64_t nk = (K + kBK - 1) / kBK;

  float16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  TileLoad la = load_tile_part(a, K, m0, 0, t);
  TileLoad lb = load_tile_part(b, K, n0, 0, t);
  store_tile_part(lds_a[0], la, t);
  store_tile_part(lds_b[0], lb, t);
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt & 1);
    const bool more = kt + 1 < nk;
    if (more) {
      la = load_tile_part(a, K, m0, (kt + 1) * kBK, t);
      lb = load_tile_part(b, K, n0, (kt + 1) * kBK, t);
    }
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int chunk = kk * 2 + (lane >> 5);
      half8_t fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = read_frag(lds_a[cur], wm * 64 + i * 32 + (lane & 31), chunk);
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = read_frag(lds_b[cur], wn * 64 + j * 32 + (lane & 31), chunk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      store_tile_part(lds_a[cur ^ 1], la, t);
      store_tile_part(lds_b[cur ^ 1], lb, t);
    }
    __syncthreads();
  }

  const float gab = (*a.global) * (*b.global);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
        if (m < a.rows && n < b.rows) {
          const float v = acc[i][j][r] * gab;
          if (OUT_BF16)
            static_cast<uint16_t*>(c)[m * ldc + n] = f32_to_bf16_rne(v);
          else
            static_cast<float*>(c)[m * ldc + n] = v;
        }
      }
}

hipError_t launch_gemm(const GemmOperand& a, const GemmOperand& b, int64_t K, void* c, int c_dtype,
                       int64_t ldc, hipStream_t s) {
  const dim3 grid((unsigned)((b.rows + kBN - 1) / kBN), (unsigned)((a.rows + kBM - 1) / kBM));
  if (c_dtype == kDtypeBF16)
    hipLaunchKernelGGL(gemm_kernel<true>, grid, dim3(kGemmThreads), 0, s, a, b, K, c, ldc);
  else
    hipLaunchKernelGGL(gemm_kernel<false>, grid, dim3(kGemmThreads), 0, s, a, b, K, c, ldc);
  return hipGetLastError();
}

}  // namespace nvfp4
