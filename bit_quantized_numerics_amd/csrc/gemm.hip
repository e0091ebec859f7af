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
//
// Structure.  A workgroup of 4 waves computes a 256 x 256 tile of C; each
// wave owns 128 x 128 (4 x 4 MFMA blocks of 32 x 32; 256 FP32 accumulators
// per lane, held in AGPRs).  There is no LDS stage and no barrier: each wave
// loads the NVFP4 codes of its own 4 A and 4 B 32-row blocks straight from
// global memory (L1/L2 absorb the sharing between the two waves that read the
// same rows) into registers, three K-steps ahead, and dequantises them one
// MFMA sub-step ahead, so that on gfx950 -- where a 16-byte LDS store runs at
// well under half the rate of a load and the fp4->f16 convert costs two issue
// passes -- the only per-element work left is 2 VALU instructions per pair of
// elements, about 4 per MFMA, issued in the MFMA's shadow.
//
// K order inside a step.  A K-step covers 64 k.  For MFMA sub-step s (0..3)
// lane-half h (lanes 32h..32h+31) supplies k = 32h + 8s + (0..7) instead of
// the natural 16s + 8h + (0..7).  A and B use the same permutation, so every
// product still pairs equal k, and each lane's 32 codes of a row are one
// contiguous 16-byte load.
//
// Block scales.  The fp16 whose bit pattern is (E4M3 code << 7) has the value
// d * 2^-8 for every E4M3 code, subnormals included; the dequantised operands
// therefore carry a factor 2^-8 each (all values stay exact in fp16, the
// smallest being a subnormal 2^-18), and the epilogue multiplies by
// 2^16 g_A g_B.
#include "device_common.h"
#include "internal.h"

namespace nvfp4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kGemmThreads = 256;
constexpr int kGroupM = 8;  // tile-row group for L2 reuse

// The codes and scales one lane needs for one K-step: for each of its 4 A and
// 4 B 32-row blocks, 32 codes (16 bytes: k = 32h .. 32h+31 of the step) and
// the row's four E4M3 scale bytes of the step (the lane uses bytes 2h, 2h+1).
struct StepRaw {
  uint4 ca[4], cb[4];
  uint32_t sa[4], sb[4];
};

// Per-lane bases of one operand's 4 row blocks.
struct OpBase {
  const uint8_t* codes[4];
  const uint8_t* scales[4];
};

__device__ __forceinline__ OpBase op_base(const GemmOperand& op, int64_t K, int64_t row0, int h) {
  OpBase ob;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = row0 + 32 * i;
    const int64_t r = row < op.rows ? row : 0;
    ob.codes[i] = op.codes + r * (K / 2) + 16 * h;
    ob.scales[i] = op.scales + (r >> op.scale_shift) * (K / 16);
  }
  return ob;
}

// 16 code bytes + 4 scale bytes of one row block at step start k0 (the lane's
// elements are k0 + 32h .. +31).  Rows past the operand read row 0 instead:
// their products only reach rows or columns of C that are never stored.
// Steps past K read step 0 instead; their scales are zeroed where they are
// consumed (scales_of), which zeroes every dequantised value (E2M1 has no Inf
// or NaN), so they add exact zeros.  Zeroing at load time would force a wait
// for the load right after issuing it.
template <bool K_ALIGNED>
__device__ __forceinline__ void load_blk(const OpBase& ob, int i, int64_t K, int64_t k0, int h,
                                         uint4& c, uint32_t& sc) {
  if (K_ALIGNED) {  // K % 64 == 0: branch-free, the lane's 32 elements all exist
    const int64_t kc = k0 < K ? k0 : 0;
    c = *reinterpret_cast<const uint4*>(ob.codes[i] + kc / 2);
    sc = *reinterpret_cast<const uint32_t*>(ob.scales[i] + kc / 16);
    return;
  }
  c = make_uint4(0, 0, 0, 0);  // general K (multiple of 16): per 16-element block
  sc = 0;
  const int64_t kk = k0 + 32 * h;
  if (kk < K) {
    const uint2 v = *reinterpret_cast<const uint2*>(ob.codes[i] + k0 / 2);
    c.x = v.x;
    c.y = v.y;
    sc = (uint32_t)ob.scales[i][k0 / 16 + 2 * h] << (16 * h);
  }
  if (kk + 16 < K) {
    const uint2 v = *reinterpret_cast<const uint2*>(ob.codes[i] + k0 / 2 + 8);
    c.z = v.x;
    c.w = v.y;
    sc |= (uint32_t)ob.scales[i][k0 / 16 + 2 * h + 1] << (16 * h + 8);
  }
}

template <bool K_ALIGNED>
__device__ __forceinline__ void load_step(const OpBase& oa, const OpBase& obb, int64_t K, int64_t k0,
                                          int h, StepRaw& r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    load_blk<K_ALIGNED>(oa, i, K, k0, h, r.ca[i], r.sa[i]);
    load_blk<K_ALIGNED>(obb, i, K, k0, h, r.cb[i], r.sb[i]);
  }
}

// Two of the four E4M3 scale bytes in s -> two fp16 values d * 2^-8 (bit
// patterns code << 7), packed: the selector `sel` (per lane-half) places byte
// 2h at bits 0..7 and byte 2h+1 at bits 16..23; the shift by 7 then cannot
// carry across halves (codes are at most 0x7E).
__device__ __forceinline__ uint32_t scale_pair(uint32_t s, uint32_t sel) {
  return __builtin_amdgcn_perm(0u, s, sel) << 7;
}

__device__ __forceinline__ half8_t dequant8(uint32_t w, uint32_t dpair, bool hi) {
  half2_t d2;
  __builtin_memcpy(&d2, &dpair, 4);
  const _Float16 d = hi ? d2[1] : d2[0];
  const half2_t dd = {d, d};
  const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * dd;
  const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * dd;
  const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * dd;
  const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * dd;
  half8_t o = {h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
  return o;
}

// Sub-step S fragments (A and B) of a step; dp* are the converted scales.
template <int S>
__device__ __forceinline__ void dequant_sub(const StepRaw& r, const uint32_t (&dpa)[4],
                                            const uint32_t (&dpb)[4], half8_t (&fa)[4],
                                            half8_t (&fb)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t wa = S == 0 ? r.ca[i].x : S == 1 ? r.ca[i].y : S == 2 ? r.ca[i].z : r.ca[i].w;
    const uint32_t wb = S == 0 ? r.cb[i].x : S == 1 ? r.cb[i].y : S == 2 ? r.cb[i].z : r.cb[i].w;
    fa[i] = dequant8(wa, dpa[i], S >= 2);
    fb[i] = dequant8(wb, dpb[i], S >= 2);
  }
}

// Converted scales of a step; `in_k` false (a step past K) gives zeros.
__device__ __forceinline__ void scales_of(const StepRaw& r, bool in_k, uint32_t sel,
                                          uint32_t (&dpa)[4], uint32_t (&dpb)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dpa[i] = in_k ? scale_pair(r.sa[i], sel) : 0u;
    dpb[i] = in_k ? scale_pair(r.sb[i], sel) : 0u;
  }
}

__device__ __forceinline__ void mfma16(float16_t (&acc)[4][4], const half8_t (&fa)[4],
                                       const half8_t (&fb)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
}

// Instruction-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008, kSchedVmemRead = 0x020;

// Interleave 16 MFMAs with VALU VALU instructions each and VMEM loads.
template <int VALU, int VMEM>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int g = 0; g < 16; ++g) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedValu, VALU, 0);
    if (g < VMEM) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
  }
}

// One K-step.  On entry `fa/fb` hold sub-step 0 of step k (from `cur`) and
// `cdp*` its scales; `nxt` holds step k+1 (loaded earlier).  The loads of step
// k+2 go into `fill`, issued during sub-step 0.  On exit fa/fb hold sub-step 0
// of step k+1 and cdp* its scales.
template <bool K_ALIGNED>
__device__ __forceinline__ void k_step(float16_t (&acc)[4][4], half8_t (&fa)[4], half8_t (&fb)[4],
                                       uint32_t (&cdpa)[4], uint32_t (&cdpb)[4], const StepRaw& cur,
                                       const StepRaw& nxt, StepRaw& fill, const OpBase& oa,
                                       const OpBase& ob, int64_t K, int64_t k_fill, int h,
                                       uint32_t sel) {
  const bool nxt_in_k = k_fill - kBK < K;  // step k+1 starts one step before k+2
  half8_t ga[4], gb[4];
  load_step<K_ALIGNED>(oa, ob, K, k_fill, h, fill);
  mfma16(acc, fa, fb);
  dequant_sub<1>(cur, cdpa, cdpb, ga, gb);
  interleave<4, 16>();
  mfma16(acc, ga, gb);
  dequant_sub<2>(cur, cdpa, cdpb, fa, fb);
  interleave<4, 0>();
  mfma16(acc, fa, fb);
  dequant_sub<3>(cur, cdpa, cdpb, ga, gb);
  interleave<4, 0>();
  mfma16(acc, ga, gb);
  scales_of(nxt, nxt_in_k, sel, cdpa, cdpb);
  dequant_sub<0>(nxt, cdpa, cdpb, fa, fb);
  interleave<4, 0>();
}

// Workgroup -> output tile.  Workgroups are dispatched round-robin over the 8
// XCDs; consecutive ids are first regrouped so that each XCD works on one
// contiguous range, then ordered in groups of kGroupM tile rows so that the
// tiles an XCD runs together share A and B rows in its L2.
__device__ __forceinline__ void tile_of(int tiles_m, int tiles_n, int* tm, int* tn) {
  const int nwg = (int)gridDim.x;
  int b = (int)blockIdx.x;
  if ((nwg & 7) == 0) b = (b & 7) * (nwg >> 3) + (b >> 3);
  const int per_group = kGroupM * tiles_n;
  const int group = b / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_group = b - group * per_group;
  *tm = first_m + in_group % gsize;
  *tn = in_group / gsize;
}

template <bool OUT_BF16, bool K_ALIGNED>
__global__ __launch_bounds__(kGemmThreads, 1) void gemm_kernel(GemmOperand a, GemmOperand b,
                                                               int64_t K, void* __restrict__ c,
                                                               int64_t ldc, int tiles_m,
                                                               int tiles_n) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_of(tiles_m, tiles_n, &tm, &tn);
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
  const int64_t nk = (K + kBK - 1) / kBK;
  const int h = lane >> 5;
  const OpBase oa = op_base(a, K, m0 + wm * 128 + (lane & 31), h);
  const OpBase ob = op_base(b, K, n0 + wn * 128 + (lane & 31), h);

  float16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Three raw buffers rotate: step k (being dequantised), k+1 (loaded), k+2
  // (in flight).  Steps past K load zeros; the loop runs a multiple of 3.
  StepRaw r0, r1, r2;
  load_step<K_ALIGNED>(oa, ob, K, 0, h, r0);
  load_step<K_ALIGNED>(oa, ob, K, kBK, h, r1);
  half8_t fa[4], fb[4];
  uint32_t dpa[4], dpb[4];
  // v_perm selector picking scale bytes 2h and 2h+1 (0x0C selects zero)
  const uint32_t sel = h ? 0x0C030C02u : 0x0C010C00u;
  scales_of(r0, true, sel, dpa, dpb);
  dequant_sub<0>(r0, dpa, dpb, fa, fb);
  for (int64_t kt = 0; kt < nk; kt += 3) {
    k_step<K_ALIGNED>(acc, fa, fb, dpa, dpb, r0, r1, r2, oa, ob, K, (kt + 2) * kBK, h, sel);
    k_step<K_ALIGNED>(acc, fa, fb, dpa, dpb, r1, r2, r0, oa, ob, K, (kt + 3) * kBK, h, sel);
    k_step<K_ALIGNED>(acc, fa, fb, dpa, dpb, r2, r0, r1, oa, ob, K, (kt + 4) * kBK, h, sel);
  }

  const float gab = (*a.global) * (*b.global) * 65536.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t n = n0 + wn * 128 + j * 32 + (lane & 31);
        if (m < a.rows && n < b.rows) {
          const float v = acc[i][j][r] * gab;
          if (OUT_BF16)
            static_cast<uint16_t*>(c)[m * ldc + n] = f32_to_bf16_rne(v);
          else
            static_cast<float*>(c)[m * ldc + n] = v;
        }
      }
}

template <bool OUT_BF16, bool K_ALIGNED>
static hipError_t launch_gemm_t(const GemmOperand& a, const GemmOperand& b, int64_t K, void* c,
                                int64_t ldc, hipStream_t s) {
  const int tiles_m = (int)((a.rows + kBM - 1) / kBM);
  const int tiles_n = (int)((b.rows + kBN - 1) / kBN);
  hipLaunchKernelGGL((gemm_kernel<OUT_BF16, K_ALIGNED>), dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(kGemmThreads), 0, s, a, b, K, c, ldc, tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmOperand& a, const GemmOperand& b, int64_t K, void* c, int c_dtype,
                       int64_t ldc, hipStream_t s) {
  const bool aligned = (K % kBK) == 0;
  if (c_dtype == kDtypeBF16)
    return aligned ? launch_gemm_t<true, true>(a, b, K, c, ldc, s)
                   : launch_gemm_t<true, false>(a, b, K, c, ldc, s);
  return aligned ? launch_gemm_t<false, true>(a, b, K, c, ldc, s)
                 : launch_gemm_t<false, false>(a, b, K, c, ldc, s);
}

}  // namespace nvfp4
