// api.hip -- the C ABI declared in include/nvfp4.h: argument validation,
// workspace slots and kernel orchestration.  Every argument check happens
// before anything is enqueued.
//
// Citations: [Review] = web page "NVFP4 4-bit Pretraining, Made Practical: 12B
// up to 10T Tokens, Effectively On Par with FP8" (review of arXiv 2509.25149),
// by numbered section; [Captions] = that paper's figure-caption list.
#include "nvfp4.h"

#include <hip/hip_runtime.h>

#include "internal.h"

#include <cmath>
#include <mutex>

// Reduction slots of nvfp4_quantize_static: a fixed 8 KB (two tensor-amax
// regions) per GPU, whatever the input size.  Host code never uses this name
// as an address (on the host it is only a stand-in): each device's copy is
// reached through hipGetSymbolAddress, once per device, and that pointer is
// what the kernels receive.
static __device__ __align__(256) uint32_t scratch[2 * nvfp4::kAmaxRegionWords];

namespace {

using namespace nvfp4;

// Workspace: 8 regions of kAmaxRegionWords words (4 KB).  Word 0 of region 0
// is the sticky device status; each other region holds the slots of one
// tensor amax (bit patterns of non-negative floats, reduced with atomicMax,
// kAmaxSlots words on separate 128-byte lines).
constexpr int kRegions = 8;
constexpr size_t kWorkspaceBytes = (size_t)kRegions * kAmaxRegionWords * 4;
constexpr int kWsWords = (int)(kWorkspaceBytes / 4);
enum Slot {
  kSlotStatus = 0,
  kSlotQRaw = 1,   // nvfp4_quantize / rowcol / 2d: plain amax
  kSlotQRht = 2,   //   ... amax after the RHT
  kSlotXRaw = 3,   // layer forward: X
  kSlotXRht = 4,   //   (R X)
  kSlotW = 5,      //   W
  kSlotDyRaw = 6,  // layer backward: dY
  kSlotDyRht = 7,  //   (R dY)
};

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }
inline uint32_t* ws_word(void* ws, int slot) {
  return static_cast<uint32_t*>(ws) + (size_t)slot * kAmaxRegionWords;
}
// Zero `n` consecutive amax regions starting at `slot`.
inline hipError_t zero_slots(void* ws, int slot, int n, hipStream_t s) {
  return launch_zero_words(ws_word(ws, slot), n * kAmaxRegionWords, s);
}
// Largest source row count (the limit the API has always stated; the kernels'
// one-dimensional grids would allow more).
constexpr int64_t kMaxRows = (int64_t)65535 * 128;
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline size_t elem_bytes(int dtype) { return dtype == NVFP4_BF16 ? 2 : 4; }

nvfp4_status hip_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

nvfp4_status check_workspace(void* ws, size_t bytes) {
  if (!ws || bytes < kWorkspaceBytes) return NVFP4_ERR_WORKSPACE;
  if (!aligned(ws, 4)) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

nvfp4_status check_source(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld) {
  if (!x) return NVFP4_ERR_NULL;
  if (dtype != NVFP4_F32 && dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
  if (rows <= 0 || cols <= 0 || cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (rows > kMaxRows) return NVFP4_ERR_SHAPE;
  if (ld < cols) return NVFP4_ERR_SHAPE;
  // a 256-row tile of the source must be addressable with 32-bit offsets
  if (ld * (int64_t)elem_bytes(dtype) * 256 >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
  if (!aligned(x, 16) || (ld * (int64_t)elem_bytes(dtype)) % 16 != 0) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

// A dense bf16 GEMM operand [rows, K]: K a whole number of 32-wide slabs and
// at least three of them (the kernel's prologue loads three), and every
// 256-row tile addressable with 32-bit buffer offsets.
nvfp4_status check_bf16_operand(int64_t rows, int64_t K) {
  if (rows <= 0 || K < 96 || K % 32 != 0) return NVFP4_ERR_SHAPE;
  if ((rows + 255) / 256 * 256 * K * 2 >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
  return NVFP4_OK;
}

nvfp4_status check_out(const nvfp4_tensor* t) {
  if (!t || !t->codes || !t->scales || !t->global_scale) return NVFP4_ERR_NULL;
  if (!aligned(t->codes, 16) || !aligned(t->global_scale, 4)) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

nvfp4_status check_opts(const nvfp4_quant_opts* o) {
  if (!o) return NVFP4_ERR_NULL;
  if (o->round != NVFP4_RN && o->round != NVFP4_SR) return NVFP4_ERR_DTYPE;
  if (o->transpose != 0 && o->transpose != 1) return NVFP4_ERR_DTYPE;
  if (o->rht != 0 && o->rht != 1) return NVFP4_ERR_DTYPE;
  if (o->rht_signs > 0xFFFFu) return NVFP4_ERR_DTYPE;
  if (o->rht_d != 0 && o->rht_d != 4 && o->rht_d != 16) return NVFP4_ERR_DTYPE;
  if (o->offset % 16 != 0) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

CopyArgs copy_args(const nvfp4_tensor* t, void* ws, int slot, const nvfp4_quant_opts* o) {
  CopyArgs c;
  c.codes = t->codes;
  c.scales = t->scales;
  c.global = t->global_scale;
  c.amax = ws_word(ws, slot);
  if (o) {
    c.seed = o->seed;
    c.offset = o->offset;
    c.stream = o->stream_id;
  }
  return c;
}

#define NVFP4_TRY(expr)                 \
  do {                                  \
    const nvfp4_status st_ = (expr);    \
    if (st_ != NVFP4_OK) return st_;    \
  } while (0)
#define NVFP4_HIP(expr)                              \
  do {                                               \
    if ((expr) != hipSuccess) return NVFP4_ERR_HIP;  \
  } while (0)

// Philox4x32-10 on the host (for the RHT sign diagonal).
void philox_host(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[1] = (uint32_t)p1;
    c[3] = (uint32_t)p0;
    c[0] = n0;
    c[2] = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

nvfp4_status check_gemm_operand(const nvfp4_tensor* t) {
  if (!t || !t->codes || !t->scales) return NVFP4_ERR_NULL;
  if (t->scale_mode != NVFP4_SCALE_MX32 && !t->global_scale) return NVFP4_ERR_NULL;
  if (t->rows <= 0 || t->cols <= 0 || t->cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (t->scale_mode != NVFP4_SCALE_1X16 && t->scale_mode != NVFP4_SCALE_16X16 &&
      t->scale_mode != NVFP4_SCALE_MX32)
    return NVFP4_ERR_DTYPE;
  if (t->scale_mode == NVFP4_SCALE_MX32 && t->cols % 32 != 0) return NVFP4_ERR_SHAPE;
  if (t->scale_mode == NVFP4_SCALE_16X16 && t->rows % 16 != 0) return NVFP4_ERR_SHAPE;
  if (!aligned(t->codes, 16) || !aligned(t->scales, 4) || !aligned(t->global_scale, 4))
    return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

GemmOperand gemm_operand(const nvfp4_tensor* t) {
  GemmOperand g;
  g.codes = t->codes;
  g.scales = t->scales;
  g.global = t->global_scale;
  g.rows = t->rows;
  g.scale_shift = t->scale_mode == NVFP4_SCALE_16X16 ? 4 : 0;
  return g;
}

void set_shape(nvfp4_tensor* t, int64_t rows, int64_t cols, int32_t mode) {
  t->rows = rows;
  t->cols = cols;
  t->scale_mode = mode;
}

}  // namespace

namespace {

// The six operands of a layer step in ctx order, with their shapes: xq [M, K],
// wq [N, K], wqt [K, N], xqt [K, M], dyq [M, N], dyqt [N, M].  Scale arrays
// are sized for 1x16 blocks so that either weight recipe fits.
void ctx_shapes(int64_t M, int64_t K, int64_t N, int64_t (&rc)[6][2]) {
  const int64_t s[6][2] = {{M, K}, {N, K}, {K, N}, {K, M}, {M, N}, {N, M}};
  for (int i = 0; i < 6; ++i) {
    rc[i][0] = s[i][0];
    rc[i][1] = s[i][1];
  }
}
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// a * b for positive a, b, or false when it would pass 2^62 (sizes beyond any
// device; keeps every size sum below in range).
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a > ((int64_t)1 << 62) / b) return false;
  *out = a * b;
  return true;
}

// ---- nvfp4_quantize and its allocation-free variant

nvfp4_status check_quantize_args(const void* x, int32_t dtype, int64_t rows, int64_t cols,
                                 int64_t ld, const nvfp4_quant_opts* opts,
                                 const nvfp4_tensor* out) {
  NVFP4_TRY(check_source(x, dtype, rows, cols, ld));
  NVFP4_TRY(check_opts(opts));
  NVFP4_TRY(check_out(out));
  // The RHT runs along the operand's block axis; the recipe applies it to the
  // column-wise (token-axis) Wgrad copies only [Review s3], which is the
  // supported placement.
  if (opts->rht && !opts->transpose) return NVFP4_ERR_SHAPE;
  if (opts->transpose && rows % 16 != 0) return NVFP4_ERR_SHAPE;
  return NVFP4_OK;
}

// Enqueues the amax pass and the emit pass of one quantisation; `slots` is
// two consecutive amax regions (plain amax, then amax after the RHT) and
// `status` the word a non-finite amax is reported in.
nvfp4_status quantize_enqueue(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                              const nvfp4_quant_opts* opts, nvfp4_tensor* out, uint32_t* slots,
                              uint32_t* status, hipStream_t s) {
  uint32_t* slot_raw = slots;
  uint32_t* slot_rht = slots + kAmaxRegionWords;
  TileArgs a;
  a.x = x;
  a.rows = rows;
  a.cols = cols;
  a.ld = ld;
  a.signs = opts->rht_signs;
  a.status = status;
  uint32_t* slot = opts->rht ? slot_rht : slot_raw;
  const bool rht4 = opts->rht && opts->rht_d == 4;
  int flags = 0;
  CopyArgs c;
  c.codes = out->codes;
  c.scales = out->scales;
  c.global = out->global_scale;
  c.amax = slot;
  c.seed = opts->seed;
  c.offset = opts->offset;
  c.stream = opts->stream_id;
  if (opts->transpose) {
    set_shape(out, cols, rows, NVFP4_SCALE_1X16);
    a.col = c;
    flags = kFCol | (opts->rht ? (rht4 ? kFRht4 : kFRht) : 0) |
            (opts->round == NVFP4_SR ? kFSrCol : 0);
  } else {
    set_shape(out, rows, cols, NVFP4_SCALE_1X16);
    a.row = c;
    flags = kFRow | (opts->round == NVFP4_SR ? kFSrRow : 0);
  }
  NVFP4_HIP(launch_zero_words(slots, 2 * kAmaxRegionWords, s));
  NVFP4_HIP(launch_amax(x, dtype, rows, cols, ld, opts->rht_signs, opts->rht ? nullptr : slot_raw,
                        opts->rht ? slot_rht : nullptr, s, rht4 ? 4 : 16));
  NVFP4_HIP(launch_quant_tile(dtype, flags, a, s));
  return NVFP4_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint32_t* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of `scratch` (the stream's device must be the current
// one); looked up on the first call on each device and kept until the
// process ends.
nvfp4_status static_scratch(hipStream_t s, uint32_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_HIP;
  if (s) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess || sdev != dev) return NVFP4_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return NVFP4_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<uint32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return NVFP4_OK;
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_tensor_bytes(int64_t rows, int64_t cols, int32_t scale_mode, size_t* codes_bytes,
                                size_t* scales_bytes) {
  if (!codes_bytes || !scales_bytes) return NVFP4_ERR_NULL;
  if (rows <= 0 || cols <= 0 || cols % 16 != 0) return NVFP4_ERR_SHAPE;
  int64_t codes = 0;
  if (!mul_ok(rows, cols / 2, &codes)) return NVFP4_ERR_SHAPE;
  if (scale_mode == NVFP4_SCALE_MX32) {
    if (cols % 32 != 0) return NVFP4_ERR_SHAPE;
    *scales_bytes = (size_t)(rows * (cols / 32));
  } else if (scale_mode == NVFP4_SCALE_1X16) {
    *scales_bytes = (size_t)(rows * (cols / 16));
  } else if (scale_mode == NVFP4_SCALE_16X16) {
    if (rows % 16 != 0) return NVFP4_ERR_SHAPE;
    *scales_bytes = (size_t)((rows / 16) * (cols / 16));
  } else {
    return NVFP4_ERR_DTYPE;
  }
  *codes_bytes = (size_t)codes;
  return NVFP4_OK;
}

size_t nvfp4_workspace_bytes(void) { return kWorkspaceBytes; }

nvfp4_status nvfp4_linear_ctx_bytes(int64_t M, int64_t K, int64_t N, size_t* bytes) {
  if (!bytes) return NVFP4_ERR_NULL;
  if (M <= 0 || K <= 0 || N <= 0 || M % 16 || K % 16 || N % 16) return NVFP4_ERR_SHAPE;
  int64_t rc[6][2];
  ctx_shapes(M, K, N, rc);
  for (int i = 0; i < 6; ++i) {
    int64_t e = 0;
    if (!mul_ok(rc[i][0], rc[i][1], &e)) return NVFP4_ERR_SHAPE;
  }
  size_t total = 0;
  for (int i = 0; i < 6; ++i) {
    total += align256((size_t)(rc[i][0] * (rc[i][1] / 2)));   // codes
    total += align256((size_t)(rc[i][0] * (rc[i][1] / 16)));  // 1x16-sized scales
    total += 256;                                              // tensor scale
  }
  total += NVFP4_LINEAR_SCRATCH_BYTES;                          // backward split scratch
  *bytes = total;
  return NVFP4_OK;
}

nvfp4_status nvfp4_linear_ctx_init(nvfp4_linear_ctx* ctx, void* buffer, size_t bytes, int64_t M,
                                   int64_t K, int64_t N) {
  if (!ctx || !buffer) return NVFP4_ERR_NULL;
  size_t need = 0;
  NVFP4_TRY(nvfp4_linear_ctx_bytes(M, K, N, &need));
  if (bytes < need) return NVFP4_ERR_SHAPE;
  if (!aligned(buffer, 256)) return NVFP4_ERR_ALIGN;
  int64_t rc[6][2];
  ctx_shapes(M, K, N, rc);
  nvfp4_tensor* t[6] = {&ctx->xq, &ctx->wq, &ctx->wqt, &ctx->xqt, &ctx->dyq, &ctx->dyqt};
  const int32_t modes[6] = {NVFP4_SCALE_1X16, NVFP4_SCALE_16X16, NVFP4_SCALE_16X16,
                            NVFP4_SCALE_1X16, NVFP4_SCALE_1X16,  NVFP4_SCALE_1X16};
  uint8_t* p = static_cast<uint8_t*>(buffer);
  for (int i = 0; i < 6; ++i) {
    t[i]->codes = p;
    p += align256((size_t)(rc[i][0] * (rc[i][1] / 2)));
    t[i]->scales = p;
    p += align256((size_t)(rc[i][0] * (rc[i][1] / 16)));
    t[i]->global_scale = reinterpret_cast<float*>(p);
    p += 256;
    set_shape(t[i], rc[i][0], rc[i][1], modes[i]);
  }
  ctx->M = M;
  ctx->K = K;
  ctx->N = N;
  ctx->rht_signs = 0;
  ctx->rht = 0;
  ctx->wgrad_scratch = p;
  ctx->wgrad_scratch_bytes = NVFP4_LINEAR_SCRATCH_BYTES;
  return NVFP4_OK;
}

uint32_t nvfp4_rht_signs_from_seed(uint64_t seed) {
  uint32_t c[4] = {0u, 0u, 0u, 0u};
  philox_host(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  return c[0] & 0xFFFFu;
}

void nvfp4_rht_signs128_from_seed(uint64_t seed, uint32_t* out) {
  uint32_t c[4] = {0u, 0u, 0u, 0u};
  philox_host(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  if (out) {
    out[0] = c[0];
    out[1] = c[1];
    out[2] = c[2];
    out[3] = c[3];
  }
}

nvfp4_status nvfp4_workspace_init(void* workspace, size_t ws_bytes, void* stream) {
  NVFP4_TRY(check_workspace(workspace, ws_bytes));
  NVFP4_HIP(launch_zero_words(static_cast<uint32_t*>(workspace), kWsWords, as_stream(stream)));
  return NVFP4_OK;
}

nvfp4_status nvfp4_device_status(void* workspace, void* stream) {
  if (!workspace) return NVFP4_ERR_WORKSPACE;
  uint32_t word = 0;
  NVFP4_HIP(hipMemcpyAsync(&word, workspace, 4, hipMemcpyDeviceToHost, as_stream(stream)));
  NVFP4_HIP(hipStreamSynchronize(as_stream(stream)));
  NVFP4_HIP(launch_zero_words(static_cast<uint32_t*>(workspace), 1, as_stream(stream)));
  return word == 0 ? NVFP4_OK : (nvfp4_status)word;
}

const char* nvfp4_status_string(nvfp4_status s) {
  switch (s) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "null pointer";
    case NVFP4_ERR_SHAPE: return "unsupported or inconsistent shape";
    case NVFP4_ERR_ALIGN: return "misaligned pointer, leading dimension or offset";
    case NVFP4_ERR_DTYPE: return "unsupported dtype or enum value";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_HIP: return "HIP launch or runtime error";
    case NVFP4_ERR_NONFINITE: return "non-finite tensor amax";
  }
  return "unknown status";
}

nvfp4_status nvfp4_quantize(const void* x, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                            const nvfp4_quant_opts* opts, nvfp4_tensor* out, void* workspace,
                            size_t ws_bytes, void* stream) {
  NVFP4_TRY(check_quantize_args(x, dtype, rows, cols, ld, opts, out));
  NVFP4_TRY(check_workspace(workspace, ws_bytes));
  return quantize_enqueue(x, dtype, rows, cols, ld, opts, out, ws_word(workspace, kSlotQRaw),
                          ws_word(workspace, kSlotStatus), as_stream(stream));
}

nvfp4_status nvfp4_quantize_static(const void* x, int32_t dtype, int64_t rows, int64_t cols,
                                   int64_t ld, const nvfp4_quant_opts* opts, nvfp4_tensor* out,
                                   uint32_t* status, void* stream) {
  NVFP4_TRY(check_quantize_args(x, dtype, rows, cols, ld, opts, out));
  if (!status) return NVFP4_ERR_NULL;
  if (!aligned(status, 4)) return NVFP4_ERR_ALIGN;
  uint32_t* slots = nullptr;
  NVFP4_TRY(static_scratch(as_stream(stream), &slots));
  return quantize_enqueue(x, dtype, rows, cols, ld, opts, out, slots, status, as_stream(stream));
}

nvfp4_status nvfp4_quantize_rowcol(const void* x, int32_t dtype, int64_t rows, int64_t cols,
                                   int64_t ld, const nvfp4_quant_opts* opts_row,
                                   const nvfp4_quant_opts* opts_col, nvfp4_tensor* row,
                                   nvfp4_tensor* col, void* workspace, size_t ws_bytes,
                                   void* stream) {
  NVFP4_TRY(check_source(x, dtype, rows, cols, ld));
  NVFP4_TRY(check_opts(opts_row));
  NVFP4_TRY(check_opts(opts_col));
  NVFP4_TRY(check_out(row));
  NVFP4_TRY(check_out(col));
  NVFP4_TRY(check_workspace(workspace, ws_bytes));
  if (opts_row->transpose != 0 || opts_row->rht != 0 || opts_col->transpose != 1)
    return NVFP4_ERR_SHAPE;
  if (opts_col->rht && opts_col->rht_d == 4) return NVFP4_ERR_DTYPE;  // 16-point only here
  if (rows % 16 != 0) return NVFP4_ERR_SHAPE;
  const hipStream_t s = as_stream(stream);
  set_shape(row, rows, cols, NVFP4_SCALE_1X16);
  set_shape(col, cols, rows, NVFP4_SCALE_1X16);
  TileArgs a;
  a.x = x;
  a.rows = rows;
  a.cols = cols;
  a.ld = ld;
  a.signs = opts_col->rht_signs;
  a.status = ws_word(workspace, kSlotStatus);
  a.row = copy_args(row, workspace, kSlotQRaw, opts_row);
  a.col = copy_args(col, workspace, opts_col->rht ? kSlotQRht : kSlotQRaw, opts_col);
  const int flags = kFRow | kFCol | (opts_col->rht ? kFRht : 0) |
                    (opts_row->round == NVFP4_SR ? kFSrRow : 0) |
                    (opts_col->round == NVFP4_SR ? kFSrCol : 0);
  NVFP4_HIP(zero_slots(workspace, kSlotQRaw, 2, s));
  NVFP4_HIP(launch_amax(x, dtype, rows, cols, ld, opts_col->rht_signs, ws_word(workspace, kSlotQRaw),
                        opts_col->rht ? ws_word(workspace, kSlotQRht) : nullptr, s));
  NVFP4_HIP(launch_quant_tile(dtype, flags, a, s));
  return NVFP4_OK;
}

nvfp4_status nvfp4_quantize_2d(const void* w, int32_t dtype, int64_t rows, int64_t cols, int64_t ld,
                               nvfp4_tensor* out, nvfp4_tensor* out_t, void* workspace,
                               size_t ws_bytes, void* stream) {
  NVFP4_TRY(check_source(w, dtype, rows, cols, ld));
  NVFP4_TRY(check_out(out));
  if (out_t) NVFP4_TRY(check_out(out_t));
  NVFP4_TRY(check_workspace(workspace, ws_bytes));
  if (rows % 16 != 0) return NVFP4_ERR_SHAPE;
  const hipStream_t s = as_stream(stream);
  set_shape(out, rows, cols, NVFP4_SCALE_16X16);
  TileArgs a;
  a.x = w;
  a.rows = rows;
  a.cols = cols;
  a.ld = ld;
  a.status = ws_word(workspace, kSlotStatus);
  a.row = copy_args(out, workspace, kSlotQRaw, nullptr);
  int flags = kFRow | kF2D;
  if (out_t) {
    set_shape(out_t, cols, rows, NVFP4_SCALE_16X16);
    a.col = copy_args(out_t, workspace, kSlotQRaw, nullptr);
    flags |= kFCol;
  }
  NVFP4_HIP(zero_slots(workspace, kSlotQRaw, 1, s));
  NVFP4_HIP(launch_amax(w, dtype, rows, cols, ld, 0, ws_word(workspace, kSlotQRaw), nullptr, s));
  NVFP4_HIP(launch_quant_tile(dtype, flags, a, s));
  return NVFP4_OK;
}

nvfp4_status nvfp4_rht16(const void* x, float* y, int32_t in_dtype, int64_t rows, int64_t cols,
                         int64_t ld, int32_t axis, uint32_t rht_signs, void* stream) {
  if (!x || !y) return NVFP4_ERR_NULL;
  if (in_dtype != NVFP4_F32 && in_dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
  if (axis != 0 && axis != 1) return NVFP4_ERR_DTYPE;
  if (rht_signs > 0xFFFFu) return NVFP4_ERR_DTYPE;
  if (rows <= 0 || cols <= 0 || ld < cols) return NVFP4_ERR_SHAPE;
  if (axis == 1 && cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (axis == 0 && (rows % 16 != 0 || cols % 8 != 0)) return NVFP4_ERR_SHAPE;
  if (rows > kMaxRows) return NVFP4_ERR_SHAPE;
  if (ld * (int64_t)elem_bytes(in_dtype) * 256 >= ((int64_t)1 << 31)) return NVFP4_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(y, 16) || (ld * (int64_t)elem_bytes(in_dtype)) % 16 != 0)
    return NVFP4_ERR_ALIGN;
  NVFP4_HIP(launch_rht16(x, y, in_dtype, rows, cols, ld, axis, rht_signs, as_stream(stream)));
  return NVFP4_OK;
}

nvfp4_status nvfp4_rht(const void* x, float* y, int32_t in_dtype, int64_t rows, int64_t cols,
                       int64_t ld, int32_t axis, int32_t d, const uint32_t* signs, void* stream) {
  if (!x || !y || !signs) return NVFP4_ERR_NULL;
  if (d != 4 && d != 16 && d != 128) return NVFP4_ERR_SHAPE;
  if (d == 16) return nvfp4_rht16(x, y, in_dtype, rows, cols, ld, axis, signs[0] & 0xFFFFu, stream);
  if (in_dtype != NVFP4_F32 && in_dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
  if (axis != 0 && axis != 1) return NVFP4_ERR_DTYPE;
  if (rows <= 0 || cols <= 0 || ld < cols) return NVFP4_ERR_SHAPE;
  if (axis == 1 && cols % (d < 8 ? 8 : d) != 0) return NVFP4_ERR_SHAPE;
  if (axis == 0 && rows % d != 0) return NVFP4_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(y, 16) || (ld * (int64_t)elem_bytes(in_dtype)) % 16 != 0)
    return NVFP4_ERR_ALIGN;
  const float c = (float)(1.0 / std::sqrt((double)d));
  NVFP4_HIP(launch_rht_d(x, y, in_dtype, rows, cols, ld, axis, d, signs, c, as_stream(stream)));
  return NVFP4_OK;
}

nvfp4_status nvfp4_gemm(const nvfp4_tensor* a, const nvfp4_tensor* b, void* c, int32_t c_dtype,
                        int64_t ldc, void* workspace, size_t ws_bytes, void* stream) {
  (void)workspace;
  (void)ws_bytes;
  NVFP4_TRY(check_gemm_operand(a));
  NVFP4_TRY(check_gemm_operand(b));
  if (!c) return NVFP4_ERR_NULL;
  if (c_dtype != NVFP4_F32 && c_dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
  if (a->cols != b->cols) return NVFP4_ERR_SHAPE;
  if (ldc < b->rows) return NVFP4_ERR_SHAPE;
  if ((a->rows + 255) / 256 * ((b->rows + 255) / 256) > (int64_t)0x7FFFFFFF) return NVFP4_ERR_SHAPE;
  if (!aligned(c, 4)) return NVFP4_ERR_ALIGN;
  const bool mxa = a->scale_mode == NVFP4_SCALE_MX32, mxb = b->scale_mode == NVFP4_SCALE_MX32;
  if (mxa != mxb) return NVFP4_ERR_DTYPE;
  if (mxa) {
    const int64_t K = a->cols;
    if (K % 128 != 0 || K < 384 || a->rows * (K / 2) >= ((int64_t)1 << 31) ||
        b->rows * (K / 2) >= ((int64_t)1 << 31))
      return NVFP4_ERR_SHAPE;
    NVFP4_HIP(launch_mx_gemm(gemm_operand(a), gemm_operand(b), K, c, c_dtype, ldc,
                             as_stream(stream)));
    return NVFP4_OK;
  }
  NVFP4_HIP(launch_gemm(gemm_operand(a), gemm_operand(b), a->cols, c, c_dtype, ldc, as_stream(stream)));
  return NVFP4_OK;
}

nvfp4_status nvfp4_dequantize(const nvfp4_tensor* t, float* out, int64_t ldo, void* stream) {
  NVFP4_TRY(check_gemm_operand(t));
  if (!out) return NVFP4_ERR_NULL;
  if (ldo < t->cols || ldo % 4 != 0) return NVFP4_ERR_SHAPE;
  if (!aligned(out, 16) || !aligned(t->codes, 4)) return NVFP4_ERR_ALIGN;
  NVFP4_HIP(launch_dequant(t->codes, t->scales, t->global_scale, t->rows, t->cols, t->scale_mode,
                           out, ldo, as_stream(stream)));
  return NVFP4_OK;
}

nvfp4_status nvfp4_mx_quantize(const void* x, int32_t dtype, int64_t rows, int64_t cols,
                               int64_t ld, nvfp4_tensor* out, void* stream) {
  NVFP4_TRY(check_source(x, dtype, rows, cols, ld));
  if (cols % 32 != 0) return NVFP4_ERR_SHAPE;
  if (!out || !out->codes || !out->scales) return NVFP4_ERR_NULL;
  if (!aligned(out->codes, 16)) return NVFP4_ERR_ALIGN;
  set_shape(out, rows, cols, NVFP4_SCALE_MX32);
  NVFP4_HIP(launch_mx_quantize(x, dtype, rows, cols, ld, out->codes, out->scales,
                               as_stream(stream)));
  return NVFP4_OK;
}

nvfp4_status nvfp4_bf16_gemm(const void* a, const void* b, void* c, int64_t M, int64_t N,
                             int64_t K, int32_t c_dtype, int64_t ldc, void* stream) {
  if (!a || !b || !c) return NVFP4_ERR_NULL;
  if (c_dtype != NVFP4_F32 && c_dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
  NVFP4_TRY(check_bf16_operand(M, K));
  NVFP4_TRY(check_bf16_operand(N, K));
  if (ldc < N) return NVFP4_ERR_SHAPE;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, elem_bytes(c_dtype)))
    return NVFP4_ERR_ALIGN;
  NVFP4_HIP(launch_bf16_gemm(a, M, b, N, K, c, c_dtype == NVFP4_BF16 ? kDtypeBF16 : kDtypeF32, ldc,
                             as_stream(stream)));
  return NVFP4_OK;
}

nvfp4_status nvfp4_linear_fwd(const void* x, const void* w, void* y, int64_t M, int64_t K, int64_t N,
                              int32_t dtype, const nvfp4_recipe* recipe, nvfp4_linear_ctx* ctx,
                              void* workspace, size_t ws_bytes, void* stream) {
  if (!recipe || !ctx || !y) return NVFP4_ERR_NULL;
  if (M % 16 || K % 16 || N % 16) return NVFP4_ERR_SHAPE;
  const bool bf16_fprop = recipe->bf16_fprop != 0;
  NVFP4_TRY(check_source(x, dtype, M, K, K));
  NVFP4_TRY(check_source(w, dtype, N, K, K));
  if (bf16_fprop) {
    if (dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
    NVFP4_TRY(check_bf16_operand(M, K));
    NVFP4_TRY(check_bf16_operand(N, K));
  } else {
    NVFP4_TRY(check_out(&ctx->xq));
    NVFP4_TRY(check_out(&ctx->wq));
  }
  if (recipe->training) {
    NVFP4_TRY(check_out(&ctx->wqt));
    NVFP4_TRY(check_out(&ctx->xqt));
  }
  if (recipe->rht_signs > 0xFFFFu) return NVFP4_ERR_DTYPE;
  NVFP4_TRY(check_workspace(workspace, ws_bytes));
  if (!aligned(y, 4)) return NVFP4_ERR_ALIGN;
  const hipStream_t s = as_stream(stream);
  ctx->M = M;
  ctx->K = K;
  ctx->N = N;
  const int wmode = recipe->no_2d_weights ? NVFP4_SCALE_1X16 : NVFP4_SCALE_16X16;
  if (!bf16_fprop) {
    set_shape(&ctx->xq, M, K, NVFP4_SCALE_1X16);
    set_shape(&ctx->wq, N, K, wmode);
  }
  // W^T (the Dgrad operand) only when training; the BF16 forward of an
  // inference call quantises nothing.
  const bool want_wt = recipe->training != 0;
  if (want_wt) set_shape(&ctx->wqt, K, N, wmode);
  NVFP4_HIP(zero_slots(workspace, kSlotXRaw, 3, s));

  // X: row-wise copy for Fprop and, when training, (R X)^T for Wgrad.
  TileArgs ax;
  ax.x = x;
  ax.rows = M;
  ax.cols = K;
  ax.ld = K;
  ax.signs = recipe->rht_signs;
  ax.status = ws_word(workspace, kSlotStatus);
  int fx = 0;
  if (!bf16_fprop) {
    ax.row = copy_args(&ctx->xq, workspace, kSlotXRaw, nullptr);
    fx |= kFRow;
  }
  const bool x_rht = recipe->training && !recipe->no_rht;
  ctx->rht_signs = recipe->rht_signs;
  ctx->rht = x_rht ? 1 : 0;
  if (recipe->training) {
    set_shape(&ctx->xqt, K, M, NVFP4_SCALE_1X16);
    // without the RHT the column copy has the row copy's amax
    ax.col = copy_args(&ctx->xqt, workspace, x_rht ? kSlotXRht : kSlotXRaw, nullptr);
    fx |= kFCol | (x_rht ? kFRht : 0);
  }
  if (fx) {
    NVFP4_HIP(launch_amax(x, dtype, M, K, K, recipe->rht_signs, ws_word(workspace, kSlotXRaw),
                          x_rht ? ws_word(workspace, kSlotXRht) : nullptr, s));
  }
  // W's stats pass runs before X's emit pass: it then reads right after
  // another read (X's stats) instead of after the emit's writes, whose dirty
  // lines it would otherwise write back while it reads (measured ~20 us
  // faster per forward).
  const bool w_any = !bf16_fprop || want_wt;
  if (w_any) NVFP4_HIP(launch_amax(w, dtype, N, K, K, 0, ws_word(workspace, kSlotW), nullptr, s));
  if (fx) NVFP4_HIP(launch_quant_tile(dtype, fx, ax, s));

  // W: 16x16 scales, with the transposed copy for Dgrad when training.  The
  // BF16 forward keeps only W^T (1x16 along N on its own with no_2d_weights).
  const int fw = (bf16_fprop ? 0 : kFRow) | (want_wt ? kFCol : 0) |
                 (recipe->no_2d_weights ? 0 : kF2D);
  if (fw & (kFRow | kFCol)) {
    TileArgs aw;
    aw.x = w;
    aw.rows = N;
    aw.cols = K;
    aw.ld = K;
    aw.status = ws_word(workspace, kSlotStatus);
    if (!bf16_fprop) aw.row = copy_args(&ctx->wq, workspace, kSlotW, nullptr);
    if (want_wt) aw.col = copy_args(&ctx->wqt, workspace, kSlotW, nullptr);
    NVFP4_HIP(launch_quant_tile(dtype, fw, aw, s));
  }

  if (bf16_fprop) {
    // Fprop in BF16: Y = X W^T [Review "Core strengths" item 9; Captions Fig. 7]
    NVFP4_HIP(launch_bf16_gemm(x, M, w, N, K, y, kDtypeBF16, N, s));
  } else {
    // Fprop: Y = Q(X) Q(W)^T
    NVFP4_HIP(launch_gemm(gemm_operand(&ctx->xq), gemm_operand(&ctx->wq), K, y, kDtypeBF16, N, s));
  }
  return NVFP4_OK;
}

nvfp4_status nvfp4_linear_bwd(const void* dy, int32_t dtype, nvfp4_linear_ctx* ctx, void* dx,
                              void* dw, int32_t dw_dtype, uint64_t sr_seed,
                              const nvfp4_recipe* recipe, void* workspace, size_t ws_bytes,
                              void* stream) {
  if (!ctx || !dx || !dw || !recipe) return NVFP4_ERR_NULL;
  const int64_t M = ctx->M, K = ctx->K, N = ctx->N;
  if (M <= 0 || M % 16 || K % 16 || N % 16) return NVFP4_ERR_SHAPE;
  if (ctx->xqt.rows != K || ctx->xqt.cols != M || ctx->wqt.rows != K || ctx->wqt.cols != N)
    return NVFP4_ERR_SHAPE;  // forward with training on this ctx has not run
  NVFP4_TRY(check_source(dy, dtype, M, N, N));
  if (dw_dtype != NVFP4_F32 && dw_dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
  NVFP4_TRY(check_out(&ctx->dyq));
  NVFP4_TRY(check_out(&ctx->dyqt));
  NVFP4_TRY(check_gemm_operand(&ctx->wqt));
  NVFP4_TRY(check_gemm_operand(&ctx->xqt));
  if (recipe->rht_signs > 0xFFFFu) return NVFP4_ERR_DTYPE;
  // (R dY)^T must carry the transform (R X)^T was built with [Review s3]
  if ((recipe->no_rht ? 0 : 1) != ctx->rht || (ctx->rht && recipe->rht_signs != ctx->rht_signs))
    return NVFP4_ERR_SHAPE;
  NVFP4_TRY(check_workspace(workspace, ws_bytes));
  if (!aligned(dx, 4) || !aligned(dw, 4)) return NVFP4_ERR_ALIGN;
  const hipStream_t s = as_stream(stream);
  set_shape(&ctx->dyq, M, N, NVFP4_SCALE_1X16);
  set_shape(&ctx->dyqt, N, M, NVFP4_SCALE_1X16);
  NVFP4_HIP(zero_slots(workspace, kSlotDyRaw, 2, s));

  // dY: SR row copy (stream 0) and SR (R dY)^T (stream 1) from one read.
  TileArgs ad;
  ad.x = dy;
  ad.rows = M;
  ad.cols = N;
  ad.ld = N;
  ad.signs = recipe->rht_signs;
  ad.status = ws_word(workspace, kSlotStatus);
  const bool rht = !recipe->no_rht, sr = !recipe->no_sr;
  const int32_t rnd = sr ? NVFP4_SR : NVFP4_RN;
  nvfp4_quant_opts o_row{rnd, 0, 0, recipe->rht_signs, sr_seed, 0, 0};
  nvfp4_quant_opts o_col{rnd, 1, rht ? 1 : 0, recipe->rht_signs, sr_seed, 0, 1};
  ad.row = copy_args(&ctx->dyq, workspace, kSlotDyRaw, &o_row);
  ad.col = copy_args(&ctx->dyqt, workspace, rht ? kSlotDyRht : kSlotDyRaw, &o_col);
  NVFP4_HIP(launch_amax(dy, dtype, M, N, N, recipe->rht_signs, ws_word(workspace, kSlotDyRaw),
                        rht ? ws_word(workspace, kSlotDyRht) : nullptr, s));
  NVFP4_HIP(launch_quant_tile(
      dtype, kFRow | kFCol | (rht ? kFRht : 0) | (sr ? kFSrRow | kFSrCol : 0), ad, s));

  // Dgrad: dX = Q(dY) Q(W^T)^T [M, K];  Wgrad: dW = Q((R dY)^T) Q((R X)^T)^T [N, K]
  // (one launch: the Wgrad tiles fill the Dgrad tail)
  NVFP4_HIP(launch_gemm_pair(gemm_operand(&ctx->dyq), gemm_operand(&ctx->wqt), N, dx, kDtypeBF16,
                             K, gemm_operand(&ctx->dyqt), gemm_operand(&ctx->xqt), M, dw,
                             dw_dtype == NVFP4_BF16 ? kDtypeBF16 : kDtypeF32, K,
                             static_cast<float*>(ctx->wgrad_scratch), ctx->wgrad_scratch_bytes, s));
  return NVFP4_OK;
}

}  // extern "C"
