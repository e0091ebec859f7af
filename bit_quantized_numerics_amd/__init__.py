"""Python binding of libnvfp4.so, the MI355X (gfx950) NVFP4 linear-layer library.

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI of ``include/nvfp4.h``.  PyTorch supplies device memory and
the current HIP stream.  There is no fallback: if the built library is
missing, importing this package raises.

Functions carry the C names (``nvfp4_quantize`` ...) and take torch tensors;
``NVFP4Tensor`` owns the device buffers of one quantised operand and
``Workspace`` the small status/reduction buffer every call needs.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python -m bit_quantized_numerics_amd.build "
        "or __graft_entry__.build()); there is no non-HIP fallback")

_lib = ctypes.CDLL(LIB_PATH)

# ------------------------------------------------------------------ C types
OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DTYPE, ERR_WORKSPACE, ERR_HIP, ERR_NONFINITE = range(8)
F32, BF16 = 0, 1
RN, SR = 0, 1
SCALE_1X16, SCALE_16X16, SCALE_MX32 = 0, 1, 2


class c_tensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("global_scale", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("scale_mode", ctypes.c_int32)]


class c_quant_opts(ctypes.Structure):
    _fields_ = [("round", ctypes.c_int32), ("transpose", ctypes.c_int32), ("rht", ctypes.c_int32),
                ("rht_signs", ctypes.c_uint32), ("seed", ctypes.c_uint64),
                ("offset", ctypes.c_uint64), ("stream_id", ctypes.c_uint32),
                ("rht_d", ctypes.c_int32)]


class c_recipe(ctypes.Structure):
    _fields_ = [("rht_signs", ctypes.c_uint32), ("training", ctypes.c_int32),
                ("no_2d_weights", ctypes.c_int32), ("no_rht", ctypes.c_int32),
                ("no_sr", ctypes.c_int32), ("bf16_fprop", ctypes.c_int32)]


class c_linear_ctx(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("K", ctypes.c_int64), ("N", ctypes.c_int64),
                ("xq", c_tensor), ("wq", c_tensor), ("wqt", c_tensor), ("xqt", c_tensor),
                ("dyq", c_tensor), ("dyqt", c_tensor), ("rht_signs", ctypes.c_uint32),
                ("rht", ctypes.c_int32), ("wgrad_scratch", ctypes.c_void_p),
                ("wgrad_scratch_bytes", ctypes.c_size_t)]


LINEAR_SCRATCH_BYTES = 32 << 20  # NVFP4_LINEAR_SCRATCH_BYTES


_vp, _i64, _i32, _u32, _u64, _sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                    ctypes.c_uint32, ctypes.c_uint64, ctypes.c_size_t)
_T = ctypes.POINTER(c_tensor)
_SIGS = {
    "nvfp4_tensor_bytes": (_i32, [_i64, _i64, _i32, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
    "nvfp4_workspace_bytes": (_sz, []),
    "nvfp4_rht_signs_from_seed": (_u32, [_u64]),
    "nvfp4_workspace_init": (_i32, [_vp, _sz, _vp]),
    "nvfp4_device_status": (_i32, [_vp, _vp]),
    "nvfp4_status_string": (ctypes.c_char_p, [_i32]),
    "nvfp4_quantize": (_i32, [_vp, _i32, _i64, _i64, _i64, ctypes.POINTER(c_quant_opts), _T, _vp,
                              _sz, _vp]),
    "nvfp4_quantize_static": (_i32, [_vp, _i32, _i64, _i64, _i64, ctypes.POINTER(c_quant_opts), _T,
                                     _vp, _vp]),
    "nvfp4_quantize_rowcol": (_i32, [_vp, _i32, _i64, _i64, _i64, ctypes.POINTER(c_quant_opts),
                                     ctypes.POINTER(c_quant_opts), _T, _T, _vp, _sz, _vp]),
    "nvfp4_quantize_2d": (_i32, [_vp, _i32, _i64, _i64, _i64, _T, _T, _vp, _sz, _vp]),
    "nvfp4_rht16": (_i32, [_vp, _vp, _i32, _i64, _i64, _i64, _i32, _u32, _vp]),
    "nvfp4_mx_quantize": (_i32, [_vp, _i32, _i64, _i64, _i64, _T, _vp]),
    "nvfp4_dequantize": (_i32, [_T, _vp, _i64, _vp]),
    "nvfp4_rht": (_i32, [_vp, _vp, _i32, _i64, _i64, _i64, _i32, _i32, ctypes.POINTER(_u32), _vp]),
    "nvfp4_rht_signs128_from_seed": (None, [_u64, ctypes.POINTER(_u32)]),
    "nvfp4_gemm": (_i32, [_T, _T, _vp, _i32, _i64, _vp, _sz, _vp]),
    "nvfp4_bf16_gemm": (_i32, [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _i64, _vp]),
    "nvfp4_peak_mfma_f16": (_i32, [_i32, _u32, _i32, _vp, ctypes.POINTER(ctypes.c_double), _vp]),
    "nvfp4_peak_mfma_fp4": (_i32, [_i32, _u32, _vp, ctypes.POINTER(ctypes.c_double), _vp]),
    "nvfp4_linear_ctx_bytes": (_i32, [_i64, _i64, _i64, ctypes.POINTER(_sz)]),
    "nvfp4_linear_ctx_init": (_i32, [ctypes.POINTER(c_linear_ctx), _vp, _sz, _i64, _i64, _i64]),
    "nvfp4_linear_fwd": (_i32, [_vp, _vp, _vp, _i64, _i64, _i64, _i32, ctypes.POINTER(c_recipe),
                                ctypes.POINTER(c_linear_ctx), _vp, _sz, _vp]),
    "nvfp4_linear_bwd": (_i32, [_vp, _i32, ctypes.POINTER(c_linear_ctx), _vp, _vp, _i32, _u64,
                                ctypes.POINTER(c_recipe), _vp, _sz, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib.nvfp4_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


def _check(status: int, where: str):
    if status != OK:
        raise NVFP4Error(status, where)


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise NVFP4Error(ERR_DTYPE, f"dtype {t.dtype}")


def _ld(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise NVFP4Error(ERR_SHAPE, "expected a 2D tensor with unit column stride")
    return t.stride(0)


# ------------------------------------------------------------------ buffers
class Workspace:
    """Device status word + reduction slots (nvfp4_workspace_bytes() bytes)."""

    def __init__(self, device="cuda"):
        self.nbytes = int(_lib.nvfp4_workspace_bytes())
        self.buf = torch.zeros(self.nbytes, dtype=torch.uint8, device=device)

    @property
    def ptr(self):
        return ctypes.c_void_p(self.buf.data_ptr())


class NVFP4Tensor:
    """Device buffers of one quantised operand [rows, cols] (cols = block axis)."""

    def __init__(self, rows: int, cols: int, scale_mode: int = SCALE_1X16, device="cuda"):
        cb, sb = _sz(0), _sz(0)
        _check(_lib.nvfp4_tensor_bytes(rows, cols, scale_mode, ctypes.byref(cb), ctypes.byref(sb)),
               "nvfp4_tensor_bytes")
        self.rows, self.cols, self.scale_mode = rows, cols, scale_mode
        self.codes = torch.empty(cb.value, dtype=torch.uint8, device=device)
        self.scales = torch.empty(sb.value, dtype=torch.uint8, device=device)
        self.global_scale = torch.empty(1, dtype=torch.float32, device=device)

    def c(self) -> c_tensor:
        return c_tensor(self.codes.data_ptr(), self.scales.data_ptr(), self.global_scale.data_ptr(),
                        self.rows, self.cols, self.scale_mode)

    def update(self, ct: c_tensor):
        self.rows, self.cols, self.scale_mode = ct.rows, ct.cols, ct.scale_mode

    def codes_2d(self):
        return self.codes[:self.rows * (self.cols // 2)].view(self.rows, self.cols // 2)

    def scales_2d(self):
        """The scale grid of the current scale mode (buffers may be larger)."""
        if self.scale_mode == SCALE_MX32:
            r, c = self.rows, self.cols // 32
        elif self.scale_mode == SCALE_1X16:
            r, c = self.rows, self.cols // 16
        else:
            r, c = self.rows // 16, self.cols // 16
        return self.scales[:r * c].view(r, c)


# ------------------------------------------------------------------ calls
def nvfp4_tensor_bytes(rows: int, cols: int, scale_mode: int = SCALE_1X16):
    cb, sb = _sz(0), _sz(0)
    _check(_lib.nvfp4_tensor_bytes(rows, cols, scale_mode, ctypes.byref(cb), ctypes.byref(sb)),
           "nvfp4_tensor_bytes")
    return cb.value, sb.value


def nvfp4_workspace_bytes() -> int:
    return int(_lib.nvfp4_workspace_bytes())


def nvfp4_rht_signs_from_seed(seed: int) -> int:
    return int(_lib.nvfp4_rht_signs_from_seed(seed))


def nvfp4_status_string(status: int) -> str:
    return _lib.nvfp4_status_string(status).decode()


def nvfp4_workspace_init(ws: Workspace):
    _check(_lib.nvfp4_workspace_init(ws.ptr, ws.nbytes, _stream(ws.buf.device)), "nvfp4_workspace_init")


def nvfp4_device_status(ws: Workspace) -> int:
    return int(_lib.nvfp4_device_status(ws.ptr, _stream(ws.buf.device)))


def _opts(round_mode=RN, transpose=False, rht=False, rht_signs=0, seed=0, offset=0, stream_id=0):
    return c_quant_opts(int(round_mode), int(transpose), int(rht), int(rht_signs), int(seed),
                        int(offset), int(stream_id))


def nvfp4_quantize(x: torch.Tensor, ws: Workspace, out: NVFP4Tensor | None = None, *,
                   round_mode=RN, transpose=False, rht=False, rht_signs=0, seed=0, offset=0,
                   stream_id=0, rht_d=16) -> NVFP4Tensor:
    rows, cols = x.shape
    if out is None:
        out = (NVFP4Tensor(cols, rows, device=x.device) if transpose
               else NVFP4Tensor(rows, cols, device=x.device))
    o = _opts(round_mode, transpose, rht, rht_signs, seed, offset, stream_id)
    o.rht_d = rht_d
    ct = out.c()
    _check(_lib.nvfp4_quantize(ctypes.c_void_p(x.data_ptr()), _dtype_code(x), rows, cols, _ld(x),
                               ctypes.byref(o), ctypes.byref(ct), ws.ptr, ws.nbytes,
                               _stream(x.device)), "nvfp4_quantize")
    out.update(ct)
    return out


def nvfp4_quantize_static(x: torch.Tensor, status: torch.Tensor, out: NVFP4Tensor | None = None, *,
                          round_mode=RN, transpose=False, rht=False, rht_signs=0, seed=0, offset=0,
                          stream_id=0, rht_d=16) -> NVFP4Tensor:
    """nvfp4_quantize without a workspace (library-owned reduction slots);
    `status`: a device int32/uint32 tensor of one element that receives
    ERR_NONFINITE when the amax is not finite."""
    rows, cols = x.shape
    if out is None:
        out = (NVFP4Tensor(cols, rows, device=x.device) if transpose
               else NVFP4Tensor(rows, cols, device=x.device))
    o = _opts(round_mode, transpose, rht, rht_signs, seed, offset, stream_id)
    o.rht_d = rht_d
    ct = out.c()
    _check(_lib.nvfp4_quantize_static(ctypes.c_void_p(x.data_ptr()), _dtype_code(x), rows, cols,
                                      _ld(x), ctypes.byref(o), ctypes.byref(ct),
                                      ctypes.c_void_p(status.data_ptr()), _stream(x.device)),
           "nvfp4_quantize_static")
    out.update(ct)
    return out


def nvfp4_quantize_rowcol(x: torch.Tensor, ws: Workspace, row: NVFP4Tensor | None = None,
                          col: NVFP4Tensor | None = None, *, round_row=RN, round_col=RN,
                          rht=True, rht_signs=0, seed=0, offset_row=0, offset_col=0,
                          stream_row=0, stream_col=1):
    rows, cols = x.shape
    row = row or NVFP4Tensor(rows, cols, device=x.device)
    col = col or NVFP4Tensor(cols, rows, device=x.device)
    o_r = _opts(round_row, False, False, rht_signs, seed, offset_row, stream_row)
    o_c = _opts(round_col, True, rht, rht_signs, seed, offset_col, stream_col)
    cr, cc = row.c(), col.c()
    _check(_lib.nvfp4_quantize_rowcol(ctypes.c_void_p(x.data_ptr()), _dtype_code(x), rows, cols,
                                      _ld(x), ctypes.byref(o_r), ctypes.byref(o_c),
                                      ctypes.byref(cr), ctypes.byref(cc), ws.ptr, ws.nbytes,
                                      _stream(x.device)), "nvfp4_quantize_rowcol")
    row.update(cr)
    col.update(cc)
    return row, col


def nvfp4_quantize_2d(w: torch.Tensor, ws: Workspace, out: NVFP4Tensor | None = None,
                      out_t: NVFP4Tensor | None = None, want_t: bool = True):
    rows, cols = w.shape
    out = out or NVFP4Tensor(rows, cols, SCALE_16X16, device=w.device)
    if want_t and out_t is None:
        out_t = NVFP4Tensor(cols, rows, SCALE_16X16, device=w.device)
    co = out.c()
    ct = out_t.c() if out_t is not None else None
    _check(_lib.nvfp4_quantize_2d(ctypes.c_void_p(w.data_ptr()), _dtype_code(w), rows, cols, _ld(w),
                                  ctypes.byref(co), ctypes.byref(ct) if ct is not None else None,
                                  ws.ptr, ws.nbytes, _stream(w.device)), "nvfp4_quantize_2d")
    out.update(co)
    if out_t is not None:
        out_t.update(ct)
    return out, out_t


def nvfp4_rht16(x: torch.Tensor, axis: int, rht_signs: int, y: torch.Tensor | None = None):
    rows, cols = x.shape
    y = y if y is not None else torch.empty(rows, cols, dtype=torch.float32, device=x.device)
    _check(_lib.nvfp4_rht16(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                            _dtype_code(x), rows, cols, _ld(x), axis, rht_signs, _stream(x.device)),
           "nvfp4_rht16")
    return y


def nvfp4_rht_signs128_from_seed(seed: int) -> tuple:
    out = (_u32 * 4)()
    _lib.nvfp4_rht_signs128_from_seed(seed, out)
    return tuple(out)


def nvfp4_rht(x: torch.Tensor, axis: int, d: int, signs, y: torch.Tensor | None = None):
    """Hadamard transform of size d (4, 16, 128) along axis; signs: 4 words."""
    rows, cols = x.shape
    if y is None:
        y = torch.empty(rows, cols, dtype=torch.float32, device=x.device)
    sg = (_u32 * 4)(*[int(v) for v in signs])
    _check(_lib.nvfp4_rht(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()), _dtype_code(x),
                          rows, cols, _ld(x), axis, d, sg, _stream(x.device)), "nvfp4_rht")
    return y


def nvfp4_dequantize(t: NVFP4Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Decode an operand to fp32 [rows, cols]."""
    if out is None:
        out = torch.empty(t.rows, t.cols, dtype=torch.float32, device=t.codes.device)
    ct = t.c()
    _check(_lib.nvfp4_dequantize(ctypes.byref(ct), ctypes.c_void_p(out.data_ptr()), _ld(out),
                                 _stream(out.device)), "nvfp4_dequantize")
    return out


def nvfp4_mx_quantize(x: torch.Tensor, out: NVFP4Tensor | None = None) -> NVFP4Tensor:
    """MXFP4 comparator quantisation (32-element blocks, E8M0 scales)."""
    rows, cols = x.shape
    if out is None:
        out = NVFP4Tensor(rows, cols, SCALE_MX32, device=x.device)
    ct = out.c()
    _check(_lib.nvfp4_mx_quantize(ctypes.c_void_p(x.data_ptr()), _dtype_code(x), rows, cols, _ld(x),
                                  ctypes.byref(ct), _stream(x.device)), "nvfp4_mx_quantize")
    out.update(ct)
    return out


def nvfp4_gemm(a: NVFP4Tensor, b: NVFP4Tensor, out_dtype=torch.float32, c: torch.Tensor | None = None,
               ws: Workspace | None = None):
    if c is None:
        c = torch.empty(a.rows, b.rows, dtype=out_dtype, device=a.codes.device)
    ca, cb = a.c(), b.c()
    _check(_lib.nvfp4_gemm(ctypes.byref(ca), ctypes.byref(cb), ctypes.c_void_p(c.data_ptr()),
                           _dtype_code(c), _ld(c), ws.ptr if ws else None, ws.nbytes if ws else 0,
                           _stream(c.device)), "nvfp4_gemm")
    return c


def nvfp4_bf16_gemm(a: torch.Tensor, b: torch.Tensor, out_dtype=torch.float32,
                    c: torch.Tensor | None = None):
    """C = A B^T for dense bf16 A [M, K], B [N, K] (FP32 accumulation)."""
    if a.dtype != torch.bfloat16 or b.dtype != torch.bfloat16:
        raise NVFP4Error(ERR_DTYPE, "nvfp4_bf16_gemm: operands must be bfloat16")
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise NVFP4Error(ERR_SHAPE, "nvfp4_bf16_gemm: shapes")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise NVFP4Error(ERR_ALIGN, "nvfp4_bf16_gemm: operands must be dense row-major")
    M, K = a.shape
    N = b.shape[0]
    if c is None:
        c = torch.empty(M, N, dtype=out_dtype, device=a.device)
    _check(_lib.nvfp4_bf16_gemm(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                                ctypes.c_void_p(c.data_ptr()), M, N, K, _dtype_code(c), _ld(c),
                                _stream(a.device)), "nvfp4_bf16_gemm")
    return c


def nvfp4_peak_mfma_f16(iters: int, toggle_mask: int = 0x87FF87FF, valu_per_mfma: int = 4,
                        device="cuda") -> float:
    """Time the fp16 MFMA loop on the current stream; returns TFLOP/s."""
    sink = torch.empty(2048, dtype=torch.float32, device=device)
    flops = ctypes.c_double(0.0)
    stream = torch.cuda.current_stream(device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    _check(_lib.nvfp4_peak_mfma_f16(iters, toggle_mask, valu_per_mfma, ctypes.c_void_p(sink.data_ptr()),
                                    ctypes.byref(flops),
                                    _stream(torch.device(device))), "nvfp4_peak_mfma_f16")
    e1.record(stream)
    e1.synchronize()
    return flops.value / (e0.elapsed_time(e1) * 1e-3) / 1e12


def nvfp4_peak_mfma_fp4(iters: int, toggle_mask: int = 0xFFFFFFFF, device="cuda") -> float:
    """Time the scaled FP4 MFMA loop on the current stream; returns TFLOP/s."""
    sink = torch.empty(2048, dtype=torch.float32, device=device)
    flops = ctypes.c_double(0.0)
    stream = torch.cuda.current_stream(device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    _check(_lib.nvfp4_peak_mfma_fp4(iters, toggle_mask, ctypes.c_void_p(sink.data_ptr()),
                                    ctypes.byref(flops), _stream(torch.device(device))),
           "nvfp4_peak_mfma_fp4")
    e1.record(stream)
    e1.synchronize()
    return flops.value / (e0.elapsed_time(e1) * 1e-3) / 1e12


def nvfp4_linear_ctx_bytes(M: int, K: int, N: int) -> int:
    out = _sz(0)
    _check(_lib.nvfp4_linear_ctx_bytes(M, K, N, ctypes.byref(out)), "nvfp4_linear_ctx_bytes")
    return out.value


class LinearContext:
    """Caller-owned quantised operands of one layer step (Y = X W^T)."""

    def __init__(self, M: int, K: int, N: int, device="cuda"):
        self.M, self.K, self.N = M, K, N
        self.xq = NVFP4Tensor(M, K, device=device)
        # 1x16-sized scale buffers: large enough for either weight recipe
        self.wq = NVFP4Tensor(N, K, SCALE_1X16, device=device)
        self.wqt = NVFP4Tensor(K, N, SCALE_1X16, device=device)
        self.xqt = NVFP4Tensor(K, M, device=device)
        self.dyq = NVFP4Tensor(M, N, device=device)
        self.dyqt = NVFP4Tensor(N, M, device=device)
        self.scratch = torch.empty(LINEAR_SCRATCH_BYTES, dtype=torch.uint8, device=device)
        self.cctx = c_linear_ctx(M, K, N, self.xq.c(), self.wq.c(), self.wqt.c(), self.xqt.c(),
                                 self.dyq.c(), self.dyqt.c(), 0, 0,
                                 ctypes.c_void_p(self.scratch.data_ptr()), LINEAR_SCRATCH_BYTES)

    @classmethod
    def from_buffer(cls, M: int, K: int, N: int, device="cuda"):
        """All six operands in one device buffer laid out by nvfp4_linear_ctx_init."""
        nbytes = nvfp4_linear_ctx_bytes(M, K, N)
        buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self = cls.__new__(cls)
        self.M, self.K, self.N, self.buffer = M, K, N, buf
        self.cctx = c_linear_ctx()
        _check(_lib.nvfp4_linear_ctx_init(ctypes.byref(self.cctx), ctypes.c_void_p(buf.data_ptr()),
                                          nbytes, M, K, N), "nvfp4_linear_ctx_init")
        base = buf.data_ptr()
        for name in ("xq", "wq", "wqt", "xqt", "dyq", "dyqt"):
            ct = getattr(self.cctx, name)
            t = NVFP4Tensor.__new__(NVFP4Tensor)
            t.rows, t.cols, t.scale_mode = ct.rows, ct.cols, ct.scale_mode
            n_codes, n_scales = ct.rows * ct.cols // 2, ct.rows * ct.cols // 16
            t.codes = buf[ct.codes - base:ct.codes - base + n_codes]
            t.scales = buf[ct.scales - base:ct.scales - base + n_scales]
            t.global_scale = buf[ct.global_scale - base:ct.global_scale - base + 4].view(torch.float32)
            setattr(self, name, t)
        return self

    def sync_shapes(self):
        for name in ("xq", "wq", "wqt", "xqt", "dyq", "dyqt"):
            getattr(self, name).update(getattr(self.cctx, name))


def _recipe(rht_signs, training, no_2d_weights, no_rht, no_sr, bf16_fprop=False):
    return c_recipe(int(rht_signs), int(training), int(no_2d_weights), int(no_rht), int(no_sr),
                    int(bf16_fprop))


def nvfp4_linear_fwd(x: torch.Tensor, w: torch.Tensor, ctx: LinearContext, ws: Workspace,
                     rht_signs: int, training: bool = True, y: torch.Tensor | None = None, *,
                     no_2d_weights: bool = False, no_rht: bool = False, no_sr: bool = False,
                     bf16_fprop: bool = False):
    M, K = x.shape
    N = w.shape[0]
    if y is None:
        y = torch.empty(M, N, dtype=torch.bfloat16, device=x.device)
    rec = _recipe(rht_signs, training, no_2d_weights, no_rht, no_sr, bf16_fprop)
    _check(_lib.nvfp4_linear_fwd(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.data_ptr()),
                                 ctypes.c_void_p(y.data_ptr()), M, K, N, _dtype_code(x),
                                 ctypes.byref(rec), ctypes.byref(ctx.cctx), ws.ptr, ws.nbytes,
                                 _stream(x.device)), "nvfp4_linear_fwd")
    ctx.sync_shapes()
    return y


def nvfp4_linear_bwd(dy: torch.Tensor, ctx: LinearContext, ws: Workspace, rht_signs: int,
                     sr_seed: int, dw_dtype=torch.float32, dx: torch.Tensor | None = None,
                     dw: torch.Tensor | None = None, *, no_2d_weights: bool = False,
                     no_rht: bool = False, no_sr: bool = False):
    if dx is None:
        dx = torch.empty(ctx.M, ctx.K, dtype=torch.bfloat16, device=dy.device)
    if dw is None:
        dw = torch.empty(ctx.N, ctx.K, dtype=dw_dtype, device=dy.device)
    rec = _recipe(rht_signs, True, no_2d_weights, no_rht, no_sr)
    _check(_lib.nvfp4_linear_bwd(ctypes.c_void_p(dy.data_ptr()), _dtype_code(dy), ctypes.byref(ctx.cctx),
                                 ctypes.c_void_p(dx.data_ptr()), ctypes.c_void_p(dw.data_ptr()),
                                 _dtype_code(dw), sr_seed, ctypes.byref(rec), ws.ptr, ws.nbytes,
                                 _stream(dy.device)), "nvfp4_linear_bwd")
    ctx.sync_shapes()
    return dx, dw
