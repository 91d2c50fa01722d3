"""Python binding of the MI355X MLA paged-KV decode library (libmla_decode.so).

Argument marshalling only: every step of the decode runs in the library's
HIP kernels.  PyTorch provides device memory and the current stream.  The
library must be built (``python -m mla_paged_kv_decode_amd.build``); without
it every call raises -- there is no fallback implementation.

Entry points mirror include/mla_decode.h:
  plan(B, q_len, H, max_seq_len)            -> (num_splits, workspace_bytes)
  decode(q, kv_cache, block_table, seq_lens, softmax_scale, ...) -> (out, lse)
  decode_varlen(q, cu_seqlens_q, kv_cache, block_table, seq_lens, ...) -> (out, lse)
  decode_tensors(q, kv_cache, block_table, seq_lens, ..., out=, workspace=) -> (out, lse)
      (per-tensor descriptors: the library checks element types, extents and strides)
  kv_pack_quantize_fp8(latent, rope, kv_scale, ...) -> uint8 rows [T, 576]
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_decode.so")

D_QK = 576
D_V = 512
DTYPE_BF16 = 1
DTYPE_FP8_E4M3 = 2
DTYPE_FP16 = 3
DTYPE_BF16_Q_FP8_KV = 4  # bf16 q over an E4M3 cache

STATUS = {0: "MLA_OK", -1: "MLA_ERR_NULL", -2: "MLA_ERR_DTYPE", -3: "MLA_ERR_SHAPE", -4: "MLA_ERR_ALIGN",
          -5: "MLA_ERR_WORKSPACE", -6: "MLA_ERR_UNSUPPORTED", -7: "MLA_ERR_HIP", -8: "MLA_ERR_DEVICE",
          -9: "MLA_ERR_STRIDE"}
# mla_elem codes of the tensor descriptors
ELEM_BF16, ELEM_FP8_E4M3, ELEM_FP16, ELEM_FP32, ELEM_INT32 = 1, 2, 3, 4, 5

# every symbol include/mla_decode.h declares
EXPORTS = ["mla_get_split_kv_and_workspace", "mla_decode", "mla_decode_ex", "mla_decode_varlen",
           "mla_decode_tensors", "mla_decode_static", "mla_workspace_bytes_ex", "mla_plan_for_cus", "mla_kv_pack_quantize_fp8",
           "mla_last_error", "mla_version"]


class MlaError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code


class MlaShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_len", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class MlaOptions(ctypes.Structure):
    _fields_ = [("num_splits", ctypes.c_int32), ("no_fold", ctypes.c_int32), ("partial_fp32", ctypes.c_int32),
                ("stages", ctypes.c_int32), ("window", ctypes.c_int32), ("kernel", ctypes.c_int32),
                ("merge", ctypes.c_int32), ("reserved", ctypes.c_int32 * 1),
                ("split_event", ctypes.c_void_p)]


class MlaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class MlaWorkspace(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("bytes", ctypes.c_size_t), ("num_splits", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32)]


def options(num_splits: int = 0, no_fold: bool = False, partial_fp32: bool = False, split_event=None,
            stages: int = 0, window: int = 0, kernel: int = 0, merge: int = 0) -> MlaOptions:
    """mla_options; split_event is a raw hipEvent_t (e.g. torch.cuda.Event().cuda_event after one record);
    stages 1 / 2 launch only the split-KV / only the merge kernel; window > 0 is the sliding-window mask
    (token t sees keys [max(0, n_t - window), n_t)); kernel 1 / 2 select the four-wave / the
    role-specialised twelve-wave E4M3 split-KV kernel (0: the default, the four-wave kernel on pages of
    at least 64 keys without a window, the twelve-wave one otherwise); for rows spread over more than 16
    slices on average, merge 1 selects the workgroup-per-row merge and 2 the per-wave one (0: the wide
    merge)."""
    o = MlaOptions()
    o.num_splits = int(num_splits)
    o.no_fold = int(bool(no_fold))
    o.partial_fp32 = int(bool(partial_fp32))
    o.stages = int(stages)
    o.window = int(window)
    o.kernel = int(kernel)
    o.merge = int(merge)
    o.split_event = split_event
    return o


_lib = None


def lib():
    """Load libmla_decode.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mla_paged_kv_decode_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i32, p, sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    L.mla_get_split_kv_and_workspace.argtypes = [i32, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(sz)]
    L.mla_workspace_bytes_ex.argtypes = [i32, i32, i32, i32, ctypes.POINTER(MlaOptions), ctypes.POINTER(i32),
                                         ctypes.POINTER(sz)]
    L.mla_plan_for_cus.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(MlaOptions), ctypes.POINTER(i32),
                                   ctypes.POINTER(i32), ctypes.POINTER(sz)]
    dec = [ctypes.POINTER(MlaShape), p, p, p, p, ctypes.c_float, ctypes.c_float, ctypes.c_float, p, p, p, sz, p]
    L.mla_decode.argtypes = dec
    L.mla_decode_ex.argtypes = dec + [ctypes.POINTER(MlaOptions)]
    fl = ctypes.c_float
    L.mla_decode_varlen.argtypes = [ctypes.POINTER(MlaShape), p, p, i32, p, p, p, fl, fl, fl, p, p, p, sz, p,
                                    ctypes.POINTER(MlaOptions)]
    L.mla_kv_pack_quantize_fp8.argtypes = [p, ctypes.c_int64, p, ctypes.c_int64, p, i32, ctypes.c_float, p,
                                           ctypes.c_int64, p]
    L.mla_decode_static.argtypes = [ctypes.POINTER(MlaShape), p, p, p, p, fl, fl, fl, p, p, p,
                                    ctypes.POINTER(MlaOptions)]
    tp = ctypes.POINTER(MlaTensor)
    L.mla_decode_tensors.argtypes = [tp, tp, tp, tp, fl, fl, fl, tp, tp, ctypes.POINTER(MlaWorkspace), p,
                                     ctypes.POINTER(MlaOptions)]
    L.mla_last_error.restype = ctypes.c_char_p
    L.mla_last_error.argtypes = []
    L.mla_version.restype = ctypes.c_int
    for f in ("mla_get_split_kv_and_workspace", "mla_workspace_bytes_ex", "mla_plan_for_cus", "mla_decode",
              "mla_decode_ex", "mla_decode_varlen", "mla_decode_tensors", "mla_decode_static",
              "mla_kv_pack_quantize_fp8"):
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int):
    if rc != 0:
        raise MlaError(rc, lib().mla_last_error().decode())


def plan(batch: int, q_len: int, num_heads: int, max_seq_len: int, opts: MlaOptions | None = None):
    """(num_splits, workspace_bytes) for a shape on the current device."""
    ns, ws = ctypes.c_int32(), ctypes.c_size_t()
    if opts is None:
        _check(lib().mla_get_split_kv_and_workspace(batch, q_len, num_heads, max_seq_len, ctypes.byref(ns),
                                                    ctypes.byref(ws)))
    else:
        _check(lib().mla_workspace_bytes_ex(batch, q_len, num_heads, max_seq_len, ctypes.byref(opts),
                                            ctypes.byref(ns), ctypes.byref(ws)))
    return ns.value, ws.value


def plan_for_cus(batch: int, q_len: int, num_heads: int, max_seq_len: int, num_cus: int,
                 opts: MlaOptions | None = None):
    """Host-only plan for an explicit compute-unit count: (num_splits, fold_factor, workspace_bytes)."""
    ns, fold, ws = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_size_t()
    _check(lib().mla_plan_for_cus(batch, q_len, num_heads, max_seq_len, num_cus,
                                  ctypes.byref(opts) if opts is not None else None, ctypes.byref(ns),
                                  ctypes.byref(fold), ctypes.byref(ws)))
    return ns.value, fold.value, ws.value


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return DTYPE_FP8_E4M3
    if t.dtype == torch.float16:
        return DTYPE_FP16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _pair_code(q, kv_cache) -> int:
    """mla_dtype of a (q, kv_cache) pair: one format for both, or bf16 q over an E4M3 cache."""
    qc, kc = _dtype_code(q), _dtype_code(kv_cache)
    if qc == kc:
        return qc
    if qc == DTYPE_BF16 and kc == DTYPE_FP8_E4M3:
        return DTYPE_BF16_Q_FP8_KV
    raise TypeError("q and kv_cache must have the same dtype, or be bf16 q over an E4M3 cache")


def make_shape(q, kv_cache, block_table, max_seq_len: int) -> MlaShape:
    s = MlaShape()
    s.batch, s.q_len, s.num_heads = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
    s.num_pages, s.page_size = int(kv_cache.shape[0]), int(kv_cache.shape[1])
    s.max_pages = int(block_table.shape[1])
    s.max_seq_len = int(max_seq_len)
    s.dtype = _pair_code(q, kv_cache)
    return s


def _check_layout(q, kv_cache, block_table, seq_lens, batch=None):
    """Layouts the kernels read; `batch` is the number of sequences (q.shape[0] when None)."""
    torch = _torch()
    if q.dim() != 4 or q.shape[3] != D_QK or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, q_len, H, 576] tensor")
    if kv_cache.dim() != 3 or kv_cache.shape[2] != D_QK or not kv_cache.is_contiguous():
        raise ValueError("kv_cache must be a contiguous [num_pages, page_size, 576] tensor")
    _pair_code(q, kv_cache)
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be int32 [B, max_pages] with unit column stride")
    if block_table.stride(0) != block_table.shape[1]:
        raise ValueError("block_table rows must be packed (row stride = max_pages)")
    if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1 or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous int32 [B] tensor")
    B = int(q.shape[0]) if batch is None else int(batch)
    if block_table.shape[0] != B or seq_lens.numel() != B:
        raise ValueError(f"block_table must have {B} rows and seq_lens {B} entries (one per sequence)")


def _check_device(q, *others):
    """Every tensor on q's HIP device (the library reads and writes them there)."""
    if q.device.type != "cuda":
        raise ValueError("q must be on a HIP device")
    for name, t in others:
        if t is not None and t.device != q.device:
            raise ValueError(f"{name} must be on {q.device} (is on {t.device})")


def _check_outputs(q, out, lse, workspace, out_shape, lse_shape):
    """Caller-supplied out / lse / workspace: dtype, shape and layout the kernels write."""
    torch = _torch()
    if out is not None and (out.dtype != torch.bfloat16 or tuple(out.shape) != tuple(out_shape)
                            or not out.is_contiguous()):
        raise ValueError(f"out must be a contiguous bfloat16 tensor of shape {tuple(out_shape)}")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != tuple(lse_shape)
                            or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {tuple(lse_shape)}")
    if workspace is not None and (workspace.dtype != torch.uint8 or workspace.dim() != 1
                                  or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor")


def decode(q, kv_cache, block_table, seq_lens, softmax_scale: float, q_scale: float = 1.0, kv_scale: float = 1.0,
           *, max_seq_len: int | None = None, out=None, lse=None, return_lse: bool = True, workspace=None,
           opts: MlaOptions | None = None, stream=None):
    """MLA decode through the C ABI.  Tensors live on the current HIP device.

    q: [B, q_len, H, 576] bfloat16, float16 or float8_e4m3fn; kv_cache: [num_pages,
    page_size, 576] of the same dtype (or float8_e4m3fn under bfloat16 q); block_table: int32 [B, max_pages];
    seq_lens: int32 [B].  Returns (out bf16 [B, q_len, H, 512], lse fp32
    [B, q_len, H] or None).  max_seq_len defaults to max(seq_lens), which
    reads seq_lens back to the host (pass it to avoid that synchronisation).
    """
    torch = _torch()
    _check_layout(q, kv_cache, block_table, seq_lens)
    B, q_len, H = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
    _check_outputs(q, out, lse, workspace, (B, q_len, H, D_V), (B, q_len, H))
    _check_device(q, ("kv_cache", kv_cache), ("block_table", block_table), ("seq_lens", seq_lens), ("out", out),
                  ("lse", lse), ("workspace", workspace))
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if seq_lens.numel() else 0
    shape = make_shape(q, kv_cache, block_table, max_seq_len)
    if out is None:
        out = torch.empty((B, q_len, H, D_V), dtype=torch.bfloat16, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, q_len, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        _, ws_bytes = plan(B, q_len, H, max_seq_len, opts)
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    args = (ctypes.byref(shape), q.data_ptr(), kv_cache.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(),
            float(softmax_scale), float(q_scale), float(kv_scale), out.data_ptr(),
            lse.data_ptr() if lse is not None else None, workspace.data_ptr(), workspace.numel(), stream)
    if opts is None:
        _check(lib().mla_decode(*args))
    else:
        _check(lib().mla_decode_ex(*args, ctypes.byref(opts)))
    return out, lse


def decode_varlen(q, cu_seqlens_q, kv_cache, block_table, seq_lens, softmax_scale: float, q_scale: float = 1.0,
                  kv_scale: float = 1.0, *, max_q_len: int, max_seq_len: int, out=None, lse=None, workspace=None,
                  opts: MlaOptions | None = None, stream=None):
    """Ragged batch through mla_decode_varlen: sequence b's new tokens are rows
    [cu_seqlens_q[b], cu_seqlens_q[b+1]) of q [total_q, H, 576]; cu_seqlens_q is a device
    int32 [B+1]; max_q_len is the largest per-sequence count (host int, sizes the plan).
    Returns (out bf16 [total_q, H, 512], lse fp32 [total_q, H])."""
    torch = _torch()
    if q.dim() != 3 or q.shape[2] != D_QK or not q.is_contiguous():
        raise ValueError("q must be a contiguous [total_q, H, 576] tensor")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_q.dim() != 1 or not cu_seqlens_q.is_contiguous():
        raise ValueError("cu_seqlens_q must be a contiguous int32 [B + 1] tensor")
    B = int(cu_seqlens_q.numel()) - 1
    q4 = q.view(1, q.shape[0], q.shape[1], D_QK)  # layout checks only
    _check_layout(q4, kv_cache, block_table, seq_lens, batch=B)
    total_q, H = int(q.shape[0]), int(q.shape[1])
    _check_outputs(q, out, lse, workspace, (total_q, H, D_V), (total_q, H))
    _check_device(q, ("cu_seqlens_q", cu_seqlens_q), ("kv_cache", kv_cache), ("block_table", block_table),
                  ("seq_lens", seq_lens), ("out", out), ("lse", lse), ("workspace", workspace))
    shape = make_shape(q4, kv_cache, block_table, max_seq_len)
    shape.batch, shape.q_len, shape.num_heads = B, int(max_q_len), H
    if out is None:
        out = torch.empty((total_q, H, D_V), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((total_q, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        _, ws_bytes = plan(B, int(max_q_len), H, max_seq_len, opts)
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(lib().mla_decode_varlen(ctypes.byref(shape), q.data_ptr(), cu_seqlens_q.data_ptr(), total_q,
                                   kv_cache.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(),
                                   float(softmax_scale), float(q_scale), float(kv_scale), out.data_ptr(),
                                   lse.data_ptr(), workspace.data_ptr(), workspace.numel(), stream,
                                   ctypes.byref(opts) if opts is not None else None))
    return out, lse


class PreparedDecode:
    """One decode call with its arguments marshalled once (validated by a first call), so that repeated
    launches cost a single C call.  The tensors must stay alive and unchanged in shape."""

    def __init__(self, q, kv_cache, block_table, seq_lens, softmax_scale: float, q_scale: float, kv_scale: float,
                 *, max_seq_len: int, out, lse, workspace, opts: MlaOptions | None = None, stream=None):
        torch = _torch()
        _check_layout(q, kv_cache, block_table, seq_lens)
        B, q_len, H = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
        _check_outputs(q, out, lse, workspace, (B, q_len, H, D_V), (B, q_len, H))
        _check_device(q, ("kv_cache", kv_cache), ("block_table", block_table), ("seq_lens", seq_lens),
                      ("out", out), ("lse", lse), ("workspace", workspace))
        self._keep = (q, kv_cache, block_table, seq_lens, out, lse, workspace)
        self._shape = make_shape(q, kv_cache, block_table, max_seq_len)
        self._opts = opts if opts is not None else options()
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        self._args = (ctypes.byref(self._shape), q.data_ptr(), kv_cache.data_ptr(), block_table.data_ptr(),
                      seq_lens.data_ptr(), float(softmax_scale), float(q_scale), float(kv_scale), out.data_ptr(),
                      lse.data_ptr() if lse is not None else None, workspace.data_ptr(), workspace.numel(), stream,
                      ctypes.byref(self._opts))
        self._fn = lib().mla_decode_ex
        _check(self._fn(*self._args))

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != 0:
            _check(rc)


def decode_static(q, kv_cache, block_table, seq_lens, softmax_scale: float, q_scale: float = 1.0,
                  kv_scale: float = 1.0, *, max_seq_len: int, out, lse=None, opts: MlaOptions | None = None,
                  stream=None):
    """mla_decode_static: the decode with the library's own static workspace (no allocation in the call).
    out (and lse, if given) are caller-owned."""
    torch = _torch()
    _check_layout(q, kv_cache, block_table, seq_lens)
    B, q_len, H = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
    if out is None:
        raise ValueError("pass `out`: the static entry point writes into caller-owned outputs")
    _check_outputs(q, out, lse, None, (B, q_len, H, D_V), (B, q_len, H))
    _check_device(q, ("kv_cache", kv_cache), ("block_table", block_table), ("seq_lens", seq_lens), ("out", out),
                  ("lse", lse))
    shape = make_shape(q, kv_cache, block_table, max_seq_len)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(lib().mla_decode_static(ctypes.byref(shape), q.data_ptr(), kv_cache.data_ptr(), block_table.data_ptr(),
                                   seq_lens.data_ptr(), float(softmax_scale), float(q_scale), float(kv_scale),
                                   out.data_ptr(), lse.data_ptr() if lse is not None else None, stream,
                                   ctypes.byref(opts) if opts is not None else None))
    return out, lse


def tensor_desc(t) -> MlaTensor:
    """mla_tensor of a torch tensor (device pointer, element type, shape and strides in elements)."""
    torch = _torch()
    elem = {torch.bfloat16: ELEM_BF16, torch.float8_e4m3fn: ELEM_FP8_E4M3, torch.uint8: ELEM_FP8_E4M3,
            torch.float16: ELEM_FP16, torch.float32: ELEM_FP32, torch.int32: ELEM_INT32}
    if t.dim() > 4:
        raise ValueError("descriptors hold at most 4 dimensions")
    d = MlaTensor()
    d.data = t.data_ptr()
    d.dtype = elem.get(t.dtype, 0)
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = int(t.shape[i])
        d.stride[i] = int(t.stride(i))
    return d


def decode_tensors(q, kv_cache, block_table, seq_lens, softmax_scale: float, q_scale: float = 1.0,
                   kv_scale: float = 1.0, *, max_seq_len: int, out, lse=None, workspace=None, num_splits: int = 0,
                   opts: MlaOptions | None = None, stream=None):
    """mla_decode_tensors: the decode through per-tensor descriptors (element type, shape and strides are
    checked by the library, strided views included).  out / lse / workspace are caller-owned."""
    torch = _torch()
    ws = MlaWorkspace()
    ws.data = workspace.data_ptr() if workspace is not None else None
    ws.bytes = workspace.numel() if workspace is not None else 0
    ws.num_splits = int(num_splits)
    ws.max_seq_len = int(max_seq_len)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream if q.device.type == "cuda" else None
    descs = [tensor_desc(t) for t in (q, kv_cache, block_table, seq_lens, out)]
    ld = tensor_desc(lse) if lse is not None else None
    _check(lib().mla_decode_tensors(*(ctypes.byref(d) for d in descs[:4]), float(softmax_scale), float(q_scale),
                                    float(kv_scale), ctypes.byref(descs[4]),
                                    ctypes.byref(ld) if ld is not None else None, ctypes.byref(ws), stream,
                                    ctypes.byref(opts) if opts is not None else None))
    return out, lse


def kv_pack_quantize_fp8(latent, rope, kv_scale: float, *, slot_mapping=None, out=None, stream=None):
    """latent [T, 512] bf16 || rope [T, 64] bf16 -> E4M3 rows (uint8 [T, 576] or scattered into `out`)."""
    torch = _torch()
    if latent.dtype != torch.bfloat16 or rope.dtype != torch.bfloat16:
        raise TypeError("latent and rope must be bfloat16")
    if latent.dim() != 2 or latent.shape[1] != D_V or latent.stride(1) != 1:
        raise ValueError("latent must be [T, 512] with unit column stride")
    if rope.dim() != 2 or rope.shape[1] != D_QK - D_V or rope.stride(1) != 1 or rope.shape[0] != latent.shape[0]:
        raise ValueError("rope must be [T, 64] with unit column stride")
    T = latent.shape[0]
    if out is None:
        if slot_mapping is not None:
            raise ValueError("pass `out` when scattering through slot_mapping")
        out = torch.empty((T, D_QK), dtype=torch.uint8, device=latent.device)
    if (out.dtype not in (torch.uint8, torch.float8_e4m3fn) or not out.is_contiguous() or out.dim() < 2
            or out.shape[-1] != D_QK):
        raise ValueError("out must be a contiguous uint8 / float8_e4m3fn tensor whose last dimension is 576")
    rows = out.numel() // D_QK
    if slot_mapping is not None and (slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous()
                                     or slot_mapping.numel() != T):
        raise ValueError("slot_mapping must be a contiguous int64 tensor with one entry per token")
    _check_device(latent, ("rope", rope), ("out", out), ("slot_mapping", slot_mapping))
    if stream is None:
        stream = torch.cuda.current_stream(latent.device).cuda_stream
    _check(lib().mla_kv_pack_quantize_fp8(latent.data_ptr(), latent.stride(0), rope.data_ptr(), rope.stride(0),
                                          slot_mapping.data_ptr() if slot_mapping is not None else None, T,
                                          float(kv_scale), out.data_ptr(), rows, stream))
    return out
