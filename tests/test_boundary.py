"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/mla_decode.h declares, plans deterministically, and
rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

import mla_paged_kv_decode_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(mla_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = mla.lib()
    names = _declared_functions()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(mla.EXPORTS) == names
    assert lib.mla_version() == 100


def test_library_is_native_and_in_tree():
    assert os.path.dirname(mla.LIB_PATH) == os.path.join(ROOT, "mla_paged_kv_decode_amd")
    assert os.path.exists(mla.LIB_PATH)


# ---------------------------------------------------------------- planning (host only)
@pytest.mark.parametrize("B,q_len,H,L,F", [
    (1, 1, 16, 256, 1),
    (4, 4, 32, 81920, 4),
    (16, 4, 32, 81920, 4),
    (64, 1, 128, 65536, 1),
    (128, 4, 64, 81920, 2),
    (1, 3, 40, 900, 3),
    (2, 1, 256, 700, 1),
    (4, 1024, 16, 17408, 8),   # prefill-sized: 128 workgroup rows
    (4, 512, 128, 16896, 1),   # 512 rows
    (2, 40, 8, 4096, 10),      # 4 rows of 10 folded tokens (H*F = 80)
])
def test_plan_fold_factor_and_workspace(B, q_len, H, L, F):
    ns, fold, ws = mla.plan_for_cus(B, q_len, H, L, 256)
    assert fold == F
    assert ns >= 1
    H_eff = H * F
    U = (q_len // F) * ((H_eff + 127) // 128)
    if U <= 32:
        assert ns * U <= max(256, U)  # at most about one workgroup per compute unit
    else:
        # many rows of unequal work: about two workgroups per compute unit, two slices per row at least
        assert ns * U <= max(2 * 256 + U, 2 * U) and ns >= 2 and ns * U >= 2 * 256
    if ns > 1:
        assert ns < 8 or ns % 8 == 0  # equal share per XCD once there are enough slices
        rows = q_len * H
        need = (ns + B) * rows * (512 * 4 + 4) + U * B * 8 + U * 8  # fp32-sized partials; slice ranges, T per row
        assert need <= ws <= need + 3 * 256
    else:
        assert ws == 0
    # cached/deterministic
    assert mla.plan_for_cus(B, q_len, H, L, 256) == (ns, fold, ws)


def test_plan_small_shapes_spread_one_unit_per_slice():
    # fewer 32-key plan units than compute units: one unit per slice (then the merge)
    assert mla.plan_for_cus(1, 1, 16, 256, 256)[0] == 8
    assert mla.plan_for_cus(1, 1, 16, 32, 256)[:3:2] == (1, 0)  # one unit: no split, no workspace
    assert mla.plan_for_cus(1, 1, 16, 64, 256)[0] == 2
    assert mla.plan_for_cus(2, 1, 16, 300, 256)[0] == 16  # 2 x ceil(300/32) = 20 units, a multiple of 8 from 8 up
    assert mla.plan_for_cus(1, 4, 32, 81920, 256)[0] == 256  # capped by the compute units


def test_plan_options():
    ns, fold, ws = mla.plan_for_cus(4, 4, 32, 81920, 256, mla.options(num_splits=24, partial_fp32=True, no_fold=True))
    assert ns == 24 and fold == 1
    rows = 4 * 32
    assert ws >= (24 + 4) * rows * (512 * 4 + 4)


def test_plan_rejects_bad_sizes():
    for args in [(-1, 1, 1, 0), (1, 0, 1, 0), (1, 1, 0, 0), (1, 1, 1, -5)]:
        with pytest.raises(mla.MlaError) as e:
            mla.plan_for_cus(*args, 256)
        assert e.value.code == -3


# ---------------------------------------------------------------- validation before any device work
def _shape(**kw):
    s = mla.MlaShape()
    s.batch, s.q_len, s.num_heads, s.num_pages, s.page_size, s.max_pages, s.max_seq_len, s.dtype = (
        2, 4, 32, 100, 64, 10, 640, mla.DTYPE_FP8_E4M3)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def _decode_raw(shape, q=16, kv=16, bt=16, sl=16, out=16, lse=None, ws=None, wsb=0):
    L = mla.lib()
    return L.mla_decode(ctypes.byref(shape) if shape is not None else None, q, kv, bt, sl, 1.0, 1.0, 1.0, out, lse,
                        ws, wsb, None)


def test_validation_errors_without_device():
    assert _decode_raw(None) == -1
    assert _decode_raw(_shape(dtype=7)) == -2
    assert _decode_raw(_shape(dtype=mla.DTYPE_FP16), kv=24) == -4  # fp16 is accepted, then validated
    assert _decode_raw(_shape(dtype=mla.DTYPE_BF16_Q_FP8_KV), kv=24) == -4  # bf16 q / e4m3 cache likewise
    assert _decode_raw(_shape(dtype=5)) == -2
    assert _decode_raw(_shape(page_size=48)) == -3
    assert _decode_raw(_shape(page_size=8)) == -3
    assert _decode_raw(_shape(q_len=0)) == -3
    assert _decode_raw(_shape(num_pages=0)) == -3
    assert _decode_raw(_shape(max_seq_len=641)) == -3
    assert _decode_raw(_shape(), q=None) == -1
    assert _decode_raw(_shape(), kv=24) == -4
    assert _decode_raw(_shape(), out=8) == -4
    assert _decode_raw(_shape(), bt=2) == -4
    assert _decode_raw(_shape(batch=0)) == 0
    msg = mla.lib().mla_last_error()
    assert msg == b""
    _decode_raw(_shape(page_size=48))
    assert b"page_size" in mla.lib().mla_last_error()


def test_options_layout_matches_header():
    # mla_options: seven int32 fields, one reserved int32, then a pointer at byte 32
    o = mla.MlaOptions
    assert [o.num_splits.offset, o.no_fold.offset, o.partial_fp32.offset, o.stages.offset, o.window.offset,
            o.kernel.offset, o.merge.offset, o.reserved.offset, o.split_event.offset] == [0, 4, 8, 12, 16, 20, 24,
                                                                                         28, 32]
    assert ctypes.sizeof(o) == 40
    text = open(HEADER).read()
    body = text[text.index("typedef struct mla_options"):text.index("} mla_options;")]
    fields = re.findall(r"(int32_t|void\*)\s+(\w+)(\[\d+\])?;", body)
    assert [f[1] for f in fields] == ["num_splits", "no_fold", "partial_fp32", "stages", "window", "kernel",
                                      "merge", "reserved", "split_event"]
    assert re.search(r"int32_t\s+reserved\[1\];", body)


def test_kernel_and_merge_options_validated_before_any_device_work():
    L = mla.lib()
    shape = _shape()
    for kw, word in ((dict(kernel=3), b"kernel"), (dict(kernel=-1), b"kernel"), (dict(merge=3), b"merge"), (dict(merge=-1), b"merge")):
        opts = mla.options(**kw)
        rc = L.mla_decode_ex(ctypes.byref(shape), 16, 16, 16, 16, 1.0, 1.0, 1.0, 16, 16, None, 0, None,
                             ctypes.byref(opts))
        assert rc == -3 and word in L.mla_last_error()


def test_stages_option_validated_before_any_device_work():
    L = mla.lib()
    shape = _shape()
    for bad in (-1, 3):
        opts = mla.options(stages=bad)
        rc = L.mla_decode_ex(ctypes.byref(shape), 16, 16, 16, 16, 1.0, 1.0, 1.0, 16, 16, None, 0, None,
                             ctypes.byref(opts))
        assert rc == -3
        assert b"stages" in L.mla_last_error()


def test_window_option_validated_and_planned():
    L = mla.lib()
    shape = _shape()
    opts = mla.options(window=-5)
    rc = L.mla_decode_ex(ctypes.byref(shape), 16, 16, 16, 16, 1.0, 1.0, 1.0, 16, 16, None, 0, None,
                         ctypes.byref(opts))
    assert rc == -3 and b"window" in L.mla_last_error()
    with pytest.raises(mla.MlaError):
        mla.plan_for_cus(4, 4, 32, 81920, 256, mla.options(window=-1))
    # a window bounds each sequence's work at window + q_len - 1 keys (+ one unit of alignment),
    # so the planned slice count shrinks with it; a window past every length changes nothing
    assert mla.plan_for_cus(1, 4, 32, 81920, 256)[0] == 256
    assert mla.plan_for_cus(1, 4, 32, 81920, 256, mla.options(window=128))[0] == 6  # ceil(131/32) + 1 units
    assert mla.plan_for_cus(1, 4, 32, 81920, 256, mla.options(window=1000))[0] == 32  # ceil(1003/32) + 1 = 33
    assert mla.plan_for_cus(4, 4, 32, 8192, 256, mla.options(window=100000)) == mla.plan_for_cus(4, 4, 32, 8192, 256)


def test_pack_validation_without_device():
    L = mla.lib()
    assert L.mla_kv_pack_quantize_fp8(16, 512, 16, 64, None, -1, 1.0, 16, 10, None) == -3
    assert L.mla_kv_pack_quantize_fp8(16, 500, 16, 64, None, 4, 1.0, 16, 10, None) == -3
    assert L.mla_kv_pack_quantize_fp8(16, 516, 16, 64, None, 4, 1.0, 16, 10, None) == -4
    assert L.mla_kv_pack_quantize_fp8(16, 512, 16, 64, None, 4, 0.0, 16, 10, None) == -3
    assert L.mla_kv_pack_quantize_fp8(16, 512, 16, 64, None, 11, 1.0, 16, 10, None) == -3
    assert L.mla_kv_pack_quantize_fp8(16, 512, 16, 64, None, 0, 1.0, 16, 10, None) == 0
    assert L.mla_kv_pack_quantize_fp8(None, 512, 16, 64, None, 4, 1.0, 16, 10, None) == -1
    assert L.mla_kv_pack_quantize_fp8(8, 512, 16, 64, None, 4, 1.0, 16, 10, None) == -4


def test_device_query_fails_cleanly_without_gpu():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(mla.MlaError) as e:
        mla.plan(4, 4, 32, 81920)
    assert e.value.code in (-8, -7)


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(mla, "_lib", None)
    monkeypatch.setattr(mla, "LIB_PATH", "/nonexistent/libmla_decode.so")
    with pytest.raises(RuntimeError):
        mla.lib()


def test_dtype_pairs_of_the_binding():
    import torch

    bf = torch.empty(1, 1, 1, 576, dtype=torch.bfloat16)
    f8 = torch.empty(1, 64, 576, dtype=torch.float8_e4m3fn)
    h = torch.empty(1, 64, 576, dtype=torch.float16)
    assert mla._pair_code(bf, f8) == mla.DTYPE_BF16_Q_FP8_KV
    assert mla._pair_code(bf, bf.view(1, 1, 576).expand(1, 64, 576)) == mla.DTYPE_BF16
    with pytest.raises(TypeError):
        mla._pair_code(f8.view(64, 1, 1, 576), bf)  # fp8 q over a bf16 cache is not a supported pair
    with pytest.raises(TypeError):
        mla._pair_code(bf, h)


def test_varlen_validation_without_device():
    L = mla.lib()
    shape = _shape()

    def call(cu=16, total_q=8, q=16):
        return L.mla_decode_varlen(ctypes.byref(shape), q, cu, total_q, 16, 16, 16, 1.0, 1.0, 1.0, 16, None, None, 0,
                                   None, None)

    assert call(cu=None) == -1 and b"cu_seqlens_q" in L.mla_last_error()
    assert call(total_q=-1) == -3
    assert call(cu=18) == -4
    assert call(total_q=0) == 0  # no new token anywhere: nothing enqueued
    assert call(q=None) == -1


# ---------------------------------------------------------------- the binding's own checks (no device needed)
def _cpu_inputs(B=2, q_len=4, H=8, pages=6, max_pages=3):
    import torch

    q = torch.zeros(B, q_len, H, 576, dtype=torch.float8_e4m3fn)
    kv = torch.zeros(pages, 64, 576, dtype=torch.float8_e4m3fn)
    bt = torch.zeros(B, max_pages, dtype=torch.int32)
    sl = torch.full((B,), 100, dtype=torch.int32)
    return q, kv, bt, sl


def test_binding_rejects_batch_mismatches():
    import torch

    q, kv, bt, sl = _cpu_inputs()
    with pytest.raises(ValueError, match="block_table"):
        mla.decode(q, kv, bt[:1], sl, 0.1, max_seq_len=100)
    with pytest.raises(ValueError, match="seq_lens"):
        mla.decode(q, kv, bt, sl[:1], 0.1, max_seq_len=100)
    with pytest.raises(ValueError, match="block_table"):
        mla.decode(q, kv, torch.zeros(3, 3, dtype=torch.int32), torch.zeros(3, dtype=torch.int32), 0.1,
                   max_seq_len=100)


def test_binding_rejects_bad_outputs_and_workspace():
    import torch

    q, kv, bt, sl = _cpu_inputs()
    good_out = torch.empty(2, 4, 8, 512, dtype=torch.bfloat16)
    good_lse = torch.empty(2, 4, 8, dtype=torch.float32)
    bad_outs = [torch.empty(2, 4, 8, 512, dtype=torch.float32),      # dtype
                torch.empty(2, 4, 8, 256, dtype=torch.bfloat16),     # shape
                torch.empty(2, 4, 512, 8, dtype=torch.bfloat16).transpose(2, 3)]  # layout
    for o in bad_outs:
        with pytest.raises(ValueError, match="out"):
            mla.decode(q, kv, bt, sl, 0.1, max_seq_len=100, out=o, lse=good_lse)
    for l in [torch.empty(2, 4, 8, dtype=torch.float64), torch.empty(2, 4, 9, dtype=torch.float32),
              torch.empty(8, 4, 2, dtype=torch.float32).permute(2, 1, 0)]:
        with pytest.raises(ValueError, match="lse"):
            mla.decode(q, kv, bt, sl, 0.1, max_seq_len=100, out=good_out, lse=l)
    with pytest.raises(ValueError, match="workspace"):
        mla.decode(q, kv, bt, sl, 0.1, max_seq_len=100, out=good_out, lse=good_lse,
                   workspace=torch.empty(64, dtype=torch.float32))
    with pytest.raises(ValueError, match="out"):
        mla.PreparedDecode(q, kv, bt, sl, 0.1, 1.0, 1.0, max_seq_len=100, out=bad_outs[0], lse=good_lse,
                           workspace=torch.empty(64, dtype=torch.uint8))


def test_binding_requires_tensors_on_the_device():
    import torch

    q, kv, bt, sl = _cpu_inputs()
    out = torch.empty(2, 4, 8, 512, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device"):
        mla.decode(q, kv, bt, sl, 0.1, max_seq_len=100, out=out)
    with pytest.raises(ValueError, match="device"):
        mla.PreparedDecode(q, kv, bt, sl, 0.1, 1.0, 1.0, max_seq_len=100, out=out, lse=None,
                           workspace=torch.empty(64, dtype=torch.uint8))


def test_binding_varlen_checks():
    import torch

    q = torch.zeros(7, 8, 576, dtype=torch.bfloat16)
    kv = torch.zeros(6, 64, 576, dtype=torch.bfloat16)
    bt = torch.zeros(2, 3, dtype=torch.int32)
    sl = torch.full((2,), 100, dtype=torch.int32)
    cu = torch.tensor([0, 3, 7], dtype=torch.int32)
    with pytest.raises(ValueError, match="block_table"):
        mla.decode_varlen(q, cu, kv, bt[:1], sl, 0.1, max_q_len=4, max_seq_len=100)
    with pytest.raises(ValueError, match="out"):
        mla.decode_varlen(q, cu, kv, bt, sl, 0.1, max_q_len=4, max_seq_len=100,
                          out=torch.empty(7, 8, 500, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="device"):
        mla.decode_varlen(q, cu, kv, bt, sl, 0.1, max_q_len=4, max_seq_len=100)


def test_binding_pack_output_checks():
    import torch

    lat = torch.zeros(4, 512, dtype=torch.bfloat16)
    rope = torch.zeros(4, 64, dtype=torch.bfloat16)
    for bad in [torch.empty(4, 512, dtype=torch.uint8), torch.empty(576, 4, dtype=torch.uint8).t(),
                torch.empty(4, 576, dtype=torch.float32)]:
        with pytest.raises(ValueError, match="out"):
            mla.kv_pack_quantize_fp8(lat, rope, 1.0, out=bad)
    with pytest.raises(ValueError, match="slot_mapping"):
        mla.kv_pack_quantize_fp8(lat, rope, 1.0, out=torch.empty(8, 576, dtype=torch.uint8),
                                 slot_mapping=torch.zeros(3, dtype=torch.int64))


# ---------------------------------------------------------------- tensor descriptors through the C ABI
def _desc_args(**over):
    """Descriptors of a valid fp8 call on fake (aligned, never dereferenced) device addresses."""
    def t(dtype, shape, stride=None, data=0x10000):
        d = mla.MlaTensor()
        d.data, d.dtype, d.ndim = data, dtype, len(shape)
        if stride is None:
            stride, acc = [], 1
            for e in reversed(shape):
                stride.insert(0, acc)
                acc *= e
        for i, (e, s) in enumerate(zip(shape, stride)):
            d.shape[i], d.stride[i] = e, s
        return d

    a = dict(q=t(mla.ELEM_FP8_E4M3, [2, 4, 32, 576]), kv=t(mla.ELEM_FP8_E4M3, [100, 64, 576]),
             bt=t(mla.ELEM_INT32, [2, 10]), sl=t(mla.ELEM_INT32, [2]), out=t(mla.ELEM_BF16, [2, 4, 32, 512]),
             lse=t(mla.ELEM_FP32, [2, 4, 32]))
    a.update({k: (t(*v) if isinstance(v, tuple) else v) for k, v in over.items()})
    return a


def _call_desc(a, max_seq_len=640, num_splits=0):
    ws = mla.MlaWorkspace()
    ws.data, ws.bytes, ws.num_splits, ws.max_seq_len = 0x20000, 1 << 30, num_splits, max_seq_len
    L = mla.lib()
    ref = lambda d: ctypes.byref(d) if d is not None else None
    return L.mla_decode_tensors(ref(a["q"]), ref(a["kv"]), ref(a["bt"]), ref(a["sl"]), 1.0, 1.0, 1.0, ref(a["out"]),
                                ref(a["lse"]), ctypes.byref(ws), None, None)


def test_descriptor_strides_are_checked():
    ERR_STRIDE = -9
    # a strided q view (every other head), a padded block_table row, a transposed out, a strided seq_lens
    assert _call_desc(_desc_args(q=(mla.ELEM_FP8_E4M3, [2, 4, 32, 576], [4 * 64 * 576, 64 * 576, 2 * 576, 1]))) \
        == ERR_STRIDE
    assert b"q must be packed" in mla.lib().mla_last_error()
    assert _call_desc(_desc_args(bt=(mla.ELEM_INT32, [2, 10], [16, 1]))) == ERR_STRIDE
    assert _call_desc(_desc_args(out=(mla.ELEM_BF16, [2, 4, 32, 512], [65536, 16384, 1, 32]))) == ERR_STRIDE
    assert _call_desc(_desc_args(sl=(mla.ELEM_INT32, [2], [2]))) == ERR_STRIDE
    assert _call_desc(_desc_args(kv=(mla.ELEM_FP8_E4M3, [100, 64, 576], [64 * 640, 640, 1]))) == ERR_STRIDE
    # extents of 1 may carry any stride (torch reports such strides freely)
    rc = _call_desc(_desc_args(q=(mla.ELEM_FP8_E4M3, [2, 1, 32, 576], [32 * 576, 12345, 576, 1]),
                               out=(mla.ELEM_BF16, [2, 1, 32, 512], [32 * 512, 7, 512, 1]),
                               lse=(mla.ELEM_FP32, [2, 1, 32], [32, 3, 1])))
    assert rc not in (ERR_STRIDE, -3, -2, -1)


def test_descriptor_types_and_extents_are_checked():
    assert _call_desc(_desc_args(kv=(mla.ELEM_BF16, [100, 64, 576]))) == -2  # fp8 q over a bf16 cache
    assert _call_desc(_desc_args(bt=(mla.ELEM_FP32, [2, 10]))) == -2
    assert _call_desc(_desc_args(out=(mla.ELEM_FP32, [2, 4, 32, 512]))) == -2
    assert _call_desc(_desc_args(q=(mla.ELEM_FP8_E4M3, [2, 4, 32, 512]))) == -3
    assert _call_desc(_desc_args(bt=(mla.ELEM_INT32, [3, 10]))) == -3
    assert _call_desc(_desc_args(out=(mla.ELEM_BF16, [2, 4, 16, 512]))) == -3
    assert _call_desc(_desc_args(lse=(mla.ELEM_FP32, [2, 4]))) == -3
    a = _desc_args()
    a["q"] = None
    assert _call_desc(a) == -1
    a = _desc_args()
    a["sl"].data = None
    assert _call_desc(a) == -1
    # the mixed pair and a NULL lse pass the descriptor checks (then the device is queried)
    a = _desc_args(q=(mla.ELEM_BF16, [2, 4, 32, 576]))
    a["lse"] = None
    assert _call_desc(a) not in (-1, -2, -3, -9)
    # sizes the plain entry point validates are still validated (max_seq_len > max_pages * page_size)
    assert _call_desc(_desc_args(), max_seq_len=641) == -3


def test_descriptor_layouts_match_header():
    text = open(HEADER).read()
    for name, cls in (("mla_tensor", mla.MlaTensor), ("mla_workspace", mla.MlaWorkspace)):
        body = text[text.index(f"typedef struct {name}"):text.index(f"}} {name};")]
        fields = re.findall(r"(int32_t|int64_t|size_t|void\*)\s+(\w+)(\[\d+\])?;", body)
        assert [f[1] for f in fields] == [f[0] for f in cls._fields_], name
    assert ctypes.sizeof(mla.MlaTensor) == 8 + 4 + 4 + 32 + 32
    assert ctypes.sizeof(mla.MlaWorkspace) == 8 + 8 + 4 + 4


def test_stream_probe_library_exports_its_entry_point():
    """The HBM -> LDS streaming probe bench.py measures the achievable read rate with is built beside the
    library and exports its one C entry point; its argument checks run without a GPU."""
    import ctypes
    import os

    from mla_paged_kv_decode_amd import build as b

    if not os.path.exists(b.PROBE_LIB):
        pytest.skip("probe library not built here")
    L = ctypes.CDLL(b.PROBE_LIB)
    f = L.mla_stream_probe
    f.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    assert f(None, 1 << 20, 0, None) == -1          # no buffer
    assert f(16, 36864 - 1, 0, None) == -1          # less than one tile
    assert f(16, 1 << 20, -1, None) == -1           # negative workgroup count
