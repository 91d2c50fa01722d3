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
        need = (ns + B) * rows * (512 * 2 + 4) + U * B * 8 + U * 8  # bf16 partials; slice ranges and T per row
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
    # mla_options: five int32 fields, three reserved int32, then a pointer at byte 32
    o = mla.MlaOptions
    assert [o.num_splits.offset, o.no_fold.offset, o.partial_fp32.offset, o.stages.offset, o.window.offset,
            o.reserved.offset, o.split_event.offset] == [0, 4, 8, 12, 16, 20, 32]
    assert ctypes.sizeof(o) == 40
    text = open(HEADER).read()
    body = text[text.index("typedef struct mla_options"):text.index("} mla_options;")]
    fields = re.findall(r"(int32_t|void\*)\s+(\w+)(\[\d+\])?;", body)
    assert [f[1] for f in fields] == ["num_splits", "no_fold", "partial_fp32", "stages", "window", "reserved",
                                      "split_event"]
    assert re.search(r"int32_t\s+reserved\[3\];", body)


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
