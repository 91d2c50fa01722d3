"""mla_decode_static (the entry point that allocates nothing) against mla_decode_ex with a
caller-owned workspace: two calls in a row through the C ABI, the second with a smaller input,
each bit-identical to the workspace path (same kernels, same plan) and within the oracle bars."""
import numpy as np
import pytest
import torch

import mla_inputs as mi
import mla_paged_kv_decode_amd as mla
from tests.gpu_util import assert_parity, run_oracle, to_dev

pytestmark = pytest.mark.gpu

STATIC_BYTES = 160 << 20


def _both(x, opts=None):
    q, kv, bt, sl = to_dev(x)
    B, ql, H = x.B, x.q_len, x.H
    ref_out, ref_lse = mla.decode(q, kv, bt, sl, x.softmax_scale, x.q_scale, x.kv_scale,
                                  max_seq_len=x.max_seq_len, opts=opts)
    out = torch.full((B, ql, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.full((B, ql, H), float("nan"), dtype=torch.float32, device="cuda:0")
    mla.decode_static(q, kv, bt, sl, x.softmax_scale, x.q_scale, x.kv_scale, max_seq_len=x.max_seq_len,
                      out=out, lse=lse, opts=opts)
    torch.cuda.synchronize()
    return ref_out, ref_lse, out, lse


def test_static_entry_matches_workspace_entry_twice():
    # first call: the B=4 agentic shape at a shorter length (many slices, the workgroup-per-row merge)
    x1 = mi.make_inputs(4, 4, 32, mi.FP8_E4M3, ("list", [9000, 70, 4100, 12000]), seed=901)
    print("call 1: B=4 q_len=4 H=32 fp8 lens [9000, 70, 4100, 12000]", flush=True)
    r1, rl1, o1, l1 = _both(x1)
    assert torch.equal(o1.view(torch.int16), r1.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), rl1.view(torch.int32))
    assert_parity(x1, o1, l1, run_oracle(x1))
    # second call, smaller: fewer sequences, bf16, the per-wave merge; the array keeps call 1's bytes
    x2 = mi.make_inputs(2, 1, 16, mi.BF16, ("list", [700, 33]), seed=902)
    print("call 2: B=2 q_len=1 H=16 bf16 lens [700, 33]", flush=True)
    r2, rl2, o2, l2 = _both(x2)
    assert torch.equal(o2.view(torch.int16), r2.view(torch.int16))
    assert torch.equal(l2.view(torch.int32), rl2.view(torch.int32))
    assert_parity(x2, o2, l2, run_oracle(x2))


def test_static_entry_rejects_plans_beyond_its_array():
    # a prefill-sized shape whose plan needs more than the static array: rejected before any launch
    B, q_len, H, L = 4, 512, 128, 16896
    ns, need = mla.plan(B, q_len, H, L)
    assert need > STATIC_BYTES
    q = torch.zeros(B, q_len, H, 576, dtype=torch.bfloat16, device="cuda:0")
    kv = torch.zeros(L // 64 + 1, 64, 576, dtype=torch.bfloat16, device="cuda:0")
    bt = torch.zeros(B, L // 64, dtype=torch.int32, device="cuda:0")
    sl = torch.full((B,), L, dtype=torch.int32, device="cuda:0")
    out = torch.empty(B, q_len, H, 512, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(mla.MlaError) as e:
        mla.decode_static(q, kv, bt, sl, 0.1, max_seq_len=L, out=out)
    assert e.value.code == -5 and "static scratch" in str(e.value)
