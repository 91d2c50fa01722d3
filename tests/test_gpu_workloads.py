"""Parity on the benchmark workloads at full size, in the launch configuration
bench.py times (default plan: planned split count, folded queries, bf16 partials).

Every output element of every workload -- every sequence, query token and head
-- is compared with the fp64 oracle run on the same bytes (16 threads), against
the flat bars (bf16 O max-abs <= 1e-2, FP8 O <= 5e-2, each on top of the
bf16 rounding of the result; LSE <= 1e-3) and the derived per-element bound.  The largest errors of each sequence are printed.
"""
import dataclasses
import time

import numpy as np
import pytest
import torch

import mla_inputs as mi
import mla_paged_kv_decode_amd as mla
import oracle
from tests.gpu_util import assert_parity, out_f64, to_dev, _torch_dtype

pytestmark = pytest.mark.gpu

ORACLE_THREADS = 16


@pytest.mark.parametrize("name", list(mi.WORKLOADS))
def test_workload_parity(name):
    t0 = time.time()
    x = mi.workload_inputs(name)
    print(f"  {name}: B={x.B} q_len={x.q_len} H={x.H} dtype={x.dtype} keys={int(x.seq_lens.sum())} "
          f"(inputs {time.time() - t0:.1f} s)", flush=True)
    q, kv, bt, sl = to_dev(x)
    out, lse = mla.decode(q, kv, bt, sl, x.softmax_scale, x.q_scale, x.kv_scale, max_seq_len=x.max_seq_len)
    torch.cuda.synchronize()
    O = out_f64(out)
    L = lse.cpu().numpy().astype(np.float64)
    del q, kv, out, lse
    # a token t of sequence b sees min(L_b - q_len + t + 1, L_b) keys; none -> zero row, LSE = -inf
    vis = np.minimum(x.seq_lens[:, None] - x.q_len + np.arange(x.q_len)[None, :] + 1, x.seq_lens[:, None])
    empty = vis <= 0
    assert np.array_equal(np.isneginf(L).all(axis=-1), empty)

    t1 = time.time()
    ref = oracle.mla_decode(x.q, x.kv_cache, x.block_table, x.seq_lens, dtype=x.dtype,
                            softmax_scale=x.softmax_scale, q_scale=x.q_scale, kv_scale=x.kv_scale,
                            want_absv=True, num_threads=ORACLE_THREADS)
    print(f"    oracle over all {x.B} sequences: {time.time() - t1:.1f} s", flush=True)
    assert_parity(x, torch.from_numpy(O), torch.from_numpy(L), ref, per_seq=True)


@pytest.mark.parametrize("name", list(mi.RAGGED_PREFILL))
def test_ragged_prefill_workload(name):
    """The ragged prefill workloads bench.py times, at full size through mla_decode_varlen: every
    sequence (every one of its new tokens and heads) against the fp64 oracle run on that sequence."""
    x, new = mi.ragged_prefill_inputs(name)
    qf = mi.q_format(x.dtype)
    q_pack = np.ascontiguousarray(np.concatenate([x.q[b, :n] for b, n in enumerate(new)], axis=0))
    raw = q_pack if q_pack.dtype == np.uint8 else q_pack.view(np.int16)
    q = torch.from_numpy(raw).to("cuda:0").view(_torch_dtype(qf))
    _, kv, bt, sl = to_dev(x)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(new)]).astype(np.int32), device="cuda:0")
    out, lse = mla.decode_varlen(q, cu, kv, bt, sl, x.softmax_scale, x.q_scale, x.kv_scale, max_q_len=max(new),
                                 max_seq_len=x.max_seq_len)
    torch.cuda.synchronize()
    O = out_f64(out)
    Lg = lse.cpu().numpy().astype(np.float64)
    for b in range(len(new)):
        t1 = time.time()
        sub = dataclasses.replace(x, q=np.ascontiguousarray(x.q[b:b + 1, :new[b]]),
                                  block_table=x.block_table[b:b + 1], seq_lens=x.seq_lens[b:b + 1])
        ref = oracle.mla_decode(sub.q, sub.kv_cache, sub.block_table, sub.seq_lens, dtype=x.dtype,
                                softmax_scale=x.softmax_scale, q_scale=x.q_scale, kv_scale=x.kv_scale,
                                want_absv=True, num_threads=ORACLE_THREADS)
        print(f"    {name}: sequence {b} ({new[b]} new tokens, L={int(x.seq_lens[b])}): oracle "
              f"{time.time() - t1:.1f} s", flush=True)
        r0 = int(np.sum(new[:b]))
        assert_parity(sub, torch.from_numpy(O[r0:r0 + new[b]][None]), torch.from_numpy(Lg[r0:r0 + new[b]][None]),
                      ref)
