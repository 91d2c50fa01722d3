"""Helpers for the GPU tests: upload seeded inputs, run the HIP path, compare with the oracle."""
import numpy as np
import torch

import mla_inputs as mi
import mla_paged_kv_decode_amd as mla
import oracle

# Flat bars of the headline workloads: bf16 O max-abs <= 1e-2, FP8 O <= 5e-2, LSE <= 1e-3
# (fp16 inputs take the bf16 bar: their PV operands round more finely).

BF16_O_TOL = 1e-2
FP8_O_TOL = 5e-2
LSE_TOL = 1e-3
# Element-wise bound derived from the arithmetic (any input).  The softmax weights are
# rounded to the PV operand format before the MFMA: unit roundoff u_P = 2^-8 for bf16
# (8-bit significand), 2^-11 for fp16 (11-bit), 2^-4 for E4M3 (4-bit significand; the
# per-row power-of-two scale keeps them normal), which moves O by at most
# u_P * sum_j w_j |V_j|.  The
# result is rounded to bf16 (u = 2^-8 of the pre-rounding value).  A small absolute
# slack covers fp32 accumulation order, exp2 and flushed fp8 subnormals.
P_ROUND = {mi.BF16: 2.0 ** -8, mi.FP8_E4M3: 2.0 ** -4, mi.FP16: 2.0 ** -11, mi.BF16_Q_E4M3_KV: 2.0 ** -8}
U_OUT = 2.0 ** -8
SLACK = 2e-4


def o_tol(dtype):
    # an E4M3 cache (with either q) takes the FP8 bar
    return FP8_O_TOL if mi.kv_format(dtype) == mi.FP8_E4M3 else BF16_O_TOL


def _torch_dtype(fmt):
    return {mi.BF16: torch.bfloat16, mi.FP16: torch.float16}.get(fmt, torch.float8_e4m3fn)


def to_dev(x: "mi.DecodeInputs", dev="cuda:0"):
    qf, kvf = mi.q_format(x.dtype), mi.kv_format(x.dtype)
    raw_q = x.q if qf == mi.FP8_E4M3 else x.q.view(np.int16)
    raw_kv = x.kv_cache if kvf == mi.FP8_E4M3 else x.kv_cache.view(np.int16)
    q = torch.from_numpy(np.ascontiguousarray(raw_q)).to(dev).view(_torch_dtype(qf))
    kv = torch.from_numpy(np.ascontiguousarray(raw_kv)).to(dev).view(_torch_dtype(kvf))
    bt = torch.from_numpy(np.ascontiguousarray(x.block_table)).to(dev)
    sl = torch.from_numpy(np.ascontiguousarray(x.seq_lens)).to(dev)
    return q, kv, bt, sl


def run_gpu(x, opts=None, dev="cuda:0", tensors=None):
    q, kv, bt, sl = tensors if tensors is not None else to_dev(x, dev)
    out, lse = mla.decode(q, kv, bt, sl, x.softmax_scale, x.q_scale, x.kv_scale, max_seq_len=x.max_seq_len,
                          opts=opts)
    torch.cuda.synchronize()
    return out, lse


def out_f64(out):
    return out.float().cpu().numpy().astype(np.float64)


def run_oracle(x, **kw):
    """(O, LSE, sum_j w_j |V_j|) from the fp64 oracle."""
    return oracle.mla_decode(x.q, x.kv_cache, x.block_table, x.seq_lens, dtype=x.dtype,
                             softmax_scale=x.softmax_scale, q_scale=x.q_scale, kv_scale=x.kv_scale, want_absv=True,
                             **kw)


def assert_parity(x, out, lse, ref, flat=False, rows=None, partial_fp32=False):
    """Element-wise parity with the oracle.

    Always: rows with no visible key are exact zeros / -inf, LSE within 1e-3,
    and |dO| within the derived bound.  flat=True also enforces the flat
    headline bars (used on the benchmark workloads).
    """
    O_ref, lse_ref, absv = ref
    O = out_f64(out)
    L = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        O, L, O_ref, lse_ref, absv = O[rows], L[rows], O_ref[rows], lse_ref[rows], absv[rows]
    assert np.all(np.isfinite(O)), "non-finite output"
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(L), empty), "rows without visible keys differ"
    assert np.all(O[empty] == 0)
    err = np.abs(O - O_ref)
    pre = P_ROUND[x.dtype] * absv
    bound = pre + U_OUT * (np.abs(O_ref) + pre) + SLACK
    if not partial_fp32:  # split partials are rounded to bf16 before the merge
        bound += U_OUT * absv
    o_err = float(err.max()) if err.size else 0.0
    fin = ~empty
    l_err = float(np.max(np.abs(L[fin] - lse_ref[fin]))) if fin.any() else 0.0
    worst = float((err / bound).max()) if err.size else 0.0
    print(f"    max|dO|={o_err:.3e} max|dLSE|={l_err:.3e} worst dO/bound={worst:.3f}", flush=True)
    assert l_err <= LSE_TOL, f"max|dLSE| = {l_err}"
    assert worst <= 1.0, f"|dO| exceeds the derived bound by {worst:.3f}x (max|dO| = {o_err})"
    if flat:
        assert o_err <= o_tol(x.dtype), f"max|dO| = {o_err}"
    return o_err, l_err
