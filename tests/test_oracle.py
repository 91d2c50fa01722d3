"""Pins of the fp64 CPU oracle against things other than itself (CPU only).

* storage formats: every E4M3 code and random bf16 patterns against torch's
  conversions; the encoder against torch's round-to-nearest-even cast;
* the folding rule against the worked example the pages print
  (tests/golden/fold_examples.txt);
* the attention result against a dense scipy brute force on tiny shapes;
* closed forms: zero query => LSE = ln(n_t) and O = mean of the visible V rows
  (pins the causal alignment and the length handling per token), and the same
  with a sliding window (pins both ends of each token's window);
* invariants: split/merge at several chunk sizes, page relabelling, needles.
"""
import math
import os

import numpy as np
import pytest
import torch

import mla_inputs as mi
import oracle
from tests.brute import brute_decode, decode_values, dense_keys

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _run(x, **kw):
    return oracle.mla_decode(x.q, x.kv_cache, x.block_table, x.seq_lens, dtype=x.dtype,
                             softmax_scale=x.softmax_scale, q_scale=x.q_scale, kv_scale=x.kv_scale, **kw)


# ---------------------------------------------------------------- formats
def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_table()
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], got[fin])
    assert np.nanmax(got) == 448.0 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.dec_bf16(bits)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], got[fin])


def test_f16_table_matches_numpy():
    # every binary16 pattern, including subnormals, infinities and NaNs
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.f16_table()
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], got[fin])
    assert got[0x3C00] == 1.0 and got[0x0001] == 2.0 ** -24 and got[0x7BFF] == 65504.0 and np.isinf(got[0x7C00])


def test_e4m3_encoder_matches_torch_rne():
    table = oracle.e4m3_table()
    finite = [c for c in range(256) if not math.isnan(table[c])]
    # every finite code round-trips (both zeros keep their sign)
    assert list(oracle.enc_e4m3(table[finite])) == finite
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-448, 448, 3000), rng.normal(0, 0.02, 3000),
                        # exact midpoints between neighbouring codes: ties go to the even code
                        (table[0x01:0x7E] + table[0x02:0x7F]) / 2])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.enc_e4m3(x32.astype(np.float64))
    assert np.array_equal(ref, got)
    # saturation (the pack step clamps to +-448) and NaN
    assert list(oracle.enc_e4m3([500.0, -1e30, 449.0, float("inf"), float("nan")])) == [0x7E, 0xFE, 0x7E, 0x7E, 0x7F]


# ---------------------------------------------------------------- folding rule
def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(v) for v in line.split()])
    return rows


def test_fold_factor_worked_example():
    rows = _golden_rows("fold_examples.txt")
    assert rows
    for H, q_len, F, H_eff, q_len_eff in rows:
        f = oracle.fold_factor(q_len, H)
        assert f == F
        assert H * f == H_eff and q_len // f == q_len_eff


# ---------------------------------------------------------------- brute force
SHAPES = [
    # B, q_len, H, dtype, lens, page_size
    (1, 1, 4, mi.BF16, [5], 16),
    (2, 4, 3, mi.FP16, [3, 150], 16),
    (2, 4, 8, mi.FP8_E4M3, [3, 200], 16),
    (3, 4, 2, mi.BF16, [0, 4, 300], 64),
    (2, 3, 5, mi.FP8_E4M3, [1, 130], 64),
    (1, 2, 8, mi.BF16, [257], 1),
    (2, 4, 6, mi.BF16_Q_E4M3_KV, [3, 170], 16),  # bf16 q over an e4m3 cache
    (1, 3, 4, mi.BF16_Q_E4M3_KV, [129], 64),
]


@pytest.mark.parametrize("B,q_len,H,dtype,lens,ps", SHAPES)
def test_oracle_matches_dense_brute_force(B, q_len, H, dtype, lens, ps):
    x = mi.make_inputs(B, q_len, H, dtype, ("list", lens), page_size=ps, seed=11 + B + H)
    O, lse = _run(x)
    Ob, lseb = brute_decode(x)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lseb))
    fin = np.isfinite(lseb)
    assert np.allclose(lse[fin], lseb[fin], rtol=1e-12, atol=1e-12)
    assert np.allclose(O, Ob, rtol=1e-11, atol=1e-12)


def test_lse_is_plain_log_sum_exp():
    # small scores: the unshifted definition is safe in fp64
    x = mi.make_inputs(1, 2, 3, mi.BF16, ("list", [40]), page_size=16, seed=5)
    _, lse = _run(x)
    q = decode_values(x.q, x.dtype)
    K = dense_keys(decode_values(x.kv_cache, x.dtype), x.block_table, 0, 40)
    for t in range(2):
        n_t = 40 - 2 + t + 1
        s = x.softmax_scale * q[0, t] @ K[:n_t].T
        assert np.abs(s).max() < 30
        assert np.allclose(lse[0, t], np.log(np.exp(s).sum(axis=-1)), rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("lens,q_len", [([70, 2, 0, 129], 4), ([64], 1), ([3], 5)])
def test_zero_query_gives_log_count_and_mean(lens, q_len):
    x = mi.make_inputs(len(lens), q_len, 3, mi.BF16, ("list", lens), page_size=16, seed=9)
    x.q[:] = 0
    O, lse = _run(x)
    kv = decode_values(x.kv_cache, x.dtype)
    for b, L in enumerate(lens):
        K = dense_keys(kv, x.block_table, b, L)
        for t in range(q_len):
            n_t = min(max(L - q_len + t + 1, 0), L)
            if n_t == 0:
                assert np.all(np.isneginf(lse[b, t])) and np.all(O[b, t] == 0)
                continue
            assert np.allclose(lse[b, t], math.log(n_t), rtol=0, atol=1e-14)
            mean = K[:n_t, :512].mean(axis=0)
            assert np.allclose(O[b, t], mean[None, :], rtol=1e-13, atol=1e-14)


def test_alignment_pin_rejects_the_other_reading():
    # The zero-query closed form tells bottom-right from top-left alignment:
    # a mask planted with the other reading must disagree with the oracle.
    x = mi.make_inputs(1, 4, 2, mi.BF16, ("list", [50]), page_size=16, seed=2)
    x.q[:] = 0
    _, lse = _run(x)
    _, lse_tl = brute_decode(x, alignment="top_left")
    assert not np.allclose(lse, lse_tl)
    _, lse_br = brute_decode(x)
    assert np.allclose(lse, lse_br, atol=1e-13)


def test_single_visible_key_is_exact():
    x = mi.make_inputs(1, 1, 4, mi.FP8_E4M3, ("list", [1]), page_size=16, seed=4)
    O, lse = _run(x)
    q = decode_values(x.q, x.dtype) * x.q_scale
    k = decode_values(x.kv_cache, x.dtype)[x.block_table[0, 0], 0] * x.kv_scale
    assert np.array_equal(O[0, 0], np.broadcast_to(k[:512], (4, 512)))
    assert np.allclose(lse[0, 0], x.softmax_scale * q[0, 0] @ k, rtol=1e-14)


# ---------------------------------------------------------------- sliding window
WINDOW_SHAPES = [
    # B, q_len, H, dtype, lens, page_size, window
    (2, 4, 4, mi.FP8_E4M3, [3, 200], 16, 1),
    (3, 4, 2, mi.BF16, [0, 4, 300], 64, 5),
    (2, 3, 5, mi.FP8_E4M3, [1, 130], 64, 64),
    (1, 2, 8, mi.BF16, [257], 16, 100),
    (2, 1, 3, mi.FP8_E4M3, [40, 77], 16, 1000),
    (2, 4, 3, mi.FP16, [90, 7], 16, 30),
    (2, 4, 3, mi.BF16_Q_E4M3_KV, [60, 9], 16, 25),
]


@pytest.mark.parametrize("B,q_len,H,dtype,lens,ps,window", WINDOW_SHAPES)
def test_window_matches_dense_brute_force(B, q_len, H, dtype, lens, ps, window):
    x = mi.make_inputs(B, q_len, H, dtype, ("list", lens), page_size=ps, seed=61 + B + H)
    O, lse = _run(x, window=window)
    Ob, lseb = brute_decode(x, window=window)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lseb))
    fin = np.isfinite(lseb)
    assert np.allclose(lse[fin], lseb[fin], rtol=1e-12, atol=1e-12)
    assert np.allclose(O, Ob, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("window", [1, 3, 20, 64])
def test_window_zero_query_gives_log_count_and_mean(window):
    # constant scores: LSE = ln(#keys in the window), O = mean of exactly those V rows,
    # which pins both ends of every token's window
    lens, q_len = [70, 2, 0, 129], 4
    x = mi.make_inputs(len(lens), q_len, 3, mi.BF16, ("list", lens), page_size=16, seed=19)
    x.q[:] = 0
    O, lse = _run(x, window=window)
    kv = decode_values(x.kv_cache, x.dtype)
    for b, L in enumerate(lens):
        K = dense_keys(kv, x.block_table, b, L)
        for t in range(q_len):
            n_t = min(max(L - q_len + t + 1, 0), L)
            lo = max(0, n_t - window)
            if n_t == 0:
                assert np.all(np.isneginf(lse[b, t])) and np.all(O[b, t] == 0)
                continue
            assert np.allclose(lse[b, t], math.log(n_t - lo), rtol=0, atol=1e-14)
            assert np.allclose(O[b, t], K[lo:n_t, :512].mean(axis=0)[None, :], rtol=1e-13, atol=1e-14)


def test_window_of_one_is_the_diagonal_key():
    x = mi.make_inputs(2, 4, 3, mi.FP8_E4M3, ("list", [9, 300]), page_size=16, seed=23)
    O, lse = _run(x, window=1)
    q = decode_values(x.q, x.dtype) * x.q_scale
    kv = decode_values(x.kv_cache, x.dtype) * x.kv_scale
    for b, L in enumerate([9, 300]):
        K = dense_keys(kv, x.block_table, b, L)
        for t in range(4):
            j = L - 4 + t  # the only visible key
            assert np.array_equal(O[b, t], np.broadcast_to(K[j, :512], (3, 512)))
            assert np.allclose(lse[b, t], x.softmax_scale * q[b, t] @ K[j], rtol=1e-13)


def test_window_covering_every_key_changes_nothing():
    x = mi.make_inputs(3, 4, 4, mi.FP8_E4M3, ("list", [0, 90, 333]), page_size=16, seed=25)
    O, lse = _run(x)
    for window in (333, 334, 10 ** 6):
        Ow, lsew = _run(x, window=window)
        assert np.array_equal(O, Ow) and np.array_equal(lse, lsew)


@pytest.mark.parametrize("split_len", [1, 7, 64])
def test_window_split_merge_equals_unsplit(split_len):
    x = mi.make_inputs(3, 4, 4, mi.BF16, ("list", [0, 90, 333]), page_size=16, seed=27)
    O, lse = _run(x, window=50)
    Os, lses = _run(x, split_len=split_len, window=50)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lses))
    fin = np.isfinite(lse)
    assert np.allclose(lse[fin], lses[fin], rtol=1e-13, atol=1e-13)
    assert np.allclose(O, Os, rtol=1e-12, atol=1e-14)


def test_negative_window_is_rejected():
    x = mi.make_inputs(1, 1, 2, mi.BF16, ("list", [10]), page_size=16, seed=29)
    with pytest.raises(ValueError):
        _run(x, window=-1)


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("split_len", [1, 7, 64, 100000])
def test_split_merge_equals_unsplit(split_len):
    x = mi.make_inputs(3, 4, 4, mi.FP8_E4M3, ("list", [0, 90, 333]), page_size=16, seed=21)
    O, lse = _run(x)
    Os, lses = _run(x, split_len=split_len)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lses))
    fin = np.isfinite(lse)
    assert np.allclose(lse[fin], lses[fin], rtol=1e-13, atol=1e-13)
    assert np.allclose(O, Os, rtol=1e-12, atol=1e-14)


def test_page_relabelling_is_bit_identical():
    x = mi.make_inputs(2, 2, 4, mi.BF16, ("list", [100, 37]), page_size=16, seed=8)
    O, lse = _run(x)
    perm = np.random.default_rng(1).permutation(x.num_pages)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    kv2 = np.empty_like(x.kv_cache)
    kv2[inv] = x.kv_cache  # page p moves to inv[p]
    bt2 = inv[x.block_table].astype(np.int32)
    O2, lse2 = oracle.mla_decode(x.q, kv2, bt2, x.seq_lens, dtype=x.dtype, softmax_scale=x.softmax_scale,
                                 q_scale=x.q_scale, kv_scale=x.kv_scale)
    assert np.array_equal(O, O2) and np.array_equal(lse, lse2)


def test_needle_selects_one_row():
    B, q_len, H, L, ps = 1, 2, 4, 150, 16
    x = mi.make_inputs(B, q_len, H, mi.BF16, ("list", [L]), page_size=ps, seed=6)
    bits = lambda v: np.array([v], dtype=np.float32).view(np.uint32)[0] >> 16  # exact bf16 values
    x.q[:] = 0
    x.kv_cache[..., 3] = 0
    for t in range(q_len):
        for h in range(H):
            x.q[0, t, h, 3] = bits(1.0)
    j_star = 77
    x.kv_cache[x.block_table[0, j_star // ps], j_star % ps, 3] = bits(4096.0)
    O, _ = _run(x)
    kv = decode_values(x.kv_cache, x.dtype)
    v_star = kv[x.block_table[0, j_star // ps], j_star % ps, :512]
    for t in range(q_len):
        assert np.array_equal(O[0, t], np.broadcast_to(v_star, (H, 512)))


def test_out_of_range_page_is_reported():
    x = mi.make_inputs(1, 1, 2, mi.BF16, ("list", [40]), page_size=16, seed=1)
    x.block_table[0, 1] = x.num_pages + 5
    with pytest.raises(IndexError):
        _run(x)


# ---------------------------------------------------------------- pack + quantise
def test_kv_pack_quantize_matches_torch_cast():
    rng = np.random.default_rng(12)
    T = 37
    latent = torch.from_numpy(rng.normal(0, 3, (T, 512)).astype(np.float32)).to(torch.bfloat16)
    rope = torch.from_numpy(rng.normal(0, 3, (T, 64)).astype(np.float32)).to(torch.bfloat16)
    latent[0, :4] = torch.tensor([1e4, -1e4, float("nan"), 0.0])
    scale = 0.0173
    got = oracle.kv_pack_quantize_fp8(latent.view(torch.int16).numpy().view(np.uint16),
                                      rope.view(torch.int16).numpy().view(np.uint16), scale)
    cat = torch.cat([latent, rope], dim=1).float() / torch.tensor(scale, dtype=torch.float32)
    nan = torch.isnan(cat)
    ref = cat.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    ref[nan.numpy()] = 0x7F
    assert np.array_equal(got, ref)
    slots = np.array([5, -1] + list(range(7, 7 + T - 2)), dtype=np.int64)
    got2 = oracle.kv_pack_quantize_fp8(latent.view(torch.int16).numpy().view(np.uint16),
                                       rope.view(torch.int16).numpy().view(np.uint16), scale, slot_mapping=slots,
                                       num_rows=T + 10)
    assert np.array_equal(got2[5], ref[0]) and np.array_equal(got2[7:7 + T - 2], ref[2:])
    assert not got2[6].any()


def test_weighted_abs_v_matches_brute_force():
    x = mi.make_inputs(2, 4, 3, mi.FP8_E4M3, ("list", [33, 140]), page_size=16, seed=14)
    O, lse, absv = _run(x, want_absv=True)
    q = decode_values(x.q, x.dtype) * x.q_scale
    kv = decode_values(x.kv_cache, x.dtype) * x.kv_scale
    for b, L in enumerate([33, 140]):
        K = dense_keys(kv, x.block_table, b, L)
        for t in range(4):
            n_t = L - 4 + t + 1
            s = x.softmax_scale * q[b, t] @ K[:n_t].T
            w = np.exp(s - s.max(axis=-1, keepdims=True))
            w /= w.sum(axis=-1, keepdims=True)
            assert np.allclose(absv[b, t], w @ np.abs(K[:n_t, :512]), rtol=1e-12, atol=1e-15)
    assert np.all(absv >= np.abs(O) - 1e-12)
