"""GPU parity of the HIP decode path against the fp64 oracle (needs an MI355X).

Tolerances: bf16 O max-abs <= 1e-2 and FP8 O <= 5e-2 (the oracle runs on the
dequantised FP8 values), each beyond the bf16 rounding of the result; LSE <=
1e-3.  Index handling (paging, masking, needles, page relabelling) is checked
bit-exactly.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import mla_inputs as mi
import mla_paged_kv_decode_amd as mla
from tests.gpu_util import assert_parity, out_f64, run_gpu, run_oracle, to_dev

pytestmark = pytest.mark.gpu

# (B, q_len, H, dtype, lens, page_size): several tiles, ragged tails, every fold shape
CASES = [
    (1, 1, 16, mi.BF16, [256], 64),
    (3, 4, 32, mi.FP8_E4M3, [0, 77, 1000], 64),
    (3, 4, 32, mi.BF16, [5, 700, 64], 64),
    (2, 1, 128, mi.BF16, [4096, 300], 64),
    (2, 1, 128, mi.FP8_E4M3, [2113, 63], 64),
    (2, 4, 64, mi.FP8_E4M3, [2000, 64], 64),
    (2, 4, 64, mi.BF16, [1500, 3], 64),
    (4, 2, 16, mi.FP8_E4M3, [1, 2, 3, 130], 16),
    (4, 2, 16, mi.BF16, [1, 2, 3, 130], 16),
    (1, 3, 40, mi.FP8_E4M3, [901], 32),
    (1, 3, 40, mi.BF16, [901], 32),
    (2, 1, 256, mi.FP8_E4M3, [700, 1200], 128),
    (2, 2, 8, mi.BF16, [333, 2], 256),
    (1, 5, 24, mi.FP8_E4M3, [600], 64),
]


@pytest.mark.parametrize("B,q_len,H,dtype,lens,ps", CASES)
def test_parity_small(B, q_len, H, dtype, lens, ps):
    x = mi.make_inputs(B, q_len, H, dtype, ("list", lens), page_size=ps, seed=100 + B * 7 + H + ps)
    print(f"case B={B} q_len={q_len} H={H} dtype={dtype} lens={lens} ps={ps}", flush=True)
    out, lse = run_gpu(x)
    assert_parity(x, out, lse, run_oracle(x))


@pytest.mark.parametrize("dtype", [mi.BF16, mi.FP8_E4M3, mi.BF16_Q_E4M3_KV])
@pytest.mark.parametrize("splits", [1, 2, 3, 8, 64, 200])
def test_forced_splits(dtype, splits):
    x = mi.make_inputs(3, 4, 32, dtype, ("list", [2500, 90, 1300]), seed=31)
    print(f"splits={splits} dtype={dtype}", flush=True)
    out, lse = run_gpu(x, opts=mla.options(num_splits=splits))
    assert_parity(x, out, lse, run_oracle(x))


FP8_CASES = [c for c in CASES if c[3] == mi.FP8_E4M3]


@pytest.mark.parametrize("B,q_len,H,dtype,lens,ps", FP8_CASES)
def test_four_wave_fp8_kernel_parity(B, q_len, H, dtype, lens, ps):
    """Both E4M3 split-KV kernels, forced: the four-wave one (the default on pages of at least one
    tile without a window; here also on 16- and 32-key pages, where it runs without the second P
    term) and the twelve-wave one."""
    x = mi.make_inputs(B, q_len, H, dtype, ("list", lens), page_size=ps, seed=100 + B * 7 + H + ps)
    print(f"kernel=1 B={B} q_len={q_len} H={H} lens={lens} ps={ps}", flush=True)
    ref = run_oracle(x)
    out1, lse1 = run_gpu(x, opts=mla.options(kernel=1))
    assert_parity(x, out1, lse1, ref)
    out2, lse2 = run_gpu(x, opts=mla.options(kernel=2))
    assert_parity(x, out2, lse2, ref)


@pytest.mark.parametrize("dtype", [mi.BF16, mi.FP8_E4M3])
@pytest.mark.parametrize("splits", [5, 64, 200])
def test_four_wave_fp8_kernel_forced_splits(dtype, splits):
    x = mi.make_inputs(3, 4, 32, dtype, ("list", [2500, 90, 1300]), seed=31)
    print(f"kernel=1 splits={splits} dtype={dtype}", flush=True)
    out, lse = run_gpu(x, opts=mla.options(num_splits=splits, kernel=1))
    assert_parity(x, out, lse, run_oracle(x))


@pytest.mark.parametrize("dtype", [mi.BF16, mi.FP8_E4M3])
@pytest.mark.parametrize("partial_fp32", [False, True])
def test_both_merge_kernels(dtype, partial_fp32):
    """The wide merge (default), the workgroup-per-row merge and the per-wave merge, on rows spread
    over many slices (ragged, with empty slices; more than a chunk of the per-wave merge): all within
    the bars, and the same up to summation order."""
    x = mi.make_inputs(2, 2, 64, dtype, ("list", [9000, 37]), seed=77)
    print(f"merge dtype={dtype} partial_fp32={partial_fp32}", flush=True)
    ref = run_oracle(x)
    res = []
    for merge in (0, 1, 2):
        out, lse = run_gpu(x, opts=mla.options(num_splits=150, partial_fp32=partial_fp32, merge=merge))
        assert_parity(x, out, lse, ref, partial_fp32=partial_fp32)
        res.append((out.float(), lse))
    for k in (1, 2):
        assert float((res[0][0] - res[k][0]).abs().max()) <= 2.0 ** -7
        assert float((res[0][1] - res[k][1]).abs().max()) <= 1e-5


# The per-wave merge takes its rows' slices in chunks sized by the average slices per row
# (bf16 partials: 16 when G >= 7B, 8 when G >= 2B, else 4; fp32: 8 or 4); a long sequence among
# short ones spans more slices than a chunk, so its rows take several chunks.
PER_WAVE_MERGE_CASES = [
    (2, 24, [3000, 2500]),                                        # 16 (fp32: 8)
    (4, 16, [5000, 300, 900, 1200]),                              # 8
    (8, 8, [6000, 100, 200, 50, 300, 10, 400, 20]),              # 4
]


@pytest.mark.parametrize("dtype", [mi.BF16, mi.FP8_E4M3])
@pytest.mark.parametrize("partial_fp32", [False, True])
@pytest.mark.parametrize("B,splits,lens", PER_WAVE_MERGE_CASES)
def test_per_wave_merge_chunks(dtype, partial_fp32, B, splits, lens):
    x = mi.make_inputs(B, 1, 16, dtype, ("list", lens), seed=900 + B + splits)
    print(f"per-wave merge dtype={dtype} partial_fp32={partial_fp32} B={B} splits={splits} lens={lens}", flush=True)
    out, lse = run_gpu(x, opts=mla.options(num_splits=splits, partial_fp32=partial_fp32))
    assert_parity(x, out, lse, run_oracle(x), partial_fp32=partial_fp32)


@pytest.mark.parametrize("dtype", [mi.BF16, mi.FP8_E4M3, mi.BF16_Q_E4M3_KV])
def test_fold_and_partial_precision_options(dtype):
    x = mi.make_inputs(2, 4, 16, dtype, ("list", [1800, 650]), seed=41)
    ref = run_oracle(x)
    planned, lse_0 = run_gpu(x)
    base, lse_b = run_gpu(x, opts=mla.options(num_splits=24))
    nofold, lse_n = run_gpu(x, opts=mla.options(no_fold=True, num_splits=24))
    pf32, lse_p = run_gpu(x, opts=mla.options(partial_fp32=True, num_splits=16))
    assert_parity(x, planned, lse_0, ref)
    assert_parity(x, base, lse_b, ref)
    assert_parity(x, nofold, lse_n, ref)
    assert_parity(x, pf32, lse_p, ref, partial_fp32=True)
    # folding only re-indexes rows: with the same split count (the plan's differs, since the
    # unfolded query groups need more workgroups per slice), identical per-row arithmetic
    assert torch.equal(base, nofold) and torch.equal(lse_b, lse_n)


@pytest.mark.parametrize("dtype", [mi.BF16, mi.FP8_E4M3, mi.BF16_Q_E4M3_KV])
def test_needles_are_bit_exact(dtype):
    """One-hot queries pick exactly one visible key; a masked needle just past the limit is ignored."""
    B, q_len, H, ps = 2, 4, 8, 64
    lens = [300, 1025]
    x = mi.make_inputs(B, q_len, H, dtype, ("list", lens), page_size=ps, seed=51)
    x.softmax_scale, x.q_scale, x.kv_scale = 1.0, 1.0, 1.0
    q16, kv16 = mi.q_format(dtype) == mi.BF16, mi.kv_format(dtype) == mi.BF16
    one = np.uint16(0x3F80) if q16 else np.uint8(0x38)      # 1.0
    big = np.uint16(0x4400) if kv16 else np.uint8(0x7E)     # 512.0 / 448.0
    bigger = np.uint16(0x4480) if kv16 else np.uint8(0x7E)  # masked needle at least as large
    x.q[:] = 0
    expected = {}
    dims = [(t * H + h) % 576 for t in range(q_len) for h in range(H)]
    for b in range(B):
        L = lens[b]
        for t in range(q_len):
            for h in range(H):
                x.q[b, t, h, (t * H + h) % 576] = one
        # the needle dims are zero in every visible row of the sequence
        pg = x.block_table[b, np.arange(L) // ps]
        sl = np.arange(L) % ps
        for d in dims:
            x.kv_cache[pg, sl, d] = 0
    for b in range(B):
        L = lens[b]
        for t in range(q_len):
            n_t = L - q_len + t + 1
            for h in range(H):
                d = (t * H + h) % 576
                # needle positions: start, a page boundary, the diagonal (last visible key)
                j_star = [0, min(ps, n_t - 1), n_t - 1][(b + t + h) % 3]
                x.kv_cache[x.block_table[b, j_star // ps], j_star % ps, d] = big
                if n_t < L:  # a needle at least as large just past this token's limit must not be seen
                    x.kv_cache[x.block_table[b, n_t // ps], n_t % ps, d] = bigger
                expected[(b, t, h)] = j_star
    out, lse = run_gpu(x)
    O = out.cpu()
    kv_t = torch.from_numpy(x.kv_cache.view(np.int16) if kv16 else x.kv_cache)
    kv_t = kv_t.view(torch.bfloat16 if kv16 else torch.float8_e4m3fn)
    for (b, t, h), j in expected.items():
        v = kv_t[x.block_table[b, j // ps], j % ps, :512].float().to(torch.bfloat16)
        assert torch.equal(O[b, t, h], v), (b, t, h, j)


@pytest.mark.parametrize("dtype", [mi.BF16, mi.FP8_E4M3, mi.BF16_Q_E4M3_KV])
def test_page_relabelling_bit_identical(dtype):
    x = mi.make_inputs(3, 2, 32, dtype, ("list", [3000, 129, 2048]), seed=61)
    out, lse = run_gpu(x)
    perm = np.random.default_rng(2).permutation(x.num_pages)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    x2 = mi.DecodeInputs(**{**x.__dict__})
    x2.kv_cache = np.empty_like(x.kv_cache)
    x2.kv_cache[inv] = x.kv_cache
    x2.block_table = inv[x.block_table].astype(np.int32)
    out2, lse2 = run_gpu(x2)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("dtype", [mi.BF16, mi.FP8_E4M3, mi.BF16_Q_E4M3_KV])
def test_nan_poisoned_tails_and_spares_are_never_read(dtype):
    x = mi.make_inputs(3, 4, 16, dtype, ("list", [70, 1, 1000]), page_size=64, seed=71, poison_tail=True)
    out, lse = run_gpu(x)
    assert_parity(x, out, lse, run_oracle(x))


def test_zero_length_sequences_and_short_sequences():
    x = mi.make_inputs(4, 4, 16, mi.FP8_E4M3, ("list", [0, 1, 3, 0]), page_size=16, seed=81)
    out, lse = run_gpu(x)
    assert_parity(x, out, lse, run_oracle(x))
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))


def test_output_guards_untouched():
    x = mi.make_inputs(2, 4, 32, mi.BF16, ("list", [900, 40]), seed=91)
    q, kv, bt, sl = to_dev(x)
    B, ql, H = 2, 4, 32
    guard = 7
    out_buf = torch.full((B * ql * H * 512 + 2 * guard,), 12345.0, dtype=torch.bfloat16, device="cuda:0")
    lse_buf = torch.full((B * ql * H + 2 * guard,), -777.0, dtype=torch.float32, device="cuda:0")
    # 16-byte aligned interior views
    out = out_buf[8:8 + B * ql * H * 512].view(B, ql, H, 512)
    lse = lse_buf[guard:guard + B * ql * H].view(B, ql, H)
    ns, ws = mla.plan(B, ql, H, x.max_seq_len)
    ws_buf = torch.full((ws + 4096,), 0xA5, dtype=torch.uint8, device="cuda:0")
    mla.decode(q, kv, bt, sl, x.softmax_scale, x.q_scale, x.kv_scale, max_seq_len=x.max_seq_len, out=out, lse=lse,
               workspace=ws_buf[:ws] if ws else ws_buf[:1])
    torch.cuda.synchronize()
    assert torch.all(out_buf[:8] == 12345.0) and torch.all(out_buf[8 + B * ql * H * 512:] == 12345.0)
    assert torch.all(lse_buf[:guard] == -777.0) and torch.all(lse_buf[guard + B * ql * H:] == -777.0)
    if ws:
        assert torch.all(ws_buf[ws:] == 0xA5)
    assert_parity(x, out, lse, run_oracle(x))


def test_empty_batch_is_a_no_op():
    x = mi.make_inputs(1, 1, 16, mi.BF16, ("list", [64]), seed=3)
    q, kv, bt, sl = to_dev(x)
    out = torch.full((0, 1, 16, 512), 1.0, dtype=torch.bfloat16, device="cuda:0")
    mla.decode(q[:0], kv, bt[:0], sl[:0], 1.0, max_seq_len=0, out=out)
    torch.cuda.synchronize()


def test_workspace_errors():
    x = mi.make_inputs(2, 4, 32, mi.BF16, ("list", [2000, 2000]), seed=4)
    q, kv, bt, sl = to_dev(x)
    ns, ws = mla.plan(2, 4, 32, 2000)
    assert ns > 1 and ws > 0
    small = torch.empty(ws - 256, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(mla.MlaError) as e:
        mla.decode(q, kv, bt, sl, 1.0, max_seq_len=2000, workspace=small)
    assert e.value.code == -5


@pytest.mark.parametrize("dtype", [mi.FP8_E4M3, mi.BF16, mi.FP16, mi.BF16_Q_E4M3_KV])
def test_hip_graph_replay_matches_eager(dtype):
    """Capture one decode, then replay it with new seq_lens / block_table contents."""
    # every block_table row holds valid pages for 2240 keys; replays use shorter lengths
    x = mi.make_inputs(3, 4, 32, dtype, ("list", [2240, 2240, 2240]), seed=111)
    q, kv, bt, sl = to_dev(x)
    max_len = 2240
    out = torch.empty(3, 4, 32, 512, dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty(3, 4, 32, dtype=torch.float32, device="cuda:0")
    _, ws = mla.plan(3, 4, 32, max_len)
    wsb = torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda:0")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mla.decode(q, kv, bt, sl, x.softmax_scale, x.q_scale, x.kv_scale, max_seq_len=max_len, out=out, lse=lse,
                   workspace=wsb)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mla.decode(q, kv, bt, sl, x.softmax_scale, x.q_scale, x.kv_scale, max_seq_len=max_len, out=out, lse=lse,
                   workspace=wsb)
    rng = np.random.default_rng(5)
    for rep in range(3):
        lens = rng.integers(1, 2241, size=3).astype(np.int32)
        sl.copy_(torch.from_numpy(lens))
        x.seq_lens = lens
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        eager_o, eager_l = mla.decode(q, kv, bt, sl, x.softmax_scale, x.q_scale, x.kv_scale, max_seq_len=max_len,
                                      workspace=wsb)
        torch.cuda.synchronize()
        ref = run_oracle(x)
        print(f"  rep {rep} lens {lens.tolist()}: eager", flush=True)
        assert_parity(x, eager_o, eager_l, ref)
        print(f"  rep {rep}: graph replay", flush=True)
        assert_parity(x, got_o, got_l, ref)
        assert torch.equal(got_o, eager_o) and torch.equal(got_l, eager_l), rep


def test_kv_pack_quantize_bit_exact():
    import oracle

    rng = np.random.default_rng(13)
    T = 333
    latent = torch.from_numpy(rng.normal(0, 4, (T, 512)).astype(np.float32)).to(torch.bfloat16)
    rope = torch.from_numpy(rng.normal(0, 4, (T, 64)).astype(np.float32)).to(torch.bfloat16)
    latent[0, :6] = torch.tensor([1e6, -1e6, float("nan"), float("inf"), -0.0, 1e-30])
    scale = 0.0123
    ref = oracle.kv_pack_quantize_fp8(latent.view(torch.int16).numpy().view(np.uint16),
                                      rope.view(torch.int16).numpy().view(np.uint16), scale)
    got = mla.kv_pack_quantize_fp8(latent.cuda(), rope.cuda(), scale)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref)
    # scattered into cache rows through a slot mapping (negative = skip)
    slots = torch.from_numpy(rng.permutation(T + 50)[:T].astype(np.int64))
    slots[3] = -1
    cache = torch.zeros(T + 50, 576, dtype=torch.uint8, device="cuda:0")
    mla.kv_pack_quantize_fp8(latent.cuda(), rope.cuda(), scale, slot_mapping=slots.cuda(), out=cache)
    ref2 = oracle.kv_pack_quantize_fp8(latent.view(torch.int16).numpy().view(np.uint16),
                                       rope.view(torch.int16).numpy().view(np.uint16), scale,
                                       slot_mapping=slots.numpy(), num_rows=T + 50)
    assert np.array_equal(cache.cpu().numpy(), ref2)


@pytest.mark.parametrize("scale", [0.0123, 1.0 / 3.0, 2.0 ** -5])
def test_kv_pack_quantize_every_bf16_input(scale):
    """Every bf16 bit pattern (NaNs, infinities, subnormals, ties included) through the pack kernel,
    bit-exact against the oracle's encoder."""
    import oracle

    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    T = -(-65536 // 576)
    flat = np.zeros(T * 576, dtype=np.uint16)
    flat[:65536] = bits
    rows = flat.reshape(T, 576)
    latent_bits, rope_bits = np.ascontiguousarray(rows[:, :512]), np.ascontiguousarray(rows[:, 512:])
    ref = oracle.kv_pack_quantize_fp8(latent_bits, rope_bits, scale)
    latent = torch.from_numpy(latent_bits.view(np.int16)).view(torch.bfloat16).cuda()
    rope = torch.from_numpy(rope_bits.view(np.int16)).view(torch.bfloat16).cuda()
    got = mla.kv_pack_quantize_fp8(latent, rope, scale)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref)


def test_packed_cache_feeds_decode():
    """Rows written by the pack kernel into a paged cache decode like the oracle says."""
    import oracle

    rng = np.random.default_rng(17)
    B, L, H, ps = 2, 500, 32, 64
    pages = (L + ps - 1) // ps
    num_pages = B * pages + 3
    T = B * L
    latent = torch.from_numpy(rng.normal(0, 1, (T, 512)).astype(np.float32)).to(torch.bfloat16)
    rope = torch.from_numpy(rng.normal(0, 1, (T, 64)).astype(np.float32)).to(torch.bfloat16)
    kv_scale = 4.0 / 448.0
    perm = rng.permutation(num_pages)[:B * pages].reshape(B, pages).astype(np.int32)
    slots = np.array([perm[b, j // ps] * ps + j % ps for b in range(B) for j in range(L)], dtype=np.int64)
    cache = torch.zeros(num_pages * ps, 576, dtype=torch.uint8, device="cuda:0")
    mla.kv_pack_quantize_fp8(latent.cuda(), rope.cuda(), kv_scale, slot_mapping=torch.from_numpy(slots).cuda(),
                             out=cache)
    q32 = rng.normal(0, 1, (B, 4, H, 576)).astype(np.float32)
    q_scale = float(np.abs(q32).max() / 448.0)
    qc = torch.from_numpy(q32 / q_scale).clamp(-448, 448).to(torch.float8_e4m3fn)
    x = mi.DecodeInputs(q=qc.view(torch.uint8).numpy(), kv_cache=cache.cpu().numpy().reshape(num_pages, ps, 576),
                        block_table=perm, seq_lens=np.full(B, L, np.int32), dtype=mi.FP8_E4M3, q_scale=q_scale,
                        kv_scale=kv_scale, softmax_scale=1 / math.sqrt(192), page_size=ps)
    out, lse = run_gpu(x)
    assert_parity(x, out, lse, run_oracle(x))


# (B, lens, slices): 96 slices for 3 sequences merge with a workgroup per row, 64 for 8 sequences
# with a wave per row (fewer than 16 slices per sequence)
EMPTY_SLICE_CASES = [(3, [700, 5, 130], 96), (8, [700, 5, 130, 64, 1, 250, 0, 90], 64)]


@pytest.mark.parametrize("dtype", [mi.BF16, mi.FP8_E4M3])
@pytest.mark.parametrize("B,lens,splits", EMPTY_SLICE_CASES)
def test_empty_slices_ignore_stale_workspace(dtype, B, lens, splits):
    """More KV slices than 64-key units: empty slices write nothing and the merge must skip them."""
    x = mi.make_inputs(B, 4, 32, dtype, ("list", lens), seed=121 + B)
    print(f"B={B} lens={lens} splits={splits} dtype={dtype}", flush=True)
    q, kv, bt, sl = to_dev(x)
    opts = mla.options(num_splits=splits)
    _, ws = mla.plan(B, 4, 32, x.max_seq_len, opts)
    wsb = torch.full((ws,), 0xFF, dtype=torch.uint8, device="cuda:0")  # NaN everywhere
    out, lse = mla.decode(q, kv, bt, sl, x.softmax_scale, x.q_scale, x.kv_scale, max_seq_len=x.max_seq_len,
                          workspace=wsb, opts=opts)
    torch.cuda.synchronize()
    assert_parity(x, out, lse, run_oracle(x))


def test_stages_split_then_merge_equals_one_call():
    """The split-KV kernel alone, then the merge alone on the same workspace, gives the one-call result bit-exactly."""
    x = mi.make_inputs(3, 4, 32, mi.FP8_E4M3, ("list", [900, 2000, 64]), seed=57)
    q, kv, bt, sl = to_dev(x)
    ns, wsb = mla.plan(x.B, x.q_len, x.H, x.max_seq_len)
    assert ns > 1
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda:0")
    o1, l1 = mla.decode(q, kv, bt, sl, x.softmax_scale, x.q_scale, x.kv_scale, max_seq_len=x.max_seq_len,
                        workspace=ws)
    ws2 = torch.full((wsb,), 0xFF, dtype=torch.uint8, device="cuda:0")
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    mla.decode(q, kv, bt, sl, x.softmax_scale, x.q_scale, x.kv_scale, max_seq_len=x.max_seq_len, out=o2, lse=l2,
               workspace=ws2, opts=mla.options(stages=1))
    mla.decode(q, kv, bt, sl, x.softmax_scale, x.q_scale, x.kv_scale, max_seq_len=x.max_seq_len, out=o2, lse=l2,
               workspace=ws2, opts=mla.options(stages=2))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


# ---------------------------------------------------------------- sliding window
# (B, q_len, H, dtype, lens, page_size, window): windows of one key, within a tile, a tile, many
# tiles; short pages take the kernels for pages below a tile
WINDOW_CASES = [
    (2, 4, 32, mi.FP8_E4M3, [2500, 700], 64, 1),
    (2, 4, 32, mi.BF16, [2500, 700], 64, 37),
    (3, 4, 16, mi.FP8_E4M3, [90, 1300, 5], 64, 64),
    (1, 1, 16, mi.BF16, [3000], 64, 500),
    (2, 4, 8, mi.FP8_E4M3, [1000, 333], 16, 200),
    (2, 2, 8, mi.BF16, [333, 2], 16, 100),
]


@pytest.mark.parametrize("B,q_len,H,dtype,lens,ps,window", WINDOW_CASES)
def test_window_parity(B, q_len, H, dtype, lens, ps, window):
    x = mi.make_inputs(B, q_len, H, dtype, ("list", lens), page_size=ps, seed=200 + B * 3 + H + window)
    print(f"window={window} B={B} q_len={q_len} H={H} dtype={dtype} lens={lens} ps={ps}", flush=True)
    out, lse = run_gpu(x, opts=mla.options(window=window))
    assert_parity(x, out, lse, run_oracle(x, window=window))


@pytest.mark.parametrize("dtype", [mi.BF16, mi.FP8_E4M3, mi.BF16_Q_E4M3_KV])
@pytest.mark.parametrize("splits", [1, 3, 64])
def test_window_forced_splits(dtype, splits):
    x = mi.make_inputs(3, 4, 32, dtype, ("list", [2500, 90, 1300]), seed=211)
    print(f"window=300 splits={splits} dtype={dtype}", flush=True)
    out, lse = run_gpu(x, opts=mla.options(window=300, num_splits=splits))
    assert_parity(x, out, lse, run_oracle(x, window=300))


@pytest.mark.parametrize("dtype", [mi.BF16, mi.FP8_E4M3])
def test_window_covering_every_key_is_bit_identical(dtype):
    """A window at least as long as every sequence selects the same keys and the same plan.  (E4M3
    runs the twelve-wave kernel both ways: by default a window selects it, and no window the
    four-wave one.)"""
    x = mi.make_inputs(3, 4, 32, dtype, ("list", [700, 5, 1300]), seed=213)
    t = to_dev(x)
    kernel = 2 if dtype == mi.FP8_E4M3 else 0
    base, lse_b = run_gpu(x, opts=mla.options(kernel=kernel), tensors=t)
    win, lse_w = run_gpu(x, opts=mla.options(window=1300, kernel=kernel), tensors=t)
    assert torch.equal(base, win) and torch.equal(lse_b, lse_w)


def test_window_full_size_agentic():
    """The 80K-key FP8 workload with a 4096-key window: only the window's pages are read; every
    sequence is compared with the oracle."""
    x = mi.workload_inputs("agentic_b4_q4_h32_fp8_80k")
    t = to_dev(x)
    out, lse = run_gpu(x, opts=mla.options(window=4096), tensors=t)
    assert_parity(x, out, lse, run_oracle(x, window=4096, num_threads=16), per_seq=True)


# ---------------------------------------------------------------- fp16 inputs
FP16_CASES = [
    # B, q_len, H, lens, page_size, options
    (3, 4, 32, [0, 77, 1000], 64, {}),
    (2, 1, 128, [4096, 300], 64, {}),
    (2, 4, 64, [1500, 3], 64, {"num_splits": 3}),
    (4, 2, 16, [1, 2, 3, 130], 16, {}),
    (3, 4, 32, [2500, 90, 1300], 64, {"num_splits": 64}),
    (2, 4, 32, [2500, 700], 64, {"window": 37}),
]


@pytest.mark.parametrize("B,q_len,H,lens,ps,kw", FP16_CASES)
def test_fp16_parity(B, q_len, H, lens, ps, kw):
    x = mi.make_inputs(B, q_len, H, mi.FP16, ("list", lens), page_size=ps, seed=300 + B * 5 + H + ps)
    print(f"fp16 B={B} q_len={q_len} H={H} lens={lens} ps={ps} {kw}", flush=True)
    out, lse = run_gpu(x, opts=mla.options(**kw) if kw else None)
    assert_parity(x, out, lse, run_oracle(x, window=kw.get("window", 0)))


# ---------------------------------------------------------------- a row max that outgrows its reference
# The kernels take each row's exponentials relative to a reference fixed at the row's first tile.  When
# a later tile's row max exceeds it by more than TAU log2 units (fp16: 15, so that P stays below 65504;
# other dtypes 32), the 16-bit kernels and the four-wave E4M3 kernel recompute the segment from the
# larger reference; the twelve-wave E4M3 kernel moves that row's reference at once and scales its sums
# and accumulators by the power of two between the two references.
TAU = {mi.FP8_E4M3: 32.0, mi.BF16: 32.0, mi.BF16_Q_E4M3_KV: 32.0, mi.FP16: 15.0}


def _decode_values(codes, fmt, scale):
    t = torch.from_numpy(codes.view(np.int16) if fmt != mi.FP8_E4M3 else codes)
    t = t.view({mi.BF16: torch.bfloat16, mi.FP16: torch.float16}.get(fmt, torch.float8_e4m3fn))
    return t.float().numpy().astype(np.float64) * scale


def _encode_values(v, fmt, scale):
    t = torch.from_numpy(np.ascontiguousarray(v / scale, dtype=np.float32))
    if fmt == mi.FP8_E4M3:
        assert float(t.abs().max()) <= 448.0
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return t.to(torch.bfloat16 if fmt == mi.BF16 else torch.float16).view(torch.int16).numpy().view(np.uint16)


def _late_outlier_inputs(dtype):
    """Two sequences whose queries share a direction, with a few keys far along it placed several
    tiles in (two of them past the causal limit of the first tokens): every row's max score grows by
    ~45-60 log2 units after its first tile."""
    lens = [512, 700]
    x = mi.make_inputs(2, 4, 32, dtype, ("list", lens), page_size=64, seed=331 + dtype)
    qf, kf = mi.q_format(dtype), mi.kv_format(dtype)
    rng = np.random.default_rng(17)
    q = _decode_values(x.q, qf, x.q_scale)
    base = rng.standard_normal((2, 576))
    q = 0.5 * q + 2.0 * base[:, None, None, :]
    if qf == mi.FP8_E4M3:
        x.q_scale = float(np.abs(q).max()) / 448.0
    x.q = _encode_values(q, qf, x.q_scale)
    planted = {0: [(200, 1.25), (260, 1.35), (333, 1.45), (450, 1.40)],
               1: [(300, 1.30), (640, 1.45), (698, 1.50), (699, 1.47)]}
    for b, keys in planted.items():
        for j, g in keys:
            row = g * np.sign(base[b]) + 0.5 * rng.standard_normal(576)  # their V parts differ
            row[:512] *= 0.4  # V stays O(1): the output's absolute error scales with |V|
            x.kv_cache[x.block_table[b, j // 64], j % 64] = _encode_values(row, kf, x.kv_scale)
    return x


@pytest.mark.parametrize("dtype,kernel", [(mi.FP8_E4M3, 2), (mi.FP8_E4M3, 1), (mi.BF16, 0),
                                          (mi.BF16_Q_E4M3_KV, 0), (mi.FP16, 0)])
def test_late_large_scores_move_the_reference(dtype, kernel):
    x = _late_outlier_inputs(dtype)
    # Worked out on the host: with one slice per sequence, each row's reference comes from its first
    # tile (keys 0..63 or 0..31, a subset of 0..63), and a later key exceeds it by more than TAU + 8.
    qv = _decode_values(x.q, mi.q_format(dtype), x.q_scale)
    kvv = _decode_values(x.kv_cache, mi.kv_format(dtype), x.kv_scale)
    for b in range(x.B):
        L = int(x.seq_lens[b])
        keys = kvv[x.block_table[b, np.arange(L) // 64], np.arange(L) % 64]
        s2 = np.einsum("thd,jd->thj", qv[b], keys) * x.softmax_scale / np.log(2.0)
        for t in range(x.q_len):
            n_t = L - x.q_len + t + 1
            gap = s2[t, :, :n_t].max(axis=-1) - s2[t, :, :64].max(axis=-1)
            assert gap.min() > TAU[dtype] + 8, (b, t, float(gap.min()))
    print(f"dtype={dtype}: every row's max grows past its first tile's by > {TAU[dtype] + 8} log2 units", flush=True)
    out, lse = run_gpu(x, opts=mla.options(num_splits=1, kernel=kernel))
    ref = run_oracle(x)
    assert_parity(x, out, lse, ref)
    # the result mixes several planted keys rather than copying the largest one
    top = kvv[x.block_table[0, 333 // 64], 333 % 64, :512]
    assert float(np.abs(ref[0][0, 0, 0] - top).max()) > 2e-2


# ---------------------------------------------------------------- bf16 q over an E4M3 cache
MIXED_CASES = [
    # B, q_len, H, lens, page_size, options
    (3, 4, 32, [0, 77, 1000], 64, {}),
    (2, 1, 128, [4096, 300], 64, {}),
    (2, 4, 64, [1500, 3], 64, {"num_splits": 3}),
    (4, 2, 16, [1, 2, 3, 130], 16, {}),  # pages shorter than a tile
    (1, 3, 40, [901], 32, {}),
    (3, 4, 32, [2500, 90, 1300], 64, {"num_splits": 64}),
    (2, 4, 32, [2500, 700], 64, {"window": 37}),
    (2, 2, 8, [333, 2], 256, {"partial_fp32": True, "num_splits": 5}),
    (1, 5, 24, [97], 64, {}),  # an odd number of 32-key halves
]


@pytest.mark.parametrize("B,q_len,H,lens,ps,kw", MIXED_CASES)
def test_bf16_q_fp8_cache_parity(B, q_len, H, lens, ps, kw):
    x = mi.make_inputs(B, q_len, H, mi.BF16_Q_E4M3_KV, ("list", lens), page_size=ps, seed=500 + B * 5 + H + ps)
    print(f"bf16 q / e4m3 cache B={B} q_len={q_len} H={H} lens={lens} ps={ps} {kw}", flush=True)
    out, lse = run_gpu(x, opts=mla.options(**kw) if kw else None)
    assert_parity(x, out, lse, run_oracle(x, window=kw.get("window", 0)),
                  partial_fp32=bool(kw.get("partial_fp32", False)))


def test_bf16_q_fp8_cache_every_code_widens_exactly():
    """Every finite E4M3 code, subnormals included, sits in each key row; each row of the
    query sees one key, so O must be that row's values exactly and LSE the one score,
    which a one-hot query makes the code's value (every cache dimension is covered)."""
    B, H = 5, 128
    x = mi.make_inputs(B, 1, H, mi.BF16_Q_E4M3_KV, ("list", [1] * B), page_size=64, seed=521)
    x.softmax_scale, x.q_scale, x.kv_scale = 1.0, 1.0, 1.0
    codes = (np.arange(576) % 256).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0  # the two NaN codes
    x.kv_cache[:] = codes
    x.q[:] = 0
    dims = {}
    for b in range(B):
        for h in range(H):
            d = (b * H + h) % 576
            x.q[b, 0, h, d] = 0x3F80  # bf16 1.0
            dims[(b, h)] = d
    out, lse = run_gpu(x)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn)
    v_expect = vals[:512].to(torch.bfloat16)
    O = out.cpu()
    L = lse.cpu().numpy().astype(np.float64)
    for (b, h), d in dims.items():
        assert torch.equal(O[b, 0, h], v_expect), (b, h)
        assert abs(L[b, 0, h] - float(vals[d].float())) <= 1e-6 * max(1.0, abs(float(vals[d].float()))), (b, h, d)


# ---------------------------------------------------------------- fewer than 128 folded rows (16-bit paths
# then spread PV over all four waves, the fp8 path always does)
@pytest.mark.parametrize("dtype", [mi.BF16, mi.FP16, mi.BF16_Q_E4M3_KV, mi.FP8_E4M3])
@pytest.mark.parametrize("H,kw", [(16, {}), (40, {"window": 90}), (96, {"num_splits": 7}), (64, {"no_fold": True})])
def test_partial_row_tiles(dtype, H, kw):
    x = mi.make_inputs(3, 1, H, dtype, ("list", [1500, 33, 700]), page_size=64, seed=600 + H)
    print(f"dtype={dtype} H={H} {kw}", flush=True)
    out, lse = run_gpu(x, opts=mla.options(**kw) if kw else None)
    assert_parity(x, out, lse, run_oracle(x, window=kw.get("window", 0)))


# ---------------------------------------------------------------- large batches, long pages, short plans
@pytest.mark.parametrize("dtype", [mi.BF16, mi.FP8_E4M3, mi.BF16_Q_E4M3_KV])
@pytest.mark.parametrize("splits", [0, 37])
def test_large_batch_with_empty_and_short_sequences(dtype, splits):
    """300 sequences (several per lane of the workgroups' prefix sum), zeros and lengths below q_len
    included; the planned split and a forced odd one."""
    rng = np.random.default_rng(401)
    lens = rng.integers(0, 600, size=300)
    lens[::17] = 0
    lens[5::23] = 1
    x = mi.make_inputs(300, 2, 16, dtype, ("list", lens.tolist()), seed=402)
    print(f"B=300 splits={splits} dtype={dtype} keys={int(lens.sum())}", flush=True)
    out, lse = run_gpu(x, opts=mla.options(num_splits=splits) if splits else None)
    assert_parity(x, out, lse, run_oracle(x))


@pytest.mark.parametrize("dtype", [mi.BF16, mi.FP8_E4M3, mi.BF16_Q_E4M3_KV])
def test_pages_of_many_tiles(dtype):
    x = mi.make_inputs(2, 4, 32, dtype, ("list", [3000, 1100]), page_size=1024, seed=403)
    out, lse = run_gpu(x)
    assert_parity(x, out, lse, run_oracle(x))


def test_lengths_above_the_planned_maximum():
    """A sequence longer than the max_seq_len the plan was made for is still decoded correctly
    (only the balance of the split suffers)."""
    x = mi.make_inputs(3, 4, 32, mi.FP8_E4M3, ("list", [1000, 50, 2500]), seed=404)
    q, kv, bt, sl = to_dev(x)
    out, lse = mla.decode(q, kv, bt, sl, x.softmax_scale, x.q_scale, x.kv_scale, max_seq_len=100)
    torch.cuda.synchronize()
    assert_parity(x, out, lse, run_oracle(x))


# ---------------------------------------------------------------- many new tokens per sequence (prefill-sized q_len)
@pytest.mark.parametrize("dtype", [mi.BF16, mi.FP8_E4M3])
@pytest.mark.parametrize("B,q_len,H,lens", [(2, 96, 16, [700, 300]), (1, 256, 8, [1024]), (2, 60, 32, [60, 2000]),
                                             (2, 264, 16, [300, 264]),  # 33 workgroup rows: the many-rows plan
                                             (2, 20, 256, [150, 300])])  # 20 groups x 2 row tiles = 40 rows
def test_prefill_sized_query_counts(dtype, B, q_len, H, lens):
    """q_len in the hundreds: the causal mask runs across the new tokens, folded groups stream
    only the keys they can see (sequences as long as q_len see no cached prefix at all)."""
    x = mi.make_inputs(B, q_len, H, dtype, ("list", lens), page_size=64, seed=700 + q_len + H)
    print(f"dtype={dtype} B={B} q_len={q_len} H={H} lens={lens}", flush=True)
    out, lse = run_gpu(x)
    assert_parity(x, out, lse, run_oracle(x))


# ---------------------------------------------------------------- ragged batches: each sequence its own query count
def _ragged(x, q_lens, dev="cuda:0"):
    """Sequence b keeps the first q_lens[b] of the max(q_lens) query tokens drawn for it; returns
    the packed device tensors and the fp64 reference, one oracle call per sequence."""
    from tests.gpu_util import _torch_dtype
    qf = mi.q_format(x.dtype)
    rows = [x.q[b, :ql] for b, ql in enumerate(q_lens)]
    q_pack = np.ascontiguousarray(np.concatenate(rows, axis=0))  # [total_q, H, 576]
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    raw = q_pack if qf == mi.FP8_E4M3 else q_pack.view(np.int16)
    q = torch.from_numpy(raw).to(dev).view(_torch_dtype(qf))
    O, L, A = [], [], []
    for b, ql in enumerate(q_lens):
        if ql == 0:
            continue
        sub = dataclasses.replace(x, q=np.ascontiguousarray(x.q[b:b + 1, :ql]), block_table=x.block_table[b:b + 1],
                                  seq_lens=x.seq_lens[b:b + 1])
        o, l, a = run_oracle(sub, window=0)
        O.append(o[0]), L.append(l[0]), A.append(a[0])
    H = x.q.shape[2]
    ref = tuple(np.concatenate(v, axis=0) if v else np.zeros((0, H, 512) if i != 1 else (0, H))
                for i, v in enumerate((O, L, A)))
    return q, torch.from_numpy(cu).to(dev), ref


RAGGED_CASES = [
    # dtype, H, q_lens, lens, options
    (mi.BF16, 16, [1, 7, 0, 33], [300, 7, 40, 2000], {}),
    (mi.FP8_E4M3, 32, [4, 1, 3, 4], [81920 // 64, 100, 2, 700], {}),
    (mi.BF16_Q_E4M3_KV, 16, [12, 5, 1], [900, 5, 3000], {"num_splits": 40}),
    (mi.FP16, 128, [2, 9, 1], [1500, 300, 64], {}),
    (mi.FP8_E4M3, 64, [6, 2, 5, 1, 6], [700, 1, 1300, 64, 6], {"partial_fp32": True}),
    # many workgroup rows (query groups x row tiles > 32): a partition per row, ~2 workgroups per CU
    (mi.FP8_E4M3, 16, [300, 8, 129], [1200, 8, 500], {}),                 # F = 6, 50 rows, G = 8
    (mi.BF16, 8, [150, 0, 37, 150], [400, 5, 90, 150], {"no_fold": True}),  # 150 rows, G = 4
    (mi.FP8_E4M3, 16, [64, 200], [3000, 300], {"no_fold": True, "num_splits": 5}),
]


@pytest.mark.parametrize("dtype,H,q_lens,lens,kw", RAGGED_CASES)
def test_ragged_query_counts(dtype, H, q_lens, lens, kw):
    x = mi.make_inputs(len(q_lens), max(q_lens), H, dtype, ("list", lens), page_size=64, seed=800 + H + len(q_lens))
    print(f"dtype={dtype} H={H} q_lens={q_lens} lens={lens} {kw}", flush=True)
    q, cu, ref = _ragged(x, q_lens)
    kv, bt, sl = to_dev(x)[1:]
    opts = mla.options(**kw) if kw else None
    out, lse = mla.decode_varlen(q, cu, kv, bt, sl, x.softmax_scale, x.q_scale, x.kv_scale,
                                 max_q_len=max(q_lens), max_seq_len=x.max_seq_len, opts=opts)
    torch.cuda.synchronize()
    assert_parity(x, out, lse, ref, partial_fp32=bool(kw.get("partial_fp32", False)))


@pytest.mark.parametrize("dtype", [mi.BF16, mi.FP8_E4M3])
def test_ragged_entry_with_equal_counts_matches_decode(dtype):
    """Equal counts through the ragged entry point: the same kernels and plan, bit-identical."""
    x = mi.make_inputs(3, 4, 32, dtype, ("list", [1000, 77, 2500]), seed=811)
    q4, kv, bt, sl = to_dev(x)
    out_u, lse_u = run_gpu(x, tensors=(q4, kv, bt, sl))
    cu = torch.arange(0, 13, 4, dtype=torch.int32, device="cuda:0")
    out_r, lse_r = mla.decode_varlen(q4.reshape(12, 32, 576), cu, kv, bt, sl, x.softmax_scale, x.q_scale, x.kv_scale,
                                     max_q_len=4, max_seq_len=x.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(out_r.view(3, 4, 32, 512), out_u) and torch.equal(lse_r.view(3, 4, 32), lse_u)


def test_ragged_window_and_more_tokens_than_keys():
    """A sliding window over a ragged batch whose sequences hold fewer keys than new tokens."""
    q_lens, lens = [8, 3, 8], [5, 900, 1200]
    x = mi.make_inputs(3, 8, 16, mi.BF16, ("list", lens), page_size=16, seed=821)
    q, cu, _ = _ragged(x, q_lens)
    O, L, A = [], [], []
    for b, ql in enumerate(q_lens):
        sub = dataclasses.replace(x, q=np.ascontiguousarray(x.q[b:b + 1, :ql]), block_table=x.block_table[b:b + 1],
                                  seq_lens=x.seq_lens[b:b + 1])
        o, l, a = run_oracle(sub, window=50)
        O.append(o[0]), L.append(l[0]), A.append(a[0])
    ref = tuple(np.concatenate(v, axis=0) for v in (O, L, A))
    kv, bt, sl = to_dev(x)[1:]
    out, lse = mla.decode_varlen(q, cu, kv, bt, sl, x.softmax_scale, x.q_scale, x.kv_scale, max_q_len=8,
                                 max_seq_len=x.max_seq_len, opts=mla.options(window=50, num_splits=9))
    torch.cuda.synchronize()
    assert_parity(x, out, lse, ref)


def test_stream_probe_runs():
    """The HBM -> LDS streaming probe bench.py reports the achievable read rate with: one pass over
    a 64 MiB buffer (a partial last round of tiles included) completes."""
    import ctypes

    from mla_paged_kv_decode_amd import build as b

    L = ctypes.CDLL(b.PROBE_LIB)
    f = L.mla_stream_probe
    f.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    buf = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda:0")
    print("stream probe over 64 MiB", flush=True)
    assert f(buf.data_ptr(), buf.numel(), 0, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
