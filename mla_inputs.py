"""Seeded synthetic inputs for MLA paged-KV decode.

This module is shared by the tests, the benchmark and the oracle checks.  It
holds none of the attention arithmetic: it only draws random numbers, casts
them to the storage formats with library routines (torch's bf16 and
float8_e4m3fn casts) and lays them out as a paged cache.

Recipe (numpy PCG64, ``seed = 1000 + workload index`` by default), in this
order of draws:
  1. sequence lengths;
  2. a permutation of the page pool (block_table rows take consecutive pages
     of it; unreferenced pool pages are spares);
  3. q ~ N(0, 1), shape [B, q_len, H, 576];
  4. the page pool ~ N(0, 1), shape [num_pages, page_size, 576], drawn in
     chunks of 256 pages in page order (for FP8 the stream is replayed: a
     first pass finds the pool's amax, a second quantises).
bf16 inputs are cast round-to-nearest-even (fp16 likewise); FP8 inputs use one per-tensor
scale amax/448 each for q and for the cache, clamp to +-448 and cast to OCP
E4M3 (e4m3fn), so dequantised value = code * scale.  The mixed code takes bf16
q and an E4M3 cache (the same draws).  Spare pages are filled
with NaN codes; block_table entries past a sequence's last page point at a
spare page; rows past seq_len inside a sequence's last page keep their N(0,1)
draws (optionally NaN with ``poison_tail``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

D_QK = 576
D_V = 512
BF16 = 1
FP8_E4M3 = 2
FP16 = 3
BF16_Q_E4M3_KV = 4  # bf16 q over an OCP E4M3 cache
NAN_BF16 = 0x7FC0
NAN_F16 = 0x7E00
NAN_E4M3 = 0x7F

# The five decode workloads (sizes from the headline benchmark definition).
WORKLOADS = {
    "tiny_b1_h16_bf16": dict(index=1, B=1, q_len=1, H=16, dtype=BF16, lens=("fixed", 256), pool_pages=8),
    "agentic_b4_q4_h32_fp8_80k": dict(index=2, B=4, q_len=4, H=32, dtype=FP8_E4M3, lens=("fixed", 81920), spare_pages=64),
    "agentic_b16_q4_h32_fp8_80k": dict(index=3, B=16, q_len=4, H=32, dtype=FP8_E4M3, lens=("fixed", 81920), spare_pages=64),
    "dsv3_b64_q1_h128_bf16_ragged": dict(index=4, B=64, q_len=1, H=128, dtype=BF16, lens=("uniform", 4096, 65536), spare_pages=64),
    "spec_b128_q4_h64_fp8_ragged": dict(index=5, B=128, q_len=4, H=64, dtype=FP8_E4M3, lens=("loguniform", 1024, 81920), spare_pages=64),
    # bf16 queries over the FP8 cache of the batch-4 agentic shape (mixed inputs; not one of the five
    # configurations above)
    "agentic_b4_q4_h32_bf16q_fp8kv_80k": dict(index=6, B=4, q_len=4, H=32, dtype=BF16_Q_E4M3_KV,
                                              lens=("fixed", 81920), spare_pages=64),
}
WORKLOAD_ORDER = list(WORKLOADS)


@dataclass
class DecodeInputs:
    q: np.ndarray              # uint16 bf16 / fp16 bits or uint8 e4m3 codes, [B, q_len, H, 576]
    kv_cache: np.ndarray       # same format (e4m3 for the mixed code), [num_pages, page_size, 576]
    block_table: np.ndarray    # int32 [B, max_pages]
    seq_lens: np.ndarray       # int32 [B]
    dtype: int                 # BF16, FP16, FP8_E4M3 or BF16_Q_E4M3_KV
    q_scale: float
    kv_scale: float
    softmax_scale: float
    page_size: int
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def q_len(self):
        return self.q.shape[1]

    @property
    def H(self):
        return self.q.shape[2]

    @property
    def num_pages(self):
        return self.kv_cache.shape[0]

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max()) if self.seq_lens.size else 0


def _cast_bf16(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _cast_f16(x: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16)


def _cast_e4m3(x: np.ndarray, scale: float) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)) / np.float32(scale)
    t = t.clamp_(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def q_format(dtype: int) -> int:
    """Storage format of q for a dtype code (bf16 for the mixed code)."""
    return BF16 if dtype == BF16_Q_E4M3_KV else dtype


def kv_format(dtype: int) -> int:
    """Storage format of the cache rows for a dtype code (E4M3 for the mixed code)."""
    return FP8_E4M3 if dtype == BF16_Q_E4M3_KV else dtype


def _quantize(x: np.ndarray, dtype: int):
    if dtype == BF16:
        return _cast_bf16(x), 1.0
    if dtype == FP16:
        return _cast_f16(x), 1.0
    amax = float(np.max(np.abs(x))) if x.size else 1.0
    scale = amax / 448.0 if amax > 0 else 1.0
    return _cast_e4m3(x, scale), scale


POOL_CHUNK_PAGES = 256


def _draw_pool(rng, num_pages, page_size, dtype):
    """N(0,1) pool drawn chunk by chunk into a preallocated output (no large temporaries)."""
    shape = (num_pages, page_size, D_QK)
    buf = np.empty((POOL_CHUNK_PAGES, page_size, D_QK), dtype=np.float32)
    if dtype in (BF16, FP16):
        cast = _cast_bf16 if dtype == BF16 else _cast_f16
        out = np.empty(shape, dtype=np.uint16)
        for p0 in range(0, num_pages, POOL_CHUNK_PAGES):
            n = min(POOL_CHUNK_PAGES, num_pages - p0)
            rng.standard_normal(out=buf[:n], dtype=np.float32)
            out[p0:p0 + n] = cast(buf[:n])
        return out, 1.0
    state = rng.bit_generator.state
    amax = 0.0
    for p0 in range(0, num_pages, POOL_CHUNK_PAGES):
        n = min(POOL_CHUNK_PAGES, num_pages - p0)
        rng.standard_normal(out=buf[:n], dtype=np.float32)
        amax = max(amax, float(buf[:n].max()), float(-buf[:n].min()))
    scale = amax / 448.0 if amax > 0 else 1.0
    rng.bit_generator.state = state
    out = np.empty(shape, dtype=np.uint8)
    for p0 in range(0, num_pages, POOL_CHUNK_PAGES):
        n = min(POOL_CHUNK_PAGES, num_pages - p0)
        rng.standard_normal(out=buf[:n], dtype=np.float32)
        out[p0:p0 + n] = _cast_e4m3(buf[:n], scale)
    return out, scale


def _draw_lens(rng, B, spec):
    kind = spec[0]
    if kind == "fixed":
        return np.full(B, spec[1], dtype=np.int64)
    if kind == "uniform":
        return rng.integers(spec[1], spec[2], size=B, endpoint=True).astype(np.int64)
    if kind == "loguniform":
        u = rng.uniform(math.log(spec[1]), math.log(spec[2]), size=B)
        return np.floor(np.exp(u)).astype(np.int64)
    if kind == "list":
        return np.asarray(spec[1], dtype=np.int64)
    raise ValueError(kind)


def make_inputs(B, q_len, H, dtype, lens, *, page_size=64, seed=0, spare_pages=8, pool_pages=None,
                softmax_scale=1.0 / math.sqrt(192.0), poison_tail=False, max_pages=None, name="") -> DecodeInputs:
    """Build one seeded paged-decode input set (see the module docstring)."""
    rng = np.random.default_rng(seed)
    seq_lens = _draw_lens(rng, B, lens)
    pages_per_seq = (seq_lens + page_size - 1) // page_size
    needed = int(pages_per_seq.sum())
    num_pages = int(pool_pages) if pool_pages is not None else needed + int(spare_pages)
    if num_pages < needed + 1 and needed > 0:
        num_pages = needed + 1  # keep at least one spare page for the unused block_table entries
    if num_pages == 0:
        num_pages = 1
    perm = rng.permutation(num_pages).astype(np.int32)
    if max_pages is None:
        max_pages = max(1, int(pages_per_seq.max()) if B else 1)
    if pool_pages is not None and B == 1 and max_pages < num_pages:
        max_pages = num_pages  # a tiny pool: the whole permutation is the block_table row
    spare = perm[needed:]
    block_table = np.empty((B, max_pages), dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(pages_per_seq[b])
        block_table[b, :n] = perm[off:off + n]
        off += n
        if max_pages > n:
            block_table[b, n:] = np.resize(spare, max_pages - n) if spare.size else perm[0]
    if pool_pages is not None and B == 1:
        block_table[0, :] = perm[:max_pages]
    q32 = rng.standard_normal((B, q_len, H, D_QK), dtype=np.float32)
    q, q_scale = _quantize(q32, q_format(dtype))
    del q32
    kv, kv_scale = _draw_pool(rng, num_pages, page_size, kv_format(dtype))
    nan_code = {BF16: NAN_BF16, FP16: NAN_F16}.get(kv_format(dtype), NAN_E4M3)
    used = np.zeros(num_pages, dtype=bool)
    for b in range(B):
        used[block_table[b, :int(pages_per_seq[b])]] = True
    kv[~used] = nan_code
    if poison_tail:
        for b in range(B):
            L = int(seq_lens[b])
            if L % page_size:
                kv[block_table[b, L // page_size], L % page_size:] = nan_code
    return DecodeInputs(q=q, kv_cache=kv, block_table=block_table, seq_lens=seq_lens.astype(np.int32), dtype=dtype,
                        q_scale=float(q_scale), kv_scale=float(kv_scale), softmax_scale=float(softmax_scale),
                        page_size=page_size, name=name, meta=dict(seed=seed))


def workload_inputs(name: str, seed=None, **overrides) -> DecodeInputs:
    """The named workload with its default seed (1000 + index)."""
    w = dict(WORKLOADS[name])
    idx = w.pop("index")
    if seed is None:
        seed = 1000 + idx
    kw = dict(page_size=64, seed=seed, name=name)
    if "pool_pages" in w:
        kw["pool_pages"] = w.pop("pool_pages")
    if "spare_pages" in w:
        kw["spare_pages"] = w.pop("spare_pages")
    kw.update(overrides)
    return make_inputs(w["B"], w["q_len"], w["H"], w["dtype"], w["lens"], **kw)


# Ragged prefill workloads (the pages name a varlen ragged prefill but give no shapes): sequence b
# gets new[b] new tokens over ctx[b] cached keys, so seq_lens = ctx + new.
RAGGED_PREFILL = {
    "ragged_prefill_b4_h16_fp8": dict(H=16, dtype=FP8_E4M3, new=[512, 1024, 256, 768], ctx=[8192, 4096, 16384, 2048]),
    "ragged_prefill_b4_h128_bf16": dict(H=128, dtype=BF16, new=[128, 512, 64, 256], ctx=[8192, 4096, 16384, 2048]),
}


def ragged_prefill_inputs(name: str, seed: int = 1100):
    """(inputs of a uniform batch of max(new) tokens, new): sequence b keeps its first new[b] tokens."""
    w = RAGGED_PREFILL[name]
    lens = [c + n for c, n in zip(w["ctx"], w["new"])]
    x = make_inputs(len(lens), max(w["new"]), w["H"], w["dtype"], ("list", lens), page_size=64, seed=seed,
                    spare_pages=64, name=name)
    return x, list(w["new"])


def workload_lens(name: str, seed=None) -> np.ndarray:
    """Only the sequence lengths of a workload (first draw of its stream)."""
    w = WORKLOADS[name]
    if seed is None:
        seed = 1000 + w["index"]
    return _draw_lens(np.random.default_rng(seed), w["B"], w["lens"])
