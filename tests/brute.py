"""Dense brute-force MLA decode for tiny shapes: an independent pin of the oracle.

It shares nothing with ``oracle/``: stored values are decoded with torch's
own bf16 / float16 / float8_e4m3fn conversions (q and the cache each in its own format), the paged cache is first gathered into
a dense [L, 576] key matrix in logical order, the causal (and sliding-window)
mask is an explicit boolean matrix, and the softmax / log-sum-exp come from scipy.
"""
import numpy as np
import scipy.special
import torch

import mla_inputs as mi


def decode_values(raw: np.ndarray, dtype: int) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(raw))
    if dtype == mi.BF16:
        return t.view(torch.bfloat16).to(torch.float64).numpy()
    if dtype == mi.FP16:
        return t.view(torch.float16).to(torch.float64).numpy()
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def dense_keys(kv: np.ndarray, block_table: np.ndarray, b: int, L: int) -> np.ndarray:
    page_size = kv.shape[1]
    rows = [kv[block_table[b, j // page_size], j % page_size] for j in range(L)]
    return np.stack(rows) if rows else np.zeros((0, kv.shape[2]))


def brute_decode(x: "mi.DecodeInputs", *, alignment: str = "bottom_right", window: int = 0):
    q = decode_values(x.q, mi.q_format(x.dtype)) * x.q_scale
    kv = decode_values(x.kv_cache, mi.kv_format(x.dtype)) * x.kv_scale
    B, q_len, H, _ = q.shape
    O = np.zeros((B, q_len, H, 512))
    lse = np.full((B, q_len, H), -np.inf)
    for b in range(B):
        L = int(x.seq_lens[b])
        K = dense_keys(kv, x.block_table, b, L)
        if L == 0:
            continue
        scores = x.softmax_scale * np.einsum("thd,jd->thj", q[b], K)
        j = np.arange(L)[None, :]
        t = np.arange(q_len)[:, None]
        if alignment == "bottom_right":
            mask = j <= (L - q_len + t)
        else:  # the other reading of "causal": token t sees keys 0..t
            mask = j <= t
        if window > 0:  # sliding window: only the last `window` keys a token can see
            mask = mask & (j > (L - q_len + t) - window)
        scores = np.where(mask[:, None, :], scores, -np.inf)
        for tt in range(q_len):
            if not mask[tt].any():
                continue
            s = scores[tt]
            lse[b, tt] = scipy.special.logsumexp(s, axis=-1)
            P = scipy.special.softmax(s, axis=-1)
            O[b, tt] = P @ K[:, :512]
    return O, lse
