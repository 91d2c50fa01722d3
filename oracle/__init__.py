"""CPU fp64 oracle for MLA decode over a paged latent KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product library
(``mla_paged_kv_decode_amd``) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (fp64, OpenMP over (batch, query token));
this module only builds/loads it and marshals numpy arrays.  What it computes
is the plain definition of MLA decode attention (see the header of
``oracle.c`` for the passages each step follows):

* tokenspeed-mla package page, "Quickstart" and "What it is": the decode call's
  arguments (query, kv_cache, block_tables, seq_lens, softmax_scale,
  kv_lora_rank = 512, qk_rope_head_dim = 64) and the BF16 output.
* TokenSpeed MLA article (gtnt.cn), section 2: split-KV partial O + LSE per KV
  segment, merged by a second reduction; section 3: query-token folding;
  section 6: tensor layouts ``query [B, q_len, H, D_qk]``,
  ``kv_cache [num_pages, page_size, D_total]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BF16 = 1
FP8_E4M3 = 2
FP16 = 3
BF16_Q_E4M3_KV = 4  # bf16 q over an e4m3 cache
D_QK = 576
D_V = 512


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    p = ctypes.c_void_p
    i = ctypes.c_int
    d = ctypes.c_double
    lib.oracle_mla_decode.argtypes = [p, p, i, p, i, p, i, i, i, i, i, d, d, d, i, i, p, p, p, i]
    lib.oracle_mla_decode.restype = i
    lib.oracle_dec_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_dec_bf16.restype = d
    lib.oracle_dec_f16.argtypes = [ctypes.c_uint16]
    lib.oracle_dec_f16.restype = d
    lib.oracle_dec_e4m3.argtypes = [ctypes.c_uint8]
    lib.oracle_dec_e4m3.restype = d
    lib.oracle_enc_e4m3.argtypes = [d]
    lib.oracle_enc_e4m3.restype = ctypes.c_uint8
    lib.oracle_fold_factor.argtypes = [i, i, i]
    lib.oracle_fold_factor.restype = i
    lib.oracle_kv_pack_quantize_fp8.argtypes = [p, p, i, d, p, p]
    lib.oracle_kv_pack_quantize_fp8.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def dec_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, from the format definition."""
    lib = _load()
    a = np.asarray(bits, dtype=np.uint16)
    return np.array([lib.oracle_dec_bf16(int(x)) for x in a.ravel()], dtype=np.float64).reshape(a.shape)


def f16_table() -> np.ndarray:
    """All 65536 IEEE binary16 patterns decoded to float64 (index = bit pattern), from the format definition."""
    lib = _load()
    return np.array([lib.oracle_dec_f16(h) for h in range(65536)], dtype=np.float64)


def e4m3_table() -> np.ndarray:
    """All 256 OCP E4M3 codes decoded to float64 (index = code)."""
    lib = _load()
    return np.array([lib.oracle_dec_e4m3(c) for c in range(256)], dtype=np.float64)


def dec_e4m3(codes) -> np.ndarray:
    a = np.asarray(codes, dtype=np.uint8)
    return e4m3_table()[a]


def enc_e4m3(x) -> np.ndarray:
    """float -> OCP E4M3 code, round-to-nearest-even, saturating to +-448."""
    lib = _load()
    a = np.asarray(x, dtype=np.float64)
    return np.array([lib.oracle_enc_e4m3(float(v)) for v in a.ravel()], dtype=np.uint8).reshape(a.shape)


def fold_factor(q_len: int, H: int, tile_m: int = 128) -> int:
    """Largest F with q_len % F == 0 and H*F <= tile_m (article section 3)."""
    return int(_load().oracle_fold_factor(int(q_len), int(H), int(tile_m)))


def mla_decode(q, kv_cache, block_table, seq_lens, *, dtype: int, softmax_scale: float,
               q_scale: float = 1.0, kv_scale: float = 1.0, split_len: int = 0, window: int = 0,
               num_threads: int = 0, want_absv: bool = False):
    """fp64 MLA decode.

    q: uint16 (bf16 or fp16 bits) or uint8 (e4m3 codes) array [B, q_len, H, 576]; dtype BF16, FP16, FP8_E4M3
    or BF16_Q_E4M3_KV (bf16 q bits, e4m3 cache codes).
    kv_cache: same format as q (e4m3 for BF16_Q_E4M3_KV), [num_pages, page_size, 576].
    block_table: int32 [B, max_pages]; seq_lens: int32 [B].
    Returns (O float64 [B, q_len, H, 512], LSE float64 [B, q_len, H]).
    split_len > 0 computes per-chunk partials and merges them by LSE.
    window > 0 is the sliding-window mask: token t sees keys [max(0, n_t - window), n_t).
    want_absv=True also returns sum_j softmax_j * |V_j| (same shape as O): the
    scale of the output's sensitivity to rounding the softmax weights.
    """
    lib = _load()
    q = np.ascontiguousarray(q)
    kv_cache = np.ascontiguousarray(kv_cache)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    want_q = np.uint8 if dtype == FP8_E4M3 else np.uint16
    want_kv = np.uint8 if dtype in (FP8_E4M3, BF16_Q_E4M3_KV) else np.uint16
    if q.dtype != want_q or kv_cache.dtype != want_kv:
        raise TypeError("q and kv_cache must hold raw bf16 / fp16 bits (uint16) or e4m3 codes (uint8)")
    B, q_len, H, dq = q.shape
    num_pages, page_size, dk = kv_cache.shape
    if dq != D_QK or dk != D_QK:
        raise ValueError("rows must be 576 wide")
    if block_table.ndim != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    out = np.zeros((B, q_len, H, D_V), dtype=np.float64)
    lse = np.zeros((B, q_len, H), dtype=np.float64)
    absv = np.zeros((B, q_len, H, D_V), dtype=np.float64) if want_absv else None
    rc = lib.oracle_mla_decode(_ptr(q), _ptr(kv_cache), int(dtype), _ptr(block_table), int(block_table.shape[1]),
                               _ptr(seq_lens), B, q_len, H, num_pages, page_size, float(softmax_scale),
                               float(q_scale), float(kv_scale), int(split_len), int(window), _ptr(out), _ptr(lse),
                               None if absv is None else _ptr(absv), int(num_threads))
    if rc == -1:
        raise IndexError("block_table entry out of range for a visible key")
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (rc={rc})")
    if want_absv:
        return out, lse, absv
    return out, lse


def kv_pack_quantize_fp8(latent_bits, rope_bits, kv_scale: float, slot_mapping=None, num_rows=None):
    """Reference for the fused pack + E4M3 quantise step.

    latent_bits: uint16 bf16 bits [T, 512]; rope_bits: uint16 [T, 64].
    Without slot_mapping returns uint8 [T, 576]; with it, writes row t to
    cache row slot_mapping[t] of a zero-filled [num_rows, 576] array.
    """
    lib = _load()
    latent_bits = np.ascontiguousarray(latent_bits, dtype=np.uint16)
    rope_bits = np.ascontiguousarray(rope_bits, dtype=np.uint16)
    T = latent_bits.shape[0]
    if slot_mapping is None:
        out = np.zeros((T, D_QK), dtype=np.uint8)
        sm = None
    else:
        sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
        out = np.zeros((int(num_rows), D_QK), dtype=np.uint8)
    lib.oracle_kv_pack_quantize_fp8(_ptr(latent_bits), _ptr(rope_bits), T, float(kv_scale),
                                    None if sm is None else _ptr(sm), _ptr(out))
    return out
