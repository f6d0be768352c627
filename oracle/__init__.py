"""FP64 CPU reference for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the attention library never does, and
the two share no code.  The arithmetic lives in ``cqsa_oracle.c`` (plain C,
FP64, two passes per row, Neumaier-compensated sums); this module only
marshals tensors into it.

Definition followed (the SDPA-equivalent call of the Stream-CQSA pages, stream-cqsa
2.2.0 -> 2.2.2 diff, ``stream_cqsa/api.py``, ``attention()``): for query head h
and key/value head h' = h // (Hq // Hkv),
``O_i = sum_{j in V(i)} softmax_j(scale * q_i . k_j) v_j`` and ``lse_i = ln sum_j exp(scale * q_i . k_j)``,
with V(i) all keys, or ``{j <= i + Nk - Nq}`` when causal (query block at the end of the keys).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cqsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libcqsa_oracle.so")
_lib = None


class _Problem(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64),
        ("Nq", ctypes.c_int64), ("Nk", ctypes.c_int64), ("D", ctypes.c_int64),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3), ("v_stride", ctypes.c_int64 * 3),
        ("scale", ctypes.c_float),
    ]


# IEEE double arithmetic as written: no fast-math, no contraction of a * b + c into a fused
# multiply-add, and the baseline x86-64 instruction set (the library is built here and run on
# whatever host the tests run on).
CFLAGS = ["-O3", "-fPIC", "-shared", "-pthread", "-fno-fast-math", "-ffp-contract=off"]


def build(force: bool = True) -> str:
    """Compile the reference with gcc into ``oracle/libcqsa_oracle.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_rows.argtypes = [ctypes.POINTER(_Problem), ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, dp, dp, dp, dp, ctypes.c_int32]
        lib.oracle_rows.restype = ctypes.c_int
        lib.oracle_merge.argtypes = [ctypes.c_int64, ctypes.c_int64, dp, dp, dp, dp, dp, dp, dp, dp, dp]
        lib.oracle_merge.restype = None
        lib.oracle_backward.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
                                        dp, dp, dp, ctypes.c_int32]
        lib.oracle_backward.restype = ctypes.c_int
        lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_double.restype = ctypes.c_double
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def f16_to_double(bits: int) -> float:
    return float(_load().oracle_f16_to_double(int(bits)))


def bf16_to_double(bits: int) -> float:
    return float(_load().oracle_bf16_to_double(int(bits)))


def _dp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _problem(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool, scale: float) -> _Problem:
    for t in (q, k, v):
        if t.device.type != "cpu" or t.dim() != 4 or t.stride(3) != 1:
            raise ValueError("oracle inputs are CPU [B, H, N, D] tensors with a unit head-dim stride")
        if t.dtype != q.dtype or t.dtype not in (torch.float16, torch.bfloat16):
            raise ValueError("oracle inputs are all fp16 or all bf16")
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nk, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D or Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("shape mismatch")
    p = _Problem()
    p.q, p.k, p.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    p.dtype = 0 if q.dtype == torch.float16 else 1
    p.causal = 1 if causal else 0
    p.B, p.Hq, p.Hkv, p.Nq, p.Nk, p.D = B, Hq, Hkv, Nq, Nk, D
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v)):
        arr = getattr(p, name)
        arr[0], arr[1], arr[2] = t.stride(0), t.stride(1), t.stride(2)
    p.scale = float(np.float32(scale))
    return p


def all_rows(B: int, H: int, N: int) -> np.ndarray:
    b, h, i = np.meshgrid(np.arange(B), np.arange(H), np.arange(N), indexing="ij")
    return np.stack([b.ravel(), h.ravel(), i.ravel()], axis=1).astype(np.int64)


def attention_rows(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool, scale: float,
                   rows: np.ndarray | None = None, key_range: tuple | None = None, partial: bool = False,
                   threads: int | None = None) -> dict:
    """Reference attention for selected rows.

    ``rows`` is an (n, 3) int64 array of (b, h, i); all rows when None.  ``key_range`` = (lo, hi)
    narrows the keys (a KV chunk).  Returns a dict with ``o`` (n, D) float64 and ``m``, ``l``,
    ``lse`` (n,) float64; with ``partial=True`` ``o`` is the unnormalised sum and ``lse`` is absent.
    ``scale`` is rounded to fp32 first, as the library receives it."""
    p = _problem(q, k, v, causal, scale)
    if rows is None:
        rows = all_rows(p.B, p.Hq, p.Nq)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    n = rows.shape[0]
    lo, hi = (0, p.Nk) if key_range is None else (int(key_range[0]), int(key_range[1]))
    o = np.zeros((n, p.D), dtype=np.float64)
    m = np.zeros(n, dtype=np.float64)
    lsum = np.zeros(n, dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    rc = _load().oracle_rows(ctypes.byref(p), rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), n, lo, hi,
                             1 if partial else 0, _dp(o), _dp(m), _dp(lsum), _dp(lse),
                             int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_rows failed ({rc})")
    out = {"o": o, "m": m, "l": lsum, "rows": rows}
    if not partial:
        out["lse"] = lse
    return out


def attention(q, k, v, *, causal: bool, scale: float, threads: int | None = None):
    """Full reference output as float64 tensors: (O [B, Hq, Nq, D], lse [B, Hq, Nq])."""
    B, Hq, Nq, D = q.shape
    r = attention_rows(q, k, v, causal=causal, scale=scale, threads=threads)
    o = torch.from_numpy(r["o"]).reshape(B, Hq, Nq, D)
    lse = torch.from_numpy(r["lse"]).reshape(B, Hq, Nq)
    return o, lse


def backward(q, k, v, dout, *, causal: bool, scale: float, threads: int | None = None):
    """Reference gradients (dq, dk, dv) as float64 tensors for the upstream gradient ``dout``
    (q's dtype and shape, unit head-dim stride)."""
    p = _problem(q, k, v, causal, scale)
    if dout.dtype != q.dtype or dout.shape != q.shape or dout.stride(3) != 1 or dout.device.type != "cpu":
        raise ValueError("dout must be a CPU tensor of q's dtype and shape with a unit head-dim stride")
    dq = np.zeros(tuple(q.shape), dtype=np.float64)
    dk = np.zeros(tuple(k.shape), dtype=np.float64)
    dv = np.zeros(tuple(v.shape), dtype=np.float64)
    st = (ctypes.c_int64 * 3)(dout.stride(0), dout.stride(1), dout.stride(2))
    rc = _load().oracle_backward(ctypes.byref(p), dout.data_ptr(), st, _dp(dq), _dp(dk), _dp(dv),
                                 int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_backward failed ({rc})")
    return torch.from_numpy(dq), torch.from_numpy(dk), torch.from_numpy(dv)


def merge(a: dict, b: dict) -> dict:
    """Exact log-sum-exp merge of two partial triples (dicts with o, m, l)."""
    oa, ma, la = (np.ascontiguousarray(a[x], dtype=np.float64) for x in ("o", "m", "l"))
    ob, mb, lb = (np.ascontiguousarray(b[x], dtype=np.float64) for x in ("o", "m", "l"))
    n, D = oa.shape
    o = np.empty_like(oa)
    m = np.empty_like(ma)
    lsum = np.empty_like(la)
    _load().oracle_merge(n, D, _dp(oa), _dp(ma), _dp(la), _dp(ob), _dp(mb), _dp(lb), _dp(o), _dp(m), _dp(lsum))
    return {"o": o, "m": m, "l": lsum}


def normalise(t: dict) -> dict:
    """Turn an unnormalised triple into (o / l, lse = m + ln l)."""
    with np.errstate(divide="ignore", invalid="ignore"):
        return {"o": t["o"] / t["l"][:, None], "lse": t["m"] + np.log(t["l"])}
