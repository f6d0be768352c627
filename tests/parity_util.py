"""Shared helpers for the GPU parity tests: sampled rows and the tolerance check against the oracle.

Tolerances: max |O_gpu(fp32) - O_ref| <= 4e-3 for fp16 inputs and <= 2e-2 for bf16 inputs;
|lse_gpu - lse_ref| / max(1, |lse_ref|) <= 1e-4.  An fp16/bf16 output adds one unit in the last
place of the output format at the reference value.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

O_TOL = {torch.float16: 4e-3, torch.bfloat16: 2e-2}
LSE_RTOL = 1e-4


def sample_rows(B: int, H: int, N: int, *, seed: int = 0, n_random: int = 512, edge: int = 64,
                boundaries=(), tiles=(), cap: int = 256, heads=None) -> np.ndarray:
    """Rows checked at scale, in every (b, h): the first and last `edge` rows, rows +-1 around each
    chunk boundary and around evenly spread tile boundaries (at most `cap` boundary rows, chunk
    boundaries first), and `n_random` seeded rows."""
    rng = np.random.default_rng(seed)
    idx = set(range(min(edge, N))) | set(range(max(0, N - edge), N))
    bl = sorted({int(x) for x in boundaries if 0 < x < N})
    if len(bl) > cap // 2:
        bl = list(np.array(bl)[np.linspace(0, len(bl) - 1, cap // 2).astype(int)])
    tl = sorted({int(x) for x in tiles if 0 < x < N} - set(bl))
    room = cap // 2 - len(bl)
    if len(tl) > room:
        tl = list(np.array(tl)[np.linspace(0, len(tl) - 1, room).astype(int)]) if room > 0 else []
    for x in bl + tl:
        idx |= {x - 1, x}
    idx |= set(rng.integers(0, N, size=min(n_random, N)).tolist())
    idx = np.array(sorted(i for i in idx if 0 <= i < N), dtype=np.int64)
    hs = range(H) if heads is None else heads
    rows = [(b, h, i) for b in range(B) for h in hs for i in idx]
    return np.array(rows, dtype=np.int64).reshape(-1, 3)


def ulp_at(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Spacing of the output format at |x| (0 for fp32 output)."""
    if dtype == torch.float32:
        return np.zeros_like(x)
    mant = 10 if dtype == torch.float16 else 7
    ax = np.maximum(np.abs(x), 2.0 ** -14)
    return 2.0 ** (np.floor(np.log2(ax)) - mant)


def compare(out: torch.Tensor, lse: torch.Tensor | None, ref: dict, in_dtype: torch.dtype, rows: np.ndarray | None = None,
            label: str = "") -> dict:
    """Compare GPU output (and lse) with oracle rows; raises AssertionError with the worst row."""
    o = out.detach().float().cpu()
    if rows is None:
        got = o.reshape(-1, o.shape[-1]).double().numpy()
        got_lse = lse.detach().cpu().reshape(-1).double().numpy() if lse is not None else None
    else:
        b, h, i = (torch.from_numpy(rows[:, c]) for c in range(3))
        got = o[b, h, i].double().numpy()
        got_lse = lse.detach().cpu()[b, h, i].double().numpy() if lse is not None else None
    want = ref["o"]
    err = np.abs(got - want)
    tol = O_TOL[in_dtype] + ulp_at(want, out.dtype)
    res = {"max_abs": float(err.max()) if err.size else 0.0}
    bad = err > tol
    if bad.any():
        r, c = np.unravel_index(np.argmax(err - tol), err.shape)
        where = tuple(rows[r]) if rows is not None else r
        raise AssertionError(f"{label}: max_abs {err.max():.3e} > tol (row {where}, dim {c}: got {got[r, c]:.6f} "
                             f"want {want[r, c]:.6f}); {int(bad.sum())} elements out of tolerance")
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    if got_lse is not None:
        rel = np.abs(got_lse - ref["lse"]) / np.maximum(1.0, np.abs(ref["lse"]))
        res["lse_rel"] = float(rel.max()) if rel.size else 0.0
        if rel.size and rel.max() > LSE_RTOL:
            r = int(np.argmax(rel))
            raise AssertionError(f"{label}: lse rel error {rel.max():.3e} > {LSE_RTOL} at row "
                                 f"{tuple(rows[r]) if rows is not None else r}: got {got_lse[r]} want {ref['lse'][r]}")
    return res


def reference(q, k, v, *, causal, scale, rows=None, threads=None) -> dict:
    return oracle.attention_rows(q, k, v, causal=causal, scale=scale, rows=rows, threads=threads)
