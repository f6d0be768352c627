"""Seeded random problems against the FP64 oracle, element by element: shapes drawn across the
parameter space (batch, GQA ratio, ragged Nq and Nk from 1 to 2500, D = 64 or 128, fp16 or bf16,
causal or not, a scale or the default) and, for each, one way of running it: the single pass, forced
query and key chunks with either merge, KV splits, the quorum-set schedule, pinned host operands
(head-major or token-major) or split-P.  The backward gets its own draw: the single pass, forced chunks
on the device, and pinned host or mixed operands, each with ragged chunk sizes (down to one row).  The
draws are fixed by their seeds, so a failure names a case that can be rerun on its own."""
import math
import sys

import numpy as np
import pytest
import torch

import synth
from parity_util import compare, reference

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MODES = ["plain", "kv_chunk", "q_kv_chunk", "fused", "kv_splits", "cqs", "host", "host_token_major", "split_p"]


def draw_cases(n: int, seed: int = 0xC05A0123) -> list:
    rng = np.random.default_rng(seed)
    cases = []
    for idx in range(n):
        D = int(rng.choice([64, 128]))
        dtype = [torch.float16, torch.bfloat16][int(rng.integers(0, 2))]
        causal = bool(rng.random() < 0.6)
        Hkv = int(rng.choice([1, 2, 3]))
        group = int(rng.choice([1, 2, 4, 5]))
        B = int(rng.choice([1, 2])) if Hkv * group <= 6 else 1
        Nk = int(rng.integers(1, 2501))
        Nq = int(rng.integers(1, Nk + 1)) if causal else int(rng.integers(1, 2501))
        mode = MODES[idx % len(MODES)]          # every mode appears
        if mode == "cqs" and min(Nq, Nk) < 13:
            mode = "plain"
        scale = None if rng.random() < 0.5 else float(rng.uniform(0.03, 0.3))
        sigma = float(rng.choice([1.0, 2.0]))
        opt = {}
        if mode in ("kv_chunk", "q_kv_chunk", "fused"):
            opt["kv_chunk"] = int(rng.integers(max(1, Nk // 8), Nk + 1))
        if mode == "q_kv_chunk":
            opt["q_chunk"] = int(rng.integers(max(1, Nq // 6), Nq + 1))
        if mode == "fused":
            opt["merge"] = 2
        if mode == "kv_chunk":
            opt["merge"] = 1   # the merge kernel (the planner's choice for chunks is the fused fold)
        if mode == "kv_splits":
            opt["kv_splits"] = int(rng.integers(2, 5))
        if mode == "cqs":
            opt["cqs"] = int(rng.choice([7, 13]))
        if mode == "split_p":
            opt["precision"] = 1
        cases.append(dict(idx=idx, B=B, Hq=Hkv * group, Hkv=Hkv, Nq=Nq, Nk=Nk, D=D, dtype=dtype, causal=causal,
                          scale=scale, sigma=sigma, mode=mode, opt=opt, seed=7000 + idx))
    return cases


CASES = draw_cases(36)


def _name(c):
    return (f"{c['idx']}-{c['mode']}-B{c['B']}H{c['Hq']}x{c['Hkv']}q{c['Nq']}k{c['Nk']}d{c['D']}"
            f"{'f16' if c['dtype'] == torch.float16 else 'bf16'}{'c' if c['causal'] else 'n'}")


def _token_major_pinned(t):
    x = torch.empty((t.shape[0], t.shape[2], t.shape[1], t.shape[3]), dtype=t.dtype, pin_memory=True)
    x.copy_(t.transpose(1, 2))
    return x.transpose(1, 2)


def test_case_table_covers_the_space():
    modes = {c["mode"] for c in CASES}
    assert {"plain", "kv_chunk", "q_kv_chunk", "fused", "kv_splits", "host", "host_token_major", "split_p"} <= modes
    assert any(c["mode"] == "cqs" for c in CASES)
    assert {c["D"] for c in CASES} == {64, 128} and {c["causal"] for c in CASES} == {True, False}
    assert {c["Hq"] // c["Hkv"] for c in CASES} >= {1, 2, 4, 5}
    assert min(c["Nq"] for c in CASES) < 64 and max(c["Nk"] for c in CASES) > 2000


@pytest.mark.parametrize("c", CASES, ids=_name)
def test_random_problem_against_oracle(c):
    print("[gpu-case] random", _name(c), c["opt"], f"scale={c['scale']} sigma={c['sigma']}", file=sys.stderr,
          flush=True)
    import exact_long_context_cqsa_amd as m
    q = synth.normal((c["B"], c["Hq"], c["Nq"], c["D"]), seed=c["seed"], tensor_id=0, sigma=c["sigma"], dtype=c["dtype"])
    k = synth.normal((c["B"], c["Hkv"], c["Nk"], c["D"]), seed=c["seed"], tensor_id=1, sigma=c["sigma"], dtype=c["dtype"])
    v = synth.normal((c["B"], c["Hkv"], c["Nk"], c["D"]), seed=c["seed"], tensor_id=2, dtype=c["dtype"])
    scale = c["scale"] if c["scale"] is not None else 1.0 / math.sqrt(c["D"])
    ref = reference(q, k, v, causal=c["causal"], scale=float(np.float32(scale)))
    if c["mode"] == "host":
        qi, ki, vi = q.pin_memory(), k.pin_memory(), v.pin_memory()
    elif c["mode"] == "host_token_major":
        qi, ki, vi = _token_major_pinned(q), _token_major_pinned(k), _token_major_pinned(v)
    else:
        qi, ki, vi = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse = m.attention(qi, ki, vi, is_causal=c["causal"], scale=c["scale"], out_dtype=torch.float32,
                           return_lse=True, **c["opt"])
    if out.is_cuda:
        torch.cuda.synchronize()
    compare(out, lse, ref, c["dtype"], label=_name(c))


# ---------------------------------------------------------------- the backward

U = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}
BWD_MODES = ["single", "chunked", "host", "mixed"]


def draw_backward_cases(n: int, seed: int = 0xC05A0B0D) -> list:
    rng = np.random.default_rng(seed)
    cases = []
    for idx in range(n):
        D = int(rng.choice([64, 128]))
        dtype = [torch.float16, torch.bfloat16][int(rng.integers(0, 2))]
        causal = bool(rng.random() < 0.6)
        Hkv = int(rng.choice([1, 2]))
        group = int(rng.choice([1, 2, 3, 4]))
        B = int(rng.choice([1, 2])) if Hkv * group <= 4 else 1
        Nk = int(rng.integers(1, 1201))
        Nq = int(rng.integers(1, Nk + 1)) if causal else int(rng.integers(1, 1201))
        mode = BWD_MODES[idx % len(BWD_MODES)]
        opt = {}
        if mode != "single":
            opt["q_chunk"] = int(rng.integers(max(1, Nq // 5), Nq + 1))
            opt["kv_chunk"] = int(rng.integers(max(1, Nk // 5), Nk + 1))
        cases.append(dict(idx=idx, B=B, Hq=Hkv * group, Hkv=Hkv, Nq=Nq, Nk=Nk, D=D, dtype=dtype, causal=causal,
                          mode=mode, opt=opt, seed=8000 + idx))
    return cases


BWD_CASES = draw_backward_cases(16)


def _bname(c):
    return (f"{c['idx']}-{c['mode']}-B{c['B']}H{c['Hq']}x{c['Hkv']}q{c['Nq']}k{c['Nk']}d{c['D']}"
            f"{'f16' if c['dtype'] == torch.float16 else 'bf16'}{'c' if c['causal'] else 'n'}")


@pytest.mark.parametrize("c", BWD_CASES, ids=_bname)
def test_random_backward_against_oracle(c):
    """Gradients within 8 u of the FP64 oracle (max |g - g_ref| / max(1, max |g_ref|)), u the unit
    roundoff of the input format: every product takes operands rounded to it once."""
    print("[gpu-case] random backward", _bname(c), c["opt"], file=sys.stderr, flush=True)
    import exact_long_context_cqsa_amd as m
    import oracle
    shp_q, shp_k = (c["B"], c["Hq"], c["Nq"], c["D"]), (c["B"], c["Hkv"], c["Nk"], c["D"])
    q = synth.normal(shp_q, seed=c["seed"], tensor_id=0, dtype=c["dtype"])
    k = synth.normal(shp_k, seed=c["seed"], tensor_id=1, dtype=c["dtype"])
    v = synth.normal(shp_k, seed=c["seed"], tensor_id=2, dtype=c["dtype"])
    do = synth.normal(shp_q, seed=c["seed"], tensor_id=synth.TENSOR_DO, dtype=c["dtype"])
    scale = 1.0 / math.sqrt(c["D"])
    rq, rk, rv = oracle.backward(q, k, v, do, causal=c["causal"], scale=scale)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    out, lse = m.attention(qd, kd, vd, is_causal=c["causal"], return_lse=True)
    if c["mode"] == "host":
        args = [t.cpu().pin_memory() for t in (qd, kd, vd, out, dod, lse)]
    elif c["mode"] == "mixed":
        args = [qd.cpu().pin_memory(), kd.cpu().pin_memory(), vd, out, dod, lse]
    else:
        args = [qd, kd, vd, out, dod, lse]
    dq, dk, dv = m.attention_backward(*args, is_causal=c["causal"], grad_dtype=torch.float32, **c["opt"])
    torch.cuda.synchronize()
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        gd = g.detach().double().cpu()
        assert torch.isfinite(gd).all(), name
        err = float((gd - r).abs().max()) / max(1.0, float(r.abs().max())) if r.numel() else 0.0
        assert err <= 8 * U[c["dtype"]], (_bname(c), name, err)
