"""GPU parity of the backward (dQ, dK, dV through cqsa_attention_backward) against the FP64 oracle.

Metric: max |g - g_ref| / max(1, max |g_ref|) per gradient tensor (the floor keeps a gradient that is
exactly zero, e.g. dQ and dK of a row that sees one key, measured in absolute terms: the inputs are
N(0, 1), so gradients are of order one).  Bound: each product takes its operands rounded to the input
format (P, dS and the forward output rounded with unit u = 2^-11 for fp16, 2^-8 for bf16), so the
error is a few u of the gradient's scale; the tests allow 8 u.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}


def cqsa():
    import exact_long_context_cqsa_amd as m
    return m


def say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def gen(B, Hq, Hkv, Nq, Nk, D, dtype, seed):
    q = synth.normal((B, Hq, Nq, D), seed=seed, tensor_id=0, dtype=dtype)
    k = synth.normal((B, Hkv, Nk, D), seed=seed, tensor_id=1, dtype=dtype)
    v = synth.normal((B, Hkv, Nk, D), seed=seed, tensor_id=2, dtype=dtype)
    do = synth.normal((B, Hq, Nq, D), seed=seed, tensor_id=synth.TENSOR_DO, dtype=dtype)
    return q, k, v, do


def rel_err(got, ref):
    g = got.detach().double().cpu()
    return float((g - ref).abs().max()) / max(1.0, float(ref.abs().max()))


CASES = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal
    (1, 1, 1, 1024, 1024, 64, torch.float16, True),
    (1, 2, 2, 300, 300, 64, torch.float16, True),        # ragged tails
    (2, 3, 3, 77, 513, 64, torch.float16, False),        # Nq < Nk
    (1, 2, 2, 700, 129, 64, torch.bfloat16, False),      # Nq > Nk
    (1, 4, 1, 257, 1000, 128, torch.bfloat16, True),     # GQA 4:1, bottom-right causal
    (2, 8, 2, 130, 130, 128, torch.float16, True),       # GQA, square causal
    (1, 2, 2, 1, 1, 64, torch.float16, True),            # one query, one key
    (1, 2, 2, 1, 4099, 128, torch.float16, True),        # one query at the end of 4099 keys
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}x{c[2]}q{c[3]}k{c[4]}d{c[5]}"
                         f"{'f16' if c[6] == torch.float16 else 'bf16'}{'c' if c[7] else 'n'}")
def test_backward_parity(case):
    B, Hq, Hkv, Nq, Nk, D, dtype, causal = case
    say("backward", case)
    q, k, v, do = gen(B, Hq, Hkv, Nq, Nk, D, dtype, seed=5000 + Nq + Nk + D)
    scale = 1.0 / math.sqrt(D)
    rq, rk, rv = oracle.backward(q, k, v, do, causal=causal, scale=scale)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    out, lse = cqsa().attention(qd, kd, vd, is_causal=causal, return_lse=True)   # out in the input dtype
    dq, dk, dv = cqsa().attention_backward(qd, kd, vd, out, dod, lse, is_causal=causal, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    errs = {n: rel_err(g, r) for n, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv))}
    say("errors", errs)
    for n, e in errs.items():
        assert e <= 8 * U[dtype], (n, e)
    assert all(torch.isfinite(g).all() for g in (dq, dk, dv))


SCALE_CASES = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal, scale
    (1, 2, 2, 600, 600, 64, torch.float16, True, 4.0),       # logits with sd 32: near one-key rows
    (1, 4, 2, 300, 900, 128, torch.bfloat16, True, 2.0),     # GQA, bottom-right causal
    (1, 2, 2, 500, 700, 64, torch.bfloat16, False, 1e-3),    # nearly uniform weights
]


@pytest.mark.parametrize("case", SCALE_CASES, ids=lambda c: f"q{c[3]}k{c[4]}d{c[5]}{'c' if c[7] else 'n'}-s{c[8]:g}")
def test_backward_extreme_scales(case):
    """The backward at softmax scales far from 1/sqrt(D): sharp rows (dS concentrated on a few keys per
    row) and nearly uniform ones, against the FP64 oracle at the same bound."""
    B, Hq, Hkv, Nq, Nk, D, dtype, causal, scale = case
    say("backward scale", case)
    q, k, v, do = gen(B, Hq, Hkv, Nq, Nk, D, dtype, seed=5300 + Nq + D)
    rq, rk, rv = oracle.backward(q, k, v, do, causal=causal, scale=scale)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    out, lse = cqsa().attention(qd, kd, vd, is_causal=causal, scale=scale, return_lse=True)
    dq, dk, dv = cqsa().attention_backward(qd, kd, vd, out, dod, lse, is_causal=causal, scale=scale,
                                           grad_dtype=torch.float32)
    torch.cuda.synchronize()
    errs = {n: rel_err(g, r) for n, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv))}
    say("errors", errs)
    for n, e in errs.items():
        assert e <= 8 * U[dtype], (n, e)
    assert all(torch.isfinite(g).all() for g in (dq, dk, dv))


def test_backward_deterministic_and_grad_dtypes():
    B, Hq, Hkv, N, D = 1, 4, 2, 777, 64
    q, k, v, do = gen(B, Hq, Hkv, N, N, D, torch.float16, seed=77)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    out, lse = cqsa().attention(qd, kd, vd, is_causal=True, return_lse=True)
    a = cqsa().attention_backward(qd, kd, vd, out, dod, lse, is_causal=True, grad_dtype=torch.float32)
    b = cqsa().attention_backward(qd, kd, vd, out, dod, lse, is_causal=True, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    h = cqsa().attention_backward(qd, kd, vd, out, dod, lse, is_causal=True)   # fp16 gradients
    torch.cuda.synchronize()
    for x, y in zip(a, h):
        assert y.dtype == torch.float16
        assert (x - y.float()).abs().max().item() <= 2e-3 * max(1.0, x.abs().max().item())


def test_backward_errors():
    m = cqsa()
    q, k, v, do = (t.to(DEV) for t in gen(1, 2, 2, 64, 64, 64, torch.float16, seed=1))
    out, lse = m.attention(q, k, v, is_causal=True, return_lse=True)
    # a pinned host operand takes the chunked path (dq then lives on the host); pageable memory is refused
    dq, dk, dv = m.attention_backward(q.cpu().pin_memory(), k, v, out, do, lse, is_causal=True)
    assert not dq.is_cuda and dk.is_cuda
    with pytest.raises(m.CqsaError, match="INVALID.*pinned"):
        m.attention_backward(q.cpu(), k, v, out, do, lse, is_causal=True)
    with pytest.raises(m.CqsaError, match="INVALID"):
        m.attention_backward(q, k, v, out, do.to(torch.bfloat16), lse, is_causal=True)


def test_autograd_through_attention():
    """attention() with requires_grad records the backward: loss = sum(out * dO) gives the oracle's
    gradients for dO."""
    B, Hq, Hkv, N, D = 1, 4, 2, 513, 64
    q, k, v, do = gen(B, Hq, Hkv, N, N, D, torch.float16, seed=91)
    rq, rk, rv = oracle.backward(q, k, v, do, causal=True, scale=1.0 / math.sqrt(D))
    qd, kd, vd = (t.to(DEV).requires_grad_(True) for t in (q, k, v))
    out = cqsa().attention(qd, kd, vd, is_causal=True)
    (out.float() * do.to(DEV).float()).sum().backward()
    torch.cuda.synchronize()
    for g, r in ((qd.grad, rq), (kd.grad, rk), (vd.grad, rv)):
        assert g.dtype == torch.float16
        assert rel_err(g.float(), r) <= 8 * U[torch.float16] + 2 ** -11   # + the fp16 rounding of the gradient


# The chunked backward (cqsa_attention_backward_ex): host-resident operands streamed in query chunks x
# key chunks (key chunks outermost, fp32 dQ/dK/dV accumulation), or forced chunks on the device.
STREAM_CASES = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal, q_chunk, kv_chunk, placement
    (1, 2, 2, 1300, 1300, 64, torch.float16, True, 512, 256, "host"),
    (1, 4, 1, 700, 2100, 128, torch.bfloat16, True, 256, 768, "host"),     # GQA 4:1, bottom-right causal
    (2, 2, 2, 900, 1100, 64, torch.float16, False, 384, 512, "host"),      # non-causal, ragged chunks
    (1, 4, 2, 1024, 1024, 128, torch.float16, True, 256, 256, "mixed"),    # device inputs, host gradients
    (1, 2, 2, 1536, 1536, 64, torch.bfloat16, True, 512, 512, "device"),   # forced chunks, resident
]


@pytest.mark.parametrize("case", STREAM_CASES, ids=lambda c: f"q{c[3]}k{c[4]}d{c[5]}{'c' if c[7] else 'n'}-{c[10]}")
def test_chunked_backward_parity(case):
    B, Hq, Hkv, Nq, Nk, D, dtype, causal, qc, kc, place = case
    say("chunked backward", case)
    q, k, v, do = gen(B, Hq, Hkv, Nq, Nk, D, dtype, seed=6000 + Nq + Nk + D)
    scale = 1.0 / math.sqrt(D)
    rq, rk, rv = oracle.backward(q, k, v, do, causal=causal, scale=scale)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    out, lse = cqsa().attention(qd, kd, vd, is_causal=causal, return_lse=True)
    if place == "host":
        args = [t.cpu().pin_memory() for t in (qd, kd, vd, out, dod, lse)]
    elif place == "mixed":
        args = [qd.cpu().pin_memory(), kd.cpu().pin_memory(), vd, out, dod, lse]   # grads follow q and k
    else:
        args = [qd, kd, vd, out, dod, lse]
    dq, dk, dv, info = cqsa().attention_backward(*args, is_causal=causal, grad_dtype=torch.float32, q_chunk=qc,
                                                 kv_chunk=kc, return_info=True)
    torch.cuda.synchronize()
    assert info["q_chunk"] == qc and info["kv_chunk"] == kc and info["chunk_pairs"] >= 2
    assert info["streamed"] == (0 if place == "device" else 1)
    if place != "device":
        assert not dq.is_cuda
    errs = {n: rel_err(g, r) for n, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv))}
    say("errors", errs)
    for n, e in errs.items():
        assert e <= 8 * U[dtype], (n, e)
    # against the single-pass backward on the same device inputs: equal up to the fp32 summation order
    g1 = cqsa().attention_backward(qd, kd, vd, out, dod, lse, is_causal=causal, grad_dtype=torch.float32)
    for n, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), g1):
        diff = float((a.cpu() - b.cpu()).abs().max()) / max(1.0, float(b.abs().max()))
        assert diff <= 1e-5, (n, diff)


def test_chunked_backward_budget_and_dtypes():
    """A budget that forces the planner's own chunking, fp16 gradients on the host (bitwise the same on
    a second call), and the budget error when even the smallest chunks do not fit."""
    B, H, N, D = 1, 4, 4096, 64
    q, k, v, do = gen(B, H, H, N, N, D, torch.float16, seed=6100)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    out, lse = cqsa().attention(qd, kd, vd, is_causal=True, return_lse=True)
    host = [t.cpu().pin_memory() for t in (qd, kd, vd, out, dod, lse)]
    # dq accumulator 4 MiB + statistics 128 KiB; 12 MB leaves room only for chunks below the full length
    dq, dk, dv, info = cqsa().attention_backward(*host, is_causal=True, mem_budget=12_000_000, return_info=True)
    assert dq.dtype == torch.float16 and not dq.is_cuda
    assert info["n_q_chunks"] * info["n_kv_chunks"] > 1 and info["workspace_bytes"] <= 0.85 * 12_000_000
    again = cqsa().attention_backward(*host, is_causal=True, mem_budget=12_000_000)
    assert all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip((dq, dk, dv), again))  # bitwise
    g1 = cqsa().attention_backward(qd, kd, vd, out, dod, lse, is_causal=True)
    for a, b in zip((dq, dk, dv), g1):
        assert float((a.float() - b.float().cpu()).abs().max()) <= 2 * 2.0 ** -11 * max(1.0, float(b.float().abs().max()))
    with pytest.raises(cqsa().CqsaError, match="BUDGET"):
        cqsa().attention_backward(*host, is_causal=True, mem_budget=1_000_000)


def test_chunked_backward_token_major_host_tensors():
    """Pinned host inputs stored token-major ([B, N, H, D]) move as one block per batch entry and chunk
    (the gradients are head-major pinned tensors here: each operand keeps its own layout)."""
    B, Hq, Hkv, N, D = 2, 4, 2, 1100, 64
    say("chunked backward, token-major host")
    q, k, v, do = gen(B, Hq, Hkv, N, N, D, torch.float16, seed=6200)
    rq, rk, rv = oracle.backward(q, k, v, do, causal=True, scale=1.0 / math.sqrt(D))
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    out, lse = cqsa().attention(qd, kd, vd, is_causal=True, return_lse=True)

    def tm(t):   # [B, N, H, D] storage in pinned memory, viewed as [B, H, N, D]
        x = torch.empty((t.shape[0], t.shape[2], t.shape[1], t.shape[3]), dtype=t.dtype, pin_memory=True)
        x.copy_(t.transpose(1, 2))
        return x.transpose(1, 2)

    args = [tm(t.cpu()) for t in (qd, kd, vd, out, dod)] + [lse.cpu().pin_memory()]
    dq, dk, dv = cqsa().attention_backward(*args, is_causal=True, grad_dtype=torch.float32, q_chunk=256, kv_chunk=512)
    for n, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        assert not g.is_cuda
        e = rel_err(g, r)
        assert e <= 8 * U[torch.float16], (n, e)
