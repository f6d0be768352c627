"""Pins of the FP64 oracle's gradients (oracle.backward) to things other than itself: PyTorch's
float64 autograd through the SDPA math on the CPU, finite differences of the oracle's own forward,
closed forms and invariants of the softmax derivative."""
import math

import numpy as np
import pytest
import torch

import oracle


def grid(shape, seed, step=2.0 ** -4, lim=3.0, dtype=torch.float16):
    """Values on a coarse grid (exact in fp16 and bf16; x +- 2^-8 stays exact for |x| < 4 in fp16)."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randint(int(-lim / step), int(lim / step) + 1, shape, generator=g).double() * step
    return x.to(dtype)


def torch_grads(q, k, v, dout, causal, scale):
    Hq, Hkv = q.shape[1], k.shape[1]
    qd, kd, vd = (t.double().clone().requires_grad_(True) for t in (q, k, v))
    kr = kd.repeat_interleave(Hq // Hkv, dim=1)
    vr = vd.repeat_interleave(Hq // Hkv, dim=1)
    s = scale * qd @ kr.transpose(-1, -2)
    if causal:
        Nq, Nk = q.shape[2], k.shape[2]
        i = torch.arange(Nq)[:, None]
        j = torch.arange(Nk)[None, :]
        s = s.masked_fill(j > i + (Nk - Nq), float("-inf"))
    o = torch.softmax(s, dim=-1) @ vr
    o.backward(dout.double())
    return qd.grad, kd.grad, vd.grad


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,causal,D,dtype", [
    (1, 2, 2, 7, 11, False, 16, torch.float16),
    (2, 2, 2, 13, 13, True, 8, torch.bfloat16),
    (1, 4, 2, 9, 17, True, 16, torch.float16),     # GQA, bottom-right causal
    (1, 3, 1, 5, 5, False, 32, torch.bfloat16),
])
def test_backward_matches_float64_autograd(B, Hq, Hkv, Nq, Nk, causal, D, dtype):
    q = grid((B, Hq, Nq, D), 1, dtype=dtype)
    k = grid((B, Hkv, Nk, D), 2, dtype=dtype)
    v = grid((B, Hkv, Nk, D), 3, dtype=dtype)
    do = grid((B, Hq, Nq, D), 4, dtype=dtype)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    dq, dk, dv = oracle.backward(q, k, v, do, causal=causal, scale=scale)
    tq, tk, tv = torch_grads(q, k, v, do, causal, scale)
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        assert torch.allclose(a, b, rtol=1e-10, atol=1e-11)


def test_backward_matches_finite_differences_of_the_forward():
    """L = sum(O * R): dL/dx from the oracle's backward with dO = R against central differences of the
    oracle's forward, with perturbations exactly representable in fp16."""
    B, Hq, Hkv, Nq, Nk, D = 1, 2, 1, 5, 6, 8
    q = grid((B, Hq, Nq, D), 11, lim=1.0)
    k = grid((B, Hkv, Nk, D), 12, lim=1.0)
    v = grid((B, Hkv, Nk, D), 13, lim=1.0)
    R = grid((B, Hq, Nq, D), 14, lim=1.0)
    scale = 0.5
    dq, dk, dv = oracle.backward(q, k, v, R, causal=True, scale=scale)
    h = 2.0 ** -8

    def loss(qq, kk, vv):
        o, _ = oracle.attention(qq, kk, vv, causal=True, scale=scale)
        return float((o * R.double()).sum())

    rng = np.random.default_rng(0)
    for name, t, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in t.shape)
            tp, tm = t.clone(), t.clone()
            tp[idx] = float(t[idx]) + h
            tm[idx] = float(t[idx]) - h
            assert float(tp[idx]) - float(t[idx]) == h and float(t[idx]) - float(tm[idx]) == h
            args_p = [q, k, v]
            args_m = [q, k, v]
            pos = "qkv".index(name)
            args_p[pos], args_m[pos] = tp, tm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - float(g[idx])) <= 1e-4 * max(1.0, abs(float(g[idx]))), (name, idx, fd, float(g[idx]))


def test_closed_forms_and_invariants():
    B, Hq, Hkv, N, D = 1, 4, 2, 24, 16
    q = grid((B, Hq, N, D), 21)
    k = grid((B, Hkv, N, D), 22)
    v = grid((B, Hkv, N, D), 23)
    do = grid((B, Hq, N, D), 24)
    scale = 0.25
    for causal in (False, True):
        dq, dk, dv = oracle.backward(q, k, v, do, causal=causal, scale=scale)
        # each row's dS sums to 0, so sum_j dK_j = 0 for every key/value head
        assert dk.sum(dim=2).abs().max().item() < 1e-10
        # each row's P sums to 1, so sum_j dV_j = sum over the group's heads and rows of dO
        want = do.double().reshape(B, Hkv, Hq // Hkv, N, D).sum(dim=(2, 3))
        assert torch.allclose(dv.sum(dim=2), want, atol=1e-10)
        # shifting every key by one vector leaves dQ unchanged (the shift cancels inside dS)
        k2 = (k.double() + 0.5).to(k.dtype)
        assert torch.equal(k2.double(), k.double() + 0.5)
        dq2, _, _ = oracle.backward(q, k2, v, do, causal=causal, scale=scale)
        assert torch.allclose(dq, dq2, atol=1e-10)
    # causal row 0 sees one key: P = 1, dS = 0, so dQ_0 = 0
    dq, _, _ = oracle.backward(q, k, v, do, causal=True, scale=scale)
    assert dq[:, :, 0].abs().max().item() == 0.0
    # q = 0: uniform P; dK = 0 and dV_j = (sum_i dO_i) / N for every j (non-causal)
    z = torch.zeros_like(q)
    dq, dk, dv = oracle.backward(z, k, v, do, causal=False, scale=scale)
    assert dk.abs().max().item() == 0.0
    want = do.double().reshape(B, Hkv, Hq // Hkv, N, D).sum(dim=(2, 3))[:, :, None, :] / N
    assert torch.allclose(dv, want.expand_as(dv), atol=1e-12)


def test_gqa_gradients_equal_mha_on_repeated_kv():
    B, Hq, Hkv, N, D = 1, 4, 2, 10, 8
    q = grid((B, Hq, N, D), 31)
    k = grid((B, Hkv, N, D), 32)
    v = grid((B, Hkv, N, D), 33)
    do = grid((B, Hq, N, D), 34)
    dq, dk, dv = oracle.backward(q, k, v, do, causal=True, scale=0.3)
    kr, vr = k.repeat_interleave(2, dim=1), v.repeat_interleave(2, dim=1)
    dq2, dk2, dv2 = oracle.backward(q, kr, vr, do, causal=True, scale=0.3)
    assert torch.allclose(dq, dq2, atol=1e-12)
    assert torch.allclose(dk, dk2.reshape(B, Hkv, 2, N, D).sum(dim=2), atol=1e-12)
    assert torch.allclose(dv, dv2.reshape(B, Hkv, 2, N, D).sum(dim=2), atol=1e-12)
