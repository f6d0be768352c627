"""Pins for the FP64 reference: each test checks it against something other than itself.

- library routines: PyTorch's scaled_dot_product_attention and logsumexp in float64;
- brute force in long double with no max subtraction on tiny inputs;
- closed forms (q = 0, constant v, a single visible key, causal row 0);
- invariants (weights sum to 1, any KV split merged equals the unsplit result, GQA equals
  MHA on repeated K/V, key permutations in the non-causal case);
- hand-derived worked examples stored under tests/golden/.
A dropped term, a wrong sign or index, a transposed operand or a wrong causal offset in the
reference fails at least one of these.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def rand_qkv(B, Hq, Hkv, Nq, Nk, D, dtype=torch.float16, seed=0, sigma=1.0):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(B, Hq, Nq, D, generator=g) * sigma).to(dtype)
    k = (torch.randn(B, Hkv, Nk, D, generator=g) * sigma).to(dtype)
    v = torch.randn(B, Hkv, Nk, D, generator=g).to(dtype)
    return q, k, v


def f32(x):
    return float(np.float32(x))


def scores64(q, k, scale):
    """Plain float64 scores with K/V heads repeated to the query heads."""
    g = q.shape[1] // k.shape[1]
    kk = k.double().repeat_interleave(g, dim=1)
    return f32(scale) * (q.double() @ kk.transpose(-1, -2))


def causal_mask(Nq, Nk):
    i = torch.arange(Nq)[:, None]
    j = torch.arange(Nk)[None, :]
    return j <= i + (Nk - Nq)


# ---------------------------------------------------------------- exact input decoding

def test_fp16_decode_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_double(int(b)) for b in bits])
    both_nan = np.isnan(want) & np.isnan(got)
    assert np.array_equal(want[~both_nan], got[~both_nan])
    assert np.array_equal(np.isnan(want), np.isnan(got))


def test_bf16_decode_every_bit_pattern():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    want = bits.view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_to_double(int(b) & 0xFFFF) for b in bits.numpy()])
    both_nan = np.isnan(want) & np.isnan(got)
    assert np.array_equal(want[~both_nan], got[~both_nan])
    assert np.array_equal(np.isnan(want), np.isnan(got))


# ---------------------------------------------------------------- hand-derived examples

def _eval(expr):
    return eval(expr, {"__builtins__": {}}, {"e": math.e, "log": math.log})


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_golden_worked_examples(dtype):
    data = json.load(open(GOLDEN))
    assert len(data["examples"]) >= 4
    for ex in data["examples"]:
        q = torch.tensor(ex["q"], dtype=torch.float64).to(dtype)
        k = torch.tensor(ex["k"], dtype=torch.float64).to(dtype)
        v = torch.tensor(ex["v"], dtype=torch.float64).to(dtype)
        o, lse = oracle.attention(q, k, v, causal=ex["causal"], scale=ex["scale"])
        want_o = np.vectorize(_eval, otypes=[np.float64])(np.array(ex["o"], dtype=object)).astype(np.float64)
        want_lse = np.vectorize(_eval, otypes=[np.float64])(np.array(ex["lse"], dtype=object)).astype(np.float64)
        np.testing.assert_allclose(o.numpy(), want_o, rtol=1e-14, atol=1e-15, err_msg=ex["name"])
        np.testing.assert_allclose(lse.numpy(), want_lse, rtol=1e-14, atol=1e-15, err_msg=ex["name"])


# ---------------------------------------------------------------- brute force (long double)

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 1, 1), (1, 2, 1, 5, 7, 3), (2, 4, 2, 8, 8, 4), (1, 3, 3, 3, 6, 2)])
def test_bruteforce_longdouble(causal, shape):
    B, Hq, Hkv, Nq, Nk, D = shape
    q, k, v = rand_qkv(B, Hq, Hkv, Nq, Nk, D, seed=sum(shape) + causal)
    scale = 0.7
    o, lse = oracle.attention(q, k, v, causal=causal, scale=scale)
    ld = np.longdouble
    qn = q.double().numpy().astype(ld)
    kn = k.double().numpy().astype(ld)
    vn = v.double().numpy().astype(ld)
    g = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            for i in range(Nq):
                vis = [j for j in range(Nk) if (not causal) or j <= i + Nk - Nq]
                s = np.array([ld(f32(scale)) * np.sum(qn[b, h, i] * kn[b, h // g, j]) for j in vis], dtype=ld)
                assert np.all(np.abs(s) <= 5)
                e = np.exp(s)                       # no max subtraction
                w = e / np.sum(e)
                want = np.sum(w[:, None] * vn[b, h // g, vis], axis=0)
                np.testing.assert_allclose(o[b, h, i].numpy(), want.astype(np.float64), rtol=1e-14, atol=1e-15)
                assert abs(lse[b, h, i].item() - float(np.log(np.sum(e)))) < 1e-14


# ---------------------------------------------------------------- library routine: torch SDPA in float64

@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("case", ["noncausal_rect", "causal_square", "gqa_causal", "gqa_noncausal"])
def test_matches_torch_sdpa_float64(dtype, case):
    if case == "noncausal_rect":
        B, Hq, Hkv, Nq, Nk, D, causal = 2, 3, 3, 37, 91, 64, False
    elif case == "causal_square":
        B, Hq, Hkv, Nq, Nk, D, causal = 1, 2, 2, 130, 130, 64, True
    elif case == "gqa_causal":
        B, Hq, Hkv, Nq, Nk, D, causal = 1, 8, 2, 67, 67, 128, True
    else:
        B, Hq, Hkv, Nq, Nk, D, causal = 2, 4, 1, 19, 45, 128, False
    q, k, v = rand_qkv(B, Hq, Hkv, Nq, Nk, D, dtype=dtype, seed=11)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attention(q, k, v, causal=causal, scale=scale)
    ref = F.scaled_dot_product_attention(q.double(), k.double(), v.double(), is_causal=causal, scale=f32(scale),
                                         enable_gqa=(Hq != Hkv))
    torch.testing.assert_close(o, ref, rtol=1e-12, atol=1e-12)
    s = scores64(q, k, scale)
    if causal:
        s = s.masked_fill(~causal_mask(Nq, Nk), float("-inf"))
    torch.testing.assert_close(lse, torch.logsumexp(s, dim=-1), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- invariants and closed forms

@pytest.mark.parametrize("causal", [False, True])
def test_weights_sum_to_one(causal):
    q, k, v = rand_qkv(1, 2, 1, 50, 80, 64, seed=5, sigma=2.0)
    scale = 0.125
    _, lse = oracle.attention(q, k, v, causal=causal, scale=scale)
    s = scores64(q, k, scale)
    w = torch.exp(s - lse[..., None])
    if causal:
        w = w.masked_fill(~causal_mask(50, 80), 0.0)
    torch.testing.assert_close(w.sum(-1), torch.ones_like(lse), rtol=0, atol=1e-13)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_causal_row0_is_v0(dtype):
    q, k, v = rand_qkv(2, 4, 2, 33, 33, 64, dtype=dtype, seed=3)
    scale = 0.125
    o, lse = oracle.attention(q, k, v, causal=True, scale=scale)
    vrep = v.double().repeat_interleave(2, dim=1)
    assert torch.equal(o[:, :, 0, :], vrep[:, :, 0, :])
    s00 = scores64(q, k, scale)[:, :, 0, 0]
    torch.testing.assert_close(lse[:, :, 0], s00, rtol=0, atol=1e-14)


@pytest.mark.parametrize("nq,nk", [(16, 16), (5, 23), (1, 9)])
def test_q_zero_closed_form(nq, nk):
    """q = 0: every visible weight is 1, so O_i is the mean of the visible values and
    lse_i = ln(#visible), with #visible = Nk - Nq + i + 1 under the causal mask."""
    _, k, v = rand_qkv(1, 2, 2, nq, nk, 64, seed=9)
    q = torch.zeros(1, 2, nq, 64, dtype=torch.float16)
    o, lse = oracle.attention(q, k, v, causal=True, scale=0.125)
    for i in range(nq):
        cnt = nk - nq + i + 1
        torch.testing.assert_close(o[:, :, i], v[:, :, :cnt].double().mean(2), rtol=1e-14, atol=1e-14)
        torch.testing.assert_close(lse[:, :, i], torch.full((1, 2), math.log(cnt), dtype=torch.float64),
                                   rtol=0, atol=1e-15)


def test_bottom_right_is_tail_of_square():
    q, k, v = rand_qkv(1, 2, 2, 40, 40, 64, seed=21)
    o_sq, lse_sq = oracle.attention(q, k, v, causal=True, scale=0.125)
    o_t, lse_t = oracle.attention(q[:, :, 25:].contiguous(), k, v, causal=True, scale=0.125)
    assert torch.equal(o_t, o_sq[:, :, 25:])
    assert torch.equal(lse_t, lse_sq[:, :, 25:])


def test_gqa_equals_mha_on_repeated_kv():
    q, k, v = rand_qkv(2, 8, 2, 21, 34, 64, seed=4)
    o, lse = oracle.attention(q, k, v, causal=True, scale=0.125)
    kr = k.repeat_interleave(4, dim=1).contiguous()
    vr = v.repeat_interleave(4, dim=1).contiguous()
    o2, lse2 = oracle.attention(q, kr, vr, causal=True, scale=0.125)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_constant_v_and_single_key():
    q, k, _ = rand_qkv(1, 1, 1, 12, 12, 64, seed=8)
    v = torch.full((1, 1, 12, 64), 0.375, dtype=torch.float16)
    o, _ = oracle.attention(q, k, v, causal=False, scale=0.125)
    torch.testing.assert_close(o, torch.full_like(o, 0.375), rtol=0, atol=1e-15)
    q1, k1, v1 = rand_qkv(1, 1, 1, 3, 1, 64, seed=8)
    o1, lse1 = oracle.attention(q1, k1, v1, causal=False, scale=0.125)
    assert torch.equal(o1[0, 0], v1[0, 0, 0].double().expand(3, 64))
    torch.testing.assert_close(lse1, scores64(q1, k1, 0.125)[..., 0], rtol=0, atol=1e-15)


def test_zero_scale_gives_uniform_weights():
    q, k, v = rand_qkv(1, 1, 1, 7, 19, 64, seed=12)
    o, lse = oracle.attention(q, k, v, causal=False, scale=0.0)
    torch.testing.assert_close(o[0, 0], v[0, 0].double().mean(0).expand(7, 64), rtol=1e-14, atol=1e-14)
    torch.testing.assert_close(lse, torch.full_like(lse, math.log(19)), rtol=0, atol=1e-15)


def test_noncausal_key_permutation_invariance():
    q, k, v = rand_qkv(1, 2, 2, 9, 31, 64, seed=13)
    perm = torch.randperm(31, generator=torch.Generator().manual_seed(1))
    o, lse = oracle.attention(q, k, v, causal=False, scale=0.125)
    o2, lse2 = oracle.attention(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), causal=False, scale=0.125)
    torch.testing.assert_close(o, o2, rtol=1e-13, atol=1e-14)
    torch.testing.assert_close(lse, lse2, rtol=1e-14, atol=1e-14)


def test_strided_token_major_layout():
    q, k, v = rand_qkv(2, 4, 2, 17, 29, 64, seed=14)
    o, lse = oracle.attention(q, k, v, causal=True, scale=0.125)
    tm = lambda t: t.transpose(1, 2).contiguous().transpose(1, 2)   # [B,N,H,D] storage, [B,H,N,D] view
    o2, lse2 = oracle.attention(tm(q), tm(k), tm(v), causal=True, scale=0.125)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


# ---------------------------------------------------------------- partial triples and the exact merge

def test_identity_partial_and_merge_identity():
    q, k, v = rand_qkv(1, 1, 1, 8, 8, 64, seed=15)
    empty = oracle.attention_rows(q, k, v, causal=False, scale=0.125, key_range=(3, 3), partial=True)
    assert np.all(empty["m"] == -np.inf) and np.all(empty["l"] == 0) and np.all(empty["o"] == 0)
    full = oracle.attention_rows(q, k, v, causal=False, scale=0.125, partial=True)
    for a, b in ((empty, full), (full, empty)):
        mg = oracle.merge(a, b)
        assert np.array_equal(mg["o"], full["o"]) and np.array_equal(mg["l"], full["l"])
    both = oracle.merge(empty, empty)
    assert np.all(both["m"] == -np.inf) and not np.any(np.isnan(both["o"])) and np.all(both["l"] == 0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("trial", range(4))
def test_any_split_merged_equals_unsplit(causal, trial):
    rng = np.random.default_rng(100 + trial)
    Nq, Nk = 23, 57
    q, k, v = rand_qkv(1, 2, 1, Nq, Nk, 64, seed=trial, sigma=1.5)
    full = oracle.attention_rows(q, k, v, causal=causal, scale=0.125)
    cuts = sorted(set([0, Nk] + list(rng.integers(0, Nk + 1, size=rng.integers(1, 9)))))
    cuts = cuts[:1] + [cuts[1]] * (trial % 2) + cuts[1:]        # sometimes an empty chunk
    if trial == 3:
        cuts = [0, 1, 2] + [c for c in cuts if c > 2]            # size-1 chunks
    parts = [oracle.attention_rows(q, k, v, causal=causal, scale=0.125, key_range=(a, b), partial=True)
             for a, b in zip(cuts[:-1], cuts[1:])]
    order = rng.permutation(len(parts))
    acc = parts[order[0]]
    for idx in order[1:]:
        acc = oracle.merge(acc, parts[idx])
    fin = oracle.normalise(acc)
    np.testing.assert_allclose(fin["o"], full["o"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(fin["lse"], full["lse"], rtol=1e-13, atol=1e-13)


def test_partial_normalises_to_full():
    q, k, v = rand_qkv(1, 2, 2, 10, 30, 64, seed=16)
    p = oracle.attention_rows(q, k, v, causal=True, scale=0.125, partial=True)
    f = oracle.attention_rows(q, k, v, causal=True, scale=0.125)
    n = oracle.normalise(p)
    np.testing.assert_allclose(n["o"], f["o"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(n["lse"], f["lse"], rtol=1e-15, atol=1e-15)


def test_sampled_rows_equal_full_rows():
    q, k, v = rand_qkv(2, 2, 1, 40, 40, 64, seed=17)
    o, lse = oracle.attention(q, k, v, causal=True, scale=0.125)
    rows = np.array([[1, 0, 39], [0, 1, 0], [1, 1, 17]], dtype=np.int64)
    r = oracle.attention_rows(q, k, v, causal=True, scale=0.125, rows=rows)
    for n, (b, h, i) in enumerate(rows):
        assert np.array_equal(r["o"][n], o[b, h, i].numpy())
        assert r["lse"][n] == lse[b, h, i].item()


def test_thread_count_does_not_change_results():
    q, k, v = rand_qkv(1, 4, 4, 64, 64, 64, seed=18)
    a = oracle.attention_rows(q, k, v, causal=True, scale=0.125, threads=1)
    b = oracle.attention_rows(q, k, v, causal=True, scale=0.125, threads=7)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])


def test_large_logits_stay_finite():
    """Logits near +-200 overflow exp() without the max subtraction; the reference must not."""
    q, k, v = rand_qkv(1, 1, 1, 16, 64, 64, seed=19, sigma=6.0)
    o, lse = oracle.attention(q, k, v, causal=False, scale=0.5)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    ref = F.scaled_dot_product_attention(q.double(), k.double(), v.double(), scale=0.5)
    torch.testing.assert_close(o, ref, rtol=1e-12, atol=1e-12)
