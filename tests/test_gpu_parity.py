"""GPU parity: the HIP library (through its C ABI) against the FP64 oracle on the same seeded inputs.

Small problems are compared element by element; the large measured shapes are compared on sampled
rows (first/last rows, rows around chunk and tile edges, seeded random rows in every head).
"""
import math
import sys

import numpy as np
import pytest
import torch

import synth
from parity_util import compare, reference, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def cqsa():
    import exact_long_context_cqsa_amd as m
    return m


def say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def gen(B, Hq, Hkv, Nq, Nk, D, dtype, seed, sigma=1.0):
    q = synth.normal((B, Hq, Nq, D), seed=seed, tensor_id=0, sigma=sigma, dtype=dtype)
    k = synth.normal((B, Hkv, Nk, D), seed=seed, tensor_id=1, sigma=sigma, dtype=dtype)
    v = synth.normal((B, Hkv, Nk, D), seed=seed, tensor_id=2, dtype=dtype)
    return q, k, v


SMALL = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal
    (1, 1, 1, 1024, 1024, 64, torch.float16, True),
    (1, 2, 2, 300, 300, 64, torch.float16, True),        # ragged query and key tails
    (2, 3, 3, 77, 513, 64, torch.float16, False),        # non-causal, Nq < Nk
    (1, 2, 2, 700, 129, 64, torch.bfloat16, False),      # non-causal, Nq > Nk
    (1, 4, 1, 257, 1000, 128, torch.bfloat16, True),     # GQA 4:1, bottom-right causal
    (2, 8, 2, 130, 130, 128, torch.float16, True),       # GQA, square causal
    (1, 2, 2, 1, 1, 64, torch.float16, True),            # one query, one key
    (1, 2, 2, 1, 4099, 128, torch.float16, True),        # one query at the end of 4099 keys
    (1, 1, 1, 64, 64, 64, torch.bfloat16, True),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"B{c[0]}H{c[1]}x{c[2]}q{c[3]}k{c[4]}d{c[5]}"
                         f"{'f16' if c[6] == torch.float16 else 'bf16'}{'c' if c[7] else 'n'}")
def test_small_full_parity(case):
    B, Hq, Hkv, Nq, Nk, D, dtype, causal = case
    say("small", case)
    q, k, v = gen(B, Hq, Hkv, Nq, Nk, D, dtype, seed=1000 + Nq + Nk + D)
    scale = 1.0 / math.sqrt(D)
    ref = reference(q, k, v, causal=causal, scale=scale)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse = cqsa().attention(qd, kd, vd, is_causal=causal, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    compare(out, lse, ref, dtype, label=f"mono {case}")
    # a forced split (LSE merges) in both merge modes, and forced Q chunks
    for kw in ({"kv_chunk": 96, "merge": 1}, {"kv_chunk": 200, "merge": 2}, {"kv_chunk": 128, "q_chunk": 100}):
        out2, lse2 = cqsa().attention(qd, kd, vd, is_causal=causal, out_dtype=torch.float32, return_lse=True, **kw)
        torch.cuda.synchronize()
        compare(out2, lse2, ref, dtype, label=f"{kw} {case}")


VARIANT_CASES = [SMALL[1], SMALL[2], SMALL[3], SMALL[4], SMALL[7]]


@pytest.mark.parametrize("variant", [1, 2, 3, 4, 5, 6, 7])
def test_every_forward_kernel_variant(variant, test_controls):
    """The non-default forward kernels (selected by cqsa_set_test_controls) on ragged, GQA,
    non-causal and long-key cases, monolithic and with a forced KV split."""
    test_controls(variant, -1)
    for case in VARIANT_CASES:
        B, Hq, Hkv, Nq, Nk, D, dtype, causal = case
        say("variant", variant, case)
        q, k, v = gen(B, Hq, Hkv, Nq, Nk, D, dtype, seed=2000 + Nq + Nk + D)
        ref = reference(q, k, v, causal=causal, scale=1.0 / math.sqrt(D))
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        for kw in ({}, {"kv_chunk": 200, "merge": 2}):
            out, lse = cqsa().attention(qd, kd, vd, is_causal=causal, out_dtype=torch.float32, return_lse=True, **kw)
            torch.cuda.synchronize()
            compare(out, lse, ref, dtype, label=f"variant {variant} {kw} {case}")


CQS_CASES = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal, cqs
    (1, 2, 2, 1000, 1000, 64, torch.float16, True, 7),                  # c = 7, set (0, 1, 3)
    (1, 2, 2, 1001, 1001, 64, torch.float16, False, 7),                 # ragged parts, non-causal
    (1, 4, 1, 513, 1300, 128, torch.bfloat16, True, (3, (0, 1))),       # GQA, bottom-right causal
    (2, 2, 2, 777, 777, 64, torch.bfloat16, True, (10, (0, 1, 2, 3, 6))),  # a covering, non-perfect set
    (1, 1, 1, 30, 30, 64, torch.float16, True, 31),                     # parts of zero and one row
]


@pytest.mark.parametrize("case", CQS_CASES, ids=lambda c: f"q{c[3]}k{c[4]}d{c[5]}{'c' if c[7] else 'n'}-cqs{c[8]}")
def test_cqs_schedule_parity(case):
    """The cyclic quorum-set schedule against the oracle, device-resident and streamed from pinned
    host memory (out and lse on the host too)."""
    B, Hq, Hkv, Nq, Nk, D, dtype, causal, cqs = case
    say("cqs", case)
    q, k, v = gen(B, Hq, Hkv, Nq, Nk, D, dtype, seed=3000 + Nq + Nk + D)
    ref = reference(q, k, v, causal=causal, scale=1.0 / math.sqrt(D))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse, info = cqsa().attention(qd, kd, vd, is_causal=causal, out_dtype=torch.float32, return_lse=True,
                                      return_info=True, cqs=cqs)
    torch.cuda.synchronize()
    compare(out, lse, ref, dtype, label=f"cqs device {case}")
    c = cqs if isinstance(cqs, int) else cqs[0]
    assert info["cqs_c"] == c and info["chunk_pairs"] >= 1
    qh, kh, vh = q.pin_memory(), k.pin_memory(), v.pin_memory()
    out_h, lse_h, info_h = cqsa().attention(qh, kh, vh, is_causal=causal, out_dtype=torch.float32,
                                            return_lse=True, return_info=True, cqs=cqs)
    assert not out_h.is_cuda and info_h["streamed"] == 1 and info_h["h2d_bytes"] > 0
    compare(out_h, lse_h, ref, dtype, label=f"cqs host {case}")


def test_cqs_causal_n32768_matches_grid_and_oracle():
    """The 32K causal bench shape under the quorum-set schedule (c = 7 and c = 31): sampled rows
    against the oracle, and the whole output against the monolithic pass."""
    w = synth.workload(1)
    say("cqs workload", w.name)
    q, k, v, _ = synth.make_inputs(w)
    rows = sample_rows(1, w.Hq, w.Nq, seed=7, n_random=64, edge=16,
                       boundaries=[w.Nq * p // 7 for p in range(8)] + [w.Nq * p // 31 for p in range(32)])
    ref = reference(q, k, v, causal=True, scale=w.scale, rows=rows)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    mono = cqsa().attention(qd, kd, vd, is_causal=True, out_dtype=torch.float32)
    for c in (7, 31):
        out, lse, info = cqsa().attention(qd, kd, vd, is_causal=True, out_dtype=torch.float32, return_lse=True,
                                          return_info=True, cqs=c)
        torch.cuda.synchronize()
        assert info["chunk_pairs"] == c * (c + 1) // 2
        compare(out, lse, ref, w.dtype, rows=rows, label=f"cqs c={c}")
        assert (out - mono).abs().max().item() <= 1e-3


def test_cqs_streamed_from_host_reduced():
    """Host-resident 131072-token causal case (the 4M recipe, shrunk) under c = 13 with a small budget."""
    w = synth.workload(3)
    say("cqs streamed reduced")
    q, k, v, _ = synth.make_inputs(w, nq=131072, nk=131072, pin=True)
    out, lse, info = cqsa().attention(q, k, v, is_causal=True, mem_budget=2 * 10**9, return_lse=True,
                                      return_info=True, cqs=13)
    assert info["streamed"] == 1 and info["cqs_subproblems"] == 13
    rows = sample_rows(1, w.Hq, 131072, seed=9, n_random=48, edge=8,
                       boundaries=[131072 * p // 13 for p in range(14)], heads=range(0, w.Hq, 3))
    ref = reference(q, k, v, causal=True, scale=w.scale, rows=rows)
    compare(out, lse, ref, w.dtype, rows=rows, label="cqs streamed 131072")


# Split-P mode (P = hi + lo, two PV accumulator chains): error bound from the arithmetic that
# remains (fp32 score accumulation, v_exp_f32, the lo part's rounding: 2^-22 of p for fp16, 2^-16 for
# bf16, fp32 accumulation), with a margin of about ten.
SPLIT_TOL = {torch.float16: 2e-5, torch.bfloat16: 1e-4}


@pytest.mark.parametrize("case", [SMALL[0], SMALL[2], SMALL[3], SMALL[4], SMALL[5], SMALL[7]],
                         ids=lambda c: f"q{c[3]}k{c[4]}d{c[5]}{'f16' if c[6] == torch.float16 else 'bf16'}")
def test_split_p_precision(case):
    """precision=1 against the oracle at the tight bound, and tighter than the default mode;
    monolithic, with a forced KV split, and streamed from pinned host memory."""
    B, Hq, Hkv, Nq, Nk, D, dtype, causal = case
    say("split-P", case)
    q, k, v = gen(B, Hq, Hkv, Nq, Nk, D, dtype, seed=4000 + Nq + Nk + D)
    ref = reference(q, k, v, causal=causal, scale=1.0 / math.sqrt(D))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)

    def err(out):
        return float(np.abs(out.detach().double().cpu().numpy() - ref["o"].reshape(out.shape)).max())

    base = cqsa().attention(qd, kd, vd, is_causal=causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    e_base = err(base)
    for kw in ({}, {"kv_chunk": 200}, {"kv_chunk": 200, "merge": 1}):   # the fused fold, then the merge kernel
        out, lse = cqsa().attention(qd, kd, vd, is_causal=causal, out_dtype=torch.float32, return_lse=True,
                                    precision=1, **kw)
        torch.cuda.synchronize()
        compare(out, lse, ref, dtype, label=f"split {kw} {case}")
        e = err(out)
        assert e <= SPLIT_TOL[dtype], (kw, e)
        assert e < e_base or e_base <= SPLIT_TOL[dtype] / 4, (e, e_base)
    outh = cqsa().attention(q.pin_memory(), k.pin_memory(), v.pin_memory(), is_causal=causal,
                            out_dtype=torch.float32, precision=1)
    assert err(outh) <= SPLIT_TOL[dtype]


def test_split_p_bench_shape_sampled():
    """The 32K causal D=64 fp16 workload in split-P mode, sampled rows, at the tight bound."""
    w = synth.workload(1)
    q, k, v, _ = synth.make_inputs(w)
    rows = sample_rows(1, w.Hq, w.Nq, seed=11, n_random=48, edge=8)
    ref = reference(q, k, v, causal=True, scale=w.scale, rows=rows)
    out = cqsa().attention(q.to(DEV), k.to(DEV), v.to(DEV), is_causal=True, out_dtype=torch.float32, precision=1)
    torch.cuda.synchronize()
    b, h, i = (torch.from_numpy(rows[:, c]) for c in range(3))
    got = out.cpu()[b, h, i].double().numpy()
    assert float(np.abs(got - ref["o"]).max()) <= SPLIT_TOL[torch.float16]


def test_causal_n1024_four_kv_chunks_merged():
    """1024 causal rows, D=64, fp16, KV chunk 256: each Q block folds its visible chunks by LSE."""
    w = synth.workload(0)
    say("workload", w.name)
    q, k, v, _ = synth.make_inputs(w)
    ref = reference(q, k, v, causal=True, scale=w.scale)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for merge in (1, 2):
        out, lse, info = cqsa().attention(qd, kd, vd, is_causal=True, kv_chunk=256, merge=merge,
                                          out_dtype=torch.float32, return_lse=True, return_info=True)
        torch.cuda.synchronize()
        assert info["n_kv_chunks"] == 4 and info["chunk_pairs"] == 4 and info["merges"] == 3
        compare(out, lse, ref, torch.float16, label=f"causal 1024 merge={merge}")
    # the default output dtype is the input's
    out16 = cqsa().attention(qd, kd, vd, is_causal=True, kv_chunk=256)
    assert out16.dtype == torch.float16
    compare(out16, None, ref, torch.float16, label="causal 1024 fp16 out")


def test_fwd_partial_matches_oracle_partial():
    q, k, v = gen(1, 2, 1, 200, 333, 64, torch.float16, seed=7)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for lo, hi in ((0, 333), (50, 150), (10, 10), (300, 333), (0, 1)):
        say("partial", lo, hi)
        o, ml = cqsa().fwd_partial(qd, kd, vd, is_causal=True, scale=0.125, kv_begin=lo, kv_end=hi)
        torch.cuda.synchronize()
        ref = reference(q, k, v, causal=True, scale=0.125)  # normalised, for the O scale
        part = __import__("oracle").attention_rows(q, k, v, causal=True, scale=0.125, key_range=(lo, hi),
                                                   partial=True)
        m = ml[..., 0].reshape(-1).double().cpu().numpy()
        l = ml[..., 1].reshape(-1).double().cpu().numpy()
        oo = o.reshape(-1, 64).double().cpu().numpy()
        empty = part["l"] == 0
        assert np.all(np.isneginf(m[empty])) and np.all(l[empty] == 0) and np.all(oo[empty] == 0)
        ne = ~empty
        if ne.any():
            # compare the normalised partial and its lse, which do not depend on the choice of m
            np.testing.assert_allclose(oo[ne] / l[ne, None], part["o"][ne] / part["l"][ne, None], atol=4e-3, rtol=0)
            lse_g = m[ne] + np.log(l[ne])
            lse_r = part["m"][ne] + np.log(part["l"][ne])
            assert np.max(np.abs(lse_g - lse_r) / np.maximum(1, np.abs(lse_r))) < 1e-4
        del ref


def test_lse_merge_kernel_matches_oracle_merge():
    rng = np.random.default_rng(3)
    rows, D = 1000, 128
    parts64 = []
    for p in range(3):
        m = rng.normal(0, 5, rows)
        m[rng.random(rows) < 0.2] = -np.inf                  # identities
        l = np.where(np.isinf(m), 0.0, rng.uniform(1, 50, rows))
        o = np.where(np.isinf(m)[:, None], 0.0, rng.normal(0, 3, (rows, D)))
        parts64.append({"o": o.astype(np.float32).astype(np.float64), "m": m.astype(np.float32).astype(np.float64),
                        "l": l.astype(np.float32).astype(np.float64)})
    oracle = __import__("oracle")
    want = oracle.merge(oracle.merge(parts64[0], parts64[1]), parts64[2])
    dev_parts = [(torch.from_numpy(p["o"]).float().to(DEV),
                  torch.from_numpy(np.stack([p["m"], p["l"]], 1)).float().to(DEV)) for p in parts64]
    o, ml = cqsa().lse_merge(dev_parts)
    torch.cuda.synchronize()
    got_m = ml[:, 0].double().cpu().numpy()
    got_l = ml[:, 1].double().cpu().numpy()
    got_o = o.double().cpu().numpy()
    empty = want["l"] == 0
    assert np.all(np.isneginf(got_m[empty])) and np.all(got_l[empty] == 0) and not np.isnan(got_o).any()
    ne = ~empty
    # the merged m is the max; compare o/l and lse
    np.testing.assert_allclose(got_o[ne] / got_l[ne, None], want["o"][ne] / want["l"][ne, None], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(got_m[ne] + np.log(got_l[ne]), want["m"][ne] + np.log(want["l"][ne]), rtol=1e-6,
                               atol=1e-5)
    # in place: output aliases part 0
    o0, ml0 = dev_parts[0][0].clone(), dev_parts[0][1].clone()
    cqsa().lse_merge([(o0, ml0), dev_parts[1], dev_parts[2]], out=(o0, ml0))
    torch.cuda.synchronize()
    assert torch.equal(o0, o) and torch.equal(ml0, ml)


def test_finalize():
    """The finalize kernel against the oracle's normalise (o / l, m + ln l) of the same triples, and the
    identity triple (l = 0, m = -inf), which the library delivers as out = 0, lse = -inf."""
    import oracle
    rng = np.random.default_rng(4)
    B, H, N, D = 2, 3, 50, 64
    o = torch.from_numpy(rng.normal(0, 1, (B, H, N, D))).float()
    m = torch.from_numpy(rng.normal(0, 1, (B, H, N))).float()
    l = torch.from_numpy(rng.uniform(0.5, 9, (B, H, N))).float()
    m[1, 2, 7], l[1, 2, 7], o[1, 2, 7] = -math.inf, 0.0, 0.0
    ml = torch.stack([m, l], -1)
    out, lse = cqsa().finalize(o.to(DEV), ml.to(DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = oracle.normalise({"o": o.double().reshape(-1, D).numpy(), "m": m.double().reshape(-1).numpy(),
                             "l": l.double().reshape(-1).numpy()})
    got_o, got_lse = out.cpu().double().reshape(-1, D).numpy(), lse.cpu().double().reshape(-1).numpy()
    ok = l.reshape(-1).numpy() > 0
    np.testing.assert_allclose(got_o[ok], want["o"][ok], rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(got_lse[ok], want["lse"][ok], rtol=1e-6, atol=1e-6)
    assert np.all(got_o[~ok] == 0) and np.all(np.isneginf(got_lse[~ok]))


def test_causal_n32768_monolithic_and_8way_split_agree():
    """B=1, H=8, N=32768, D=64 causal fp16: one pass, and a forced split into 8 KV chunks (merge kernel
    and fused merges), each checked in full (all 262,144 rows) against the FP64 reference."""
    w = synth.workload(1)
    say("workload", w.name, "every row")
    q, k, v, _ = synth.make_inputs(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    mono, lse_m = cqsa().attention(qd, kd, vd, is_causal=True, out_dtype=torch.float32, return_lse=True)
    split, lse_s, info = cqsa().attention(qd, kd, vd, is_causal=True, kv_chunk=4096, merge=1, out_dtype=torch.float32,
                                          return_lse=True, return_info=True)
    fused, lse_f = cqsa().attention(qd, kd, vd, is_causal=True, kv_chunk=4096, merge=2, out_dtype=torch.float32,
                                    return_lse=True)
    torch.cuda.synchronize()
    assert info["n_kv_chunks"] == 8 and info["chunk_pairs"] == 8
    ref = reference(q, k, v, causal=True, scale=w.scale)
    r1 = compare(mono, lse_m, ref, torch.float16, label="causal 32K mono")
    r2 = compare(split, lse_s, ref, torch.float16, label="causal 32K split")
    r3 = compare(fused, lse_f, ref, torch.float16, label="causal 32K fused")
    agree = (mono - split).abs().max().item()
    say("causal 32K", r1, r2, r3, "max|mono-split|", agree)
    assert agree <= 1e-3
    assert (fused - split).abs().max().item() <= 1e-3


# Rows checked at the sizes the reference cannot finish in full within the test's time: every (b, h),
# with the first and last EDGE rows, rows +-1 around Q-chunk, KV-chunk and 128-row tile edges (at most
# CAP rows of them), and RANDOM seeded rows.  (edge, random, cap) per workload; the row count per
# (b, h) is logged.  64 edge rows and 512 random rows in every (b, h); the boundary rows are capped where
# the oracle's cost per row is largest (up to 4M visible keys a row).
LARGE_SAMPLED = {"prompt_131072": (64, 512, 256), "streamed_4m": (64, 512, 64), "stress_full": (64, 512, 64)}


@pytest.mark.parametrize("nk", [8192, 32768, 131072])
def test_prompt_q2048_gqa(nk):
    """2048 queries at the end of the context, 32 query heads over 8 KV heads, D=128, bf16: every row
    at 8K and 32K keys; at 131K, sampled rows in every head."""
    w = synth.workload(2, nk=nk)
    say("workload", w.name)
    q, k, v, _ = synth.make_inputs(w)
    if nk <= 32768:
        rows = None
    else:
        edge, n_random, cap = LARGE_SAMPLED["prompt_131072"]
        rows = sample_rows(1, 32, 2048, seed=3, n_random=n_random, edge=edge, boundaries=range(0, 2048, 128), cap=cap)
        say("prompt", nk, "rows per head", len(rows) // 32)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse, info = cqsa().attention(qd, kd, vd, is_causal=True, out_dtype=torch.float32, return_lse=True,
                                      return_info=True)
    # split-KV across the GPU merges to the same answer
    out2, lse2 = cqsa().attention(qd, kd, vd, is_causal=True, kv_splits=4, out_dtype=torch.float32,
                                  return_lse=True)
    torch.cuda.synchronize()
    ref = reference(q, k, v, causal=True, scale=w.scale, rows=rows)
    say("prompt", nk, info["kv_splits"], compare(out, lse, ref, torch.bfloat16, rows=rows, label=f"prompt {nk}"))
    compare(out2, lse2, ref, torch.bfloat16, rows=rows, label=f"prompt {nk} splits=4")


# (Hq, Hkv, N, D, dtype, causal, key chunks): past 512K keys, with several rounds of workgroups
LONG_KEY_CASES = [
    (2, 1, 532000, 64, torch.float16, True, 5),      # GQA 2/1, a ragged last chunk
    (4, 2, 540000, 128, torch.bfloat16, False, 5),   # D=128 bf16, non-causal
]


@pytest.mark.parametrize("case", LONG_KEY_CASES, ids=lambda c: f"n{c[2]}d{c[3]}{'c' if c[5] else 'n'}")
def test_resident_long_key_range_runs_in_key_chunks(case):
    """Device-resident attention over more than 512K keys: by default the plan runs one launch per
    128K-key chunk, folded into one fp32 accumulator by the kernel epilogue.  Sampled rows in every
    head (chunk edges included) match the oracle, and the forced single pass (kv_splits=1) agrees up to
    the fp32 summation order."""
    Hq, Hkv, N, D, dtype, causal, nchunks = case
    say("resident long keys", case)
    q, k, v = gen(1, Hq, Hkv, N, N, D, dtype, seed=41 + D)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse, info = cqsa().attention(qd, kd, vd, is_causal=causal, out_dtype=torch.float32, return_lse=True,
                                      return_info=True)
    one, lse1, info1 = cqsa().attention(qd, kd, vd, is_causal=causal, kv_splits=1, out_dtype=torch.float32,
                                        return_lse=True, return_info=True)
    torch.cuda.synchronize()
    assert (info["kv_chunk"], info["n_kv_chunks"], info["n_q_chunks"], info["merge_mode"]) == (131072, nchunks, 1, 2)
    assert info1["n_kv_chunks"] == 1 and info1["workspace_bytes"] == 0
    rows = sample_rows(1, Hq, N, seed=5, n_random=256, edge=64, boundaries=range(131072, N, 131072), cap=64)
    ref = reference(q, k, v, causal=causal, scale=1.0 / math.sqrt(D), rows=rows)
    say("resident long keys", len(rows) // Hq, "rows per head",
        compare(out, lse, ref, dtype, rows=rows, label="key chunks"))
    compare(one, lse1, ref, dtype, rows=rows, label="one pass")
    assert (out - one).abs().max().item() <= 1e-4
    assert (lse - lse1).abs().max().item() <= 1e-4


DECODE_CASES = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal, options, side-by-side KV splits (0: the planner's, more than one)
    (1, 32, 8, 1, 131075, 128, torch.bfloat16, True, {}, 0),     # one query per head at the end of 131K keys
    (1, 8, 1, 16, 150001, 64, torch.float16, True, {}, 0),       # 16 queries, one KV head
    (1, 4, 4, 7, 65537, 64, torch.bfloat16, False, {"kv_splits": 16}, 16),
    (1, 8, 2, 3, 100000, 128, torch.float16, True, {"kv_chunk": 30000, "merge": 2}, 1),   # the fused fold
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"q{c[3]}k{c[4]}d{c[5]}{'c' if c[7] else 'n'}"
                         f"{'-' + '-'.join(c[8]) if c[8] else ''}")
def test_decode_shapes_over_long_keys(case):
    """A few queries against a long key range: the planner runs side-by-side KV splits (one pass per
    split, folded by the merge kernel) so that the CUs are filled; with a forced KV chunk, the chunks
    are folded in the kernel epilogue.  Every row against the FP64 oracle."""
    B, Hq, Hkv, Nq, Nk, D, dtype, causal, opt, splits = case
    say("decode", case)
    q, k, v = gen(B, Hq, Hkv, Nq, Nk, D, dtype, seed=4400 + Nq + D)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse, info = cqsa().attention(qd, kd, vd, is_causal=causal, out_dtype=torch.float32, return_lse=True,
                                      return_info=True, **opt)
    torch.cuda.synchronize()
    if splits == 0:
        assert info["kv_splits"] > 1
    else:
        assert info["kv_splits"] == splits
    if info["kv_splits"] > 1:
        assert info["merge_mode"] == 1 and info["n_kv_chunks"] == 1
    ref = reference(q, k, v, causal=causal, scale=1.0 / math.sqrt(D))
    say("decode", compare(out, lse, ref, dtype, label=f"decode {case[:8]}"))


SCALE_CASES = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal, scale
    (1, 2, 2, 1000, 1000, 64, torch.float16, True, 8.0),      # logits with sd 64: one key per row dominates
    (1, 4, 2, 700, 1300, 128, torch.bfloat16, True, 4.0),     # sd 45, bottom-right causal, GQA
    (1, 2, 2, 900, 900, 64, torch.bfloat16, False, 1e-4),     # nearly uniform weights
    (2, 2, 1, 333, 2048, 128, torch.float16, False, 1e-3),
]


@pytest.mark.parametrize("case", SCALE_CASES, ids=lambda c: f"q{c[3]}k{c[4]}d{c[5]}{'c' if c[7] else 'n'}-s{c[8]:g}")
def test_extreme_softmax_scales(case):
    """Softmax scales far outside the default: at 4 and 8 the scaled logits have standard deviations of
    45-64, so the running shift moves by large steps and all but a few keys underflow; at 1e-3 and
    1e-4 the weights are almost uniform and the output is close to the mean of the visible values.
    Single pass and forced KV chunks (both merges), every row against the FP64 oracle."""
    B, Hq, Hkv, Nq, Nk, D, dtype, causal, scale = case
    say("scale", case)
    q, k, v = gen(B, Hq, Hkv, Nq, Nk, D, dtype, seed=4500 + D + Nq)
    ref = reference(q, k, v, causal=causal, scale=scale)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for kw in ({}, {"kv_chunk": 300, "merge": 1}, {"kv_chunk": 300, "merge": 2}):
        out, lse = cqsa().attention(qd, kd, vd, is_causal=causal, scale=scale, out_dtype=torch.float32,
                                    return_lse=True, **kw)
        torch.cuda.synchronize()
        say("scale", compare(out, lse, ref, dtype, label=f"scale {case} {kw}"))


def test_softmax_stress_reduced():
    """Large logits (N(0, 9^2)) with +20 spikes on 5% of keys, uniform v, non-causal, bf16, KV chunk
    16384; the batch, heads and length are cut so the reference runs in seconds."""
    w = synth.workload(4)
    say("workload", w.name, "reduced")
    q, k, v, pos = synth.make_inputs(w, nq=2048, nk=65536, batch=2, heads=(2, 2))
    rows = sample_rows(2, 2, 2048, seed=5, n_random=48, edge=16)
    ref = reference(q, k, v, causal=False, scale=w.scale, rows=rows)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse, info = cqsa().attention(qd, kd, vd, is_causal=False, kv_chunk=16384, out_dtype=torch.float32,
                                      return_lse=True, return_info=True)
    torch.cuda.synchronize()
    assert info["n_kv_chunks"] == 4
    say("stress", compare(out, lse, ref, torch.bfloat16, rows=rows, label="stress reduced"))


SHIFT_CASES = [
    # D, dtype, causal
    (64, torch.float16, True),
    (64, torch.bfloat16, False),
    (128, torch.float16, False),
    (128, torch.bfloat16, True),
]


@pytest.mark.parametrize("variant", [0, 4, 5, 6, 7])
@pytest.mark.parametrize("case", SHIFT_CASES, ids=lambda c: f"d{c[0]}{'f16' if c[1] == torch.float16 else 'bf16'}"
                         f"{'c' if c[2] else 'n'}")
def test_shift_moves_inside_a_tile(case, variant, test_controls):
    """The running maximum jumps at the start of the second 32-key block of many 64-key tiles (and at
    the start of other tiles), by growing amounts, so the exact path of the online softmax runs in the
    middle of a tile, after the first block's probabilities were formed (and, in the pipelined kernel,
    after its PV products were issued).  Every query gets q[..., 0] = 3; the chosen keys get
    k[..., 0] raised so that their logit rises by 8 + 1.5 t (natural log) in tile t.  The kernels whose
    softmax runs per 32-key block (the ping-pong DMA kernel in both shapes, variants 0 and 7, and the
    DMA kernel's pipelined shapes) and the DMA kernel's plain order are compared with the FP64
    reference."""
    D, dtype, causal = case
    test_controls(variant, -1)
    B, H, N = 1, 2, 1100
    say("shift", case, "variant", variant)
    q, k, v = gen(B, H, H, N, N, D, dtype, seed=4100 + D + variant)
    scale = 1.0 / math.sqrt(D)
    q[..., 0] = 3.0
    for t in range(N // 64 + 1):
        j = 64 * t + (32 + t % 5 if t % 3 else t % 7)     # second block in two tiles of three, else the first
        if j < N:
            k[:, :, j, 0] = (k[:, :, j, 0].float() + (8.0 + 1.5 * t) / (3.0 * scale)).to(dtype)
    ref = reference(q, k, v, causal=causal, scale=scale)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse = cqsa().attention(qd, kd, vd, is_causal=causal, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    say("shift", compare(out, lse, ref, dtype, label=f"shift {case} variant {variant}"))
    # the spike keys dominate the rows that see them: the output is far from the plain average
    assert float((out.float().cpu() - v.float().mean(2, keepdim=True)).abs().max()) > 0.5


@pytest.mark.parametrize("layout", ["bhnd", "bnhd"])
def test_streamed_from_pinned_host(layout):
    """Host-resident q/k/v/out under a small budget: the planner must chunk Q and KV."""
    B, Hq, Hkv, N, D = 1, 4, 2, 6000, 64
    q, k, v = gen(B, Hq, Hkv, N, N, D, torch.float16, seed=44)
    ref = reference(q, k, v, causal=True, scale=0.125)

    def host(t):
        if layout == "bhnd":
            h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
        else:
            h = torch.empty((t.shape[0], t.shape[2], t.shape[1], t.shape[3]), dtype=t.dtype,
                            pin_memory=True).transpose(1, 2)
        h.copy_(t)
        return h

    qh, kh, vh = host(q), host(k), host(v)
    out = host(torch.zeros(B, Hq, N, D, dtype=torch.float32))
    budget = 2_000_000
    say("streamed", layout)
    o, lse, info = cqsa().attention(qh, kh, vh, is_causal=True, mem_budget=budget, out=out, return_lse=True,
                                    return_info=True)
    assert info["streamed"] == 1 and info["n_q_chunks"] > 1 and info["n_kv_chunks"] > 1
    assert info["workspace_bytes"] <= budget * 0.85
    assert o.data_ptr() == out.data_ptr() and not o.is_cuda
    compare(o, lse, ref, torch.float16, label=f"streamed {layout}")
    # the resident call gives the same numbers up to the merge order
    od = cqsa().attention(q.to(DEV), k.to(DEV), v.to(DEV), is_causal=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert (od.cpu() - o).abs().max().item() <= 1e-3


def test_mixed_residency_device_q_host_kv():
    q, k, v = gen(1, 2, 2, 3000, 5000, 128, torch.bfloat16, seed=45)
    ref = reference(q, k, v, causal=True, scale=1 / math.sqrt(128))
    kh, vh = k.pin_memory(), v.pin_memory()
    out, lse, info = cqsa().attention(q.to(DEV), kh, vh, is_causal=True, mem_budget=12_000_000,
                                      out_dtype=torch.float32, return_lse=True, return_info=True)
    assert info["streamed"] == 1 and out.is_cuda
    compare(out, lse, ref, torch.bfloat16, label="device q, host kv")


def test_deterministic():
    q, k, v = gen(1, 4, 4, 2000, 2000, 64, torch.float16, seed=46)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    a = cqsa().attention(qd, kd, vd, is_causal=True, kv_chunk=512)
    b = cqsa().attention(qd, kd, vd, is_causal=True, kv_chunk=512)
    c = cqsa().attention(qd, kd, vd, is_causal=True)
    d = cqsa().attention(qd, kd, vd, is_causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(c, d)


def test_q_zero_gives_mean_of_visible_values():
    """q = 0: every probability is exactly 1, so row i is the mean of its visible values."""
    Nq, Nk = 100, 300
    _, k, v = gen(1, 2, 2, Nq, Nk, 64, torch.float16, seed=47)
    q = torch.zeros(1, 2, Nq, 64, dtype=torch.float16)
    out, lse = cqsa().attention(q.to(DEV), k.to(DEV), v.to(DEV), is_causal=True, out_dtype=torch.float32,
                                return_lse=True)
    torch.cuda.synchronize()
    for i in (0, 1, 50, 99):
        cnt = Nk - Nq + i + 1
        torch.testing.assert_close(out[:, :, i].cpu().double(), v[:, :, :cnt].double().mean(2), rtol=0, atol=1e-5)
        torch.testing.assert_close(lse[:, :, i].cpu().double(), torch.full((1, 2), math.log(cnt), dtype=torch.float64),
                                   rtol=0, atol=1e-5)


def test_strided_device_inputs():
    q, k, v = gen(2, 4, 2, 333, 333, 64, torch.bfloat16, seed=48)
    ref = reference(q, k, v, causal=True, scale=0.125)
    tm = lambda t: t.transpose(1, 2).contiguous().transpose(1, 2).to(DEV)   # [B,N,H,D] storage
    out, lse = cqsa().attention(tm(q), tm(k), tm(v), is_causal=True, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    compare(out, lse, ref, torch.bfloat16, label="token-major device inputs")


def test_errors():
    m = cqsa()
    q, k, v = gen(1, 2, 2, 64, 64, 64, torch.float16, seed=49)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    with pytest.raises(m.CqsaError, match="INVALID.*pinned"):
        m.attention(q, k, v, is_causal=True, out=torch.empty(1, 2, 64, 64, dtype=torch.float16, device=DEV))
    with pytest.raises(m.CqsaError, match="UNSUPPORTED"):
        m.attention(qd[..., :32].contiguous(), kd[..., :32].contiguous(), vd[..., :32].contiguous())
    with pytest.raises(m.CqsaError, match="INVALID"):
        m.attention(torch.cat([qd, qd[:, :1]], 1), kd, vd)           # 3 query heads over 2
    with pytest.raises(m.CqsaError, match="INVALID"):
        m.attention(torch.cat([qd, qd], 2), kd, vd, is_causal=True)  # causal Nq > Nk
    with pytest.raises(m.CqsaError, match="BUDGET"):
        m.attention(q.pin_memory(), k.pin_memory(), v.pin_memory(), mem_budget=1000)
    # empty query set: nothing to do, no error
    e = m.attention(qd[:, :, :0], kd, vd, is_causal=True)
    assert e.shape == (1, 2, 0, 64)


def test_streamed_causal_n4194304_full_size():
    """4,194,304-token causal attention, H=8, D=64, fp16, q/k/v and out in pinned host memory, device budget
    16e9 bytes: the planner must cut Q in two and stream KV; sampled rows in every head against the FP64
    reference."""
    w = synth.workload(3)
    say("workload", w.name, "full size")
    q, k, v, _ = synth.make_inputs(w, pin=True)
    out = torch.empty((w.B, w.Hq, w.Nq, w.D), dtype=torch.float16, pin_memory=True)
    o, lse, info = cqsa().attention(q, k, v, is_causal=True, mem_budget=w.mem_budget, out=out, return_lse=True,
                                    return_info=True)
    say("streamed 4M", {x: info[x] for x in ("q_chunk", "kv_chunk", "chunk_pairs", "workspace_bytes", "h2d_bytes",
                                         "h2d_ms")})
    assert info["streamed"] == 1 and info["n_q_chunks"] == 2
    assert info["workspace_bytes"] <= 16e9 * 0.85
    assert info["h2d_bytes"] == 16 * 2**30
    edge, n_random, cap = LARGE_SAMPLED["streamed_4m"]
    rows = sample_rows(1, 8, w.Nq, seed=6, n_random=n_random, edge=edge, boundaries=[info["q_chunk"]] +
                       list(range(0, w.Nq, info["kv_chunk"])), tiles=range(0, w.Nq, 128), cap=cap)
    say("streamed 4M", "rows per head", len(rows) // 8)
    ref = reference(q, k, v, causal=True, scale=w.scale, rows=rows)
    say("streamed 4M", compare(o, lse, ref, torch.float16, rows=rows, label="streamed 4M"))


def test_softmax_stress_full_size():
    """B=2, H=16, N=262,144, D=128, bf16, non-causal, logits N(0, 9^2) with +20 spikes on 5% of keys,
    KV chunk 16,384 (16 LSE merges); sampled rows in every (b, h) against the FP64 reference."""
    w = synth.workload(4)
    say("workload", w.name, "full size")
    q, k, v, pos = synth.make_inputs(w)
    assert len(pos) == 13107
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse, info = cqsa().attention(qd, kd, vd, is_causal=False, kv_chunk=16384, out_dtype=torch.float32,
                                      return_lse=True, return_info=True)
    torch.cuda.synchronize()
    assert info["n_kv_chunks"] == 16 and info["merges"] == 15
    edge, n_random, cap = LARGE_SAMPLED["stress_full"]
    rows = sample_rows(2, 16, w.Nq, seed=7, n_random=n_random, edge=edge,
                       boundaries=range(0, w.Nq, 16384), tiles=range(0, w.Nq, 128), cap=cap)
    say("stress full", "rows per (b, h)", len(rows) // 32)
    ref = reference(q, k, v, causal=False, scale=w.scale, rows=rows)
    say("stress full", compare(out, lse, ref, torch.bfloat16, rows=rows, label="stress full"))


def test_launch_failure_mid_stream_is_reported_and_the_next_call_is_exact(test_controls):
    """A forward launch that fails partway through a host-streamed call is reported as CQSA_ERR_HIP.  The
    failure is forced from the host (cqsa_set_test_controls with 3: the call's Q and KV copies and its
    first three launches are already issued when the fourth launch fails), so no kernel faults.  The
    call returns only after its streams have drained; nothing of it is left running, and the next
    call on the same pinned buffers is exact."""
    m = cqsa()
    B, Hq, Hkv, N, D = 1, 4, 2, 6000, 64
    q, k, v = gen(B, Hq, Hkv, N, N, D, torch.float16, seed=45)
    qh, kh, vh = q.pin_memory(), k.pin_memory(), v.pin_memory()
    out = torch.full((B, Hq, N, D), 7.0, dtype=torch.float32, pin_memory=True)
    budget = 2_000_000
    say("injected launch failure, streamed")
    test_controls(0, 3)
    with pytest.raises(m.CqsaError, match="HIP.*injected"):
        m.attention(qh, kh, vh, is_causal=True, mem_budget=budget, out=out)
    torch.cuda.synchronize()                      # no GPU error left behind
    test_controls(0, -1)
    o, lse, info = m.attention(qh, kh, vh, is_causal=True, mem_budget=budget, out=out, return_lse=True,
                               return_info=True)
    assert info["streamed"] == 1 and info["kernel_launches"] > 3
    rows = sample_rows(B, Hq, N, seed=45, n_random=64, edge=8)
    ref = reference(q, k, v, causal=True, scale=0.125, rows=rows)
    compare(o, lse, ref, torch.float16, rows=rows, label="after an injected failure")


def test_allocation_failure_is_reported_and_leaves_nothing_behind():
    """With no caller workspace the library allocates its own; when the device cannot hold it the call
    returns CQSA_ERR_OOM (no retry) and the free memory afterwards is what it was.  The device is
    filled by a PyTorch allocation first, leaving 1 GiB, and the plan needs more than that."""
    import ctypes
    m = cqsa()
    B, H, N, D = 1, 8, 1 << 20, 64
    q = torch.zeros((B, H, N, D), dtype=torch.float16, pin_memory=True)
    k = torch.zeros_like(q).pin_memory()
    v = torch.zeros_like(q).pin_memory()
    out = torch.empty_like(q).pin_memory()
    opt = m._options()                                   # no workspace: the library calls hipMalloc
    budget = 16 * 10**9
    plan = m.plan(q, k, v, True, budget)
    assert plan["workspace_bytes"] > 2 * (1 << 30)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    free0, _ = torch.cuda.mem_get_info()
    hog = torch.empty(free0 - (1 << 30), dtype=torch.uint8, device=DEV)
    try:
        st = m._lib.cqsa_attention_ex(ctypes.byref(m._desc(q)), ctypes.byref(m._desc(k)), ctypes.byref(m._desc(v)),
                                      1, ctypes.c_float(0.0), budget, ctypes.byref(m._desc(out)), None,
                                      ctypes.byref(opt), None)
        msg = m._lib.cqsa_last_error().decode()
    finally:
        del hog
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    assert st == -4 and "hipMalloc" in msg, (st, msg)
    free1, _ = torch.cuda.mem_get_info()
    # nothing of the library is left allocated; the runtime may release cached memory of its own when
    # an allocation fails, so more memory can be free afterwards than before
    assert free1 >= free0 - (64 << 20), (free0, free1)
    # and the same call succeeds once the memory is back
    o2 = m.attention(q[:, :, :4096], k[:, :, :4096], v[:, :, :4096], is_causal=True, mem_budget=budget)
    assert torch.isfinite(o2.float()).all()
