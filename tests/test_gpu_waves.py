"""The wave engine of the quorum-set schedule on the GPU: subproblems packed into waves, one batched
launch per wave (per 32 query and 32 key parts), each query part attending to the union of its key
parts in one pass, folded into the accumulator on the device.  Compared with the FP64 oracle at
several wave budgets, from one subproblem per wave to a single wave, with device-resident and
pinned-host inputs (head-major and token-major host layouts); and the schedule at depth 2 and 3
(c^itr parts)."""
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


def gen(B, Hq, Hkv, Nq, Nk, D, dtype, seed):
    q = synth.normal((B, Hq, Nq, D), seed=seed, tensor_id=0, dtype=dtype)
    k = synth.normal((B, Hkv, Nk, D), seed=seed, tensor_id=1, dtype=dtype)
    v = synth.normal((B, Hkv, Nk, D), seed=seed, tensor_id=2, dtype=dtype)
    return q, k, v


WAVE_CASES = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal, cqs
    (1, 2, 2, 1500, 1500, 64, torch.float16, True, 7),
    (1, 2, 2, 1201, 1201, 64, torch.float16, False, 13),               # ragged parts, non-causal
    (1, 4, 1, 513, 2000, 128, torch.bfloat16, True, 7),                # GQA 4:1, bottom-right causal
    (2, 2, 2, 900, 900, 128, torch.float16, True, 31),                 # parts of 29-30 rows
    (1, 1, 1, 40, 40, 64, torch.bfloat16, True, 31),                   # parts of one or two rows
]


@pytest.mark.parametrize("case", WAVE_CASES, ids=lambda c: f"B{c[0]}H{c[1]}x{c[2]}q{c[3]}k{c[4]}d{c[5]}"
                         f"{'c' if c[7] else 'n'}-cqs{c[8]}")
def test_wave_budgets_against_oracle(case):
    B, Hq, Hkv, Nq, Nk, D, dtype, causal, c = case
    say("waves", case)
    q, k, v = gen(B, Hq, Hkv, Nq, Nk, D, dtype, seed=5000 + Nq + Nk + D + c)
    ref = reference(q, k, v, causal=causal, scale=1.0 / math.sqrt(D))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    outs, waves = [], []
    for wt in (1, (Nq + Nk) // 3, None):
        out, lse, info = cqsa().attention(qd, kd, vd, is_causal=causal, out_dtype=torch.float32, return_lse=True,
                                          return_info=True, cqs=c, wave_tokens=wt)
        torch.cuda.synchronize()
        compare(out, lse, ref, dtype, label=f"waves device wave_tokens={wt} {case}")
        assert info["kernel_launches"] >= info["cqs_waves"] + 2
        outs.append(out)
        waves.append(info["cqs_waves"])
    assert waves[0] == info["cqs_subproblems"] and waves[2] == 1 and waves[0] >= waves[1] >= waves[2]
    # different budgets fold the parts in different groupings, so P is rounded against different
    # running maxima: the outputs agree to the rounding of P (2^-11 fp16, 2^-8 bf16, times |v| <~ 4)
    agree = 2e-3 if dtype == torch.float16 else 1.6e-2
    for o in outs[1:]:
        assert (o - outs[0]).abs().max().item() <= agree
    qh, kh, vh = q.pin_memory(), k.pin_memory(), v.pin_memory()
    for wt in (1, None):
        out_h, lse_h, info_h = cqsa().attention(qh, kh, vh, is_causal=causal, out_dtype=torch.float32,
                                                return_lse=True, return_info=True, cqs=c, wave_tokens=wt)
        assert not out_h.is_cuda and info_h["streamed"] == 1
        compare(out_h, lse_h, ref, dtype, label=f"waves host wave_tokens={wt} {case}")


def test_wave_launches_of_32_parts():
    """c = 57 (a perfect difference set of 8 elements): a single wave holds all 57 query parts and
    runs as several launches of at most 32 query and 32 key parts, so a query part folds more than
    once per wave."""
    iset = (0, 1, 3, 13, 32, 36, 43, 52)
    B, Hq, Hkv, N, D = 1, 2, 1, 57 * 23 + 5, 64
    for causal in (True, False):
        say("waves c=57", causal)
        q, k, v = gen(B, Hq, Hkv, N, N, D, torch.float16, seed=5100 + causal)
        ref = reference(q, k, v, causal=causal, scale=0.125)
        out, lse, info = cqsa().attention(q.to(DEV), k.to(DEV), v.to(DEV), is_causal=causal, out_dtype=torch.float32,
                                          return_lse=True, return_info=True, cqs=(57, iset))
        torch.cuda.synchronize()
        assert info["cqs_waves"] == 1 and info["kernel_launches"] - 2 >= 2
        compare(out, lse, ref, torch.float16, label=f"waves c=57 causal={causal}")
        out_h, lse_h = cqsa().attention(q.pin_memory(), k.pin_memory(), v.pin_memory(), is_causal=causal,
                                        out_dtype=torch.float32, return_lse=True, cqs=(57, iset), wave_tokens=400)
        compare(out_h, lse_h, ref, torch.float16, label=f"waves c=57 host causal={causal}")


def test_wave_token_major_host_inputs():
    """Pinned host tensors stored token-major ([B, N, H, D]) are staged per part in that order; the
    wave kernel reads the compact token-major copy."""
    B, Hq, Hkv, N, D = 2, 4, 2, 1100, 128
    say("waves token-major host")
    q, k, v = gen(B, Hq, Hkv, N, N, D, torch.bfloat16, seed=5200)
    ref = reference(q, k, v, causal=True, scale=1.0 / math.sqrt(D))

    def tm(t):   # [B, N, H, D] storage in pinned memory, viewed as [B, H, N, D]
        x = torch.empty((t.shape[0], t.shape[2], t.shape[1], t.shape[3]), dtype=t.dtype, pin_memory=True)
        x.copy_(t.transpose(1, 2))
        return x.transpose(1, 2)

    qh, kh, vh = tm(q), tm(k), tm(v)
    assert qh.stride(1) < qh.stride(2)
    for wt in (1, None):
        out, lse = cqsa().attention(qh, kh, vh, is_causal=True, out_dtype=torch.float32, return_lse=True, cqs=13,
                                    wave_tokens=wt)
        compare(out, lse, ref, torch.bfloat16, label=f"waves token-major host wave_tokens={wt}")


def test_wave_split_p():
    """precision=1 (split P) through the wave kernel: within the tight split-P bound."""
    B, Hq, Hkv, N, D = 1, 2, 2, 1300, 64
    say("waves split-P")
    q, k, v = gen(B, Hq, Hkv, N, N, D, torch.float16, seed=5300)
    ref = reference(q, k, v, causal=True, scale=0.125)
    out, lse = cqsa().attention(q.to(DEV), k.to(DEV), v.to(DEV), is_causal=True, out_dtype=torch.float32,
                                return_lse=True, cqs=7, precision=1)
    torch.cuda.synchronize()
    compare(out, lse, ref, torch.float16, label="waves split-P")
    err = float(np.abs(out.cpu().double().numpy() - ref["o"].reshape(out.shape)).max())
    assert err <= 2e-5, err


def test_wave_bench_shape_one_launch_matches_monolithic():
    """The 32K causal D=64 workload under c = 31 with the default budget: one wave, one launch; sampled
    rows against the oracle and the whole output against the monolithic pass."""
    w = synth.workload(1)
    say("waves workload", w.name)
    q, k, v, _ = synth.make_inputs(w)
    rows = sample_rows(1, w.Hq, w.Nq, seed=17, n_random=48, edge=8,
                       boundaries=[w.Nq * p // 31 for p in range(32)])
    ref = reference(q, k, v, causal=True, scale=w.scale, rows=rows)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    mono = cqsa().attention(qd, kd, vd, is_causal=True, out_dtype=torch.float32)
    out, lse, info = cqsa().attention(qd, kd, vd, is_causal=True, out_dtype=torch.float32, return_lse=True,
                                      return_info=True, cqs=31)
    torch.cuda.synchronize()
    assert info["cqs_waves"] == 1 and info["kernel_launches"] == 3
    compare(out, lse, ref, w.dtype, rows=rows, label="waves c=31 32K")
    assert (out - mono).abs().max().item() <= 1e-3


def test_wave_units_per_query_part_streamed():
    """131072 host-resident tokens under c = 31 with a 0.48 GB budget: whole subproblems do not fit two
    staging sets but a subproblem's pairs of one query part do, so the waves are cut per query part
    (more waves than subproblems), double-buffered; sampled rows against the oracle."""
    w = synth.workload(3)
    say("waves per query part, streamed 131072")
    q, k, v, _ = synth.make_inputs(w, nq=131072, nk=131072, pin=True)
    out, lse, info = cqsa().attention(q, k, v, is_causal=True, mem_budget=480_000_000, return_lse=True,
                                      return_info=True, cqs=31)
    assert info["streamed"] == 1 and info["cqs_waves"] > info["cqs_subproblems"] == 31
    rows = sample_rows(1, w.Hq, 131072, seed=19, n_random=48, edge=8,
                       boundaries=[131072 * p // 31 for p in range(32)], heads=range(0, w.Hq, 3))
    ref = reference(q, k, v, causal=True, scale=w.scale, rows=rows)
    compare(out, lse, ref, w.dtype, rows=rows, label="waves per query part, streamed 131072")


DEPTH_CASES = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, causal, c, itr
    (1, 2, 2, 1500, 1500, 64, torch.float16, True, 3, 2),       # 9 parts
    (1, 4, 1, 700, 2100, 128, torch.bfloat16, True, 7, 2),      # 49 parts, GQA 4:1, bottom-right causal
    (2, 2, 2, 900, 900, 64, torch.float16, False, 3, 3),        # 27 parts, non-causal
    (1, 2, 2, 1201, 1201, 128, torch.float16, True, 13, 2),     # 169 parts of 7-8 rows: several launches per wave
]


@pytest.mark.parametrize("case", DEPTH_CASES, ids=lambda c: f"q{c[3]}k{c[4]}d{c[5]}{'c' if c[7] else 'n'}-cqs{c[8]}^{c[9]}")
def test_depth_against_oracle(case):
    """The quorum-set schedule itr levels deep (c^itr parts): against the oracle with device-resident
    inputs at the default wave budget and one subproblem per wave, and with pinned host inputs; and
    against the single-level schedule and the monolithic pass."""
    B, Hq, Hkv, Nq, Nk, D, dtype, causal, c, itr = case
    say("depth", case)
    q, k, v = gen(B, Hq, Hkv, Nq, Nk, D, dtype, seed=5400 + Nq + Nk + c + itr)
    ref = reference(q, k, v, causal=causal, scale=1.0 / math.sqrt(D))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    agree = 2e-3 if dtype == torch.float16 else 1.6e-2
    mono = cqsa().attention(qd, kd, vd, is_causal=causal, out_dtype=torch.float32)
    for wt in (None, 1):
        out, lse, info = cqsa().attention(qd, kd, vd, is_causal=causal, out_dtype=torch.float32, return_lse=True,
                                          return_info=True, cqs=c, cqs_itr=itr, wave_tokens=wt)
        torch.cuda.synchronize()
        assert info["n_q_chunks"] == c ** itr and info["cqs_c"] == c
        compare(out, lse, ref, dtype, label=f"depth wave_tokens={wt} {case}")
        assert (out - mono).abs().max().item() <= agree
    out_h, lse_h, info_h = cqsa().attention(q.pin_memory(), k.pin_memory(), v.pin_memory(), is_causal=causal,
                                            out_dtype=torch.float32, return_lse=True, return_info=True, cqs=c,
                                            cqs_itr=itr)
    assert info_h["streamed"] == 1 and not out_h.is_cuda
    compare(out_h, lse_h, ref, dtype, label=f"depth host {case}")
