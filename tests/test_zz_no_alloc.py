"""cqsa_attention_noalloc, the entry point for callers that cannot allocate: through the C ABI it must give
what cqsa_attention_ex gives for the same split (the same kernels; its partials live in the library's
fixed device array instead of a workspace), on two calls in a row with the second one smaller, and both
must match the FP64 oracle at the fp16 / bf16 tolerances.  Sizes it cannot hold, and host operands, are
refused before any device work."""
import math
import sys

import pytest
import torch

import exact_long_context_cqsa_amd as m
import synth
from parity_util import compare, reference

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def gen(B, Hq, Hkv, Nq, Nk, D, dtype, seed):
    q = synth.normal((B, Hq, Nq, D), seed=seed, tensor_id=0, dtype=dtype)
    k = synth.normal((B, Hkv, Nk, D), seed=seed, tensor_id=1, dtype=dtype)
    v = synth.normal((B, Hkv, Nk, D), seed=seed, tensor_id=2, dtype=dtype)
    return q, k, v


CASES = [
    # B, Hq, Hkv, Nq, Nk, D, dtype, kv_splits: the second case is smaller than the first
    (1, 32, 8, 512, 32768, 128, torch.bfloat16, 4),
    (1, 4, 2, 300, 20000, 64, torch.float16, 3),
]


def test_noalloc_matches_attention_ex_on_two_calls_in_a_row():
    for n, (B, Hq, Hkv, Nq, Nk, D, dtype, splits) in enumerate(CASES):
        say("noalloc call", n, (B, Hq, Hkv, Nq, Nk, D, dtype, splits))
        q, k, v = gen(B, Hq, Hkv, Nq, Nk, D, dtype, seed=80 + n)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        out = torch.full((B, Hq, Nq, D), float("nan"), dtype=torch.float32, device=DEV)
        lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=DEV)
        info = m.attention_noalloc(qd, kd, vd, out, lse, is_causal=True, kv_splits=splits)
        assert info["kv_splits"] == splits and 0 < info["workspace_bytes"] <= 128 << 20
        ref_out, ref_lse = m.attention(qd, kd, vd, is_causal=True, kv_splits=splits, out_dtype=torch.float32,
                                       return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), "noalloc differs from attention_ex"
        ref = reference(q, k, v, causal=True, scale=1.0 / math.sqrt(D))
        say("noalloc call", n, compare(out, lse, ref, dtype, label=f"noalloc call {n}"))


def test_noalloc_planner_split_and_single_pass():
    B, Hq, Hkv, Nq, Nk, D = 1, 32, 8, 256, 65536, 128
    q, k, v = gen(B, Hq, Hkv, Nq, Nk, D, torch.bfloat16, seed=90)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.empty((B, Hq, Nq, D), dtype=torch.bfloat16, device=DEV)
    info = m.attention_noalloc(qd, kd, vd, out, None, is_causal=True)     # the planner's split
    assert info["kv_splits"] > 1
    ref_out = m.attention(qd, kd, vd, is_causal=True, kv_splits=info["kv_splits"])
    one = torch.empty_like(out)
    info1 = m.attention_noalloc(qd, kd, vd, one, None, is_causal=True, kv_splits=1)
    assert info1["kv_splits"] == 1 and info1["workspace_bytes"] == 0
    ref_one = m.attention(qd, kd, vd, is_causal=True, kv_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(one, ref_one)
    ref = reference(q, k, v, causal=True, scale=1.0 / math.sqrt(D))
    compare(out, None, ref, torch.bfloat16, label="noalloc planner split, bf16 out")


def test_noalloc_long_key_range_stays_single_pass():
    """Past 512K keys the planner cuts a resident key range into chunks with an accumulator; the
    no-allocation entry point keeps its single-pass plan (here the planner's side-by-side split) and
    matches cqsa_attention_ex with that split exactly and the oracle within tolerance."""
    B, Hq, Hkv, Nq, Nk, D = 1, 2, 1, 256, 600000, 64
    q, k, v = gen(B, Hq, Hkv, Nq, Nk, D, torch.float16, seed=92)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.empty((B, Hq, Nq, D), dtype=torch.float16, device=DEV)
    info = m.attention_noalloc(qd, kd, vd, out, None, is_causal=True)
    assert info["n_kv_chunks"] == 1 and info["kv_splits"] > 1
    ref_out = m.attention(qd, kd, vd, is_causal=True, kv_splits=info["kv_splits"])
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    ref = reference(q, k, v, causal=True, scale=1.0 / math.sqrt(D))
    say("noalloc long keys", info["kv_splits"], compare(out, None, ref, torch.float16, label="noalloc long keys"))


def test_noalloc_refuses_what_it_cannot_hold():
    B, Hq, Hkv, Nq, Nk, D = 1, 32, 8, 2048, 65536, 128
    q, k, v = gen(B, Hq, Hkv, Nq, Nk, D, torch.bfloat16, seed=91)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.zeros((B, Hq, Nq, D), dtype=torch.float32, device=DEV)
    with pytest.raises(m.CqsaError, match="BUDGET.*CQSA_NOALLOC_SCRATCH_BYTES"):
        m.attention_noalloc(qd, kd, vd, out, None, is_causal=True, kv_splits=8)   # 8 x 68 MB of partials
    with pytest.raises(m.CqsaError, match="UNSUPPORTED"):
        m.attention_noalloc(q.pin_memory(), kd, vd, out, None, is_causal=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0                                          # nothing ran
