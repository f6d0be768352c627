"""The entry point cqsa_attention(q, k, v, is_causal, scale, mem_budget, out, lse) called directly through
the C ABI, with no options: the library plans, allocates its own workspace with hipMalloc, runs on the
null stream and returns once the work is done.  Each case is compared element by element with the
FP64 oracle at the fp16 / bf16 tolerances.  This is the SDPA drop-in of the Stream-CQSA pages
(stream-cqsa 2.2.0 -> 2.2.2 diff, stream_cqsa/api.py, the attention() docstring), and below and above
the memory boundary it must give the monolithic answer (stream-cqsa 2.2.2 -> 2.2.3 diff, README.md
"Use")."""
import ctypes
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


def call(q, k, v, causal, scale, budget, out, lse):
    """cqsa_attention itself: tensor descriptors and raw pointers, nothing else."""
    dq, dk, dv, do = m._desc(q), m._desc(k), m._desc(v), m._desc(out)
    lp = None if lse is None else ctypes.cast(ctypes.c_void_p(lse.data_ptr()), ctypes.POINTER(ctypes.c_float))
    st = m._lib.cqsa_attention(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), 1 if causal else 0,
                               float(scale), int(budget), ctypes.byref(do), lp)
    if st != 0:
        raise m.CqsaError(st, m._lib.cqsa_last_error().decode())


def gen(B, Hq, Hkv, Nq, Nk, D, dtype, seed):
    q = synth.normal((B, Hq, Nq, D), seed=seed, tensor_id=0, dtype=dtype)
    k = synth.normal((B, Hkv, Nk, D), seed=seed, tensor_id=1, dtype=dtype)
    v = synth.normal((B, Hkv, Nk, D), seed=seed, tensor_id=2, dtype=dtype)
    return q, k, v


def test_device_resident_prompt_with_kv_splits():
    """A GQA prompt (256 queries at the end of 32,768 keys, 32 query heads over 8, D=128, bf16) with every
    operand on the device and mem_budget = 0 (the free memory): the planner splits the key range across
    the GPU, which needs partial buffers, so the library allocates them itself."""
    B, Hq, Hkv, Nq, Nk, D = 1, 32, 8, 256, 32768, 128
    q, k, v = gen(B, Hq, Hkv, Nq, Nk, D, torch.bfloat16, seed=71)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    info = m.plan(qd, kd, vd, is_causal=True, want_lse=True)
    say("cqsa_attention device", info["kv_splits"], info["workspace_bytes"])
    assert info["kv_splits"] > 1 and info["workspace_bytes"] > 0
    out = torch.full((B, Hq, Nq, D), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    call(qd, kd, vd, True, 0.0, 0, out, lse)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] >= free0 - (64 << 20)     # the library freed its workspace
    ref = reference(q, k, v, causal=True, scale=1.0 / math.sqrt(D))
    say("cqsa_attention device", compare(out, lse, ref, torch.bfloat16, label="cqsa_attention device kv_splits"))
    # the same call with the input dtype as output: within the tolerance plus one output ulp
    out16 = torch.empty((B, Hq, Nq, D), dtype=torch.bfloat16, device=DEV)
    call(qd, kd, vd, True, 0.0, 0, out16, None)
    torch.cuda.synchronize()
    compare(out16, None, ref, torch.bfloat16, label="cqsa_attention device bf16 out")


@pytest.mark.parametrize("place", ["all_host", "device_out_host_lse"])
def test_streamed_under_a_small_budget(place):
    """Causal fp16, 6000 tokens, 4 query heads over 2, D=64, under a 3 MB budget that forces Q chunks (and KV
    chunks, where K and V are on the host).  all_host: q, k, v, out and lse in pinned host memory.  device_out_host_lse: q, k, v and out
    on the device and lse in pinned host memory, so every Q chunk's lse goes through the one staging
    buffer and back to the host while the next Q chunk runs."""
    B, Hq, Hkv, N, D = 1, 4, 2, 6000, 64
    budget = 3_000_000
    q, k, v = gen(B, Hq, Hkv, N, N, D, torch.float16, seed=72)
    if place == "all_host":
        qx, kx, vx = q.pin_memory(), k.pin_memory(), v.pin_memory()
        out = torch.full((B, Hq, N, D), float("nan"), dtype=torch.float32, pin_memory=True)
        where = {"q": "host", "k": "host", "v": "host", "out": "host"}
        want_lse = "host"
    else:
        qx, kx, vx = q.to(DEV), k.to(DEV), v.to(DEV)
        out = torch.full((B, Hq, N, D), float("nan"), dtype=torch.float32, device=DEV)
        where = {"q": "device", "k": "device", "v": "device", "out": "device"}
        want_lse = "host"
    lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, pin_memory=True)
    info = m.plan(((B, Hq, N, D), torch.float16), ((B, Hkv, N, D), torch.float16), ((B, Hkv, N, D), torch.float16),
                  is_causal=True, mem_budget=budget, out=((B, Hq, N, D), torch.float32), want_lse=want_lse,
                  where=where, num_cus=256)
    say("cqsa_attention", place, {x: info[x] for x in ("n_q_chunks", "n_kv_chunks", "workspace_bytes", "d2h_bytes")})
    assert info["streamed"] == 1 and info["n_q_chunks"] > 1
    if place == "all_host":          # device K/V is read in place, so only host K/V is cut into chunks
        assert info["n_kv_chunks"] > 1
    assert info["d2h_bytes"] >= B * Hq * N * 4
    call(qx, kx, vx, True, 0.125, budget, out, lse)
    torch.cuda.synchronize()
    ref = reference(q, k, v, causal=True, scale=0.125)
    say("cqsa_attention", place, compare(out, lse, ref, torch.float16, label=f"cqsa_attention {place}"))
