"""The seeded input generator: Philox4x32-10 known answers, rounding, determinism, recipes."""
import math

import numpy as np
import pytest
import torch

import synth


def test_philox_known_answer_vectors():
    """Known-answer vectors of Philox4x32 with 10 rounds (Salmon et al., SC'11; the Random123 KAT set)."""
    assert synth.philox4x32_10([0, 0, 0, 0], [0, 0]) == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    assert synth.philox4x32_10([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2) == [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]
    assert synth.philox4x32_10([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0]) == \
        [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]


def test_f16_rounding_matches_numpy():
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.standard_normal(20000) * s for s in (1e-7, 1e-5, 1e-3, 1.0, 100.0, 7e4)])
    xs = np.concatenate([xs, [0.0, -0.0, 65504.0, 65520.0, 65519.99, 2.0**-24, 2.0**-25, 3 * 2.0**-26, np.inf, -np.inf]])
    xs = xs.astype(np.float32)
    want = xs.astype(np.float16).view(np.uint16)
    got = np.array([synth.f32_to_f16_bits(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(want, got)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.standard_normal(20000) * s for s in (1e-30, 1e-3, 1.0, 1e30)]).astype(np.float32)
    want = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([synth.f32_to_bf16_bits(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(want, got)


def test_deterministic_across_threads_and_pieces():
    a = synth.normal((3, 5, 7001), seed=7, tensor_id=1, threads=1)
    b = synth.normal((3, 5, 7001), seed=7, tensor_id=1, threads=8)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    flat = a.reshape(-1)
    piece = torch.empty(1000, dtype=torch.float16)
    synth.fill_(piece, seed=7, tensor_id=1, element_offset=5000)
    assert torch.equal(piece.view(torch.int16), flat[5000:6000].view(torch.int16))
    c = synth.normal((3, 5, 7001), seed=7, tensor_id=2)
    assert not torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_moments():
    x = synth.normal((1 << 20,), seed=3, tensor_id=0, sigma=3.0, dtype=torch.float32).double()
    assert abs(x.mean().item()) < 0.02 and abs(x.std().item() - 3.0) < 0.02
    u = synth.uniform((1 << 20,), seed=3, tensor_id=2, dtype=torch.float32).double()
    assert u.min().item() >= -1.0 and u.max().item() <= 1.0 and abs(u.mean().item()) < 0.01
    assert abs(u.var().item() - 1.0 / 3.0) < 0.01


def test_sampling_without_replacement():
    pos = synth.choose_without_replacement(262144, 13107, seed=synth.SEED_BASE + 4)
    assert len(pos) == 13107 and len(np.unique(pos)) == 13107
    assert pos.min() >= 0 and pos.max() < 262144
    again = synth.choose_without_replacement(262144, 13107, seed=synth.SEED_BASE + 4)
    assert np.array_equal(pos, again)


def test_workload_table():
    w = [synth.workload(i) for i in range(5)]
    assert (w[0].Nq, w[0].D, w[0].kv_chunk, w[0].causal) == (1024, 64, 256, True)
    assert (w[1].Hq, w[1].Nq, w[1].D, w[1].dtype) == (8, 32768, 64, torch.float16)
    assert (w[2].Hq, w[2].Hkv, w[2].Nq, w[2].D, w[2].dtype) == (32, 8, 2048, 128, torch.bfloat16)
    assert (w[3].Nq, w[3].mem_budget, w[3].host_resident) == (4194304, 16 * 10**9, True)
    assert (w[4].B, w[4].Hq, w[4].Nq, w[4].kv_chunk, w[4].causal) == (2, 16, 262144, 16384, False)
    # algorithmic FLOPs: 4 * D per visible pair
    assert w[1].flops() == 4 * 64 * (32768 * 32769 // 2) * 8
    assert w[0].flops() == 4 * 64 * 524800
    w2 = synth.workload(2, nk=8192)
    assert w2.visible_pairs() == sum(8192 - 2048 + i + 1 for i in range(2048))


def test_spike_recipe_raises_logits_by_twenty():
    w = synth.workload(4)
    q, k, v, pos = synth.make_inputs(w, nq=64, nk=2000, batch=1, heads=(2, 2))
    assert len(pos) == 100
    assert torch.all(q[..., 0].float() == 3.0)
    assert v.float().abs().max().item() <= 1.0
    # the same draw without the spike: logit difference towards spike keys is ~+20 (bf16 rounding of k)
    k_plain = synth.normal((1, 2, 2000, 128), seed=w.seed, tensor_id=synth.TENSOR_K, sigma=3.0,
                           dtype=torch.float64)
    s_spk = w.scale * (q.double() @ k.double().transpose(-1, -2))
    s_pln = w.scale * (q.double() @ k_plain.transpose(-1, -2))
    diff = (s_spk - s_pln)[..., torch.from_numpy(pos)]
    assert abs(diff.mean().item() - 20.0) < 0.5
    others = np.setdiff1d(np.arange(2000), pos)
    assert (s_spk - s_pln)[..., torch.from_numpy(others)].abs().max().item() < 1.5
