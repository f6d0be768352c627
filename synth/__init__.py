"""Seeded synthetic inputs for exact attention (shared by the checker and the GPU path).

This module only draws numbers: it holds none of the attention arithmetic.  The
C generator (``synth_gen.c``) is Philox4x32-10 (Salmon et al., SC'11) with
Box-Muller normals, rounded to binary32 and then to fp16/bf16 (round to nearest
even).  Values depend only on (seed, tensor id, logical element index), so a
tensor can be regenerated piecewise and in any storage layout.

The five workloads (``workload(i)``) follow the input recipe of the method's
measured cases: fp16/bf16 q/k/v drawn i.i.d. from N(0, sigma^2), causal or not,
GQA for the prompt case, large logits with +20 spikes for the softmax-stress
case.  Seeds are ``0xC05A0000 + i``; tensor ids are q=0, k=1, v=2, spikes=3, upstream gradient=4.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth_gen.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_SPIKES, TENSOR_DO = 0, 1, 2, 3, 4
SEED_BASE = 0xC05A0000

_DT = {torch.float16: 0, torch.bfloat16: 1, torch.float32: 2, torch.float64: 3}


def build(force: bool = True) -> str:
    """Compile the generator with gcc into ``synth/libsynth.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_double, ctypes.c_double, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int]
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_philox4x32_10.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint32),
                                            ctypes.POINTER(ctypes.c_uint32)]
        lib.synth_f32_to_f16_bits.argtypes = [ctypes.c_float]
        lib.synth_f32_to_f16_bits.restype = ctypes.c_uint16
        lib.synth_f32_to_bf16_bits.argtypes = [ctypes.c_float]
        lib.synth_f32_to_bf16_bits.restype = ctypes.c_uint16
        lib.synth_raw_u32.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint32]
        _lib = lib
    return _lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def philox4x32_10(counter, key):
    """One Philox4x32-10 block: four 32-bit counter words, two key words -> four words."""
    lib = _load()
    c = (ctypes.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in counter])
    k = (ctypes.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    o = (ctypes.c_uint32 * 4)()
    lib.synth_philox4x32_10(c, k, o)
    return [int(x) for x in o]


def f32_to_f16_bits(x: float) -> int:
    return int(_load().synth_f32_to_f16_bits(ctypes.c_float(x)))


def f32_to_bf16_bits(x: float) -> int:
    return int(_load().synth_f32_to_bf16_bits(ctypes.c_float(x)))


def fill_(t: torch.Tensor, *, seed: int, tensor_id: int, dist: str = "normal", a: float = 0.0, b: float = 1.0,
          element_offset: int = 0, threads: int | None = None) -> torch.Tensor:
    """Fill a contiguous CPU tensor in place with elements element_offset.. of the stream."""
    if t.device.type != "cpu" or not t.is_contiguous():
        raise ValueError("fill_ needs a contiguous CPU tensor")
    rc = _load().synth_fill(ctypes.c_void_p(t.data_ptr()), t.numel(), int(element_offset),
                            0 if dist == "normal" else 1, _DT[t.dtype], float(a), float(b),
                            int(seed) & 0xFFFFFFFF, int(tensor_id) & 0xFFFFFFFF, threads or default_threads())
    if rc != 0:
        raise RuntimeError("synth_fill failed")
    return t


def normal(shape, *, seed: int, tensor_id: int, sigma: float = 1.0, dtype=torch.float16, pin: bool = False,
           threads: int | None = None) -> torch.Tensor:
    """A [*shape] tensor of N(0, sigma^2) draws, contiguous, on the CPU (pinned if asked)."""
    t = torch.empty(tuple(shape), dtype=dtype, pin_memory=pin)
    return fill_(t, seed=seed, tensor_id=tensor_id, dist="normal", a=0.0, b=sigma, threads=threads)


def uniform(shape, *, seed: int, tensor_id: int, lo: float = -1.0, hi: float = 1.0, dtype=torch.float16,
            pin: bool = False, threads: int | None = None) -> torch.Tensor:
    t = torch.empty(tuple(shape), dtype=dtype, pin_memory=pin)
    return fill_(t, seed=seed, tensor_id=tensor_id, dist="uniform", a=lo, b=hi, threads=threads)


def choose_without_replacement(n: int, count: int, *, seed: int, tensor_id: int = TENSOR_SPIKES) -> np.ndarray:
    """``count`` distinct positions out of range(n): rank every position by its own Philox word
    (ties broken by position) and keep the smallest ``count``; returned sorted."""
    if count > n:
        raise ValueError("count > n")
    words = (ctypes.c_uint32 * n)()
    _load().synth_raw_u32(words, n, int(seed) & 0xFFFFFFFF, int(tensor_id) & 0xFFFFFFFF)
    w = np.frombuffer(words, dtype=np.uint32).astype(np.uint64)
    key = (w << np.uint64(32)) | np.arange(n, dtype=np.uint64)
    sel = np.argpartition(key, count - 1)[:count] if count > 0 else np.zeros(0, dtype=np.int64)
    return np.sort(sel.astype(np.int64))


@dataclass
class Workload:
    """One measured attention case: shapes, dtype, distribution and the split it forces."""
    index: int
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    D: int
    dtype: torch.dtype
    causal: bool
    kv_chunk: int | None = None
    host_resident: bool = False
    mem_budget: int | None = None
    q_sigma: float = 1.0
    k_sigma: float = 1.0
    v_dist: str = "normal"
    spikes: float = 0.0         # fraction of key positions that get a +20 logit spike
    spike_logit: float = 20.0
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def visible_pairs(self) -> int:
        """Exact (query, key) pairs that enter the softmax, per (batch, head)."""
        if not self.causal:
            return self.Nq * self.Nk
        off = self.Nk - self.Nq
        return self.Nq * (off + 1) + self.Nq * (self.Nq - 1) // 2

    def flops(self) -> float:
        """Algorithmic FLOPs: two products of 2 FLOP per multiply-add over visible pairs only."""
        return 4.0 * self.D * self.visible_pairs() * self.B * self.Hq


def workload(i: int, *, nk: int | None = None) -> Workload:
    """The five measured cases (index 0..4)."""
    if i == 0:
        return Workload(0, "causal_n1024_h1_d64_f16_kvchunk256", 1, 1, 1, 1024, 1024, 64, torch.float16, True,
                        kv_chunk=256, notes="4 KV chunks of 256, merged by log-sum-exp; fp32 output")
    if i == 1:
        return Workload(1, "causal_n32768_h8_d64_f16", 1, 8, 8, 32768, 32768, 64, torch.float16, True,
                        notes="monolithic pass, and a forced 8-chunk split (kv_chunk=4096)",
                        extra={"split_kv_chunk": 4096})
    if i == 2:
        n = nk or 32768
        return Workload(2, f"prompt_q2048_k{n}_gqa32x8_d128_bf16", 1, 32, 8, 2048, n, 128, torch.bfloat16, True,
                        notes="2048 queries at the end of the context (bottom-right causal), 4 query heads per KV head")
    if i == 3:
        return Workload(3, "streamed_causal_n4194304_h8_d64_f16", 1, 8, 8, 4194304, 4194304, 64, torch.float16,
                        True, host_resident=True, mem_budget=16 * 10**9,
                        notes="q/k/v in pinned host memory, 16e9-byte device budget")
    if i == 4:
        return Workload(4, "stress_nc_n262144_h16_b2_d128_bf16", 2, 16, 16, 262144, 262144, 128, torch.bfloat16,
                        False, kv_chunk=16384, q_sigma=3.0, k_sigma=3.0, v_dist="uniform", spikes=0.05,
                        notes="logits ~N(0, 9^2), 5% of keys carry +20 logit spikes, KV chunk 16384")
    raise ValueError(i)


def make_inputs(w: Workload, *, nq: int | None = None, nk: int | None = None, batch: int | None = None,
                heads: tuple | None = None, pin: bool = False, threads: int | None = None):
    """Generate (q, k, v) for a workload as contiguous [B, H, N, D] CPU tensors.

    ``nq``/``nk``/``batch``/``heads`` shrink the problem (same recipe, same seed), for tests that
    need a size the checker finishes quickly.  The spike recipe (softmax stress) realises the +20
    logit spikes in the inputs: every query gets q[..., 0] = q_sigma, and the chosen keys get
    k[..., 0] += spike_logit / (q_sigma * scale) (added to the fp32-rounded draw), so each logit
    towards a spike key rises by spike_logit before k is rounded to the storage format."""
    B = batch if batch is not None else w.B
    Hq, Hkv = heads if heads is not None else (w.Hq, w.Hkv)
    Nq = nq if nq is not None else w.Nq
    Nk = nk if nk is not None else w.Nk
    D = w.D
    seed = w.seed
    spike_pos = None
    if w.spikes > 0.0:
        # one (b, h) slice at a time: draws rounded to fp32, the spike added in fp32, then one
        # rounding to the storage format (the same two roundings as every other draw)
        count = int(math.floor(w.spikes * Nk))
        spike_pos = choose_without_replacement(Nk, count, seed=seed)
        sp = torch.from_numpy(spike_pos)
        delta = w.spike_logit / (w.q_sigma * w.scale)
        q = torch.empty((B, Hq, Nq, D), dtype=w.dtype, pin_memory=pin)
        k = torch.empty((B, Hkv, Nk, D), dtype=w.dtype, pin_memory=pin)
        tmp_q = torch.empty((Nq, D), dtype=torch.float32)
        tmp_k = torch.empty((Nk, D), dtype=torch.float32)
        for b in range(B):
            for h in range(Hq):
                fill_(tmp_q, seed=seed, tensor_id=TENSOR_Q, dist="normal", a=0.0, b=w.q_sigma,
                      element_offset=((b * Hq + h) * Nq) * D, threads=threads)
                tmp_q[:, 0] = w.q_sigma
                q[b, h].copy_(tmp_q)
            for h in range(Hkv):
                fill_(tmp_k, seed=seed, tensor_id=TENSOR_K, dist="normal", a=0.0, b=w.k_sigma,
                      element_offset=((b * Hkv + h) * Nk) * D, threads=threads)
                tmp_k[sp, 0] += delta
                k[b, h].copy_(tmp_k)
    else:
        q = normal((B, Hq, Nq, D), seed=seed, tensor_id=TENSOR_Q, sigma=w.q_sigma, dtype=w.dtype, pin=pin,
                   threads=threads)
        k = normal((B, Hkv, Nk, D), seed=seed, tensor_id=TENSOR_K, sigma=w.k_sigma, dtype=w.dtype, pin=pin,
                   threads=threads)
    if w.v_dist == "uniform":
        v = uniform((B, Hkv, Nk, D), seed=seed, tensor_id=TENSOR_V, lo=-1.0, hi=1.0, dtype=w.dtype, pin=pin,
                    threads=threads)
    else:
        v = normal((B, Hkv, Nk, D), seed=seed, tensor_id=TENSOR_V, sigma=1.0, dtype=w.dtype, pin=pin,
                   threads=threads)
    return q, k, v, spike_pos


