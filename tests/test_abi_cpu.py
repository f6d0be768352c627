"""The C ABI without a GPU: the library loads, exports what include/cqsa.h declares, its structs
match the binding, and the planner (pure host logic) sizes chunks, skips causal chunks and rejects
impossible budgets.  No compute call is made here."""
import ctypes
import importlib.util
import os
import re
import shutil
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cqsa.h")
GB = 10**9


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cqsa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    import exact_long_context_cqsa_amd as m
    names = declared_functions()
    assert len(names) >= 9
    lib = ctypes.CDLL(m.library_path())
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    nm = subprocess.run(["nm", "-D", "--defined-only", m.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (cqsa_\w+)", nm))
    assert set(names) <= exported


def test_forward_kernel_name(test_controls):
    import exact_long_context_cqsa_amd as m
    test_controls(0, -1)
    # the default at both head dims is the ping-pong DMA kernel; variant 6 is the DMA kernel's best
    # shape (pipelined and lean at D=64, plain at D=128), variants 4 and 5 its other choices
    assert m.fwd_kernel_name(64).startswith("fwd_pp_dma_kernel waves=8 ")
    assert m.fwd_kernel_name(128).startswith("fwd_pp_dma_kernel waves=8 ")
    assert m.fwd_kernel_name(96) == ""
    test_controls(6, -1)
    assert m.fwd_kernel_name(64).startswith("fwd_dma_kernel ")
    assert "pipelined" in m.fwd_kernel_name(64) and "lean" in m.fwd_kernel_name(64)
    assert "pipelined" not in m.fwd_kernel_name(128) and "lean" not in m.fwd_kernel_name(128)
    test_controls(5, -1)
    assert "pipelined" in m.fwd_kernel_name(64) and "lean" not in m.fwd_kernel_name(64)
    assert "lean" in m.fwd_kernel_name(128)
    test_controls(2, -1)
    assert m.fwd_kernel_name(64).startswith("fwd_kernel ")
    test_controls(4, -1)
    assert m.fwd_kernel_name(64).startswith("fwd_dma_kernel ") and "pipelined" not in m.fwd_kernel_name(64)
    assert m.fwd_kernel_name(128).startswith("fwd_dma_kernel ") and "pipelined" in m.fwd_kernel_name(128)
    test_controls(7, -1)
    assert m.fwd_kernel_name(64).startswith("fwd_pp_dma_kernel ")
    assert "keys_per_tile=32" in m.fwd_kernel_name(128)
    for bad in ((99, -1), (-1, -1), (0, -2), (8, -1)):   # out of range: rejected, nothing changes
        with pytest.raises(m.CqsaError, match="INVALID"):
            test_controls(*bad)
        assert m.fwd_kernel_name(64).startswith("fwd_pp_dma_kernel ")
    # split-P runs the DMA kernel in its own shape whatever the variant
    test_controls(2, -1)
    assert m.fwd_kernel_name(64, 1).startswith("fwd_dma_kernel ") and m.fwd_kernel_name(64, 1).endswith("split_p")
    assert m.fwd_kernel_name(128, 1).endswith("split_p")
    test_controls(0, -1)
    assert m.fwd_kernel_name(64).startswith("fwd_pp_dma_kernel ")


def test_struct_layout_and_version():
    import exact_long_context_cqsa_amd as m
    lib = m._lib
    assert lib.cqsa_version() == 5
    assert lib.cqsa_struct_size(0) == ctypes.sizeof(m.CqsaTensor) == 80
    assert lib.cqsa_struct_size(1) == ctypes.sizeof(m.CqsaOptions) == 88
    assert [f for f, _ in m.CqsaOptions._fields_][-3:] == ["cqs_set", "wave_tokens", "cqs_itr"]
    assert [f for f, _ in m.CqsaPlanInfo._fields_][-3:] == ["cqs_waves", "reserved0", "wave_tokens"]
    assert lib.cqsa_struct_size(2) == ctypes.sizeof(m.CqsaPlanInfo) == 152
    assert lib.cqsa_struct_size(3) == ctypes.sizeof(m.CqsaProbeResult) == 72
    assert lib.cqsa_struct_size(7) == 0


def test_probe_rejects_bad_arguments_before_any_hip_call():
    """cqsa_probe_device validates its arguments first, so these fail the same way with or without a
    GPU (a HIP call here, with no device, would give CQSA_ERR_HIP instead)."""
    import exact_long_context_cqsa_amd as m
    lib, r = m._lib, m.CqsaProbeResult()
    for copy_bytes, repeats in [(1 << 30, 0), (1 << 30, 101), (1000, 5), ((1 << 20) + 8, 5), ((1 << 34) + 16, 5)]:
        assert lib.cqsa_probe_device(copy_bytes, repeats, ctypes.byref(r)) == -1, (copy_bytes, repeats)
        assert lib.cqsa_last_error()
    assert lib.cqsa_probe_device(1 << 30, 5, None) == -1


def test_missing_library_fails_loudly(tmp_path):
    """Without libcqsa.so the package refuses to import: there is no CPU fallback."""
    src = os.path.join(ROOT, "exact_long_context_cqsa_amd")
    dst = tmp_path / "exact_long_context_cqsa_amd"
    shutil.copytree(src, dst, ignore=shutil.ignore_patterns("*.so", "__pycache__", "csrc"))
    spec = importlib.util.spec_from_file_location("cqsa_copy", dst / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError, match="not built"):
        spec.loader.exec_module(mod)


def plan(q, k, v, causal, budget, where=None, **kw):
    import exact_long_context_cqsa_amd as m
    return m.plan(q, k, v, causal, budget, where=where or {}, num_cus=256, **kw)


def shp(B, H, N, D, dt=torch.float16):
    return ((B, H, N, D), dt)


def test_plan_streamed_4m_context():
    """4,194,304 tokens, 8 heads, D=64 in pinned host memory under a 16e9-byte budget: Q must be cut in
    two, every KV chunk streams once per Q chunk that sees it, and the plan stays inside 85% of the budget."""
    s = shp(1, 8, 4194304, 64)
    host = {"q": "host", "k": "host", "v": "host", "out": "host"}
    p = plan(s, s, s, True, 16 * GB, where=host)
    assert p["streamed"] == 1 and p["merge_mode"] == 2
    assert p["n_q_chunks"] == 2 and p["q_chunk"] == 2097152
    assert p["workspace_bytes"] <= p["budget_bytes"] == int(16 * GB * 0.85)
    # H2D: Q once (4 GiB) + KV prefix for each Q chunk (K+V: 4 GiB, then 8 GiB)
    assert p["h2d_bytes"] == 16 * 2**30
    assert p["d2h_bytes"] == 4 * 2**30
    kv = p["kv_chunk"]
    assert p["chunk_pairs"] == -(-2097152 // kv) + -(-4194304 // kv)


def test_plan_forced_splits():
    s = shp(1, 1, 1024, 64)
    p = plan(s, s, s, True, 16 * GB, kv_chunk=256)
    assert (p["n_kv_chunks"], p["chunk_pairs"], p["merges"], p["merge_mode"]) == (4, 4, 3, 2)
    assert plan(s, s, s, True, 16 * GB, kv_chunk=256, merge=1)["merge_mode"] == 1
    s2 = shp(1, 8, 32768, 64)
    p2 = plan(s2, s2, s2, True, 16 * GB, kv_chunk=4096)
    assert (p2["n_kv_chunks"], p2["chunk_pairs"], p2["merges"]) == (8, 8, 7)
    p3 = plan(s2, s2, s2, True, 16 * GB)
    assert (p3["chunk_pairs"], p3["merges"], p3["workspace_bytes"], p3["kernel_launches"]) == (1, 0, 0, 1)
    # causal skipping with Q chunks: chunk pairs above the diagonal are not scheduled
    p4 = plan(s2, s2, s2, True, 16 * GB, kv_chunk=4096, q_chunk=4096)
    assert p4["chunk_pairs"] == sum(range(1, 9))
    p5 = plan(s2, s2, s2, False, 16 * GB, kv_chunk=4096, q_chunk=4096)
    assert p5["chunk_pairs"] == 64


def test_plan_split_kv_when_few_query_tiles():
    q = shp(1, 4, 256, 128, torch.bfloat16)
    kv = shp(1, 1, 131072, 128, torch.bfloat16)
    p = plan(q, kv, kv, True, 16 * GB)
    assert p["kv_splits"] > 1 and p["merge_mode"] == 1
    # side-by-side splits run at the same time: the merge kernel folds them whatever is requested
    assert plan(q, kv, kv, True, 16 * GB, kv_splits=4, merge=2)["merge_mode"] == 1
    p1 = plan(q, kv, kv, True, 16 * GB, kv_splits=1)
    assert p1["kv_splits"] == 1 and p1["workspace_bytes"] == 0


def test_plan_resident_long_key_range():
    """Device-resident inputs over more than 512K keys run one launch per 128K-key chunk, folded by the
    kernel epilogue into one fp32 accumulator, when that accumulator fits the budget and the query tiles
    make several rounds of workgroups; otherwise, with forced kv_splits, or at 512K keys and below, one
    pass."""
    s = shp(1, 8, 4194304, 64)
    p = plan(s, s, s, True, 16 * GB)
    assert (p["q_chunk"], p["kv_chunk"], p["n_kv_chunks"], p["merge_mode"]) == (4194304, 131072, 32, 2)
    assert (p["chunk_pairs"], p["merges"], p["kernel_launches"]) == (32, 31, 33)
    assert p["workspace_bytes"] == 8 * 4194304 * (64 + 2) * 4 and p["h2d_bytes"] == 0
    for kw, budget in (({}, 8 * GB), ({"kv_splits": 1}, 16 * GB)):
        p1 = plan(s, s, s, True, budget, **kw)
        assert (p1["n_kv_chunks"], p1["workspace_bytes"], p1["kernel_launches"]) == (1, 0, 1)
    s2 = shp(1, 8, 524288, 64)
    assert plan(s2, s2, s2, True, 16 * GB)["n_kv_chunks"] == 1
    # few query tiles (8 heads, one query): side-by-side splits fill the GPU instead
    p3 = plan(shp(1, 8, 1, 64), shp(1, 8, 1 << 20, 64), shp(1, 8, 1 << 20, 64), False, 16 * GB)
    assert p3["n_kv_chunks"] == 1 and p3["kv_splits"] > 1
    # one round of workgroups (a 2,048-query prompt over 1M keys at D=128): one pass
    p4 = plan(shp(1, 32, 2048, 128), shp(1, 8, 1 << 20, 128), shp(1, 8, 1 << 20, 128), True, 16 * GB)
    assert p4["n_kv_chunks"] == 1 and p4["kv_splits"] == 1


def test_plan_split_target_is_the_workgroups_the_cus_hold():
    """Side-by-side KV splits fill the CUs with as many workgroups as they hold at once: one 8-wave
    workgroup per CU at D=128, two at D=64 (256 CUs here)."""
    bf, f16 = torch.bfloat16, torch.float16
    prompt = lambda nk, D, dt: (shp(1, 32, 2048, D, dt), shp(1, 8, nk, D, dt))
    for nk in (32768, 131072):        # 256 workgroups at D=128 already fill the CUs
        q, kv = prompt(nk, 128, bf)
        assert plan(q, kv, kv, True, 16 * GB)["kv_splits"] == 1
    q, kv = prompt(131072, 64, f16)   # 256 workgroups at D=64: two per CU wanted
    assert plan(q, kv, kv, True, 16 * GB)["kv_splits"] == 2
    q, kv = shp(1, 8, 2048, 128, bf), shp(1, 8, 65536, 128, bf)   # 64 workgroups at D=128
    assert plan(q, kv, kv, True, 16 * GB)["kv_splits"] == 4


def test_plan_errors():
    import exact_long_context_cqsa_amd as m
    s = shp(1, 8, 4194304, 64)
    host = {"q": "host", "k": "host", "v": "host", "out": "host"}
    with pytest.raises(m.CqsaError, match="BUDGET.*needs"):
        plan(s, s, s, True, 10_000, where=host)
    with pytest.raises(m.CqsaError, match="UNSUPPORTED"):
        plan(shp(1, 2, 64, 96), shp(1, 2, 64, 96), shp(1, 2, 64, 96), False, GB)
    with pytest.raises(m.CqsaError, match="INVALID"):
        plan(shp(1, 3, 64, 64), shp(1, 2, 64, 64), shp(1, 2, 64, 64), False, GB)
    with pytest.raises(m.CqsaError, match="INVALID"):
        plan(shp(1, 2, 65, 64), shp(1, 2, 64, 64), shp(1, 2, 64, 64), True, GB)
    with pytest.raises(m.CqsaError, match="BUDGET"):
        plan(shp(1, 2, 64, 64), shp(1, 2, 64, 64), shp(1, 2, 64, 64), True, 1000, kv_chunk=16)
    with pytest.raises(m.CqsaError, match="precision"):
        plan(shp(1, 2, 64, 64), shp(1, 2, 64, 64), shp(1, 2, 64, 64), True, GB, precision=2)


def test_plan_split_p_block_m():
    """The split-P product runs in its own kernel shape: 128-row workgroups (4 waves, pipelined) at
    D=64, 256-row workgroups at D=128."""
    a = plan(shp(1, 2, 1000, 64), shp(1, 2, 1000, 64), shp(1, 2, 1000, 64), True, GB, precision=1)
    assert a["block_m"] == 128
    b = plan(shp(1, 2, 1000, 128), shp(1, 2, 1000, 128), shp(1, 2, 1000, 128), True, GB, precision=1)
    assert b["block_m"] == 256


def test_plan_budget_monotone():
    """A larger budget never gives more Q chunks or smaller KV chunks."""
    s = shp(1, 8, 1 << 20, 64)
    host = {"q": "host", "k": "host", "v": "host", "out": "host"}
    prev = None
    for gb in (1, 2, 4, 8, 16, 32):
        p = plan(s, s, s, True, gb * GB, where=host)
        assert p["workspace_bytes"] <= p["budget_bytes"]
        if prev:
            assert p["n_q_chunks"] <= prev["n_q_chunks"]
            if p["n_q_chunks"] == prev["n_q_chunks"]:
                assert p["kv_chunk"] >= prev["kv_chunk"]
        prev = p


def test_header_is_plain_c(tmp_path):
    """include/cqsa.h is a C header: it compiles as C99 with warnings as errors, with no HIP header."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "use.c"
    src.write_text('#include "cqsa.h"\nint main(void) { cqsa_options o; cqsa_plan_info i; (void)o; (void)i; '
                   'return (int)cqsa_struct_size(0) * 0; }\n')
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
