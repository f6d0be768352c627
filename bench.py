"""Benchmark: exact causal attention forward on one MI355X.

Default workload: causal self-attention, B=1, H=8, N=32,768, D=64, fp16 q/k/v drawn N(0,1) from
a fixed seed, all tensors resident in HBM, one monolithic pass per step (the path's steps a1-a6
in one call: validate, plan, forward kernel with the in-kernel finalise).  Prints one JSON line.

  value         algorithmic TFLOP/s = 4 * D * (visible (query, key) pairs) * B * H / step time
  roofline      the forward kernel against the dense fp16 matrix-core peak (2.5 PFLOP/s), timed
                per launch with HIP events on the stream the kernel runs on; with the rates this
                device measures (matrix cores, LDS, HBM copy) and the clock they ran at beside it
                (roofline.profile: the same kernel's average and matrix-core counters from the committed
                rocprofv3 summaries under profiles/)
  configs       the other measured cases, inputs in HBM: the 1,024-token parity case, the 2,048-query
                GQA prompt at 8K/32K/131K keys, the full-size softmax-stress case (--no-configs skips)
  cpu_baseline  the FP64 reference on this host's cores: time-bounded samples of every case (the
                1,024-token case in full; --cpu-full times the bench workload and the prompt at 8K
                and 32K in full too)
  streamed_4m   4,194,304-token causal attention from pinned host memory under a 16e9-byte device
                budget: tokens/s and H2D GB/s (the metric's second figure; --no-streamed skips it)
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2500.0   # MI355X dense fp16/bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=1, help="index of the measured case (default 1)")
    ap.add_argument("--nk", type=int, default=None, help="context length for the prompt case")
    ap.add_argument("--kv-chunk", type=int, default=None, help="force a KV split (LSE merges)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--streamed", dest="streamed", action="store_true", default=True,
                    help="also run the 4M-token host-streamed case (the default; it adds about a minute)")
    ap.add_argument("--no-streamed", dest="streamed", action="store_false",
                    help="skip the 4M-token host-streamed case")
    ap.add_argument("--backward", action="store_true",
                    help="also time the backward (dQ, dK, dV) on the resident workload")
    ap.add_argument("--streamed-backward", action="store_true",
                    help="also run the 4M-token backward from pinned host memory (about two minutes)")
    ap.add_argument("--split-p", action="store_true",
                    help="also time the split-P precision mode on the resident workload and check it on sampled rows")
    ap.add_argument("--wave-tokens", type=int, default=None,
                    help="packed-row budget of a wave of the quorum-set schedule (default: the library's)")
    ap.add_argument("--cqs", type=int, default=0,
                    help="also time the cyclic quorum-set schedule with this many parts (resident workload, "
                         "and the streamed case with --streamed)")
    ap.add_argument("--cqs-itr", type=int, default=1,
                    help="depth of the quorum-set schedule of --cqs (c**itr parts; default 1)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, copy 1 GiB device to device once (scales HBM byte counters)")
    ap.add_argument("--merge", action="store_true",
                    help="also time the exact merge and the finalize (HBM-bound steps) at 8.4M rows")
    ap.add_argument("--no-probe", dest="probe", action="store_false", default=True,
                    help="skip the device probe (matrix-core, LDS and HBM rates with the clock they ran at)")
    ap.add_argument("--no-configs", dest="configs", action="store_false", default=True,
                    help="skip the other measured configurations (the 1,024-token parity case, the 2,048-query "
                         "prompt at 8K/32K/131K keys, the full-size softmax-stress case)")
    ap.add_argument("--cpu-full", action="store_true",
                    help="time the FP64 reference in full on the 1,024-token case, the bench workload and the "
                         "prompt at 8K and 32K keys whatever their predicted time (by default each runs in full "
                         "only when a short sample predicts it within --cpu-full-limit seconds)")
    ap.add_argument("--cpu-full-limit", type=float, default=45.0,
                    help="longest predicted whole-workload oracle time that the default run still takes in full")
    ap.add_argument("--fwd-variant", type=int, default=0,
                    help="forward kernel shape (0 = the default; see cqsa_set_test_controls), for A/B runs")
    ap.add_argument("--profile", default=None, help="profile summary holding the measured traffic "
                    "(default profiles/<forward kernel>_<workload>.md)")
    return ap.parse_args()


def _oracle_rate(w, q, k, v, seconds: float, threads: int, rng, full: bool = False) -> dict:
    """The FP64 reference on rows of one workload: every row (full), or seeded random rows until
    `seconds` pass.  Returns rows, visible pairs, seconds and the algorithmic TFLOP/s."""
    import numpy as np
    import oracle
    t0 = time.perf_counter()
    if full:
        oracle.attention_rows(q, k, v, causal=w.causal, scale=w.scale, threads=threads)
        n = w.B * w.Hq * w.Nq
        pairs = w.visible_pairs() * w.B * w.Hq
    else:
        n = pairs = 0
        batch = 2 * threads
        while time.perf_counter() - t0 < seconds:
            b = rng.integers(0, w.B, batch)
            h = rng.integers(0, w.Hq, batch)
            i = rng.integers(0, w.Nq, batch)
            rows = np.stack([b, h, i], 1).astype(np.int64)
            oracle.attention_rows(q, k, v, causal=w.causal, scale=w.scale, rows=rows, threads=threads)
            n += batch
            pairs += int(np.sum(np.minimum(i + (w.Nk - w.Nq) + 1, w.Nk))) if w.causal else batch * w.Nk
    dt = time.perf_counter() - t0
    rate = 4.0 * w.D * pairs / dt
    return {"rows": int(n), "seconds": round(dt, 2), "tflops": round(rate / 1e12, 6),
            "mode": "every row" if full else "seeded random rows",
            "full_workload_s": round(w.flops() / rate, 1),
            "full_workload_s_is": "measured" if full else "extrapolated from the sampled rate"}


def cpu_baseline(w, q, k, v, seconds: float, others: dict, full: bool = False, limit: float = 45.0) -> dict:
    """The FP64 reference on this host's cores, reported beside the GPU figures (never a target).  The
    headline is the bench workload, timed in full when a 2 s sample predicts at most `limit` seconds for
    it (always with full=True), else sampled for `seconds`.  `others` maps the names of the other
    configurations to (workload, q, k, v): the 1,024-token case always runs in full, the prompt at 8K
    and 32K keys in full under the same rule, the rest on a 3 s sample.  A one-thread figure of the
    headline workload is given too."""
    import numpy as np
    import oracle
    threads = oracle.default_threads()
    rng = np.random.default_rng(12345)
    first = _oracle_rate(w, q, k, v, 2.0, threads, rng)
    head = _oracle_rate(w, q, k, v, seconds, threads, rng, full=full or first["full_workload_s"] <= limit)
    one = _oracle_rate(w, q, k, v, min(2.0, seconds / 4), 1, rng)
    per = {w.name: head}
    for name, (w2, q2, k2, v2) in others.items():
        whole = w2.index == 0
        if w2.index == 2 and w2.Nk <= 32768:
            whole = full or _oracle_rate(w2, q2, k2, v2, 1.0, threads, rng)["full_workload_s"] <= limit
        per[name] = _oracle_rate(w2, q2, k2, v2, 3.0, threads, rng, full=whole)
    return {"value": head["tflops"], "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"{head['rows']} {head['mode']} of {w.name} (all their visible keys), {head['seconds']} s, "
                       f"FP64 C reference on {threads} threads"),
            "single_thread_value": one["tflops"], "single_thread_sample": f"{one['rows']} rows, {one['seconds']} s",
            "extrapolated_full_workload_s": head["full_workload_s"] if head["mode"] != "every row" else None,
            "full_workload_s": head["full_workload_s"] if head["mode"] == "every row" else None,
            "per_config": per, "cpu_model": _cpu_model(), "nproc": os.cpu_count(), "threads": threads}


def _cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def profile_figures(kernel_prof: str, mfma_prof: str, flops: float) -> dict:
    """The same kernel's figures from the committed rocprofv3 summaries: the kernel-trace average over
    the timed dispatches (and the fraction of the peak it gives) and the matrix-core counters
    (MfmaUtil, clock); each marked with whether the kernel source is still the one measured."""
    from exact_long_context_cqsa_amd import profiling
    out = {}
    sha = profiling.kernel_source_sha256()
    kt = profiling.read_profile(kernel_prof)
    if kt.get("avg_ns"):
        ns = float(kt["avg_ns"])
        out.update({"trace_source": os.path.relpath(kernel_prof, ROOT), "trace_avg_ms": round(ns / 1e6, 4),
                    "trace_frac": round(flops / (ns * 1e-9) / 1e12 / PEAK_F16_TFLOPS, 4),
                    "trace_same_kernel_source": kt.get("kernel_source_sha256") == sha})
    mf = profiling.read_profile(mfma_prof)
    if mf.get("mfma_util_pct"):
        out.update({"mfma_source": os.path.relpath(mfma_prof, ROOT), "mfma_util_pct": float(mf["mfma_util_pct"]),
                    "clock_ghz": float(mf["clock_ghz"]),
                    "mfma_same_kernel_source": mf.get("kernel_source_sha256") == sha})
    return out


def measured_traffic(path: str):
    """HBM bytes per launch from a committed rocprofv3 summary, if it measured the current kernel source."""
    from exact_long_context_cqsa_amd import profiling
    prof = profiling.read_profile(path)
    if not prof or prof.get("kernel_source_sha256") != profiling.kernel_source_sha256():
        return None, ("no profile" if not prof else "kernel changed since the counters were taken")
    return int(float(prof["traffic_bytes_per_launch"])), os.path.relpath(path, ROOT)


def run_configs(cqsa, torch, synth, steps: int) -> tuple[dict, dict]:
    """The other measured configurations, each with its inputs in HBM: the 1,024-token parity case (4 KV
    chunks of 256 merged by log-sum-exp; a time, no roofline claim), the 2,048-query GQA prompt at 8K,
    32K and 131K keys, and the full-size softmax-stress case (16 KV chunks of 16,384, 15 folds).  Each
    call is timed with HIP events on the current stream; TFLOP/s and the fraction of the 2.5 PFLOP/s
    dense peak use the algorithmic count.  Sampled rows are checked against the FP64 reference (every
    row for the 1,024-token case).  Returns (figures, inputs kept for the CPU baseline)."""
    import numpy as np
    import oracle
    dev = "cuda:0"
    res, keep = {}, {}
    st = torch.cuda.current_stream()
    cases = [(0, None), (2, 8192), (2, 32768), (2, 131072), (4, None)]
    for idx, nk in cases:
        w = synth.workload(idx, nk=nk)
        t0 = time.perf_counter()
        q, k, v, _ = synth.make_inputs(w)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        kw = {"kv_chunk": w.kv_chunk} if w.kv_chunk else {}
        odt = torch.float32 if idx == 0 else w.dtype
        out = torch.empty((w.B, w.Hq, w.Nq, w.D), dtype=odt, device=dev)
        reps = 3 if idx == 4 else max(5, steps)
        cqsa.attention(qd, kd, vd, is_causal=w.causal, out=out, **kw)
        info = cqsa.attention(qd, kd, vd, is_causal=w.causal, out=out, return_info=True, **kw)[1]
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a_, b_ in ev:
            a_.record(st)
            cqsa.attention(qd, kd, vd, is_causal=w.causal, out=out, **kw)
            b_.record(st)
        torch.cuda.synchronize()
        ms = sorted(a_.elapsed_time(b_) for a_, b_ in ev)
        med = ms[len(ms) // 2]
        # parity: every row of the 1,024-token case, else seeded rows in several heads
        o32, lse = cqsa.attention(qd, kd, vd, is_causal=w.causal, out_dtype=torch.float32, return_lse=True, **kw)
        torch.cuda.synchronize()
        rng = np.random.default_rng(77 + idx)
        if idx == 0:
            rows = None
        else:
            n_r = 16 if idx == 4 else 48
            rows = np.stack([rng.integers(0, w.B, n_r), rng.integers(0, w.Hq, n_r), rng.integers(0, w.Nq, n_r)],
                            1).astype(np.int64)
        ref = oracle.attention_rows(q, k, v, causal=w.causal, scale=w.scale, rows=rows)
        if rows is None:
            got = o32.cpu().reshape(-1, w.D).double().numpy()
            gl = lse.cpu().reshape(-1).double().numpy()
        else:
            b_, h_, i_ = (torch.from_numpy(rows[:, c]) for c in range(3))
            got = o32.cpu()[b_, h_, i_].double().numpy()
            gl = lse.cpu()[b_, h_, i_].double().numpy()
        max_abs = float(np.abs(got - ref["o"]).max())
        lse_rel = float((np.abs(gl - ref["lse"]) / np.maximum(1.0, np.abs(ref["lse"]))).max())
        tol = 4e-3 if w.dtype == torch.float16 else 2e-2
        entry = {"ms": round(med, 4), "ms_min": round(ms[0], 4), "calls_timed": reps,
                 "algorithmic_flop": w.flops(), "kernel": cqsa.fwd_kernel_name(w.D),
                 "plan": {x: info[x] for x in ("kv_splits", "n_kv_chunks", "chunk_pairs", "merges", "kernel_launches")},
                 "parity_rows": "all" if rows is None else int(len(rows)), "max_abs_vs_fp64": max_abs,
                 "lse_rel_vs_fp64": lse_rel, "tolerance": tol, "parity_ok": max_abs <= tol and lse_rel <= 1e-4}
        if idx == 0:
            entry["note"] = "launch-bound parity case: a time, no roofline claim"
        else:
            tf = w.flops() / (med / 1e3) / 1e12
            entry.update({"tflops": round(tf, 2), "frac": round(tf / PEAK_F16_TFLOPS, 4),
                          "tokens_per_s": round(w.B * w.Nq / (med / 1e3), 1)})
        res[w.name] = entry
        print(f"[bench] {w.name}: {med:.3f} ms" + (f" ({entry['tflops']} TFLOP/s)" if idx else "")
              + f", max_abs {max_abs:.2e}, lse_rel {lse_rel:.1e} ({time.perf_counter() - t0:.1f} s)",
              file=sys.stderr, flush=True)
        keep[w.name] = (w, q, k, v)
        del qd, kd, vd, out, o32, lse
        torch.cuda.empty_cache()
    return res, keep


def run_streamed(cqsa, torch, synth, cqs=None, cqs_itr=1, keep=None) -> dict:
    w = synth.workload(3)
    t0 = time.perf_counter()
    q, k, v, _ = synth.make_inputs(w, pin=True)
    if keep is not None:
        keep[w.name] = (w, q, k, v)
    out = torch.empty((w.B, w.Hq, w.Nq, w.D), dtype=torch.float16, pin_memory=True)
    gen_s = time.perf_counter() - t0
    print(f"[bench] streamed inputs ready ({gen_s:.1f} s)", file=sys.stderr, flush=True)
    res = streamed_run(cqsa, torch, w, q, k, v, out, None)
    if cqs:
        res["cqs"] = streamed_run(cqsa, torch, w, q, k, v, out, cqs, cqs_itr)
    return res


def run_merge(cqsa, torch, steps: int) -> dict:
    """The exact log-sum-exp merge (step a5) and the finalize (step a6) at the softmax-stress workload's
    row count (B=2, Hq=16, Nq=262144, D=128: 8.4M rows), the unit its 16 KV chunks repeat: one two-way
    fold of fp32 partial triples, then the normalisation into bf16 with lse.  Both are HBM-bound.
    Algorithmic bytes: a J-way merge reads J (D + 2) 4 and writes (D + 2) 4 bytes per row; the finalize
    reads (D + 2) 4 and writes 2 D + 4.  Also a 16-way merge at 1/8 of the rows.  Partials are seeded
    random (O ~ N(0, 1), m ~ N(0, 16), l ~ U[1, 101]); times are HIP events on the current stream."""
    dev = "cuda:0"
    B, Hq, N, D = 2, 16, 262144, 128
    g = torch.Generator(device=dev)
    g.manual_seed(0xC05A0005)

    def part(n):
        o = torch.randn(B, Hq, n, D, device=dev, generator=g)
        ml = torch.empty(B, Hq, n, 2, device=dev)
        ml[..., 0] = torch.randn(B, Hq, n, device=dev, generator=g) * 4.0
        ml[..., 1] = torch.rand(B, Hq, n, device=dev, generator=g) * 100.0 + 1.0
        return o, ml

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for i in range(reps):
            e[2 * i].record(st)
            fn()
            e[2 * i + 1].record(st)
        torch.cuda.synchronize()
        return sum(e[2 * i].elapsed_time(e[2 * i + 1]) for i in range(reps)) / reps

    reps = max(3, steps // 2)
    res = {"workload": f"merge_b{B}_h{Hq}_n{N}_d{D}_f32", "rows": B * Hq * N, "peak_gbs": PEAK_HBM_GBS}
    parts = [part(N), part(N)]
    out = (torch.empty_like(parts[0][0]), torch.empty_like(parts[0][1]))
    ms = timed(lambda: cqsa.lse_merge(parts, out=out), reps)
    nbytes = 3 * B * Hq * N * (D + 2) * 4
    res["merge2"] = {"ms": round(ms, 4), "bytes": nbytes, "gbs": round(nbytes / ms / 1e6, 1),
                     "frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4)}
    ms = timed(lambda: cqsa.finalize(out[0], out[1], out_dtype=torch.bfloat16), reps)
    nbytes = B * Hq * N * ((D + 2) * 4 + 2 * D + 4)
    res["finalize_bf16"] = {"ms": round(ms, 4), "bytes": nbytes, "gbs": round(nbytes / ms / 1e6, 1),
                            "frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4)}
    del parts, out
    n16 = N // 8
    parts = [part(n16) for _ in range(16)]
    out = (torch.empty_like(parts[0][0]), torch.empty_like(parts[0][1]))
    ms = timed(lambda: cqsa.lse_merge(parts, out=out), reps)
    nbytes = 17 * B * Hq * n16 * (D + 2) * 4
    res["merge16_rows_div8"] = {"ms": round(ms, 4), "bytes": nbytes, "gbs": round(nbytes / ms / 1e6, 1),
                                "frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4)}
    del parts, out
    torch.cuda.empty_cache()
    print(f"[bench] merge: 2-way {res['merge2']['gbs']} GB/s, finalize {res['finalize_bf16']['gbs']} GB/s, "
          f"16-way {res['merge16_rows_div8']['gbs']} GB/s", file=sys.stderr, flush=True)
    return res


def run_streamed_backward(cqsa, torch, synth) -> dict:
    """dQ, dK, dV of the 4M-token causal case from pinned host memory under the 16e9-byte budget (fp32
    gradients on the host).  At this size the FP64 reference is out of reach, so the check is two
    identities that hold at any size: sum_j dV_j = sum_i dO_i (each row of P sums to one) and
    sum_j dK_j = 0 (each row of dS sums to zero)."""
    w = synth.workload(3)
    q, k, v, _ = synth.make_inputs(w, pin=True)
    do = torch.empty(q.shape, dtype=q.dtype, pin_memory=True)
    synth.fill_(do, seed=w.seed, tensor_id=synth.TENSOR_DO)
    out, lse = cqsa.attention(q, k, v, is_causal=True, mem_budget=w.mem_budget, return_lse=True)
    t0 = time.perf_counter()
    dq, dk, dv, info = cqsa.attention_backward(q, k, v, out, do, lse, is_causal=True, mem_budget=w.mem_budget,
                                               grad_dtype=torch.float32, return_info=True)
    wall = time.perf_counter() - t0
    sdo = do.sum(2, dtype=torch.float64)
    e_v = float((dv.sum(2, dtype=torch.float64) - sdo).abs().max() / sdo.abs().max())
    e_k = float(dk.sum(2, dtype=torch.float64).abs().max() / dk.abs().sum(2, dtype=torch.float64).max())
    print(f"[bench] streamed backward: {wall:.1f} s; sum dV vs sum dO {e_v:.1e}, sum dK {e_k:.1e}",
          file=sys.stderr, flush=True)
    return {"workload": w.name, "seconds": round(wall, 2), "tokens_per_s": round(w.B * w.Nq / wall, 1),
            "tflops": round(2.5 * w.flops() / wall / 1e12, 2),
            "note": "10 D FLOP per visible pair (2.5x the forward); fp32 gradients streamed back to pinned host memory",
            "q_chunk": info["q_chunk"], "kv_chunk": info["kv_chunk"], "chunk_pairs": info["chunk_pairs"],
            "h2d_bytes": info["h2d_bytes"], "h2d_seconds_busy": round(info["h2d_ms"] / 1e3, 3),
            "d2h_bytes": info["d2h_bytes"], "workspace_bytes": info["workspace_bytes"],
            "identity_sum_dv_rel": e_v, "identity_sum_dk_rel": e_k}


def streamed_run(cqsa, torch, w, q, k, v, out, cqs, cqs_itr=1) -> dict:
    # link peak: one pinned 1 GiB H2D copy timed by the host clock between two synchronisations
    src = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(3):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    link = 3 * (1 << 30) / (time.perf_counter() - t1) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    base_alloc = torch.cuda.memory_allocated()
    t2 = time.perf_counter()
    _, info = cqsa.attention(q, k, v, is_causal=True, mem_budget=w.mem_budget, out=out, return_info=True, cqs=cqs,
                             cqs_itr=cqs_itr if cqs else None)
    wall = time.perf_counter() - t2
    # the call's device memory: its workspace comes from PyTorch's allocator (the library then allocates
    # nothing itself), so the allocator's high-water mark over the call is the call's peak
    peak = torch.cuda.max_memory_allocated() - base_alloc
    print(f"[bench] streamed {'grid' if not cqs else f'cqs c={cqs} itr={cqs_itr}'}: {wall:.2f} s", file=sys.stderr,
          flush=True)
    tok = w.B * w.Nq / wall
    h2d_gbs = info["h2d_bytes"] / (info["h2d_ms"] / 1e3) / 1e9 if info["h2d_ms"] > 0 else None
    # parity on sampled rows against the FP64 reference (first/last rows, Q-chunk edges, seeded rows)
    import numpy as np
    import oracle
    rng = np.random.default_rng(4)
    qc = info["q_chunk"]
    edges = [w.Nq * p // cqs ** cqs_itr for p in range(1, cqs ** cqs_itr)][:6] if cqs else [qc - 1, qc]
    idx = sorted({0, 1, w.Nq - 1, w.Nq - 2, *edges, *[e - 1 for e in edges], *rng.integers(0, w.Nq, 10).tolist()})
    rows = np.array([(0, h, i) for h in (0, 5) for i in idx if 0 <= i < w.Nq], dtype=np.int64)
    t3 = time.perf_counter()
    ref = oracle.attention_rows(q, k, v, causal=True, scale=w.scale, rows=rows)
    got = out[0, torch.from_numpy(rows[:, 1]), torch.from_numpy(rows[:, 2])].double().numpy()
    max_abs = float(np.abs(got - ref["o"]).max())
    print(f"[bench] streamed parity on {len(rows)} rows: max_abs {max_abs:.2e} ({time.perf_counter() - t3:.1f} s)",
          file=sys.stderr, flush=True)
    # the same call with every tensor already in HBM, for the overlap score of the BlockStreamer README
    # ("Profiler and validation status"): 1 - (streamed - resident) / isolated H2D time, not clamped
    resident = overlap = None
    if not cqs:
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        od = torch.empty(qd.shape, dtype=qd.dtype, device="cuda")
        torch.cuda.synchronize()
        t4 = time.perf_counter()
        cqsa.attention(qd, kd, vd, is_causal=True, out=od)
        torch.cuda.synchronize()
        resident = time.perf_counter() - t4
        overlap = 1.0 - (wall - resident) / (info["h2d_bytes"] / (link * 1e9))
        del qd, kd, vd, od
        torch.cuda.empty_cache()
        print(f"[bench] same call with the tensors in HBM: {resident:.2f} s; overlap score {overlap:.3f}",
              file=sys.stderr, flush=True)
    return {"workload": w.name, "schedule": "grid" if not cqs else f"cyclic quorum sets, c={cqs}, itr={cqs_itr}",
            "seconds": round(wall, 3), "tokens_per_s": round(tok, 1),
            "tflops": round(w.flops() / wall / 1e12, 2), "h2d_bytes": info["h2d_bytes"],
            "h2d_gbs_during_copies": round(h2d_gbs, 2) if h2d_gbs else None,
            "h2d_link_peak_gbs_host_timed": round(link, 2),
            "h2d_frac_of_link": round(h2d_gbs / link, 3) if h2d_gbs else None,
            "q_chunk": info["q_chunk"], "kv_chunk": info["kv_chunk"], "chunk_pairs": info["chunk_pairs"],
            "cqs_subproblems": info["cqs_subproblems"],
            "workspace_bytes": info["workspace_bytes"], "budget_bytes": info["budget_bytes"],
            "peak_device_bytes": int(peak), "mem_budget": w.mem_budget,
            "resident_seconds": round(resident, 3) if resident else None,
            "overlap_score": round(overlap, 3) if overlap is not None else None,
            "parity_rows": int(len(rows)), "parity_max_abs_fp16_out": max_abs,
            "note": "wall time includes PCIe transfers from/to pinned host memory; not the headline value"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the attention path has no "
                                   "multi-GPU component (one GPU's share is the measured kernel)",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    import synth
    import exact_long_context_cqsa_amd as cqsa

    if args.fwd_variant:
        cqsa.set_test_controls(args.fwd_variant, -1)
    w = synth.workload(args.workload, nk=args.nk)
    if w.host_resident:
        raise SystemExit("use --streamed for the host-resident case")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.perf_counter()
    q, k, v, _ = synth.make_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty((w.B, w.Hq, w.Nq, w.D), dtype=w.dtype, device=dev)
    print(f"[bench] {w.name}: inputs ready in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)

    kw = {"kv_chunk": args.kv_chunk or w.kv_chunk} if (args.kv_chunk or w.kv_chunk) else {}
    for _ in range(args.warmup):
        cqsa.attention(qd, kd, vd, is_causal=w.causal, out=out, **kw)
    torch.cuda.synchronize()
    info = cqsa.attention(qd, kd, vd, is_causal=w.causal, out=out, return_info=True, **kw)[1]
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        cqsa.attention(qd, kd, vd, is_causal=w.causal, out=out, **kw)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ms_step = wall * 1e3 / args.steps
    ms_kernel = sum(per) / len(per)
    flops = w.flops()
    value = flops / (ms_step / 1e3) / 1e12
    achieved = flops / (ms_kernel / 1e3) / 1e12
    print(f"[bench] step {ms_step:.3f} ms (events {ms_kernel:.3f} ms, min {min(per):.3f}) -> {value:.1f} TFLOP/s",
          file=sys.stderr, flush=True)

    measured = None
    if args.probe:
        # the rates this device delivers, measured after the timed steps so that they do not warm it
        # first: the fraction of the measured matrix-core rate is the kernel's efficiency at the clock
        # the chip holds, which the datasheet peak (2.4 GHz) does not reflect
        pr = cqsa.probe_device(copy_bytes=1 << 30, repeats=5)
        measured = {"mfma_f16_tflops": round(pr["mfma_f16_tflops"], 1),
                    "mfma_clock_ghz": round(pr["mfma_clock_ghz"], 3),
                    "mfma_flop_per_clk_per_cu": round(pr["mfma_flop_per_clk_per_cu"] or 0.0, 1),
                    "frac_of_measured_mfma": round(achieved / pr["mfma_f16_tflops"], 4),
                    "lds_read_tbs": round(pr["lds_read_tbs"], 2),
                    "lds_bytes_per_clk_per_cu": round(pr["lds_bytes_per_clk_per_cu"] or 0.0, 1),
                    "hbm_copy_gbs": round(pr["hbm_copy_gbs"], 1),
                    "compute_units": pr["compute_units"],
                    "source": "cqsa_probe_device: back-to-back v_mfma_f32_32x32x16_f16, ds_read_b128 and a "
                              "1 GiB copy on this device, fastest of 5 launches each"}
        print(f"[bench] probe: MFMA {measured['mfma_f16_tflops']} TFLOP/s at {measured['mfma_clock_ghz']} GHz "
              f"({measured['mfma_flop_per_clk_per_cu']} FLOP/clk/CU), LDS {measured['lds_read_tbs']} TB/s "
              f"({measured['lds_bytes_per_clk_per_cu']} B/clk/CU), HBM copy {measured['hbm_copy_gbs']} GB/s",
              file=sys.stderr, flush=True)

    cqs_resident = None
    if args.cqs:
        for _ in range(2):
            cqsa.attention(qd, kd, vd, is_causal=w.causal, out=out, cqs=args.cqs, wave_tokens=args.wave_tokens,
                           cqs_itr=args.cqs_itr)
        torch.cuda.synchronize()
        c0 = time.perf_counter()
        n_cqs = max(3, args.steps // 4)
        for _ in range(n_cqs):
            cinfo = cqsa.attention(qd, kd, vd, is_causal=w.causal, out=out, cqs=args.cqs, wave_tokens=args.wave_tokens,
                                   cqs_itr=args.cqs_itr, return_info=True)[1]
        torch.cuda.synchronize()
        cms = (time.perf_counter() - c0) * 1e3 / n_cqs
        cqs_resident = {"c": args.cqs, "itr": args.cqs_itr, "ms_per_call": round(cms, 4), "tflops": round(flops / (cms / 1e3) / 1e12, 2),
                        "pairs": cinfo["chunk_pairs"], "subproblems": cinfo["cqs_subproblems"],
                        "waves": cinfo["cqs_waves"], "wave_tokens": cinfo["wave_tokens"],
                        "kernel_launches": cinfo["kernel_launches"]}
        print(f"[bench] cqs c={args.cqs}: {cms:.3f} ms per call ({cinfo['cqs_waves']} waves, "
              f"{cinfo['kernel_launches']} launches)", file=sys.stderr, flush=True)
    split_p = None
    if args.split_p:
        import numpy as np
        import oracle
        for _ in range(2):
            cqsa.attention(qd, kd, vd, is_causal=w.causal, out=out, precision=1)
        torch.cuda.synchronize()
        s0 = time.perf_counter()
        n_sp = max(3, args.steps // 2)
        for _ in range(n_sp):
            cqsa.attention(qd, kd, vd, is_causal=w.causal, out=out, precision=1)
        torch.cuda.synchronize()
        sms = (time.perf_counter() - s0) * 1e3 / n_sp
        rng = np.random.default_rng(12)
        rows = np.array([(0, h, int(i)) for h in range(0, w.Hq, 3) for i in rng.integers(0, w.Nq, 24)], dtype=np.int64)
        ref = oracle.attention_rows(q, k, v, causal=w.causal, scale=w.scale, rows=rows)
        errs = {}
        for prec in (0, 1):
            o32 = cqsa.attention(qd, kd, vd, is_causal=w.causal, out_dtype=torch.float32, precision=prec)
            b_, h_, i_ = (torch.from_numpy(rows[:, c]) for c in range(3))
            errs[prec] = float(np.abs(o32.cpu()[b_, h_, i_].double().numpy() - ref["o"]).max())
            del o32
        split_p = {"kernel": cqsa.fwd_kernel_name(w.D, 1), "ms_per_call": round(sms, 4),
                   "tflops": round(flops / (sms / 1e3) / 1e12, 2), "rows_checked": int(len(rows)),
                   "max_abs_vs_fp64_split": errs[1], "max_abs_vs_fp64_default": errs[0]}
        print(f"[bench] split-P: {sms:.3f} ms per call, max_abs {errs[1]:.2e} (default {errs[0]:.2e})",
              file=sys.stderr, flush=True)
    backward = None
    if args.backward:
        out_b, lse_b = cqsa.attention(qd, kd, vd, is_causal=w.causal, return_lse=True)
        dout = torch.randn_like(out_b)
        for _ in range(2):
            cqsa.attention_backward(qd, kd, vd, out_b, dout, lse_b, is_causal=w.causal)
        torch.cuda.synchronize()
        b0 = time.perf_counter()
        n_b = max(3, args.steps // 2)
        for _ in range(n_b):
            grads = cqsa.attention_backward(qd, kd, vd, out_b, dout, lse_b, is_causal=w.causal)
        torch.cuda.synchronize()
        bms = (time.perf_counter() - b0) * 1e3 / n_b
        bflops = 2.5 * flops      # the five products of the derivative: 10 D per visible pair
        backward = {"ms_per_call": round(bms, 4), "tflops": round(bflops / (bms / 1e3) / 1e12, 2),
                    "algorithmic_flop": bflops,
                    "note": "dQ, dK, dV from the forward's out and lse; 10 D FLOP per visible pair (the dQ "
                            "kernel recomputes S and dP, so 14 D per pair are executed)"}
        del grads, out_b, lse_b, dout
        print(f"[bench] backward: {bms:.3f} ms per call ({backward['tflops']} TFLOP/s)", file=sys.stderr, flush=True)
    kernel = cqsa.fwd_kernel_name(w.D)
    prof_path = args.profile or os.path.join(ROOT, "profiles", f"{kernel.split()[0]}_{w.name}.md")
    traffic, traffic_src = measured_traffic(prof_path)
    prof = profile_figures(prof_path, os.path.join(ROOT, "profiles", f"{kernel.split()[0]}_mfma_counters_{w.name}.md"),
                           flops)
    line = {
        "metric": "causal attention fwd TFLOP/s & % MFMA peak (1 GPU); tokens/s at 4M ctx",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if w.dtype == torch.float16 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk, "D": w.D,
                   "causal": w.causal, "kv_chunk": kw.get("kv_chunk"), "plan": {
                       k_: info[k_] for k_ in ("kv_splits", "n_kv_chunks", "chunk_pairs", "kernel_launches",
                                               "block_m")},
                   "tokens_per_s": round(w.B * w.Nq / (ms_step / 1e3), 1),
                   "algorithmic_flop_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_F16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4), "traffic": traffic,
                     "traffic_source": traffic_src,
                     "kernel": kernel,
                     "kernel_ms": round(ms_kernel, 4),
                     "launches_per_step": info["kernel_launches"]},
    }
    if prof:
        line["roofline"]["profile"] = prof
    if measured:
        line["roofline"]["measured_on_this_device"] = measured
    if cqs_resident:
        line["cqs_resident"] = cqs_resident
    if split_p:
        line["split_p"] = split_p
    if backward:
        line["backward"] = backward
    kept = {}
    if args.configs and args.workload == 1 and not args.kv_chunk:
        line["configs"], kept = run_configs(cqsa, torch, synth, args.steps)
    if args.streamed:
        line["streamed_4m"] = run_streamed(cqsa, torch, synth, cqs=args.cqs or None, cqs_itr=args.cqs_itr,
                                           keep=kept if args.configs else None)
    if args.merge:
        line["merge"] = run_merge(cqsa, torch, args.steps)
    if args.streamed_backward:
        line["streamed_backward_4m"] = run_streamed_backward(cqsa, torch, synth)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_seconds, kept, full=args.cpu_full, limit=args.cpu_full_limit)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
