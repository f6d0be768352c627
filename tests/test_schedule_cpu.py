"""The race test of the executors, on the CPU: cqsa_schedule_trace records the copies, launches, event
records and waits a call would issue (nothing runs), and a happens-before analysis over the streams
and events checks that every two operations touching one device byte, one of them writing, are
ordered; that every workspace read follows a write of it; and that everything is finished before the
call returns.  Run over the grid schedule (forced Q and KV chunks, both merge modes, host and device
operands, token-major host layouts, lse), single-pass KV splits, the quorum-set waves and the
chunked backward."""
import re

import pytest
import torch

GB = 1 << 30
ADDR = {"q": 1 << 36, "k": 2 << 36, "v": 3 << 36, "out": 4 << 36,   # stand-in addresses, far apart
        "dout": 5 << 36, "lse": 6 << 36, "dq": 7 << 36, "dk": 8 << 36, "dv": 9 << 36}


def m():
    import exact_long_context_cqsa_amd as mod
    return mod


class Op:
    __slots__ = ("idx", "kind", "stream", "reads", "writes", "vc")

    def __init__(self, idx, kind, stream):
        self.idx, self.kind, self.stream = idx, kind, stream
        self.reads, self.writes, self.vc = [], [], None


def analyse(text):
    """Vector clocks over the trace: returns (ops, workspace range, final-sync op or None)."""
    clocks, events, ops, ws, last_sync = {}, {}, [], None, None

    def tick(s):
        c = clocks.setdefault(s, {})
        c[s] = c.get(s, 0) + 1
        return dict(c)

    for ln in text.splitlines():
        f = ln.split()
        if not f:
            continue
        if f[0] == "workspace":
            _, lo, hi = f[1].split(":")
            ws = (int(lo), int(hi))
        elif f[0] == "record":
            events[f[2]] = dict(clocks.get(f[1], {}))
        elif f[0] == "wait":
            if f[2] in events:                   # a wait on a never-recorded event orders nothing
                c = clocks.setdefault(f[1], {})
                for s, t in events[f[2]].items():
                    c[s] = max(c.get(s, 0), t)
        elif f[0] in ("copy", "kernel", "sync"):
            op = Op(len(ops), f[0] if f[0] != "kernel" else f[2], f[1])
            for tok in f[2:]:
                mm = re.match(r"^([RW]):(\d+):(\d+)$", tok)
                if mm:
                    (op.reads if mm.group(1) == "R" else op.writes).append((int(mm.group(2)), int(mm.group(3))))
            op.vc = tick(f[1])
            ops.append(op)
            if f[0] == "sync":
                last_sync = op
        else:
            raise AssertionError(f"unknown trace line {ln!r}")
    return ops, ws, last_sync


def hb(a, b):
    return a.idx != b.idx and b.vc.get(a.stream, 0) >= a.vc[a.stream]


def overlap(r, s):
    return r[0] < s[1] and s[0] < r[1]


def check(text, streamed):
    ops, ws, last_sync = analyse(text)
    assert ops, "empty trace"
    races, unwritten = [], []
    for i, a in enumerate(ops):
        for b in ops[i + 1:]:
            conflict = any(overlap(w, x) for w in a.writes for x in b.reads + b.writes) or \
                any(overlap(w, x) for w in b.writes for x in a.reads)
            if conflict and not hb(a, b) and not hb(b, a):
                races.append((a.idx, a.kind, a.stream, b.idx, b.kind, b.stream))
    if ws:
        for b in ops:
            for r in b.reads:
                if overlap(r, ws) and not any(hb(a, b) and any(overlap(w, r) for w in a.writes) for a in ops):
                    unwritten.append((b.idx, b.kind, r))
    assert not races, f"unordered conflicting operations: {races[:5]}"
    assert not unwritten, f"workspace reads with no earlier write: {unwritten[:5]}"
    if streamed:
        assert last_sync is not None, "a streamed call must synchronise before returning"
        late = [a.idx for a in ops if a is not last_sync and not hb(a, last_sync)]
        assert not late, f"operations not finished when the call returns: {late[:5]}"
    return ops


def spec(name, shape, where, dtype=torch.float16, token_major=False):
    B, H, N, D = shape
    stride = [N * H * D, D, H * D, 1] if token_major else [H * N * D, N * D, D, 1]
    return (shape, dtype, where, ADDR[name], stride)


def trace(Nq, Nk, *, H=4, Hkv=None, D=64, causal=True, where=("host", "host", "host", "host"), budget=4 * GB,
          token_major=False, **kw):
    Hkv = Hkv or H
    q = spec("q", (1, H, Nq, D), where[0], token_major=token_major)
    k = spec("k", (1, Hkv, Nk, D), where[1], token_major=token_major)
    v = spec("v", (1, Hkv, Nk, D), where[2], token_major=token_major)
    o = spec("out", (1, H, Nq, D), where[3], token_major=token_major)
    return m().schedule_trace(q, k, v, causal, budget, out=o, **kw)


GRID = [
    dict(Nq=8192, Nk=8192, q_chunk=2048, kv_chunk=1024, merge=1),               # merge kernel
    dict(Nq=8192, Nk=8192, q_chunk=2048, kv_chunk=1024, merge=2),               # fused accumulation
    dict(Nq=6000, Nk=9000, q_chunk=1536, kv_chunk=2560, merge=2, causal=False),  # ragged chunks
    dict(Nq=4096, Nk=12288, kv_chunk=1024, want_lse=True),                     # bottom-right causal, lse
    dict(Nq=8192, Nk=8192, q_chunk=4096, kv_chunk=2048, token_major=True),
    dict(Nq=8192, Nk=8192, H=8, Hkv=2, kv_chunk=2048, where=("device", "host", "host", "device")),
    dict(Nq=8192, Nk=8192, kv_chunk=2048, where=("host", "device", "device", "host"), want_lse=True),
    dict(Nq=8192, Nk=8192, kv_chunk=1024, where=("device",) * 4),               # resident, forced split
    dict(Nq=1 << 20, Nk=1 << 20, H=8, budget=3 * 10**9),                         # the planner's own chunks
    # out on the device, lse in pinned host memory: the lse staging of one Q chunk must not be
    # rewritten by the next Q chunk while its D2H copy still reads it
    dict(Nq=8192, Nk=8192, q_chunk=2048, kv_chunk=1024, merge=2, where=("device",) * 4, want_lse="host"),
    dict(Nq=8192, Nk=8192, q_chunk=2048, kv_chunk=1024, merge=1, where=("device",) * 4, want_lse="host"),
    dict(Nq=8192, Nk=8192, q_chunk=2048, kv_chunk=8192, where=("device",) * 4, want_lse="host"),  # single pass per Q chunk
    dict(Nq=8192, Nk=8192, q_chunk=2048, kv_chunk=1024, where=("host",) * 4, want_lse="device"),
]


def _streamed(kw):
    return "host" in kw.get("where", ("host",)) or kw.get("want_lse") == "host"


@pytest.mark.parametrize("kw", GRID, ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items() if k != "where")
                         + ("," + "".join(w[0] for w in d["where"]) if "where" in d else ""))
def test_grid_schedule_is_race_free(kw):
    kw = dict(kw)
    streamed = _streamed(kw)
    ops = check(trace(**kw), streamed)
    kinds = {o.kind for o in ops}
    assert "fwd" in kinds
    if streamed:
        assert "copy" in kinds and len({o.stream for o in ops}) >= 2


def test_single_pass_kv_splits_are_race_free():
    ops = check(trace(2048, 131072, H=32, Hkv=8, D=128, where=("device",) * 4, kv_splits=4), streamed=False)
    assert [o.kind for o in ops] == ["fwd", "merge"]


@pytest.mark.parametrize("c,wt,budget", [(7, None, 4 * GB), (7, 1, 4 * GB), (13, 5000, 4 * GB), (31, None, 4 * GB),
                                         (31, None, 480_000_000)])
def test_quorum_set_waves_are_race_free(c, wt, budget):
    ops = check(trace(131072, 131072, H=8, cqs=c, wave_tokens=wt, budget=budget, want_lse=True), streamed=True)
    assert sum(o.kind == "wave" for o in ops) >= 1
    resident = check(trace(30000, 30000, where=("device",) * 4, cqs=c, wave_tokens=wt), streamed=False)
    assert sum(o.kind == "wave" for o in resident) >= 1
    lse_host = check(trace(30000, 30000, where=("device",) * 4, cqs=c, wave_tokens=wt, want_lse="host"),
                     streamed=True)
    assert sum(o.kind == "copy" for o in lse_host) >= 1


@pytest.mark.parametrize("c,itr,wt", [(7, 2, None), (3, 3, 20000), (13, 2, None)])
def test_quorum_set_waves_of_depth_are_race_free(c, itr, wt):
    ops = check(trace(131072, 131072, H=8, cqs=c, cqs_itr=itr, wave_tokens=wt, want_lse=True), streamed=True)
    assert sum(o.kind == "wave" for o in ops) >= 1
    check(trace(30000, 30000, where=("device",) * 4, cqs=c, cqs_itr=itr), streamed=False)


def test_checker_catches_a_missing_wait():
    """Plant the mistake in the trace, not in the library: drop the compute stream's wait for a staged
    K/V copy (or the copy stream's wait for the compute that last used a buffer)."""
    text = trace(8192, 8192, q_chunk=4096, kv_chunk=1024)
    check(text, streamed=True)
    lines = text.splitlines()
    caught = 0
    waits = [i for i, ln in enumerate(lines) if ln.startswith("wait ")]
    for i in waits[3:9]:
        broken = "\n".join(lines[:i] + lines[i + 1:])
        try:
            check(broken, streamed=True)
        except AssertionError:
            caught += 1
    assert caught >= 4, caught


def test_trace_needs_explicit_placement_and_budget():
    s = (1, 2, 512, 64)
    with pytest.raises(m().CqsaError):
        m().schedule_trace((s, torch.float16, "detect", 1 << 36), (s, torch.float16, "host", 2 << 36),
                           (s, torch.float16, "host", 3 << 36), True, GB, out=(s, torch.float16, "host", 4 << 36))
    with pytest.raises(m().CqsaError):
        m().schedule_trace((s, torch.float16, "host", 1 << 36), (s, torch.float16, "host", 2 << 36),
                           (s, torch.float16, "host", 3 << 36), True, 0, out=(s, torch.float16, "host", 4 << 36))


BWD = [
    dict(Nq=8192, Nk=8192, q_chunk=2048, kv_chunk=1024),                       # all on the host
    dict(Nq=4096, Nk=10240, q_chunk=1024, kv_chunk=4096, H=8, Hkv=2, D=128),     # GQA, bottom-right causal
    dict(Nq=6000, Nk=6000, q_chunk=1536, kv_chunk=2560, causal=False),           # ragged chunks
    dict(Nq=8192, Nk=8192, kv_chunk=2048, place="mixed"),                       # device q/k/v/out, host grads
    dict(Nq=8192, Nk=8192, q_chunk=2048, kv_chunk=2048, place="device"),        # resident, forced chunks
    dict(Nq=1 << 20, Nk=1 << 20, H=8, budget=6 * 10**9),                          # the planner's own chunks
]


@pytest.mark.parametrize("kw", BWD, ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_chunked_backward_schedule_is_race_free(kw):
    kw = dict(kw)
    Nq, Nk, H = kw.pop("Nq"), kw.pop("Nk"), kw.pop("H", 4)
    Hkv, D, causal = kw.pop("Hkv", H), kw.pop("D", 64), kw.pop("causal", True)
    place, budget = kw.pop("place", "host"), kw.pop("budget", 4 * GB)
    qside = "device" if place in ("mixed", "device") else "host"
    grads = "device" if place == "device" else "host"
    t = lambda name, shape, where: spec(name, shape, where)
    qs, ks = (1, H, Nq, D), (1, Hkv, Nk, D)
    text = m().backward_schedule_trace(
        t("q", qs, qside), t("k", ks, qside), t("v", ks, qside), t("out", qs, qside), t("dout", qs, qside),
        (qside, ADDR["lse"]), t("dq", qs, grads), t("dk", ks, grads), t("dv", ks, grads), causal, budget, **kw)
    ops = check(text, streamed=True)
    kinds = [o.kind for o in ops]
    assert "bwd_stats" in kinds and "bwd_dq" in kinds and "bwd_dkdv" in kinds and "cast" in kinds
