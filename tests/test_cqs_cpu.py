"""The cyclic quorum-set schedule's host logic, without a GPU: the built-in interest sets, the owner
of every (query part, key part) pair, set validation, and the plan (pairs, subproblems, bytes)."""
import itertools

import pytest
import torch

GB = 10**9


def m():
    import exact_long_context_cqsa_amd as mod
    return mod


def parts_of(c, iset, i):
    return {(i + s) % c for s in iset}


@pytest.mark.parametrize("c", [3, 7, 13, 21, 31])
def test_builtin_sets_are_perfect_difference_sets(c):
    """Every nonzero residue mod c is exactly one difference of two set elements (so every pair of
    parts meets in exactly one subproblem, and the set has l = (1 + sqrt(4c - 3)) / 2 elements)."""
    s = m().cqs_default_set(c)
    assert len(s) * (len(s) - 1) == c - 1
    diffs = sorted((a - b) % c for a in s for b in s if a != b)
    assert diffs == list(range(1, c))


def test_no_builtin_set_for_other_c():
    assert m().cqs_default_set(5) == ()
    assert m().cqs_default_set(133) == ()


@pytest.mark.parametrize("c,iset", [(7, (0, 1, 3)), (13, (0, 1, 3, 9)), (31, (0, 1, 3, 8, 12, 18)),
                                    (10, (0, 1, 2, 3, 6)), (9, (0, 1, 2, 4, 6)), (4, (0, 1, 2)), (1, (0,)),
                                    (5, (0, 1, 2, 3, 4))])
def test_owner_is_the_first_subproblem_holding_both_parts(c, iset):
    own = m().cqs_assign(c, iset)
    per_sub = [0] * c
    for a, b in itertools.product(range(c), repeat=2):
        holders = [i for i in range(c) if {a, b} <= parts_of(c, iset, i)]
        assert holders, (a, b)
        assert own[a][b] == holders[0]
        per_sub[own[a][b]] += 1
    # every pair is computed once: c^2 pairs over the subproblems, none beyond l^2 in one subproblem
    assert sum(per_sub) == c * c
    assert max(per_sub) <= len(iset) ** 2


@pytest.mark.parametrize("c,iset,msg", [(7, (0, 1), "share no subproblem"), (7, (0, 1, 1), "repeated"),
                                        (7, (0, 7, 1), "outside"), (3, (0, 1, 2, 0), "size"), (0, (0,), "outside"),
                                        (8, (0, 1, 3), "share no subproblem")])
def test_invalid_sets_are_rejected(c, iset, msg):
    with pytest.raises(m().CqsaError) as e:
        m().cqs_assign(c, iset)
    assert msg in str(e.value)


def _plan(N, causal, c, iset=None, where="device", H=8, D=64, Nq=None, budget=64 * GB, **kw):
    Nq = N if Nq is None else Nq
    shp_q, shp_kv = (1, H, Nq, D), (1, H, N, D)
    w = {n: where for n in ("q", "k", "v", "out")}
    return m().plan((shp_q, torch.float16), (shp_kv, torch.float16), (shp_kv, torch.float16), causal, budget,
                    where=w, num_cus=256, cqs=c if iset is None else (c, iset), **kw)


def test_plan_pairs_and_subproblems():
    p = _plan(7000, False, 7)
    assert p["chunk_pairs"] == 49 and p["cqs_c"] == 7 and p["cqs_subproblems"] == 7
    assert p["n_q_chunks"] == 7 and p["q_chunk"] == 1000
    p = _plan(7000, True, 7)
    assert p["chunk_pairs"] == 28          # causal: key part <= query part
    # the default wave budget holds every subproblem: one launch folds each query part once
    assert p["cqs_waves"] == 1 and p["merges"] == 7 and p["kernel_launches"] == 3
    assert p["wave_tokens"] == 1 << 20
    # accumulator for every query row: fp32 O plus (m, l)
    assert p["workspace_bytes"] >= 8 * 7000 * (64 + 2) * 4
    # ragged parts: 7001 rows over 7 parts of 1000 or 1001
    p = _plan(7001, True, 7)
    assert p["q_chunk"] == 1001 and p["chunk_pairs"] == 28


def test_plan_streamed_4m_fits_16gb_with_31_parts():
    N = 4_194_304
    p = _plan(N, True, 31, where="host", budget=16 * GB)
    assert p["streamed"] == 1 and p["cqs_subproblems"] >= 1
    assert p["workspace_bytes"] <= 0.85 * 16 * GB
    # every subproblem stages only the parts of its owned non-empty pairs
    assert p["h2d_bytes"] > 3 * 8 * N * 64 * 2 // 31


def test_plan_too_small_budget_and_conflicting_options():
    with pytest.raises(m().CqsaError) as e:
        _plan(4_194_304, True, 31, where="host", budget=4 * GB)
    assert "BUDGET" in str(e.value)
    with pytest.raises(m().CqsaError):
        _plan(7000, True, 7, kv_chunk=1024)
    with pytest.raises(m().CqsaError):
        _plan(7000, True, 5)               # no built-in set for c = 5


def _waves_model(N, causal, c, iset, W):
    """The wave cut from its definition: subproblems in index order, each owning the pairs (a, b) whose
    smallest common subproblem it is; a wave takes the next subproblem while the query rows of the
    union of its query parts plus the key rows of the union of its key parts stay <= W (a wave always
    takes at least one).  Returns (waves, launches, folds) for parts of <= 32 per launch."""
    lo = [N * p // c for p in range(c + 1)]
    ln = [lo[p + 1] - lo[p] for p in range(c)]
    members = [{(i + s) % c for s in iset} for i in range(c)]
    subs = []
    for i in range(c):
        prs = []
        for a in range(c):
            for b in range(c):
                if min(j for j in range(c) if a in members[j] and b in members[j]) != i:
                    continue
                if ln[a] == 0 or ln[b] == 0 or (causal and lo[b] > lo[a + 1] - 1):
                    continue
                prs.append((a, b))
        if prs:
            subs.append(prs)
    waves, cur, qs, ks = [], [], set(), set()
    for prs in subs:
        nq, nk = qs | {a for a, _ in prs}, ks | {b for _, b in prs}
        if cur and sum(ln[a] for a in nq) + sum(ln[b] for b in nk) > W:
            waves.append(cur)
            cur, qs, ks = [], set(), set()
            nq, nk = {a for a, _ in prs}, {b for _, b in prs}
        cur = cur + prs
        qs, ks = nq, nk
    if cur:
        waves.append(cur)
    return waves, len(subs)


@pytest.mark.parametrize("W", [1, 3000, 5000, 9000, 14000, 1 << 20])
def test_wave_cut_follows_the_budget(W):
    N, c, iset = 7000, 7, (0, 1, 3)
    waves, nsub = _waves_model(N, True, c, iset, W)
    p = _plan(N, True, c, wave_tokens=W)
    assert p["cqs_waves"] == len(waves) and p["cqs_subproblems"] == nsub
    assert p["merges"] == sum(len({a for a, _ in wv}) for wv in waves)   # one fold per query part and wave
    assert p["kernel_launches"] == len(waves) + 2
    if W == 1:
        assert p["cqs_waves"] == nsub


def test_wave_launches_split_at_32_parts():
    # c = 57 (a perfect difference set of size 8 mod 57): one wave holds all 57 query parts, so its
    # pairs run as launches of at most 32 query parts and 32 key parts each
    iset = (0, 1, 3, 13, 32, 36, 43, 52)
    assert sorted({(x - y) % 57 for x in iset for y in iset if x != y}) == list(range(1, 57))
    p = _plan(57 * 64, False, 57, iset=iset)
    assert p["cqs_waves"] == 1 and p["chunk_pairs"] == 57 * 57
    assert p["kernel_launches"] - 2 >= 4      # 57 query parts x 57 key parts in 32 x 32 blocks
    assert p["merges"] >= 57


def test_wave_budget_shrinks_to_fit_memory():
    # 4M tokens from host memory over 31 parts: the default budget (4M rows) would stage too much for
    # 16 GB beside the 8.9 GB accumulator, so the planner halves it until the staging fits
    N = 4_194_304
    p = _plan(N, True, 31, where="host", budget=16 * GB)
    assert p["wave_tokens"] < 1 << 22 and p["workspace_bytes"] <= 0.85 * 16 * GB
    # one subproblem's staging (2.6 GB) fits once beside the accumulator but not twice, so the waves
    # are cut per query part of a subproblem: more copies (a key part once per unit), all double-buffered
    big = _plan(N, True, 31, where="host", budget=20 * GB)   # room for two subproblem-sized sets
    assert big["cqs_waves"] <= big["cqs_subproblems"] == 31
    assert p["cqs_waves"] > p["cqs_subproblems"] == 31
    assert p["h2d_bytes"] > big["h2d_bytes"]
    with pytest.raises(m().CqsaError):
        _plan(7000, True, 7, wave_tokens=-1)
    with pytest.raises(m().CqsaError):
        m().plan(((1, 8, 7000, 64), torch.float16), ((1, 8, 7000, 64), torch.float16),
                 ((1, 8, 7000, 64), torch.float16), True, 64 * GB, num_cus=256, wave_tokens=5000)


# ---------------------------------------------------------------- depth itr > 1

def _digits(p, c, itr):
    """Base-c digits of part p, most significant (the depth-1 part) first."""
    return [(p // c ** (itr - 1 - k)) % c for k in range(itr)]


def _holds(c, iset, itr, sub, part):
    """Subproblem `sub` holds `part` when every digit of the part is in the cyclic shift of the set by
    the subproblem's digit at the same level (the set applied again inside each part)."""
    return all(pd in parts_of(c, iset, sd) for pd, sd in zip(_digits(part, c, itr), _digits(sub, c, itr)))


@pytest.mark.parametrize("c,iset,itr", [(3, (0, 1), 2), (7, (0, 1, 3), 2), (3, (0, 1), 3), (4, (0, 1, 2), 2),
                                        (5, (0, 1, 2, 3, 4), 2)])
def test_depth_owner_is_the_first_subproblem_holding_both_parts(c, iset, itr):
    """Brute force over the definition: C = c^itr parts and subproblems; each subproblem holds l^itr
    parts; every pair of parts has a holder, and the owner is the smallest one, so each pair is
    computed exactly once."""
    C = c ** itr
    own = m().cqs_assign(c, iset, itr)
    assert len(own) == C
    held = {i: {p for p in range(C) if _holds(c, iset, itr, i, p)} for i in range(C)}
    assert all(len(h) == len(iset) ** itr for h in held.values())
    per_sub = [0] * C
    for a, b in itertools.product(range(C), repeat=2):
        holders = [i for i in range(C) if a in held[i] and b in held[i]]
        assert holders, (a, b)
        assert own[a][b] == holders[0]
        per_sub[own[a][b]] += 1
    assert sum(per_sub) == C * C and max(per_sub) <= len(iset) ** (2 * itr)


def test_depth_one_is_the_single_level_schedule():
    assert m().cqs_assign(7, (0, 1, 3), 1) == m().cqs_assign(7, (0, 1, 3))


def test_depth_plan_counts_and_errors():
    """c = 7 at depth 2: 49 parts; the plan's pairs are the visible pairs of the 49-part cut; the
    user's c is reported as such."""
    p = _plan(4900, False, 7, cqs_itr=2)
    assert p["n_q_chunks"] == 49 and p["cqs_c"] == 7 and p["chunk_pairs"] == 49 * 49
    assert p["cqs_subproblems"] == 49 and p["q_chunk"] == 100
    p = _plan(4900, True, 7, cqs_itr=2)
    assert p["chunk_pairs"] == 49 * 50 // 2                                  # key part <= query part
    p1 = _plan(4900, True, 7)
    assert p["workspace_bytes"] == p1["workspace_bytes"]                      # the same accumulator
    with pytest.raises(m().CqsaError, match="exceed 4096"):
        _plan(4900, True, 31, cqs_itr=3)
    with pytest.raises(m().CqsaError, match="cqs_itr applies"):
        m().plan(((1, 2, 64, 64), torch.float16), ((1, 2, 64, 64), torch.float16), ((1, 2, 64, 64), torch.float16),
                 True, GB, where={n: "device" for n in ("q", "k", "v", "out")}, num_cus=256, cqs_itr=2)
    with pytest.raises(m().CqsaError, match="negative"):
        _plan(4900, True, 7, cqs_itr=-1)
