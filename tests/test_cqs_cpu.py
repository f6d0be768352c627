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
    assert p["merges"] == 28
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
