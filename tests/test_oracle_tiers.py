"""Pins of the oracle's tier assignment (CPU only).

Tiers: "Toutes les pensees n'ont pas besoin de HBM" (gist.science, paper 2605.09490),
Methodologie section 1 (four tiers, protected tokens in T0, T3 = permanent tail) and
section 4 (reassignment every Delta steps).  The oracle sorts; the checks here do not:
a hand-worked example, closed-form budgets, and a pairwise characterisation that fixes
the result uniquely (sizes + "every kept candidate outranks every demoted one").
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import Policy, assign_tiers, budgets, keep_order, protected_mask
from tests import golden_io


def test_worked_example():
    g = golden_io.load("tier_worked_example.txt")
    pol = Policy(g["prompt"], g["sinks"], g["recent"], g["frac_t1"], g["frac_t2"], g["frac_t3"], 64)
    s = np.array(g["scores"], dtype=np.float64)
    n = g["n"]
    assert budgets(n, pol) == (8, 4, 3, 1)
    assert keep_order(s, [i for i in range(n) if not protected_mask(n, pol)[i]]) == g["keep_order"]
    tiers, counts = assign_tiers(s, np.zeros(n, np.uint8), n, pol)
    assert tiers.tolist() == g["tiers"]
    assert counts.tolist() == g["counts"]


def test_budget_closed_forms():
    pol = Policy(256, 4, 128, 0.30, 0.15, 0.05, 64)
    assert budgets(8192, pol) == (4098, 2457, 1228, 409)
    # the float32 fraction is what is multiplied: fl32(0.7) * 10 = 6.99999988 -> 6
    assert budgets(10, Policy(0, 0, 0, 0.7, 0.0, 0.0, 1)) == (4, 6, 0, 0)
    assert budgets(0, pol) == (0, 0, 0, 0)


def test_protected_set():
    pol = Policy(prompt=3, sinks=5, recent=2, frac_t1=0, frac_t2=0, frac_t3=0, delta=1)
    assert np.nonzero(protected_mask(10, pol))[0].tolist() == [0, 1, 2, 3, 4, 8, 9]
    assert protected_mask(4, pol).all()


def better(s, i, j):
    """i ranks above j in the keep order (score desc, then position asc)."""
    return s[i] > s[j] or (s[i] == s[j] and i < j)


def check_characterisation(s, prev, n, pol, new, counts):
    prot = protected_mask(n, pol)
    _, n1, n2, n3 = budgets(n, pol)
    E = [i for i in range(n) if prev[i] == 3]
    pool = [i for i in range(n) if not prot[i] and prev[i] <= 2]
    evicted = [i for i in pool if new[i] == 3]
    e = min(max(n3 - len(E), 0), len(pool))
    assert len(evicted) == e
    assert all(new[i] == 3 for i in E)                      # T3 is absorbing
    for x in evicted:                                       # evicted are the pool's bottom
        for y in pool:
            if new[y] != 3:
                assert better(s, y, x)
    survivors = [i for i in range(n) if prev[i] == 2 and new[i] != 3]
    assert all(new[i] == 2 for i in survivors)              # T2 only moves to T3
    live = [i for i in range(n) if not prot[i] and prev[i] <= 1 and new[i] != 3]
    to_t2 = [i for i in live if new[i] == 2]
    assert len(to_t2) == min(max(n2 - len(survivors), 0), len(live))
    rest = [i for i in live if new[i] != 2]
    for x in to_t2:
        for y in rest:
            assert better(s, y, x)
    t1 = [i for i in rest if new[i] == 1]
    t0 = [i for i in rest if new[i] == 0]
    assert len(t1) == min(n1, len(rest))
    assert len(t0) + len(t1) == len(rest)
    for x in t1:
        for y in t0:
            assert better(s, y, x)
    for i in range(n):
        if prot[i] and prev[i] <= 1:
            assert new[i] == 0
    assert counts.tolist() == [int((new == t).sum()) for t in range(4)]


@settings(max_examples=300, deadline=None)
@given(n=st.integers(0, 90), distinct=st.integers(1, 6), seed=st.integers(0, 2 ** 31),
       prompt=st.integers(0, 8), sinks=st.integers(0, 8), recent=st.integers(0, 10),
       f=st.tuples(*[st.sampled_from([0.0, 0.05, 0.1, 0.2, 0.3, 0.45, 0.6])] * 3),
       history=st.booleans())
def test_characterisation_random(n, distinct, seed, prompt, sinks, recent, f, history):
    if sum(f) > 1.0:
        f = (f[0] / 2, f[1] / 2, f[2] / 2)
    pol = Policy(prompt, sinks, recent, f[0], f[1], f[2], 8)
    r = np.random.default_rng(seed)
    s = r.integers(0, distinct, size=n).astype(np.float64) / distinct   # many ties
    prev = np.zeros(n, np.uint8)
    if history and n:
        # a reachable earlier state: the assignment at an earlier length with other scores
        n_old = int(r.integers(0, n + 1))
        s_old = r.random(n_old)
        prev[:n_old], _ = assign_tiers(s_old, np.zeros(n_old, np.uint8), n_old, pol)
    new, counts = assign_tiers(s, prev, n, pol)
    check_characterisation(s, prev, n, pol, new, counts)


def test_first_assignment_is_a_stable_sort_bottom_fill():
    r = np.random.default_rng(5)
    n = 500
    pol = Policy(20, 4, 30, 0.3, 0.15, 0.05, 64)
    s = np.round(r.random(n), 2)
    new, _ = assign_tiers(s, np.zeros(n, np.uint8), n, pol)
    prot = protected_mask(n, pol)
    cand = np.nonzero(~prot)[0]
    # numpy's stable argsort on -s keeps equal scores in position order
    ordered = cand[np.argsort(-s[cand], kind="stable")]
    _, n1, n2, n3 = budgets(n, pol)
    bottom = ordered[::-1]
    assert (new[bottom[:n3]] == 3).all()
    assert (new[bottom[n3:n3 + n2]] == 2).all()
    assert (new[bottom[n3 + n2:n3 + n2 + n1]] == 1).all()
    assert (new[bottom[n3 + n2 + n1:]] == 0).all()
    assert (new[prot] == 0).all()
