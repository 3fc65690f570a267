"""Pins of the oracle's gate (D1-D3) and token-budget selection (D4).

Sources: "SeerAttention: Learning Intrinsic Sparse Attention in Your LLMs",
abstract v1 (pool K along the sequence, learnable linear layers, multiply the
results into gating scores); "SeerAttention-R: Sparse Attention Adaptation for
Long Reasoning", abstract (no query pooling in decode; a token budget at
64/128-token block granularity).  The pages print no gate values, so the pins
are closed forms, algebraic invariants and brute-force enumeration.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16(x) -> np.ndarray:
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def widen(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


# ------------------------------------------------------------------ D1 pooling
def test_pool_constant_block_is_that_row():
    g = torch.Generator().manual_seed(0)
    L, bs, d = 256, 64, 32
    rows = torch.randn(L // bs, d, generator=g)
    k = bf16(rows.repeat_interleave(bs, dim=0))
    np.testing.assert_array_equal(oracle.pool_k(k, bs), widen(bf16(rows)))


def test_pool_ramp_closed_form():
    """K_t = t * e_c  ->  kp_j = (j*bs + (bs-1)/2) e_c  (integers <= 255 are exact in bf16)."""
    L, bs, d, c = 256, 64, 16, 5
    k = torch.zeros(L, d)
    k[:, c] = torch.arange(L, dtype=torch.float32)
    kp = oracle.pool_k(bf16(k), bs)
    expect = np.zeros((L // bs, d))
    expect[:, c] = np.arange(L // bs) * bs + (bs - 1) / 2
    np.testing.assert_array_equal(kp, expect)


def test_pool_ignores_tail_and_token_order():
    g = torch.Generator().manual_seed(1)
    L, bs, d = 64 * 3 + 17, 64, 64
    k = torch.randn(L, d, generator=g)
    kp = oracle.pool_k(bf16(k), bs)
    assert kp.shape == (3, d)                       # only complete blocks are pooled
    perm = torch.cat([torch.randperm(bs, generator=g) + j * bs for j in range(3)] + [torch.arange(192, L)])
    np.testing.assert_allclose(oracle.pool_k(bf16(k[perm]), bs), kp, rtol=0, atol=1e-15)


# --------------------------------------------------------------- D2/D3 gate
def test_gate_single_entry_projections_closed_form():
    """Wq = e_r e_c^T, Wk = e_r e_c'^T (dg != d) -> s_hj = q_h[c] * kp_j[c'] * scale.

    A transposed projection, a swapped operand or a wrong gate width fails this."""
    g = torch.Generator().manual_seed(2)
    G, d, dg, nc = 4, 64, 24, 9
    r, c, c2 = 17, 3, 41
    wq = torch.zeros(dg, d); wq[r, c] = 1.0
    wk = torch.zeros(dg, d); wk[r, c2] = 1.0
    q = bf16(torch.randn(G, d, generator=g))
    kp = torch.randn(nc, d, generator=g, dtype=torch.float64).numpy()
    s_head, S = oracle.gate_scores(q, bf16(wq), bf16(wk), kp, 0.5)
    expect = widen(q)[:, c][:, None] * kp[None, :, c2] * 0.5
    np.testing.assert_allclose(s_head, expect, rtol=1e-15, atol=0)
    np.testing.assert_allclose(S, expect.mean(axis=0), rtol=1e-14, atol=0)


def test_gate_identity_projections_score_group_mean_query():
    g = torch.Generator().manual_seed(3)
    G, d, nc = 8, 64, 12
    eye = bf16(torch.eye(d))
    q = bf16(torch.randn(G, d, generator=g))
    kp = torch.randn(nc, d, generator=g, dtype=torch.float64).numpy()
    _, S = oracle.gate_scores(q, eye, eye, kp, 1 / 8)
    np.testing.assert_allclose(S, kp @ widen(q).mean(axis=0) / 8, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("G,d,dg", [(4, 64, 64), (8, 128, 128), (2, 64, 32)])
def test_gate_matches_reassociated_form(G, d, dg):
    """Invariant: mean_h (Wq q_h).(Wk kp_j) == (Wk^T Wq qbar) . kp_j (the form the GPU evaluates)."""
    g = torch.Generator().manual_seed(G * d + dg)
    q = bf16(torch.randn(G, d, generator=g))
    wq = bf16(torch.randn(dg, d, generator=g) / math.sqrt(d))
    wk = bf16(torch.randn(dg, d, generator=g) / math.sqrt(d))
    kp = torch.randn(33, d, generator=g, dtype=torch.float64).numpy()
    s_head, S = oracle.gate_scores(q, wq, wk, kp, 1 / math.sqrt(dg))
    u = widen(wk).T @ (widen(wq) @ widen(q).mean(axis=0))
    np.testing.assert_allclose(S, (kp @ u) / math.sqrt(dg), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(s_head.mean(axis=0), S, rtol=1e-14, atol=1e-15)


# ------------------------------------------------------------------ D4 selection
def _dominant_subsets(scores, k):
    """All k-subsets S with: for i in S, j not in S -> s_i > s_j or (s_i == s_j and i < j)."""
    n = len(scores)
    found = []
    for sub in itertools.combinations(range(n), k):
        inside = set(sub)
        ok = all(scores[i] > scores[j] or (scores[i] == scores[j] and i < j)
                 for i in inside for j in range(n) if j not in inside)
        if ok:
            found.append(sub)
    return found


@pytest.mark.parametrize("seed", range(12))
def test_selection_brute_force(seed):
    """Pin (brute force): exactly one k-subset dominates the rest; it is the oracle's, and
    it has the largest score sum of all k-subsets."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 13))
    k = int(rng.integers(0, 5))
    if seed % 3 == 0:      # integer scores force exact ties
        scores = rng.integers(-2, 3, size=n).astype(np.float64)
    else:
        scores = rng.standard_normal(n)
    sel = oracle.select_blocks(scores, k)
    m = min(k, n)
    assert len(sel) == m                                   # pin: the count is min(k, nc)
    dom = _dominant_subsets(scores, m)
    assert len(dom) == 1 and tuple(sel.tolist()) == dom[0]
    best = max(sum(scores[list(s)]) for s in itertools.combinations(range(n), m)) if m else 0.0
    assert math.isclose(float(scores[sel].sum()) if m else 0.0, best, rel_tol=0, abs_tol=1e-12)


def test_selection_ties_go_to_lower_index_and_output_ascends():
    scores = np.zeros(16)
    np.testing.assert_array_equal(oracle.select_blocks(scores, 4), [0, 1, 2, 3])
    scores = np.array([1.0, 3.0, 3.0, 0.5, 3.0, 2.0])
    np.testing.assert_array_equal(oracle.select_blocks(scores, 2), [1, 2])
    np.testing.assert_array_equal(oracle.select_blocks(scores, 4), [1, 2, 4, 5])
    # ids come out ascending, not in score order (9 then 5)
    np.testing.assert_array_equal(oracle.select_blocks(np.array([5.0, 1.0, 4.0, 9.0]), 2), [0, 3])


def test_selection_counts_golden():
    """Pin: selected counts at the budgets and block sizes of the decode workloads (tests/golden)."""
    rows = [list(map(int, ln.split())) for ln in open(os.path.join(GOLDEN, "selection_counts.txt"))
            if ln.strip() and not ln.startswith("#")]
    rng = np.random.default_rng(0)
    for budget, bs, L, expect_k in rows:
        nc = L // bs
        sel = oracle.select_blocks(rng.standard_normal(nc), budget // bs)
        assert len(sel) == expect_k, (budget, bs, L)
        assert np.all(np.diff(sel) > 0)
