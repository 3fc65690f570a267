"""Pins of the oracle's block-level ground truth of decoding attention (G1).

Source: "SeerAttention: Learning Intrinsic Sparse Attention in Your LLMs",
abstract v2 (a FlashAttention variant that extracts the block-level ground
truth of the attention map with little overhead; the gate is distilled toward
it).  Reading (R22): for one decode query the block-level ground truth of block
j is the softmax weight of dense attention summed over the block's tokens,
averaged over the query heads that share the KV head; the incomplete tail gets
its own last slot.  Pins: PyTorch's fp64 softmax summed per block (a library
routine), closed forms (equal keys: weights proportional to token counts),
the normalisation, and head-duplication invariance.
"""
import math

import numpy as np
import pytest
import torch

import oracle

from test_oracle_attention import bf16, rand_case, widen


def torch_mass(q, k, bs, scale):
    """Dense softmax per head with PyTorch, summed per block and the tail, mean over heads."""
    qd, kd = widen(q), widen(k)
    w = torch.softmax((qd @ kd.T) * scale, dim=-1)          # [G, L]
    L = kd.shape[0]
    nc = L // bs
    cols = [w[:, j * bs:(j + 1) * bs].sum(-1) for j in range(nc)] + [w[:, nc * bs:].sum(-1)]
    return torch.stack(cols, dim=-1).mean(0).numpy()


@pytest.mark.parametrize("G,d,L,bs", [(4, 64, 300, 64), (1, 128, 1024, 128), (8, 64, 1000, 64), (2, 32, 7, 64),
                                      (4, 128, 512, 128)])
def test_block_mass_equals_torch_softmax_block_sums(G, d, L, bs):
    q, k, v = rand_case(G, d, L, seed=7 * L + G)
    scale = 1.0 / math.sqrt(d)
    out, lse, mass = oracle.decode_block_mass(q, k, v, bs, scale)
    np.testing.assert_allclose(mass, torch_mass(q, k, bs, scale), rtol=0, atol=1e-12)
    assert mass.shape == (L // bs + 1,)
    if L % bs == 0:
        assert mass[-1] == 0.0
    # out and lse are those of plain dense attention
    qd, kd, vd = widen(q), widen(k), widen(v)
    logits = (qd @ kd.T) * scale
    np.testing.assert_allclose(out, (torch.softmax(logits, -1) @ vd).numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, -1).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,bs", [(1, 64), (64, 64), (300, 64), (1000, 128)])
def test_block_mass_normalised_and_nonnegative(L, bs):
    q, k, v = rand_case(4, 64, L, seed=L)
    _, _, mass = oracle.decode_block_mass(q, k, v, bs, 0.125)
    assert np.all(mass >= 0)
    assert abs(mass.sum() - 1.0) < 1e-12


@pytest.mark.parametrize("L,bs", [(300, 64), (1000, 128), (128, 64)])
def test_equal_keys_give_token_count_shares(L, bs):
    """All keys equal: every token gets weight 1/L, so block j holds bs/L and the tail (L mod bs)/L."""
    g = torch.Generator().manual_seed(L)
    q = bf16(torch.randn(2, 64, generator=g))
    krow = torch.randn(1, 64, generator=g)
    k = bf16(krow.expand(L, 64).contiguous())
    v = bf16(torch.randn(L, 64, generator=g))
    _, _, mass = oracle.decode_block_mass(q, k, v, bs, 0.125)
    nc = L // bs
    expect = np.array([bs / L] * nc + [(L - nc * bs) / L])
    np.testing.assert_allclose(mass, expect, rtol=0, atol=1e-12)


def test_duplicated_query_heads_leave_the_mean_unchanged():
    q, k, v = rand_case(1, 64, 500, seed=3)
    _, _, m1 = oracle.decode_block_mass(q, k, v, 64, 0.125)
    q3 = np.concatenate([q, q, q], axis=0)
    _, _, m3 = oracle.decode_block_mass(q3, k, v, 64, 0.125)
    np.testing.assert_allclose(m1, m3, rtol=0, atol=1e-14)


def test_group_mass_is_the_mean_of_the_heads():
    q, k, v = rand_case(3, 64, 700, seed=5)
    _, _, m = oracle.decode_block_mass(q, k, v, 64, 0.125)
    per = [oracle.decode_block_mass(q[h:h + 1], k, v, 64, 0.125)[2] for h in range(3)]
    np.testing.assert_allclose(m, np.mean(per, axis=0), rtol=0, atol=1e-14)


# ---- prefill (G2): per (query block, key block) mean attention mass under dense causal attention ----

def torch_prefill_mass(q, k, bs, scale):
    qd, kd = widen(q), widen(k)
    L = qd.shape[0]
    logits = (qd @ kd.T) * scale
    causal = torch.ones(L, L, dtype=torch.bool).tril()
    w = torch.softmax(logits.masked_fill(~causal, -math.inf), dim=-1)    # [L, L]
    nb = (L + bs - 1) // bs
    out = torch.zeros(nb, nb, dtype=torch.float64)
    for i in range(nb):
        rows = w[i * bs:(i + 1) * bs]
        for j in range(i + 1):
            out[i, j] = rows[:, j * bs:(j + 1) * bs].sum(-1).mean()
    return out.numpy()


@pytest.mark.parametrize("L,bs", [(256, 64), (300, 64), (64, 64), (5, 64), (1000, 128)])
def test_prefill_mass_equals_torch_causal_softmax(L, bs):
    q, k, _ = rand_case(1, 64, L, seed=L + 1)
    q = rand_case(L, 64, 1, seed=L + 2)[0]          # L query rows
    mass = oracle.prefill_block_mass(q, k, bs, 0.125)
    np.testing.assert_allclose(mass, torch_prefill_mass(q, k, bs, 0.125), rtol=0, atol=1e-12)
    np.testing.assert_allclose(mass.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.triu(mass, 1) == 0.0)


def test_prefill_mass_equal_keys_closed_form():
    """Equal keys: row t spreads 1/(t+1) over tokens 0..t."""
    L, bs = 200, 64
    g = torch.Generator().manual_seed(9)
    q = bf16(torch.randn(L, 32, generator=g))
    k = bf16(torch.randn(1, 32, generator=g).expand(L, 32).contiguous())
    mass = oracle.prefill_block_mass(q, k, bs, 0.2)
    nb = (L + bs - 1) // bs
    expect = np.zeros((nb, nb))
    for i in range(nb):
        ts = range(i * bs, min((i + 1) * bs, L))
        for j in range(i + 1):
            expect[i, j] = np.mean([max(0, min(t + 1, (j + 1) * bs) - j * bs) / (t + 1) for t in ts])
    np.testing.assert_allclose(mass, expect, rtol=0, atol=1e-12)


def test_prefill_mass_row_range_matches_full():
    q = rand_case(500, 64, 1, seed=3)[0]
    k = rand_case(1, 64, 500, seed=4)[1]
    full = oracle.prefill_block_mass(q, k, 64, 0.125)
    part = oracle.prefill_block_mass(q, k, 64, 0.125, 3, 6)
    np.testing.assert_allclose(part, full[3:6], rtol=0, atol=0)
