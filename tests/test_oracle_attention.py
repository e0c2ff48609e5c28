"""Pins for oracle.attention: a library routine (torch SDPA on the CPU), a
second route over gathered keys, closed forms and invariants."""
import numpy as np
import pytest
import torch

from oracle import attention as A, csla, geometry as G
from varsparse_inputs import TINY_SIDES, gaussian_qkv


def _sdpa(q, k, v, scale, mask=None):
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.ascontiguousarray(q, np.float64))[None],
        torch.from_numpy(np.ascontiguousarray(k, np.float64))[None],
        torch.from_numpy(np.ascontiguousarray(v, np.float64))[None],
        attn_mask=None if mask is None else torch.from_numpy(mask)[None], scale=scale)
    return out[0].numpy()


def test_all_ones_mask_is_dense_sdpa():
    rng = np.random.default_rng(1)
    q, k, v = rng.standard_normal((3, 37, 16)), rng.standard_normal((3, 53, 16)), rng.standard_normal((3, 53, 16))
    for i in range(3):
        o, lse = A.softmax_attention(q[i], k[i], v[i], np.ones((37, 53), bool), 0.3)
        assert np.abs(o - _sdpa(q[i], k[i], v[i], 0.3)).max() < 1e-12
        s = q[i] @ k[i].T * 0.3
        # logsumexp via the library's log-sum-exp on the raw logits
        assert np.abs(lse - torch.logsumexp(torch.from_numpy(s), dim=1).numpy()).max() < 1e-12


def test_dense_attention_matches_sdpa_batched():
    q, k, v = gaussian_qkv(5, 99, 2, 3, 40, 70, 8)
    o, _ = A.dense_attention(q, k, v, 0.125)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x.astype(np.float64)) for x in (q, k, v)), scale=0.125).numpy()
    assert np.abs(o - ref).max() < 1e-12


def test_rows_sum_to_one():
    """With V = identity rows the output is the attention matrix itself."""
    rng = np.random.default_rng(2)
    nk = 24
    q, k = rng.standard_normal((10, 8)), rng.standard_normal((nk, 8))
    keep = rng.random((10, nk)) < 0.5
    keep[:, 0] = True
    p, _ = A.softmax_attention(q, k, np.eye(nk), keep, 1.0)
    assert np.abs(p.sum(axis=1) - 1).max() < 1e-12
    assert (p[~keep] == 0).all()


def test_masked_equals_gathered_keys():
    """Second route: attention over only the kept keys (library SDPA) equals
    the -inf-masked dense attention."""
    sides, qs, t = TINY_SIDES, 4, 4
    q, k, v = gaussian_qkv(0, 7, 1, 1, 256, 341, 64)
    mask = csla.block_mask(sides, qs, t, 3, [1] * 5)
    cnt, idx = csla.lists_from_mask(mask)
    o, lse = A.block_sparse_attention(q, k, v, sides, qs, t, cnt, idx, 0.125)
    for i, qt in enumerate(G.query_tiles(sides, qs, t)):
        keys = np.concatenate([G.key_tiles(sides, qs, t)[j].tokens() for j in idx[i, : cnt[i]]])
        qtok = qt.tokens()
        ref = _sdpa(q[0, 0, qtok], k[0, 0, keys], v[0, 0, keys], 0.125)
        assert np.abs(o[0, 0, qtok] - ref).max() < 1e-12


def test_identical_keys_closed_form():
    """All kept keys equal: uniform weights, O = mean of the kept values,
    lse = q.k * scale + log(number kept)."""
    rng = np.random.default_rng(3)
    kvec = rng.standard_normal(8)
    k = np.tile(kvec, (30, 1))
    v = rng.standard_normal((30, 8))
    q = rng.standard_normal((4, 8))
    keep = np.zeros((4, 30), bool)
    keep[0, :5] = keep[1, 10:30] = keep[2, ::3] = keep[3, 7] = True
    o, lse = A.softmax_attention(q, k, v, keep, 0.5)
    for r in range(4):
        assert np.abs(o[r] - v[keep[r]].mean(axis=0)).max() < 1e-12
        assert abs(lse[r] - (q[r] @ kvec * 0.5 + np.log(keep[r].sum()))) < 1e-12


def test_empty_row():
    q, k, v = np.ones((2, 4)), np.ones((3, 4)), np.ones((3, 4))
    keep = np.array([[False] * 3, [True, False, False]])
    o, lse = A.softmax_attention(q, k, v, keep, 1.0)
    assert (o[0] == 0).all() and lse[0] == -np.inf
    assert np.allclose(o[1], 1.0) and np.isclose(lse[1], 4.0)


def test_scale_matters():
    """A dropped softmax scale would be caught: the scaled result differs from
    the unscaled one and matches the library only when the scale is applied."""
    rng = np.random.default_rng(4)
    q, k, v = rng.standard_normal((5, 8)), rng.standard_normal((9, 8)), rng.standard_normal((9, 8))
    o1, _ = A.softmax_attention(q, k, v, np.ones((5, 9), bool), 0.1)
    o2, _ = A.softmax_attention(q, k, v, np.ones((5, 9), bool), 1.0)
    assert np.abs(o1 - o2).max() > 1e-3
    assert np.abs(o1 - _sdpa(q, k, v, 0.1)).max() < 1e-12


# ---- token-level CSLA mask


def _tiny_inputs(seed=5):
    from varsparse_inputs import TINY_SIDES
    rng = np.random.default_rng(seed)
    sides = list(TINY_SIDES)
    nk = sum(s * s for s in sides)
    q = rng.normal(size=(1, 1, sides[-1] ** 2, 16))
    k = rng.normal(size=(1, 1, nk, 16))
    v = rng.normal(size=(1, 1, nk, 16))
    return sides, q, k, v


def test_token_masked_wide_window_is_dense():
    from oracle import attention as OA
    sides, q, k, v = _tiny_inputs()
    qs = len(sides) - 1
    o, l = OA.token_masked_attention(q, k, v, sides, qs, 4, 0, [max(sides)] * len(sides), 0.25)
    ro, rl = OA.dense_attention(q, k, v, 0.25)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(l, rl, atol=1e-12)


def test_token_masked_sinks_only_is_attention_over_the_sink_tokens():
    from oracle import attention as OA
    sides, q, k, v = _tiny_inputs(6)
    qs, n_sink = len(sides) - 1, 2
    o, l = OA.token_masked_attention(q, k, v, sides, qs, 4, n_sink, [-1] * len(sides), 0.25)
    ns = sum(s * s for s in sides[:n_sink])
    ro, rl = OA.dense_attention(q, k[:, :, :ns], v[:, :, :ns], 0.25)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(l, rl, atol=1e-12)


def test_token_masked_matches_per_query_gather():
    """Second route: per query, gather the kept keys by the window rule
    written out with explicit loops and run textbook attention on them."""
    from oracle import attention as OA
    sides, q, k, v = _tiny_inputs(7)
    qs, n_sink, radius = len(sides) - 1, 2, [1, 1, 1, 0, 1]
    o, l = OA.token_masked_attention(q, k, v, sides, qs, 4, n_sink, radius, 0.3)
    H = sides[qs]
    offs = np.cumsum([0] + [s * s for s in sides])
    for y in range(H):
        for x in range(H):
            keys = []
            for s, h in enumerate(sides[: qs + 1]):
                py, px = (y * h) // H, (x * h) // H
                for yy in range(h):
                    for xx in range(h):
                        if s < n_sink or (radius[s] >= 0 and abs(yy - py) <= radius[s] and abs(xx - px) <= radius[s]):
                            keys.append(offs[s] + yy * h + xx)
            qi = q[0, 0, y * H + x]
            sc = np.array([qi @ k[0, 0, j] for j in keys]) * 0.3
            p = np.exp(sc - sc.max())
            ref = (p[:, None] * v[0, 0, keys]).sum(0) / p.sum()
            np.testing.assert_allclose(o[0, 0, y * H + x], ref, atol=1e-12)
            np.testing.assert_allclose(l[0, 0, y * H + x], sc.max() + np.log(p.sum()), atol=1e-12)
