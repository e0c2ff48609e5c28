"""GPU parity: CS4A scoring, top-p selection, index mapping and attention at
the mapped scales.

Stage by stage: GPU scores against the oracle's (abs 1e-5); the GPU's
selection and target lists against the oracle's select/map fed with the GPU's
own scores (bit-exact: the integer decisions are taken on the same float32
values); end to end, selections from the oracle's own scores may differ only
in rows whose decision sits within float32 rounding of the threshold."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as OA, cs4a as OC, geometry as G
from tests._common import spatial, to_device
from varsparse_inputs import workloads as W

pytestmark = pytest.mark.gpu

SCORE_TOL = 1e-5


def _vs():
    import block_sparse_cross_csla_amd as vs
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return vs


@pytest.fixture(scope="module")
def cs4a_run():
    vs = _vs()
    w = W.CS4A
    B, H = 1, 4
    D = W.CS4A_DECISION
    q_d, k, v = spatial(w, B=B, H=H, q_side=w.sides[D])
    kd = to_device(k)
    out = {}
    scores, sc, si, kc, ki = vs.map_indices(w.sides, w.tile, D, W.CS4A_TARGETS[0], w.n_sink, W.CS4A_TOP_P,
                                           q_d=to_device(q_d), k=kd, want_selection=True)
    out[W.CS4A_TARGETS[0]] = (kc, ki)
    for T in W.CS4A_TARGETS[1:]:
        _, _, _, kc, ki = vs.map_indices(w.sides, w.tile, D, T, w.n_sink, W.CS4A_TOP_P, scores=scores)
        out[T] = (kc, ki)
    torch.cuda.synchronize()
    return dict(w=w, B=B, H=H, D=D, q_d=q_d, k=k, v=v, kd=kd, scores=scores.cpu().numpy(),
                sel=(sc.cpu().numpy(), si.cpu().numpy()),
                lists={T: (a.cpu().numpy(), b.cpu().numpy()) for T, (a, b) in out.items()})


def test_scores_match_oracle(cs4a_run):
    r = cs4a_run
    w = r["w"]
    ref = OC.block_scores(r["q_d"], r["k"], w.sides, r["D"], w.tile, 1 / math.sqrt(w.d))
    err = np.abs(r["scores"] - ref).max()
    assert err <= SCORE_TOL, err
    assert np.abs(r["scores"].astype(np.float64).sum(-1) - 1).max() < 1e-4


def test_selection_bit_exact_on_gpu_scores(cs4a_run):
    r = cs4a_run
    cnt, idx = OC.top_p_select(r["scores"], W.CS4A_TOP_P)
    assert (r["sel"][0] == cnt).all()
    assert (r["sel"][1] == idx).all()


@pytest.mark.parametrize("T", W.CS4A_TARGETS)
def test_mapping_bit_exact_on_gpu_selection(cs4a_run, T):
    r = cs4a_run
    w = r["w"]
    cnt, idx = OC.map_indices(r["sel"][0], r["sel"][1], w.sides, r["D"], T, w.tile, w.n_sink)
    assert (r["lists"][T][0] == cnt).all()
    assert (r["lists"][T][1] == idx).all()


def _top_p_margin(row: np.ndarray, p: float) -> float:
    """How far, in score units, one row's top-p decision is from changing: the
    gaps between p times the row's mass and the cumulative mass of the kept
    prefix with and without its last tile, and the gap between the last kept
    and the first dropped score (a swap there changes the set)."""
    s = np.sort(row)[::-1]
    cum = np.cumsum(s)
    thr = p * cum[-1]
    k = int(np.argmax(cum >= thr)) + 1          # tiles kept
    gaps = [cum[k - 1] - thr]
    if k >= 2:
        gaps.append(thr - cum[k - 2])
    if k < s.size:
        gaps.append(s[k - 1] - s[k])
    return float(min(gaps))


def test_selection_end_to_end(cs4a_run):
    """Against the oracle's own float64 scores: a row's selection may differ
    only where the oracle's decision lies within 1e-5 of a change (its
    top-p margin, in score units); such rows are counted and reported, and
    any GPU selection still reaches the mass threshold on the oracle's
    scores."""
    r = cs4a_run
    w = r["w"]
    ref = OC.block_scores(r["q_d"], r["k"], w.sides, r["D"], w.tile, 1 / math.sqrt(w.d))
    cnt, idx = OC.top_p_select(ref.astype(np.float32), W.CS4A_TOP_P)
    gc, gi = r["sel"]
    diff = np.flatnonzero((cnt != gc).reshape(-1) | (idx != gi).reshape(-1, idx.shape[-1]).any(axis=1))
    flat_ref = ref.reshape(-1, ref.shape[-1])
    margins = [_top_p_margin(flat_ref[row], W.CS4A_TOP_P) for row in diff]
    print(f"end-to-end selection: {diff.size} of {cnt.size} rows differ; their margins {margins}")
    assert all(m < 1e-5 for m in margins), margins
    assert diff.size <= max(1, cnt.size // 50), f"{diff.size} of {cnt.size} rows differ"
    for row in diff:
        kept = gi.reshape(-1, gi.shape[-1])[row, : gc.reshape(-1)[row]]
        mass = flat_ref[row, kept].sum()
        assert mass >= W.CS4A_TOP_P - 1e-4
        assert mass - flat_ref[row, kept].min() < W.CS4A_TOP_P + 1e-4


@pytest.mark.parametrize("T", W.CS4A_TARGETS)
def test_attention_at_mapped_scales(cs4a_run, T):
    vs = _vs()
    r = cs4a_run
    w = r["w"]
    f_q = spatial(w, B=r["B"], H=r["H"], q_side=w.sides[T])[0]
    nk = G.scale_offsets(w.sides)[T + 1]
    kc, ki = r["lists"][T]
    o, lse = vs.attn_fwd(to_device(f_q), r["kd"][:, :, :nk], to_device(r["v"][:, :, :nk].copy()), w.sides, w.tile,
                         T, torch.from_numpy(kc).cuda(), torch.from_numpy(ki).cuda())
    torch.cuda.synchronize()
    ro, rl = OA.block_sparse_attention(f_q, r["k"][:, :, :nk], r["v"][:, :, :nk], w.sides, T, w.tile, kc, ki,
                                       1 / math.sqrt(w.d))
    err = np.abs(o.float().cpu().numpy() - ro).max()
    assert err <= 2e-2, err
    assert np.abs(lse.cpu().numpy() - rl).max() <= 2e-2


def test_full_size_cs4a_lists():
    """The benchmarked CS4A launch (B=2, H=16): GPU lists equal the oracle's
    select/map of the GPU scores, for every target; scores within tolerance on
    sampled heads."""
    vs = _vs()
    w = W.CS4A
    D = W.CS4A_DECISION
    q_d, k, _ = spatial(w, q_side=w.sides[D])
    scores, sc, si, _, _ = vs.map_indices(w.sides, w.tile, D, W.CS4A_TARGETS[-1], w.n_sink, W.CS4A_TOP_P,
                                         q_d=to_device(q_d), k=to_device(k), want_selection=True)
    lists = {}
    for T in W.CS4A_TARGETS:
        lists[T] = vs.map_indices(w.sides, w.tile, D, T, w.n_sink, W.CS4A_TOP_P, scores=scores)[3:]
    torch.cuda.synchronize()
    s = scores.cpu().numpy()
    cnt, idx = OC.top_p_select(s, W.CS4A_TOP_P)
    assert (sc.cpu().numpy() == cnt).all() and (si.cpu().numpy() == idx).all()
    for T in W.CS4A_TARGETS:
        mc, mi = OC.map_indices(cnt, idx, w.sides, D, T, w.tile, w.n_sink)
        assert (lists[T][0].cpu().numpy() == mc).all()
        assert (lists[T][1].cpu().numpy() == mi).all()
    ref = OC.block_scores(q_d[1:, 14:], k[1:, 14:], w.sides, D, w.tile, 1 / math.sqrt(w.d))
    assert np.abs(s[1:, 14:] - ref).max() <= SCORE_TOL


@pytest.mark.parametrize("frac", [0.2, 0.05, 1.0])
def test_top_k_selection_and_mapping_bit_exact(cs4a_run, frac):
    """The Top-K-fraction rule on the GPU's own scores: selection and every
    target's lists equal the oracle's (integer decisions on the same float32
    values), including the degenerate fractions (one tile, every tile)."""
    vs = _vs()
    r = cs4a_run
    w = r["w"]
    scores = torch.from_numpy(r["scores"]).cuda()
    gpu = {}
    for T in W.CS4A_TARGETS:
        _, sc, si, kc, ki = vs.map_indices(w.sides, w.tile, r["D"], T, w.n_sink, 0.9, scores=scores,
                                           want_selection=True, top_k=frac)
        gpu[T] = (sc.cpu().numpy(), si.cpu().numpy(), kc.cpu().numpy(), ki.cpu().numpy())
    torch.cuda.synchronize()
    cnt, idx = OC.top_k_select(r["scores"], frac)
    assert (cnt == OC.top_k_count(r["scores"].shape[-1], frac)).all()
    for T in W.CS4A_TARGETS:
        sc, si, kc, ki = gpu[T]
        assert (sc == cnt).all() and (si == idx).all()
        mc, mi = OC.map_indices(cnt, idx, w.sides, r["D"], T, w.tile, w.n_sink)
        assert (kc == mc).all() and (ki == mi).all()


def test_large_decision_scale():
    """Decision scale side 64 of the 16-scale schedule (172 key tiles: the
    score kernel's largest per-tile accumulator in these workloads), mapped to
    side 128: scores within tolerance, selection and map bit-exact on the
    GPU's own scores."""
    vs = _vs()
    w = W.HIGH_RES
    D, T = 12, 15
    q_d, k, _ = spatial(w, B=1, H=2, q_side=w.sides[D])
    scores, sc, si, kc, ki = vs.map_indices(w.sides, w.tile, D, T, w.n_sink, W.CS4A_TOP_P,
                                           q_d=to_device(q_d), k=to_device(k), want_selection=True)
    torch.cuda.synchronize()
    s = scores.cpu().numpy()
    assert s.shape[-1] == 172
    ref = OC.block_scores(q_d, k, w.sides, D, w.tile, 1 / math.sqrt(w.d))
    assert np.abs(s - ref).max() <= SCORE_TOL
    cnt, idx = OC.top_p_select(s, W.CS4A_TOP_P)
    assert (sc.cpu().numpy() == cnt).all() and (si.cpu().numpy() == idx).all()
    mc, mi = OC.map_indices(cnt, idx, w.sides, D, T, w.tile, w.n_sink)
    assert (kc.cpu().numpy() == mc).all() and (ki.cpu().numpy() == mi).all()


@pytest.mark.parametrize("rule,param", [("top_p", W.CS4A_TOP_P), ("top_k", 0.2)])
def test_multi_target_map_bit_exact(cs4a_run, rule, param):
    """One launch mapping onto the decision scale itself and the three targets
    writes exactly the lists of one launch per target, and those equal the
    oracle's select/map of the GPU's own scores."""
    vs = _vs()
    r = cs4a_run
    w = r["w"]
    D = r["D"]
    targets = [D, *W.CS4A_TARGETS]
    scores = torch.from_numpy(r["scores"]).cuda()
    _, multi = vs.map_indices_multi(w.sides, w.tile, D, targets, w.n_sink, param, rule=rule, scores=scores)
    torch.cuda.synchronize()
    s = r["scores"]
    cnt, idx = OC.top_p_select(s, param) if rule == "top_p" else OC.top_k_select(s, param)
    for T, (kc, ki) in zip(targets, multi):
        kw = {"top_k": param} if rule == "top_k" else {}
        one = vs.map_indices(w.sides, w.tile, D, T, w.n_sink, W.CS4A_TOP_P, scores=scores, **kw)[3:]
        torch.cuda.synchronize()
        assert torch.equal(kc, one[0]) and torch.equal(ki, one[1]), T
        mc, mi = OC.map_indices(cnt, idx, w.sides, D, T, w.tile, w.n_sink)
        assert (kc.cpu().numpy() == mc).all() and (ki.cpu().numpy() == mi).all(), T


def test_multi_target_map_computes_scores():
    """With q_d and k the multi-target launch computes the scores first, as
    the single-target entry point does (identical scores and lists)."""
    vs = _vs()
    w = W.CS4A
    D = W.CS4A_DECISION
    q_d, k, _ = spatial(w, B=2, H=4, q_side=w.sides[D])
    qd, kd = to_device(q_d), to_device(k)
    s1, multi = vs.map_indices_multi(w.sides, w.tile, D, list(W.CS4A_TARGETS), w.n_sink, W.CS4A_TOP_P, q_d=qd, k=kd)
    s2, _, _, kc, ki = vs.map_indices(w.sides, w.tile, D, W.CS4A_TARGETS[-1], w.n_sink, W.CS4A_TOP_P, q_d=qd, k=kd)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert torch.equal(multi[-1][0], kc) and torch.equal(multi[-1][1], ki)


@pytest.mark.parametrize("d", [128, 64])
def test_scores_odd_tile_count_fallback_and_head_dims(d):
    """Decision scale side 40 (25 query tiles: the scoring workgroups take
    query tiles two at a time, so the last one holds a single tile) and side
    64 of the 16-scale schedule (172 key tiles: too many for the two-tile
    workgroup's accumulator in LDS, so one tile per workgroup), head dims 128
    and 64: scores within tolerance of the oracle, rows summing to 1."""
    vs = _vs()
    for w, D, T, H in ((W.CS4A, 10, 11, 3), (W.HIGH_RES, 12, 15, 1)):
        print(f"scores: side {w.sides[D]} d={d}", flush=True)
        q_d, k, _ = spatial(w, B=1, H=H, q_side=w.sides[D])
        if d != w.d:
            q_d, k = q_d[..., :d].copy(), k[..., :d].copy()
        scores, _, _, _, _ = vs.map_indices(w.sides, w.tile, D, T, w.n_sink, W.CS4A_TOP_P, q_d=to_device(q_d),
                                            k=to_device(k))
        torch.cuda.synchronize()
        s = scores.cpu().numpy()
        ref = OC.block_scores(q_d, k, w.sides, D, w.tile, 1 / math.sqrt(d))
        assert np.abs(s - ref).max() <= SCORE_TOL, (w.sides[D], d)
        assert np.abs(s.astype(np.float64).sum(-1) - 1).max() < 1e-4
