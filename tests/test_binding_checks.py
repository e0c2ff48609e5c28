"""The Python binding's host-side checks (no GPU): the library sees only
pointers and strides, so tensors whose shapes, dtypes or list sizes do not
match the geometry are refused before any call into it.  CPU tensors serve:
every case below fails a check that runs before the device check."""
import pytest
import torch

vs = pytest.importorskip("block_sparse_cross_csla_amd")
from varsparse_inputs import SCHEDULE_13  # noqa: E402

SIDES, T, QS = SCHEDULE_13, 8, 10          # side 40: 25 query tiles, 72 key tiles, 1600 x 4121 tokens
NQB, NKB, NQ, NK = vs.geom_counts(SIDES, T, QS)


def _qkv(nq=NQ, nk=NK, d=128, dtype=torch.bfloat16, B=1, H=2):
    return (torch.zeros(B, H, nq, d, dtype=dtype), torch.zeros(B, H, nk, d, dtype=dtype),
            torch.zeros(B, H, nk, d, dtype=dtype))


def _lists(B=None, H=None, nqb=NQB, nkb=NKB, dtype=torch.int32):
    lead = () if B is None else (B, H)
    return torch.zeros(*lead, nqb, dtype=dtype), torch.zeros(*lead, nqb, nkb, dtype=dtype)


@pytest.mark.parametrize("fn", [vs.attn_fwd, vs.attn_fwd_pair])
def test_attention_shape_checks(fn):
    q, k, v = _qkv()
    cnt, idx = _lists()
    with pytest.raises(ValueError, match="k holds"):
        fn(q, k[:, :, :100], v, SIDES, T, QS, cnt, idx)
    with pytest.raises(ValueError, match="q holds"):
        fn(q[:, :, :64], k, v, SIDES, T, QS, cnt, idx)
    with pytest.raises(ValueError, match="does not match q"):
        fn(q, k[..., :64].contiguous(), v, SIDES, T, QS, cnt, idx)
    with pytest.raises(ValueError, match="shared lists"):
        fn(q, k, v, SIDES, T, QS, cnt[:5], idx)
    c2, i2 = _lists(B=1, H=3)
    with pytest.raises(ValueError, match="per-head lists"):
        fn(q, k, v, SIDES, T, QS, c2, i2)
    c3, i3 = _lists(dtype=torch.int64)
    with pytest.raises(ValueError, match="int32"):
        fn(q, k, v, SIDES, T, QS, c3, i3)
    with pytest.raises(ValueError, match="one dtype"):
        fn(q, k.float(), v, SIDES, T, QS, cnt, idx)
    with pytest.raises(ValueError, match="lse"):
        fn(q, k, v, SIDES, T, QS, cnt, idx, lse=torch.zeros(1, 2, NQ, dtype=torch.float64))
    with pytest.raises(ValueError, match="one GPU"):
        fn(q, k, v, SIDES, T, QS, cnt, idx)


def test_bf16_only_entry_points():
    q, k, v = _qkv(dtype=torch.float32)
    cnt, idx = _lists()
    with pytest.raises(ValueError, match="bfloat16"):
        vs.attn_fwd_pair(q, k, v, SIDES, T, QS, cnt, idx)
    with pytest.raises(ValueError, match="bfloat16"):
        vs.attn_fwd_token(q, k, v, SIDES, T, QS, 5, [2] * (QS + 1), cnt, idx)
    f = torch.zeros(1, 2, 32 * 32, 128)
    with pytest.raises(ValueError, match="bfloat16"):
        vs.ocache_correct(f, f, torch.zeros(1, 2, 40 * 40, 128), 32, 40)


def test_token_and_mask_argument_checks():
    q, k, v = _qkv()
    cnt, idx = _lists()
    with pytest.raises(ValueError, match="both lists"):
        vs.attn_fwd_token(q, k, v, SIDES, T, QS, 5, [2] * (QS + 1), cnt, None)
    with pytest.raises(ValueError, match="radius"):
        vs.attn_fwd_token(q, k, v, SIDES, T, QS, 5, [2] * 3)
    with pytest.raises(ValueError, match="wrong shape"):
        vs.build_mask(SIDES, T, QS, 5, radius=[2] * (QS + 1), out=(cnt[:3], idx, None))
    with pytest.raises(ValueError, match="radius"):
        vs.build_mask(SIDES, T, QS, 5, radius=[2])


def test_map_indices_checks():
    D, TT = 9, 10
    nqbD, nkbD, nqD, nkD = vs.geom_counts(SIDES, T, D)
    nqbT, nkbT, _, _ = vs.geom_counts(SIDES, T, TT)
    q_d = torch.zeros(1, 2, nqD, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, nkD, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="k holds fewer"):
        vs.map_indices(SIDES, T, D, TT, 5, 0.9, q_d=q_d, k=k[:, :, :10])
    with pytest.raises(ValueError, match="decision scale's tokens"):
        vs.map_indices(SIDES, T, D, TT, 5, 0.9, q_d=q_d[:, :, :5], k=k)
    with pytest.raises(ValueError, match="scores"):
        vs.map_indices(SIDES, T, D, TT, 5, 0.9, scores=torch.zeros(1, 2, nqbD, nkbD + 1))
    bad = (torch.zeros(1, 2, nqbT, dtype=torch.int32), torch.zeros(1, 2, nqbT, nkbT - 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="per-head lists"):
        vs.map_indices(SIDES, T, D, TT, 5, 0.9, scores=torch.zeros(1, 2, nqbD, nkbD), out=bad)


def test_missing_library_fails_loudly(tmp_path):
    """Without the built library the package refuses to import: there is no
    fallback path that could compute without the HIP kernels."""
    import os
    import shutil
    import subprocess
    import sys
    src = os.path.dirname(os.path.abspath(vs.__file__))
    shutil.copytree(src, tmp_path / "block_sparse_cross_csla_amd", ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    r = subprocess.run([sys.executable, "-c", "import block_sparse_cross_csla_amd"], cwd=tmp_path,
                       capture_output=True, text=True, env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libvarsparse.so is missing" in r.stderr


def test_product_sources_never_reach_the_oracle():
    """The package (binding and kernels) neither imports nor names the CPU
    oracle, which is test infrastructure only."""
    import os
    root = os.path.dirname(os.path.abspath(vs.__file__))
    for dirpath, _, files in os.walk(root):
        for name in files:
            if name.endswith((".py", ".hip", ".h", ".cpp")):
                with open(os.path.join(dirpath, name), encoding="utf-8") as fh:
                    assert "oracle" not in fh.read(), os.path.join(dirpath, name)
