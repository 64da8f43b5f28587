"""The tuner end to end on the tiny bf16 layer: every bucket gets a config
that the library accepts, timed and gated against the built-in choice; an
expert-parallel shard only considers configs that split K like the
unsharded call."""
import pytest

import mixture_experts_ffn_align_amd as moe
from mixture_experts_ffn_align_amd import tune

pytestmark = pytest.mark.gpu


def test_tune_tiny_bf16(tmp_path):
    rows = tune.tune("tiny_bf16", [1, 16, 64], log=print)
    assert [r["bucket"] for r in rows] == [1, 16, 64]
    for r in rows:
        assert 0 <= r["config"] < 64 and r["us"] > 0 and r["candidates"] >= 2
        assert float(r["rel_l2"]) <= 1e-2 and float(r["err_ratio"]) <= 0.05
    path = tmp_path / "tiny.csv"
    tune.write_csv(rows, str(path))
    assert len(tune.read_csv(str(path))) == 3


def test_tune_tiny_bf16_shard():
    rows = tune.tune("tiny_bf16", [64], ep=2, log=print)
    assert rows[0]["E_local"] == 4 and rows[0]["us"] > 0
