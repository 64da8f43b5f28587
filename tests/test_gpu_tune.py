"""The tuner end to end on the tiny bf16 layer, gated on the CPU oracle:
every bucket gets a config that the library accepts, that matches the
oracle's rows within the bf16 bars and that is timed; a reference with a
planted mistake (the oracle's rows scaled by 1.05) rejects every config; an
expert-parallel shard only considers configs that split K like the unsharded
call, gated on the oracle with the other shards' slots dropped."""
import pytest

from mixture_experts_ffn_align_amd import tune
from tune_gated import oracle_reference

pytestmark = pytest.mark.gpu


def test_tune_tiny_bf16_oracle_gated(tmp_path):
    rows = tune.tune("tiny_bf16", [1, 16, 64], oracle_reference("tiny_bf16"), log=print)
    assert [r["bucket"] for r in rows] == [1, 16, 64]
    for r in rows:
        assert 0 <= r["config"] < 64 and r["us"] > 0 and r["candidates"] >= 2
        assert float(r["rel_l2"]) <= 1e-2 and float(r["err_ratio"]) <= 0.05
        assert r["ref_tokens"] >= 1 and r["rejected"] == ""
    path = tmp_path / "tiny.csv"
    tune.write_csv(rows, str(path))
    assert len(tune.read_csv(str(path))) == 3


def test_tune_rejects_everything_against_a_wrong_reference():
    with pytest.raises(RuntimeError, match="no config passed"):
        tune.tune("tiny_bf16", [64], oracle_reference("tiny_bf16", scale=1.05), log=print)


def test_tune_tiny_bf16_shard():
    rows = tune.tune("tiny_bf16", [64], oracle_reference("tiny_bf16"), ep=2, log=print)
    assert rows[0]["E_local"] == 4 and rows[0]["us"] > 0
    assert float(rows[0]["rel_l2"]) <= 1e-2
