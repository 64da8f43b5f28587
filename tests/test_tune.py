"""The tuned-config table on the CPU: the CSV -> table writer, and every row
of the table compiled into the library is picked for its exact layer and
bucket and passes the library's own argument checks there (host-only calls
on descriptors of the row's sizes; nothing is launched)."""
import os
import re

import torch

import mixture_experts_ffn_align_amd as moe
from mixture_experts_ffn_align_amd import tune

ROW = re.compile(r"^\{(-?\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (-?\d+), ([0-9.]+)f\},")


def _rows():
    return [tuple(int(v) for v in m.groups()[:8])
            for m in (ROW.match(line) for line in open(tune.INC)) if m]


def _view(shape, dtype, row_stride=16):
    """A descriptor-only tensor of any size: positive, 16-byte aligned strides
    over a small buffer (the library's host checks never read it)."""
    n = len(shape)
    strides = [row_stride] * (n - 1) + [1]
    numel = 1 + sum((s - 1) * st for s, st in zip(shape, strides))
    return torch.empty(numel + 64, dtype=dtype).as_strided(shape, strides)


def _query(mode, H, I, E, E_local, k, T):
    fp4 = mode == moe.MODE_MXFP4
    wdt = torch.uint8 if fp4 else torch.bfloat16
    Hw, Iw = (H // 2, I // 2) if fp4 else (H, I)
    kw = dict(mode=mode)
    if fp4:
        kw.update(gate_scale=_view((E_local, I, H // 32), torch.uint8),
                  up_scale=_view((E_local, I, H // 32), torch.uint8),
                  w2_scale=_view((E_local, H, I // 32), torch.uint8))
    if E_local != E:
        kw.update(expert_offset=0, num_global_experts=E,
                  y_rows=torch.empty(T * k * H + 64, dtype=torch.bfloat16).as_strided((T, k, H), (k * H, H, 1)))
    x = _view((T, H), torch.bfloat16)
    ids = _view((T, k), torch.int32, 1)
    w = _view((T, k), torch.float32, 1)
    out = torch.empty(T * H + 64, dtype=torch.bfloat16).as_strided((T, H), (H, 1))
    return moe.moe_query_config(x, _view((E_local, I, Hw), wdt), _view((E_local, I, Hw), wdt),
                                _view((E_local, H, Iw), wdt), ids, w, out=None if E_local != E else out, **kw)


def test_table_rows_are_chosen_and_valid():
    rows = _rows()
    for mode, H, I, E, E_local, k, bucket, cfg in rows:
        q = _query(mode, H, I, E, E_local, k, bucket)
        assert q["config_index"] == cfg, (mode, H, I, E, E_local, k, bucket)
        # any T in the bucket takes the same row
        if bucket > 2:
            assert _query(mode, H, I, E, E_local, k, bucket // 2 + 1)["config_index"] == cfg


def test_write_inc_merges_and_formats(tmp_path):
    a = tmp_path / "a.csv"
    b = tmp_path / "b.csv"
    base = {"layer": "t", "mode": 0, "H": 256, "I": 128, "E": 8, "E_local": 8, "k": 2, "default_config": 0,
            "default_us": 1.0, "candidates": 3, "rejected": "", "rel_l2": "0", "err_ratio": "0"}
    tune.write_csv([dict(base, bucket=1, config=3, us=10.0), dict(base, bucket=2, config=4, us=11.0)], str(a))
    tune.write_csv([dict(base, bucket=2, config=5, us=9.5)], str(b))
    inc = tmp_path / "t.inc"
    assert tune.write_inc([str(a), str(b)], str(inc)) == 2
    got = [ROW.match(line).groups() for line in open(inc) if ROW.match(line)]
    assert [g[6:8] for g in got] == [("1", "3"), ("2", "5")]
    assert got[1][8] == "9.5"


def test_shard_rows_split_k_like_the_unsharded_call():
    """A tuned expert-parallel row keeps the unsharded call's K split for the
    same bucket, so shard rows stay bit-identical to the unsharded result."""
    rows = _rows()
    for mode, H, I, E, E_local, k, bucket, cfg in rows:
        if E_local == E:
            continue
        s = _query(mode, H, I, E, E_local, k, bucket)
        u = _query(mode, H, I, E, E, k, bucket)
        assert (s["gemm1_split_k"], s["gemm2_split_k"]) == (u["gemm1_split_k"], u["gemm2_split_k"])


def test_rules_take_the_320_row_tile_where_one_block_holds_the_busiest_expert():
    """Outside the table (here E = 256 experts, not a tuned layer) the bf16
    rules take 320-row tiles where the typical busiest expert has 257 to 320
    rows (expected rows r with r + 3 sqrt(r) in that range), so one block
    holds every expert, and 256-row tiles on either side."""
    H, I, E, k = 4096, 1536, 256, 8

    def rows(T):
        return T * k / E

    def busy(T):
        r = rows(T)
        return r + 3 * r ** 0.5

    for T in (4096, 8192, 16384, 32768):
        q = _query(moe.MODE_BF16, H, I, E, E, k, T)
        want = 320 if rows(T) >= 128 and 256 < busy(T) <= 320 else 256
        assert q["block_m"] == want, (T, rows(T), busy(T), q)
    # T = 8192: 256 rows per expert at E = 256, the case the rule is for
    assert _query(moe.MODE_BF16, H, I, E, E, k, 8192)["block_m"] == 320
