"""Host-side checks of the bench's byte accounting (no GPU).

The algorithmic bytes per step follow the step's definition: every weight read once
(MXFP8 codes plus one E8M0 scale per 32, the FP8 shared expert with one f32 scale per
128 x 128 block, each distinct selected MXFP4 expert once), the union of the rows' KV
windows (or index-table rows) read once per layer, one record written per live row.
The per-component figures below are the ones the sizes give at hidden 4096, 16 heads of
512, q/o rank 1024, 128 experts of inter 2048, shared inter 2048.
"""
from types import SimpleNamespace

import numpy as np

import bench
from moe_transformer_layer_amd import synth

ATTN = 27_328_512     # wqkv 1536x4096, wq_b 8192x1024, wo_a 1024x8192, wo_b 4096x1024, 4 gammas
ROUTER = 2_097_152    # 128 x 4096 f32
SHARED = 25_171_968   # 3 x 4096 x 2048 fp8 + f32 scales per 128 x 128 block
EXPERT = 13_369_344   # 3 x 4096 x 2048 fp4 + one e8m0 per 32


def _kv(positions, row_req, key_table=None):
    return SimpleNamespace(positions=np.array(positions), row_req=np.array(row_req), key_table=key_table)


def test_components_full_layer():
    d = synth.CONFIGS["layer48"]
    M = 6
    ids = np.array([[[0, 1, 2, 3, 4, 5]] * M])  # every row the same 6 experts
    kv = _kv([1000 + j for j in range(M)], [0] * M)
    b = bench.algorithmic_bytes(d, M, ids, kv)
    assert (b["attention"], b["router"], b["shared"]) == (ATTN, ROUTER, SHARED)
    assert b["n_distinct"] == [6] and b["experts"] == 6 * EXPERT
    rec = d.head_dim + 16
    # rows at 1000..1005 with window 128: positions 873..1005 are read once
    assert b["kv"] == (1005 - 873 + 1) * rec + M * rec
    assert b["act"] == 2 * M * d.hidden * 2
    assert b["total"] == ATTN + ROUTER + SHARED + 6 * EXPERT + b["kv"] + b["act"]


def test_distinct_experts_and_pad_rows():
    d = synth.CONFIGS["layer48"]
    M = 4
    ids = np.array([[[0, 1, 2, 3, 4, 5], [5, 6, 7, 8, 9, 10], [0, 1, 2, 3, 4, 5], [100, 101, 102, 103, 104, 105]]])
    # the last row is a pad row: its selection is not read
    kv = _kv([10, 11, 12, -1], [0, 0, 0, 0])
    b = bench.algorithmic_bytes(d, M, ids, kv)
    assert b["n_distinct"] == [11]
    rec = d.head_dim + 16
    assert b["kv"] == 13 * rec + 3 * rec  # positions 0..12 once, three records written


def test_draft_layers_count_each_layer():
    d = synth.CONFIGS["draft"]
    M = 2
    ids = np.array([[[0, 1, 2]] * M, [[3, 4, 5], [3, 4, 6]], [[7, 8, 9]] * M])
    kt = np.full((M, d.swa_width), -1)
    kt[0, :5] = [10, 11, 12, 13, 14]
    kt[1, :6] = [10, 11, 12, 13, 14, 15]
    kv = _kv([20, 21], [0, 0], kt)
    b = bench.algorithmic_bytes(d, M, ids, kv)
    rec = d.head_dim + 16
    assert b["n_distinct"] == [3, 4, 3]
    assert b["kv"] == 3 * (6 * rec + M * rec)
    assert b["total"] == 3 * (ATTN + ROUTER + SHARED) + 10 * EXPERT + b["kv"] + b["act"]
    assert b["per_layer"] == b["total"] / 3
