"""Comparison helpers for the GPU-vs-oracle parity tests.

Bars: expert ids bit-exact (as sets per row; the order inside a row is decided by
logit ties the gap rule does not cover); every bf16 output max-abs <= 2e-2 and
cosine >= 0.9995; router weights per id within a stated tolerance; KV records equal
except rare round-to-nearest-even flips of one code step in the e4m3 codes (the
float32 inputs of the two sides differ by summation order)."""
from __future__ import annotations

import json
import os

import numpy as np

from moe_transformer_layer_amd import synth
from oracle import layer as OL
from oracle.formats import bf16_value

ATOL = 2e-2
COS_MIN = 0.9995
GAP_MIN = 1e-3
SEEDS_FILE = os.path.join(os.path.dirname(__file__), "golden", "seeds.json")


def cos(a, b) -> float:
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


def check_bf16(name: str, got, want, report: dict | None = None):
    g, w = bf16_value(got), bf16_value(want)
    assert g.shape == w.shape, (name, g.shape, w.shape)
    assert np.isfinite(g).all(), f"{name}: non-finite GPU values"
    err = np.abs(g - w)
    maxabs = float(err.max()) if g.size else 0.0
    c = cos(g, w)
    if report is not None:
        report[name] = (maxabs, c)
    if not (maxabs <= ATOL and c >= COS_MIN):
        rows = err.reshape(err.shape[0], -1).max(axis=1)
        worst = np.argsort(-rows)[:4]
        where = np.unravel_index(int(err.argmax()), err.shape)
        detail = ", ".join(f"row {int(r)}: {rows[r]:.3g}" for r in worst)
        raise AssertionError(f"{name}: max-abs {maxabs:.4g} (bar {ATOL}) at {where} got {g[where]:.5g} want "
                             f"{w[where]:.5g}, cos {c:.7f} (bar {COS_MIN}); worst rows {detail}")
    return maxabs, c


def check_routing(got_ids, got_w, want_ids, want_w, live, w_tol: float, report: dict | None = None):
    M, k = want_ids.shape
    worst = 0.0
    for m in range(M):
        if not live[m]:
            assert (got_ids[m] == -1).all() and (got_w[m] == 0).all(), f"pad row {m} routed"
            continue
        gs, ws = np.argsort(got_ids[m]), np.argsort(want_ids[m])
        assert np.array_equal(got_ids[m][gs], want_ids[m][ws]), \
            f"row {m}: ids {sorted(got_ids[m].tolist())} vs oracle {sorted(want_ids[m].tolist())}"
        d = float(np.abs(got_w[m][gs] - want_w[m][ws]).max())
        worst = max(worst, d)
        assert abs(float(got_w[m].sum()) - 1.0) < 1e-5
    if report is not None:
        report["router_w_maxdiff"] = worst
    assert worst <= w_tol, f"router weights differ by {worst:.3g} (bar {w_tol})"


def _code_index(c):
    c = c.astype(np.int64)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def check_records(d, got_cache, want_cache, before, report: dict | None = None):
    """Records the step wrote: e4m3 codes within one step (>= 99.9% identical), scales
    within 1e-5 relative, pad bytes zero; every other byte unchanged."""
    D = d.head_dim
    changed = (want_cache != before).any(axis=2) | (got_cache != before).any(axis=2)
    assert np.array_equal(got_cache[~changed], before[~changed])
    g, w = got_cache[changed], want_cache[changed]
    if g.size == 0:
        return
    gi, wi = _code_index(g[:, :D]), _code_index(w[:, :D])
    step = np.abs(gi - wi)
    same = float((step == 0).mean())
    gs = g[:, D:D + 4].copy().view(np.float32).ravel()
    ws = w[:, D:D + 4].copy().view(np.float32).ravel()
    rel = float(np.max(np.abs(gs - ws) / np.maximum(np.abs(ws), 1e-30)))
    if report is not None:
        report["kv_codes_identical"] = same
        report["kv_scale_rel"] = rel
    assert step.max() <= 1, f"KV code off by {step.max()} steps"
    assert same >= 0.999, f"only {same:.5f} of KV codes identical"
    assert rel <= 1e-5, f"KV scale relative difference {rel:.3g}"
    assert not g[:, D + 4:].any(), "KV record pad bytes not zero"


def min_gap(d, res_layers: list, live) -> float:
    g = np.inf
    for r in res_layers:
        gaps = OL.topk_gap(r["logits"], d.top_k)
        g = min(g, float(gaps[live].min()) if live.any() else np.inf)
    return g


def oracle_decode(case):
    caches = [c.copy() for c in case.kv.cache]
    res = OL.decode_step(case.dims, case.layers, case.x, case.kv, caches)
    return res, caches


def load_seeds() -> dict:
    if not os.path.exists(SEEDS_FILE):
        return {}
    with open(SEEDS_FILE) as f:
        return json.load(f)


def gap_seed(name: str, key: str, make, oracle_run, live_of, first: int = 0, tries: int = 50):
    """A seed whose oracle logits keep every live row's top-k gap >= 1e-3: the committed
    one for `key` if present, else the first passing seed from `first` on.  `make(seed)`
    draws the case, `oracle_run(case)` returns (result, per-layer results)."""
    seeds = load_seeds()
    cand = [seeds[key]["seed"]] if key in seeds else list(range(first, first + tries))
    for s in cand:
        case = make(s)
        res, per = oracle_run(case)
        if min_gap(case.dims, per, live_of(case)) >= GAP_MIN:
            return case, res
    raise AssertionError(f"{key}: no seed in {cand[:3]}... keeps the top-k gap >= {GAP_MIN}")


def decode_live(case):
    return case.kv.positions >= 0


__all__ = ["synth", "check_bf16", "check_routing", "check_records", "gap_seed", "oracle_decode", "cos",
           "decode_live", "min_gap", "ATOL", "COS_MIN", "GAP_MIN"]
