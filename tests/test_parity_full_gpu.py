"""GPU parity at the workloads' full sizes (hidden 4096, 16 heads x 512, 128 experts,
inter 2048), in the launch configuration the bench times, against the oracle on the
same seeded inputs.  Seeds come from tests/golden/seeds.json (written by
make_seeds.py with the oracle alone); each test re-checks the top-k gap rule.

  MoE stage alone, M = 6, top-3                 (moe6)
  attention half alone, M = 48 (8 x 6 rows)     (attn48)
  full layer, top-6, M = 48 and M = 6           (layer48)
  three draft layers, 192-wide index rows, top-3, M in {1, 6, 12, 24, 36, 48}, one
  handle for all widths (each width gets its own scratch)  (draft)
"""
import numpy as np
import pytest

from moe_transformer_layer_amd import synth
from oracle import layer as OL
from parity import (GAP_MIN, check_bf16, check_records, check_routing, decode_live, load_seeds, min_gap,
                    oracle_decode)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

W_TOL_MOE = 1e-5
W_TOL_LAYER = 1e-4
SEEDS = load_seeds()


def _say(msg):
    print(f"[parity-full] {msg}", flush=True)


@pytest.fixture(scope="module")
def dsl(gpu):
    from moe_transformer_layer_amd import dsl as d
    d.lib()
    return d


_weights = {}


def _device_weights(dsl, name, wseed):
    key = (name, wseed)
    if key not in _weights:
        for k in list(_weights):
            _weights.pop(k)[1].close()
        layers = synth.make_weights(name, wseed)
        _say(f"uploading {name} weights (seed {wseed})")
        _weights[key] = (layers, dsl.DeviceWeights(synth.CONFIGS[name], layers))
    return _weights[key]


def _seeded(key):
    assert key in SEEDS, f"no committed seed for {key}: run tests/golden/make_seeds.py"
    return SEEDS[key]


def _run_decode(dsl, name, key):
    sd = _seeded(key)
    layers, dw = _device_weights(dsl, name, sd["weights_seed"])
    case = synth.make_case(name, sd["seed"], M=sd["M"], layers=layers)
    res, caches = oracle_decode(case)
    live = decode_live(case)
    g = min_gap(case.dims, res["layers"], live)
    assert g >= GAP_MIN, f"{key}: top-k gap {g} below {GAP_MIN}"
    dev = dsl.LayerOnDevice(case, weights=dw)
    _say(f"{key}: decode M={case.M} layers={case.dims.n_layers}")
    got = dev.decode(case.x)
    got_caches = dev.caches_host()
    dev.close()
    rep, errors = {}, []

    def attempt(f, *a):
        try:
            f(*a)
        except AssertionError as e:
            errors.append(str(e))

    for k in ("attn_out", "hres", "moe_in", "moe_out", "out"):
        attempt(check_bf16, k, got[k], res[k], rep)
    attempt(check_routing, got["ids"], got["w"], res["ids"], res["w"], live, W_TOL_LAYER, rep)
    for l in range(case.dims.n_layers):
        attempt(check_records, case.dims, got_caches[l], caches[l], case.kv.cache[l], rep)
    _say(f"{key}: {rep}")
    assert not errors, f"{key}: " + " | ".join(errors)


def test_moe_stage_m6_top3(dsl):
    sd = _seeded("moe6")
    layers, dw = _device_weights(dsl, "moe6", sd["weights_seed"])
    case = synth.make_case("moe6", sd["seed"], layers=layers)
    d = case.dims
    want = OL.moe_step(d, layers[0], case.x)
    assert float(OL.topk_gap(want["logits"], d.top_k).min()) >= GAP_MIN
    dev = dsl.LayerOnDevice(case, weights=dw)
    _say("moe6: moe step M=6")
    got = dev.moe(case.x)
    dev.close()
    rep = {}
    check_bf16("moe_out", got["moe_out"], want["moe_out"], rep)
    check_routing(got["ids"], got["w"], want["ids"], want["w"], np.ones(case.M, bool), W_TOL_MOE, rep)
    _say(f"moe6: ok {rep}")


def test_attention_half_m48(dsl):
    layers, dw = _device_weights(dsl, "layer48", 7)
    case = synth.make_case("attn48", 3, M=48, layers=layers)
    caches = [c.copy() for c in case.kv.cache]
    want = OL.attn_step(case.dims, layers[0], case.x, case.kv, caches[0])
    dev = dsl.LayerOnDevice(case, weights=dw)
    _say("attn48: attention step M=48")
    got = dev.attn(case.x)
    gc = dev.caches_host()
    dev.close()
    rep = {}
    check_bf16("attn_out", got["attn_out"], want["attn_out"], rep)
    check_records(case.dims, gc[0], caches[0], case.kv.cache[0], rep)
    _say(f"attn48: ok {rep}")


def test_full_layer_m48_top6(dsl):
    _run_decode(dsl, "layer48", "layer48_m48")


def test_full_layer_m6_top6(dsl):
    _run_decode(dsl, "layer48", "layer48_m6")


@pytest.mark.parametrize("M", [1, 6, 12, 24, 36, 48])
def test_draft_three_layers(dsl, M):
    _run_decode(dsl, "draft", f"draft_m{M}")
