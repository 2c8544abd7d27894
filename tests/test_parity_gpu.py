"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded
inputs, element by element.  Small multi-tile shapes with ragged row counts and pad
rows first, then every workload at its full size in the launch configuration the
bench times."""
import numpy as np
import pytest

from moe_transformer_layer_amd import synth
from oracle import layer as OL
from parity import (check_bf16, check_records, check_routing, decode_live, gap_seed, min_gap,
                    oracle_decode, GAP_MIN)

pytestmark = pytest.mark.gpu

W_TOL_MOE = 1e-5     # MoE-only steps: both sides read the same bf16 input
W_TOL_LAYER = 1e-4   # full steps: the MoE input may differ by one bf16 rounding flip per element


@pytest.fixture(scope="module")
def dsl(gpu):
    from moe_transformer_layer_amd import dsl as d
    d.lib()
    return d


def _say(msg):
    print(f"[parity] {msg}", flush=True)


def run_decode(dsl, case, res, want_caches, w_tol, report=None):
    dev = dsl.LayerOnDevice(case)
    try:
        _say(f"decode dims={case.dims.hidden}/{case.dims.n_experts} layers={case.dims.n_layers} "
             f"M={case.M} seed={case.seed}")
        got = dev.decode(case.x)
        got_caches = dev.caches_host()
    finally:
        dev.close()
    rep = {} if report is None else report
    live = decode_live(case)
    for key in ("out", "attn_out", "hres", "moe_in", "moe_out"):
        check_bf16(key, got[key], res[key], rep)
    check_routing(got["ids"], got["w"], res["ids"], res["w"], live, w_tol, rep)
    for l in range(case.dims.n_layers):
        check_records(case.dims, got_caches[l], want_caches[l], case.kv.cache[l], rep)
    _say(f"ok {rep}")
    return rep


def _decode_case(name, key, first=0, **kw):
    def run(c):
        res, caches = oracle_decode(c)
        return (res, caches), res["layers"]

    return gap_seed(name, key, lambda s: synth.make_case(name, s, **kw), run, decode_live, first=first)


# ------------------------------------------------------------------ small shapes

def test_tiny_layer_m1(dsl):
    case, (res, caches) = _decode_case("tiny", "tiny")
    run_decode(dsl, case, res, caches, W_TOL_LAYER)


# M = 8 and 9 sit on either side of the width up to which every block selects the experts
# itself (no grid barrier before the routing) and up to which the down stage's last wave
# per column group combines (no grid barrier before the combine); 1x6+1 and 2x3+2 put pad
# rows in that folded combine
@pytest.mark.parametrize("n_req,rows,n_pad", [(2, 6, 1), (1, 5, 0), (3, 4, 0), (2, 4, 0), (1, 8, 1), (1, 6, 1), (2, 3, 2)])
def test_mid_layer_ragged(dsl, n_req, rows, n_pad):
    case, (res, caches) = _decode_case("mid", f"mid_{n_req}x{rows}+{n_pad}", first=100,
                                       n_req=n_req, rows_per_req=rows, n_pad=n_pad)
    run_decode(dsl, case, res, caches, W_TOL_LAYER)


def test_mid_layer_clamp_active(dsl):
    """Large gate/up weights drive the SwiGLU clamp on many elements."""
    case, (res, caches) = _decode_case("mid", "mid_clamp", first=200, gate_gain=4.0)
    assert (np.abs(res["moe"]["gu_sh"]) > case.dims.swiglu_limit).mean() > 0.01
    run_decode(dsl, case, res, caches, W_TOL_LAYER)


def test_mid_draft_two_layers(dsl):
    case, (res, caches) = _decode_case("mid_draft", "mid_draft", first=300, n_pad=1)
    run_decode(dsl, case, res, caches, W_TOL_LAYER)


# A8W4 (MXFP8 activations into the routed experts) either side of 8 rows, with a pad row
# (mid_a8mx: the matrix-core experts on the scaled MX instruction, K steps one at a time)
@pytest.mark.parametrize("name", ["mid_a8", "mid_a8mx"])
@pytest.mark.parametrize("n_req,rows,n_pad", [(1, 6, 1), (2, 6, 0)])
def test_mid_layer_a8(dsl, name, n_req, rows, n_pad):
    case, (res, caches) = _decode_case(name, f"mid_a8_{n_req}x{rows}+{n_pad}", first=800,
                                       n_req=n_req, rows_per_req=rows, n_pad=n_pad)
    assert case.dims.expert_a8 == (2 if name.endswith("mx") else 1)
    run_decode(dsl, case, res, caches, W_TOL_LAYER)


def test_mid_attention_only(dsl):
    case = synth.make_case("mid", 400, n_pad=1)
    caches = [c.copy() for c in case.kv.cache]
    want = OL.attn_step(case.dims, case.layers[0], case.x, case.kv, caches[0])
    dev = dsl.LayerOnDevice(case)
    try:
        _say(f"attn mid M={case.M}")
        got = dev.attn(case.x)
        gc = dev.caches_host()
    finally:
        dev.close()
    check_bf16("attn_out", got["attn_out"], want["attn_out"])
    check_records(case.dims, gc[0], caches[0], case.kv.cache[0])


@pytest.mark.parametrize("name", ["mid", "mid_a8", "mid_a8mx"])
def test_mid_moe_only(dsl, name):
    d = synth.CONFIGS[name]

    def make(s):
        c = synth.make_case(name, s)
        return c

    def run(c):
        r = OL.moe_step(d, c.layers[0], c.x)
        return r, [r]

    case, res = gap_seed(name, f"{name}_moe", make, run, lambda c: np.ones(c.M, bool), first=500)
    dev = dsl.LayerOnDevice(case)
    try:
        _say(f"moe mid M={case.M}")
        got = dev.moe(case.x)
    finally:
        dev.close()
    check_bf16("moe_out", got["moe_out"], res["moe_out"])
    check_routing(got["ids"], got["w"], res["ids"], res["w"], np.ones(case.M, bool), W_TOL_MOE)


def test_repeat_launch_bit_exact(dsl):
    """Two launches of the same step give bit-identical outputs (no value atomics)."""
    case = synth.make_case("mid", 600)
    dev = dsl.LayerOnDevice(case)
    try:
        a = dev.decode(case.x)
        b = dev.decode(case.x)
    finally:
        dev.close()
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_modes_and_widths_interleaved_bit_exact(dsl):
    """Decode, MoE-only and attention-only steps of two widths, interleaved on one handle,
    each give what it gave when it ran first.  Steps of up to 8 rows finish the MoE on
    counters in the handle's sync words whose starting values every launch reads for
    itself (in its first stage, whatever the step's kind); a 12-row step does not count on
    them, an attention-only step stops before them."""
    d = synth.CONFIGS["mid"]
    layers = synth.make_weights("mid", 3)
    weights = dsl.DeviceWeights(d, layers)
    small = dsl.LayerOnDevice(synth.make_case("mid", 700, layers=layers, n_req=1, rows_per_req=6, n_pad=1),
                              weights=weights)
    wide = dsl.LayerOnDevice(synth.make_case("mid", 701, layers=layers, n_req=2, rows_per_req=6), weights=weights)
    u = synth.gen_x(d, np.random.default_rng(702), 7)
    try:
        steps = {"decode7": lambda: small.decode(small.case.x), "moe7": lambda: small.moe(u),
                 "attn7": lambda: small.attn(small.case.x), "decode12": lambda: wide.decode(wide.case.x)}
        first = {k: f() for k, f in steps.items()}
        for k in ("moe7", "decode7", "decode12", "decode7", "attn7", "moe7", "decode7", "moe7"):
            got = steps[k]()
            for key in got:
                assert np.array_equal(got[key], first[k][key]), f"{k}: {key} differs from its first run"
    finally:
        small.close()
        wide.close()
        weights.close()
