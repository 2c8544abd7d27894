"""dsl_decode_step_noalloc, the decode step for callers that cannot allocate, against
dsl_decode_step on the same inputs: two calls in a row on one handle, the second with
fewer rows, every output, tap and KV record bit for bit.  Each entry point writes a cache
of its own (two uploads of the same cache), so both see the same records.  Also the
refusal of a width whose scratch does not fit the static array."""
import numpy as np
import pytest

from moe_transformer_layer_amd import synth

pytestmark = [pytest.mark.gpu]


def _say(msg):
    print(f"[noalloc] {msg}", flush=True)


@pytest.fixture(scope="module")
def dsl(gpu):
    from moe_transformer_layer_amd import dsl as d
    d.lib()
    return d


def _pair(dsl, name, layouts, wseed, seeds):
    layers = synth.make_weights(name, wseed)
    weights = dsl.DeviceWeights(synth.CONFIGS[name], layers)
    try:
        for lay, seed in zip(layouts, seeds):
            case = synth.make_case(name, seed, layers=layers, **lay)
            a = dsl.LayerOnDevice(case, weights=weights)
            b = dsl.LayerOnDevice(case, weights=weights)
            _say(f"{name}: M={case.M} layers={case.dims.n_layers}, no-allocation entry point then the usual one")
            got = a.decode(case.x, noalloc=True)
            want = b.decode(case.x)
            for k in want:
                assert np.array_equal(got[k], want[k]), f"{name} M={case.M}: {k} differs"
            for l, (ca, cb) in enumerate(zip(a.caches_host(), b.caches_host())):
                assert np.array_equal(ca, cb), f"{name} M={case.M}: layer {l} KV records differ"
            assert got["out"].any()
            a.close()
            b.close()
    finally:
        weights.close()


def test_noalloc_equals_decode_small(dsl):
    _pair(dsl, "mid_draft", (dict(n_req=2, rows_per_req=6, n_pad=1), dict(n_req=1, rows_per_req=5)), 3, (40, 41))


def test_noalloc_equals_decode_full(dsl):
    _pair(dsl, "layer48", (dict(M=48), dict(M=6)), 7, (50, 51))


def test_noalloc_refuses_scratch_beyond_the_array(dsl):
    """Three draft layers of 48 rows need about 64 MiB of scratch: refused before any
    launch, and the handle still works through both entry points afterwards."""
    name = "draft"
    layers = synth.make_weights(name, 11)
    weights = dsl.DeviceWeights(synth.CONFIGS[name], layers)
    try:
        case = synth.make_case(name, 0, layers=layers, M=48)
        dev = dsl.LayerOnDevice(case, weights=weights)
        with pytest.raises(dsl.DslError) as ei:
            dev.decode(case.x, noalloc=True)
        assert ei.value.code == dsl.DSL_EUNSUPPORTED and "scratch" in str(ei.value)
        small = synth.make_case(name, 1, layers=layers, M=6)
        a = dsl.LayerOnDevice(small, weights=weights)
        b = dsl.LayerOnDevice(small, weights=weights)
        got, want = a.decode(small.x, noalloc=True), b.decode(small.x)
        assert all(np.array_equal(got[k], want[k]) for k in want)
        for d_ in (dev, a, b):
            d_.close()
    finally:
        weights.close()
