"""GPU parity of the skinny MXFP8 linear (the draft step's head GEMMs) against the oracle's
mxfp8_linear on the same seeded inputs, through the C ABI.

Shapes: ragged K (not a multiple of 512: the one-step tile path), split K with float32
partials (few output tiles), one, two and three 16-row groups, and the full-size head at
6 rows (N = 32320, K = 4096: a 129280-row vocabulary over four ranks), whose outputs are
checked on 640 sampled columns that the oracle computes alone.

Bar: the float32 result of each output may differ from the oracle's (a float64 sum of exact
products, rounded once) by the float32 rounding of a K-term sum taken in another order:
|dy| <= 2^-20 * sum_k |w_nk xq_k| + 2^-126, where xq is the quantized row (a K-term sum in
float32 carries at most about log2(K) ulps of error per term when summed pairwise; 2^-20
leaves that margin at K = 4096)."""
import numpy as np
import pytest

from moe_transformer_layer_amd import synth
from oracle import layer as OL
from oracle.formats import bf16_value, dequant_mxfp8_weight, mx_e4m3_dequant_act, mx_e4m3_quantize

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsl(gpu):
    from moe_transformer_layer_amd import dsl as d
    d.lib()
    return d


def _check(got, x_bits, w, ws, cols=None):
    xv = bf16_value(x_bits)
    xq = mx_e4m3_dequant_act(*mx_e4m3_quantize(xv))
    if cols is None:
        wd = dequant_mxfp8_weight(w, ws)
        want = OL.mxfp8_linear(xv, w, ws)
    else:
        # the sampled rows with the E8M0 of their own tile row; the oracle's product of them
        wd = _rows_dequant(w[cols], ws[cols // 32])
        want = OL.f32(xq @ wd.T)
    bound = np.abs(xq) @ np.abs(wd).T
    g = got if cols is None else got[:, cols]
    err = np.abs(g.astype(np.float64) - want)
    bar = bound * 2.0 ** -20 + 2.0 ** -126
    worst = float((err / bar).max())
    assert np.isfinite(g).all()
    assert worst <= 1.0, f"error up to {worst:.3g} of the bar (max abs {err.max():.3g})"
    return worst


def _rows_dequant(wc, sc_rows):
    """Sampled weight rows with the E8M0 of their own tile row."""
    from oracle.formats import e4m3_value, e8m0_value
    return e4m3_value(wc) * np.repeat(e8m0_value(sc_rows), 32, axis=1)


@pytest.mark.parametrize("M,N,K", [(5, 96, 384), (13, 1024, 1024), (17, 2048, 2048), (48, 4096, 4096)])
def test_linear_matches_oracle(dsl, M, N, K):
    rng = np.random.default_rng([M, N, K])
    w, ws = synth.gen_mxfp8_weight(N, K, 1.5 / np.sqrt(K), rng)
    x = synth.gen_x(synth.CONFIGS["mid"].replace(hidden=K), rng, M)
    lin = dsl.LinearOnDevice(w, ws)
    print(f"[linear] M={M} N={N} K={K} workspace {dsl.dsl_linear_workspace_bytes(M, N, K)} bytes", flush=True)
    got = lin(x)
    worst = _check(got, x, w, ws)
    print(f"[linear] ok, worst {worst:.3g} of the bar", flush=True)


def test_linear_full_size_head_sampled(dsl):
    M, N, K = 6, 32320, 4096
    rng = np.random.default_rng(9)
    w, ws = synth.gen_mxfp8_weight(N, K, 1.5 / np.sqrt(K), rng)
    x = synth.gen_x(synth.CONFIGS["mid"].replace(hidden=K), rng, M)
    lin = dsl.LinearOnDevice(w, ws)
    got = lin(x)
    cols = np.sort(np.random.default_rng(10).choice(N, 640, replace=False))
    print(f"[linear] full-size head M={M} N={N} K={K}, {len(cols)} sampled columns", flush=True)
    worst = _check(got, x, w, ws, cols)
    # every column written (the sampled check covers the values)
    assert np.isfinite(got).all() and (got != 0).mean() > 0.99
    print(f"[linear] ok, worst {worst:.3g} of the bar", flush=True)


def test_linear_repeat_bit_exact(dsl):
    rng = np.random.default_rng(11)
    w, ws = synth.gen_mxfp8_weight(1024, 1024, 0.05, rng)
    x = synth.gen_x(synth.CONFIGS["mid"].replace(hidden=1024), rng, 7)
    lin = dsl.LinearOnDevice(w, ws)
    assert np.array_equal(lin(x), lin(x))
