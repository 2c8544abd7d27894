"""Pins of the oracle's layer composition (how attn_half, layer_step and decode_step chain
the pieces the other pin files check one by one).  CPU only.

The main pin is a second, independent derivation of the decode layer written here with
torch float64 operations: weights decoded by torch's own float8 cast (and a hand e2m1
table), MX activation quantization through torch.frexp and the float8 cast, bf16
rounding through torch's casts, keys gathered from the block table here.  It follows
the stage order of "Mono decode layer for DeepSeek-V4.1-Flash on MI355X" (vLLM PR
60397), Purpose, launch table: attention-input norm, wqkv, q/kv norms, the KV insert
before any row attends, wq_b, attention, wo_a, wo_b, then the FFN norm and the MoE;
with the plain pre-norm residual (hres = bf16(x + a), out = bf16(hres + m)) and the
MXFP8 quantization of every attention linear's input.  The oracle must agree with it
bit for bit on every bf16 output, the ids, the weights and the KV records.

Each plausible slip in the composition is then planted in a copy of the oracle's
source (on the CPU) and must make that pin fail: the FFN norm of x instead of hres, the
step's KV records inserted after attention, no MXFP8 quantization before wo_a, the
output summed without the bf16 hres, x in place of hres in the output, a skipped q norm,
and the q/kv halves of wqkv swapped.  Degenerate
weights give closed forms: one key per row (window 1) makes the attention output the
row's own dequantized record; wo_b = 0 gives hres = x; zero down projections give
out = hres."""
import inspect
import math
import types

import numpy as np
import pytest
import torch

from moe_transformer_layer_amd import synth
from oracle import layer as L

F64 = torch.float64


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a))


# ---------------------------------------------------------------- the second derivation

def _bf16r(x):
    """Round to float32, then to bf16 (torch's casts, nearest even), as float64."""
    return x.to(torch.float32).to(torch.bfloat16).to(F64)


def _f32r(x):
    return x.to(torch.float32).to(F64)


def _bf16_from_bits(bits):
    return _t(bits.view(np.int16)).view(torch.bfloat16).to(F64)


def _bits_from_bf16(x):
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _e4m3(codes):
    return _t(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(F64)


def _pow2(e):
    return torch.pow(torch.tensor(2.0, dtype=F64), e.to(F64))


def _w_mx8(codes, s):
    sc = _pow2(_t(s.astype(np.int64)) - 127).repeat_interleave(32, 0).repeat_interleave(32, 1)
    return _e4m3(codes) * sc


def _w_b128(codes, s):
    sc = _t(s.astype(np.float64)).repeat_interleave(128, 0).repeat_interleave(128, 1)
    return _e4m3(codes) * sc


_E2M1 = torch.tensor([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6], dtype=F64)


def _w_fp4(packed, s):
    p = _t(packed.astype(np.int64))
    v = torch.stack([_E2M1[p & 15], _E2M1[p >> 4]], -1).reshape(p.shape[0], -1)
    return v * _pow2(_t(s.astype(np.int64)) - 127).repeat_interleave(32, 1)


def _mxq(v):
    """MXFP8 per 1x32 block along the last axis: the block exponent is floor(log2 amax)
    of the float32 amax less 8 (e4m3's largest exponent), biased by 127, clamped to
    [0, 254]; elements v / 2^(X-127) cast to e4m3 (nearest even, saturated at 448)."""
    R, K = v.shape
    b = v.reshape(R, K // 32, 32)
    amax = b.abs().amax(-1).to(torch.float32)
    _, e = torch.frexp(amax)  # amax = m 2^e, m in [0.5, 1): floor(log2 amax) = e - 1
    X = torch.where(amax > 0, (e - 1 + 127 - 8).clamp(0, 254), torch.zeros_like(e))
    sc = _pow2(X - 127)[..., None]
    q = (b / sc).clamp(-448.0, 448.0).to(torch.float32).to(torch.float8_e4m3fn).to(F64)
    return (q * sc).reshape(R, K)


def _rms(x, g, eps):
    return _f32r(x / torch.sqrt((x * x).mean(-1, keepdim=True) + eps) * _t(g.astype(np.float64)))


def _lin8(x, codes, s):
    return _f32r(_mxq(x) @ _w_mx8(codes, s).T)


def _swiglu(g, u, lim):
    g = g.clamp(max=lim)
    u = u.clamp(-lim, lim)
    return g * torch.sigmoid(g) * u


def _record(kv, D):
    """fp8 KV records [n, D + 16] of float32 rows: s = amax / 448 in float32, codes
    e4m3(kv / s) in float32, then s, then 12 zero bytes; and their dequantized values."""
    kv32 = kv.to(torch.float32)
    s = kv32.abs().amax(-1, keepdim=True) / torch.tensor(448.0, dtype=torch.float32)
    safe = torch.where(s > 0, s, torch.ones_like(s))
    c = torch.where(s > 0, (kv32 / safe).clamp(-448.0, 448.0), torch.zeros_like(kv32)).to(torch.float8_e4m3fn)
    rec = np.zeros((kv.shape[0], D + 16), dtype=np.uint8)
    rec[:, :D] = c.view(torch.uint8).numpy()
    rec[:, D:D + 4] = s.numpy().view(np.uint8)
    return rec


def _rec_value(rec, D):
    s = _t(rec[:, D:D + 4].copy().view(np.float32).astype(np.float64))
    return _e4m3(rec[:, :D]) * s


def _keys(d, kv, r):
    p, q = int(kv.positions[r]), int(kv.row_req[r])
    if d.swa_width > 0:
        return [int(s) for s in kv.key_table[r] if s >= 0]
    out = []
    for pos in range(max(0, p - d.window + 1), p + 1):
        out.append(int(kv.block_table[q, pos // d.kv_block]) * d.kv_block + pos % d.kv_block)
    return out


def torch_layer(d, lw, x_bits, kv, cache):
    """One decode layer, independently of the oracle.  `cache` (uint8 [blocks, B, RECORD])
    receives the step's records.  Returns the bf16 outputs (as bits), ids, weights."""
    M, qr, D, H, h = x_bits.shape[0], d.q_rank, d.head_dim, d.n_heads, d.hidden
    live = torch.from_numpy(kv.positions >= 0)
    x = _bf16_from_bits(x_bits)
    # attention front
    xn = _rms(x, lw["attn_norm"], d.norm_eps)
    qkv = _lin8(xn, lw["wqkv"], lw["wqkv_s"])
    qn = _rms(qkv[:, :qr], lw["q_norm"], d.norm_eps)
    kvn = _rms(qkv[:, qr:], lw["kv_norm"], d.norm_eps)
    recs = _record(kvn, D)
    B = d.kv_block
    for r in range(M):  # every insert before any read
        if live[r]:
            p, q = int(kv.positions[r]), int(kv.row_req[r])
            slot = int(kv.block_table[q, p // B]) * B + p % B
            cache[slot // B, slot % B] = recs[r]
    qh = _lin8(qn, lw["wq_b"], lw["wq_b_s"]).reshape(M, H, D)
    o = torch.zeros((M, H, D), dtype=F64)
    for r in range(M):
        if not live[r]:
            continue
        slots = _keys(d, kv, r)
        kval = _rec_value(np.stack([cache[s // B, s % B] for s in slots]), D)
        p = torch.softmax((qh[r] @ kval.T) / math.sqrt(D), dim=-1)
        o[r] = p @ kval
    o = _f32r(o).reshape(M, H * D)
    a = _lin8(_lin8(o, lw["wo_a"], lw["wo_a_s"]), lw["wo_b"], lw["wo_b_s"])
    a[~live] = 0
    hres = _bf16r(x + a)
    u = _bf16r(_rms(hres, lw["ffn_norm"], d.norm_eps))
    # MoE
    logits = _f32r(u @ _t(lw["w_router"].astype(np.float64)).T)
    k, I, Is = d.top_k, d.inter, d.shared_inter
    ids = torch.full((M, k), -1, dtype=torch.int64)
    wt = torch.zeros((M, k), dtype=F64)
    for r in range(M):
        if not live[r]:
            continue
        order = torch.sort(-logits[r], stable=True).indices[:k]
        ids[r] = order
        wt[r] = torch.softmax(logits[r, order], dim=0)
    wt = _f32r(wt)
    gu = _f32r(u @ _w_b128(lw["sh_w13"], lw["sh_w13_s"]).T)
    zs = _bf16r(_swiglu(gu[:, :Is], gu[:, Is:], d.swiglu_limit))
    m = _f32r(zs @ _w_b128(lw["sh_wd"], lw["sh_wd_s"]).T)
    # A8W4: the routed experts' inputs (u, and the SwiGLU output z) go through MXFP8
    act = _mxq if d.expert_a8 else (lambda v: v)
    for j in range(k):
        for r in range(M):
            if not live[r]:
                continue
            e = int(ids[r, j])
            g = _f32r(act(u[r:r + 1]) @ _w_fp4(lw["ex_w13"][e], lw["ex_w13_s"][e]).T)
            z = _bf16r(_swiglu(g[:, :I], g[:, I:], d.swiglu_limit))
            y = _f32r(act(z) @ _w_fp4(lw["ex_wd"][e], lw["ex_wd_s"][e]).T)
            m[r] = m[r] + wt[r, j] * y[0]
    m = _f32r(m)
    m[~live] = 0
    out = _bf16r(hres + m)
    z16 = np.uint16(0)
    res = dict(out=_bits_from_bf16(out), attn_out=_bits_from_bf16(a), hres=_bits_from_bf16(hres),
               moe_in=_bits_from_bf16(u), moe_out=_bits_from_bf16(m), ids=ids.numpy().astype(np.int32),
               w=wt.numpy())
    for key in ("out", "hres", "moe_in"):
        res[key][~live.numpy()] = z16
    return res


def torch_decode(d, layers, x_bits, kv, caches):
    x = x_bits
    for l in range(d.n_layers):
        r = torch_layer(d, layers[l], x, kv, caches[l])
        x = r["out"]
    return r


# ---------------------------------------------------------------- comparison

def mismatches(d, orc, case) -> list:
    """Run `orc` (the oracle module, or a mutated copy) and the torch derivation on `case`;
    return what differs."""
    c1 = [x.copy() for x in case.kv.cache]
    c2 = [x.copy() for x in case.kv.cache]
    want = orc.decode_step(d, case.layers, case.x, case.kv, c1)
    got = torch_decode(d, case.layers, case.x, case.kv, c2)
    bad = []
    for key in ("out", "attn_out", "hres", "moe_in", "moe_out"):
        n = int((want[key] != got[key]).sum())
        if n:
            bad.append(f"{key}: {n} of {got[key].size} bf16 values differ")
    live = case.kv.positions >= 0
    if not np.array_equal(want["ids"][live], got["ids"][live]):
        bad.append("ids differ")
    if not np.array_equal(np.asarray(want["w"], dtype=np.float64)[live], got["w"][live]):
        bad.append("router weights differ")
    for l in range(d.n_layers):
        if not np.array_equal(c1[l], c2[l]):
            bad.append(f"layer {l} KV records differ")
    return bad


_CASES = {
    # causal window over a paged cache, two requests of 6 rows and a pad row
    "mid": dict(name="mid", seed=21, n_pad=1),
    # the same with MXFP8 activations into the routed experts (A8W4)
    "mid_a8": dict(name="mid_a8", seed=21, n_pad=1),
    # index-table rows, two chained layers (layer 1's input is layer 0's output)
    "mid_draft": dict(name="mid_draft", seed=22),
}


def _case(key):
    kw = dict(_CASES[key])
    return synth.make_case(kw.pop("name"), kw.pop("seed"), **kw)


@pytest.mark.parametrize("key", list(_CASES))
def test_oracle_equals_independent_torch_derivation(key):
    c = _case(key)
    assert mismatches(c.dims, L, c) == []


# ---------------------------------------------------------------- planted slips

def _mutant(edits) -> types.ModuleType:
    """A copy of the oracle module with each (old, new) source edit applied once."""
    src = inspect.getsource(L)
    for old, new in edits:
        assert src.count(old) == 1, f"oracle source no longer holds {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("oracle._mutant")
    mod.__package__ = "oracle"
    exec(compile(src, "oracle/layer.py (planted slip)", "exec"), mod.__dict__)
    return mod


_INSERT = """    for r in range(M):
        if live[r]:
            s = slot_of(int(kv.positions[r]), int(kv.row_req[r]), kv.block_table, d.kv_block)
            cache[s // d.kv_block, s % d.kv_block] = recs[r]
"""
_AFTER_ATTN = "    o = f32(o).reshape(M, H * D)\n"

_SLIPS = {
    "ffn norm of x": [('u_bits = bf16_encode(rmsnorm(hres, lw["ffn_norm"], d.norm_eps))',
                       'u_bits = bf16_encode(rmsnorm(x, lw["ffn_norm"], d.norm_eps))')],
    "kv insert after attention": [(_INSERT, ""), (_AFTER_ATTN, _AFTER_ATTN + _INSERT)],
    "no mxfp8 before wo_a": [('t = mxfp8_linear(o, lw["wo_a"], lw["wo_a_s"])',
                              't = f32(gemv_mxfp8(lw["wo_a"], lw["wo_a_s"], o))')],
    "out without bf16 hres": [('out_bits = bf16_encode(hres + mo["m"])',
                               'out_bits = bf16_encode(x + at["a"] + mo["m"])')],
    "q/kv halves swapped": [("q_lat, kv_lat = qkv[:, :qr], qkv[:, qr:qr + D]",
                             "kv_lat, q_lat = qkv[:, :D], qkv[:, D:D + qr]")],
    "q norm skipped": [('q_n = rmsnorm(q_lat, lw["q_norm"], d.norm_eps)', "q_n = f32(q_lat)")],
    "x instead of hres in the output": [('out_bits = bf16_encode(hres + mo["m"])',
                                         'out_bits = bf16_encode(x + mo["m"])')],
}


_A8_SLIPS = {
    "a8: gate/up input not quantized": [("u_ex = mxq(u) if a8 else u", "u_ex = u")],
    "a8: down input not quantized": [('lw["ex_wd_s"][e], mxq(z) if a8 else z))', 'lw["ex_wd_s"][e], z))')],
}


@pytest.mark.parametrize("slip", list(_A8_SLIPS))
def test_planted_a8_slip_fails_the_pin(slip):
    c = _case("mid_a8")
    bad = mismatches(c.dims, _mutant(_A8_SLIPS[slip]), c)
    assert bad, f"planted slip '{slip}' passed the composition pin"


def test_a8_changes_only_the_routed_experts():
    """A8W4 and W4A16 on the same draws: the attention half, the MoE input, the router and
    the KV records are identical; the MoE output differs (the experts' inputs are
    quantized), by no more than the MXFP8 rounding of their inputs allows."""
    c16, c8 = _case("mid"), _case("mid_a8")
    assert np.array_equal(c16.x, c8.x)
    r16 = L.decode_step(c16.dims, c16.layers, c16.x, c16.kv, [x.copy() for x in c16.kv.cache])
    r8 = L.decode_step(c8.dims, c8.layers, c8.x, c8.kv, [x.copy() for x in c8.kv.cache])
    for key in ("attn_out", "hres", "moe_in", "ids", "logits"):
        np.testing.assert_array_equal(r16[key], r8[key])
    from oracle.formats import bf16_value
    a, b = bf16_value(r16["moe_out"]), bf16_value(r8["moe_out"])
    assert (a != b).any()
    # e4m3 keeps 4 significant bits: each quantized input is within 2^-4 of its value, so
    # the branch moves by a few percent of its size, not more
    assert np.abs(a - b).max() < 0.1 * np.abs(a).max()


def test_unmutated_copy_passes():
    """The planting machinery itself changes nothing when no slip is planted."""
    c = _case("mid")
    assert mismatches(c.dims, _mutant([]), c) == []


@pytest.mark.parametrize("slip", list(_SLIPS))
def test_planted_slip_fails_the_pin(slip):
    c = _case("mid")
    bad = mismatches(c.dims, _mutant(_SLIPS[slip]), c)
    assert bad, f"planted slip '{slip}' passed the composition pin"


# ---------------------------------------------------------------- degenerate weights

def test_window_one_gives_own_record():
    """With one key per row (window 1) every head of a live row attends only to the
    record this step inserted for it, so the attention output is that record's
    dequantized latent: the insert precedes the read and lands at the row's slot."""
    c = _case("mid")
    d = c.dims.replace(window=1)
    cache = c.kv.cache[0].copy()
    at = L.attn_half(d, c.layers[0], c.x, c.kv, cache)
    o = at["o"].reshape(c.M, d.n_heads, d.head_dim)
    B = d.kv_block
    for r in range(c.M):
        if c.kv.positions[r] < 0:
            assert not o[r].any()
            continue
        p, q = int(c.kv.positions[r]), int(c.kv.row_req[r])
        slot = int(c.kv.block_table[q, p // B]) * B + p % B
        own = _rec_value(cache[slot // B, slot % B][None], d.head_dim).numpy()[0]
        assert np.abs(own).max() > 0
        for hh in range(d.n_heads):
            np.testing.assert_array_equal(o[r, hh], own.astype(np.float32).astype(np.float64))


def test_kv_rows_of_wqkv_follow_the_q_rows():
    """wqkv's rows are [q latent; kv latent]: zeroing the last head_dim rows zeroes every
    record the step writes (scale 0, codes 0), while zeroing the first q_rank rows leaves
    them nonzero."""
    c = _case("mid")
    d = c.dims
    live = c.kv.positions >= 0
    for zero_kv in (True, False):
        lw = dict(c.layers[0])
        w = lw["wqkv"].copy()
        if zero_kv:
            w[d.q_rank:] = 0
        else:
            w[:d.q_rank] = 0
        lw["wqkv"] = w
        at = L.attn_half(d, lw, c.x, c.kv, c.kv.cache[0].copy())
        recs = at["records"][live]
        assert (not recs.any()) if zero_kv else recs[:, :d.head_dim].any(axis=1).all()


def test_zero_wo_b_gives_hres_equal_x():
    c = _case("mid")
    lw = dict(c.layers[0])
    lw["wo_b"] = np.zeros_like(lw["wo_b"])
    r = L.layer_step(c.dims, lw, c.x, c.kv, c.kv.cache[0].copy())
    live = c.kv.positions >= 0
    np.testing.assert_array_equal(r["hres"][live], c.x[live])
    assert not r["attn_out"].any()


def test_zero_down_projections_give_out_equal_hres():
    c = _case("mid")
    lw = dict(c.layers[0])
    lw["sh_wd"] = np.zeros_like(lw["sh_wd"])
    lw["ex_wd"] = np.zeros_like(lw["ex_wd"])
    r = L.layer_step(c.dims, lw, c.x, c.kv, c.kv.cache[0].copy())
    np.testing.assert_array_equal(r["out"], r["hres"])
    assert not r["moe_out"].any()


def test_chained_layer_input_is_previous_output():
    """decode_step feeds layer l + 1 the bf16 output of layer l, with its own weights and
    its own cache."""
    c = _case("mid_draft")
    d = c.dims
    caches = [x.copy() for x in c.kv.cache]
    res = L.decode_step(d, c.layers, c.x, c.kv, caches)
    d1 = d.replace(n_layers=1)
    x = c.x
    for l in range(d.n_layers):
        cl = c.kv.cache[l].copy()
        one = L.layer_step(d1, c.layers[l], x, c.kv, cl)
        np.testing.assert_array_equal(one["out"], res["layers"][l]["out"])
        np.testing.assert_array_equal(cl, caches[l])
        x = one["out"]


# ---------------------------------------------------------------- the skinny head linear

@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (6, 96, 384), (13, 32, 1024)])
def test_skinny_mxfp8_linear_against_torch(M, N, K):
    """The oracle of the draft head GEMMs is mxfp8_linear: MXq(x) . W^T in float32.  Checked
    against a torch float64 product of the torch-side MX quantization and float8 decode above,
    on bf16 rows off the MXFP8 grid."""
    rng = np.random.default_rng(M * 1000 + N + K)
    w, ws = synth.gen_mxfp8_weight(N, K, 1.5 / math.sqrt(K), rng)
    x = synth.gen_x(synth.CONFIGS["mid"].replace(hidden=K), rng, M)
    got = L.mxfp8_linear(__import__("oracle.formats", fromlist=["bf16_value"]).bf16_value(x), w, ws)
    want = _f32r(_mxq(_bf16_from_bits(x)) @ _w_mx8(w, ws).T).numpy()
    np.testing.assert_array_equal(got, want)
