"""Plain CPU oracle of one DeepSeek-V4.1-style decode layer (attention front,
sliding-window attention, attention back, MoE), and of its attention and MoE
halves on their own.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  The product path never imports it.

Stage list: "Mono decode layer for DeepSeek-V4.1-Flash on MI355X" (vLLM PR
60397), Purpose, launch table: K1 = attention seam, wqkv, q/kv norms, the KV
insert, wq_b; K2 = split attention, combine, wo_a, wo_b, then the MoE (router,
top-k, shared expert, MXFP4 experts).  Numerics: same page, Layout (f32 router
logits, row-major FP8 shared-expert weights, MXFP8 activation quantization,
clamped SwiGLU) and Design (row-major MXFP8 attention weights with 32x32 E8M0
scales).  Draft layers: "Mono decode for the DSpark draft layers" (vLLM PR
62131), Details (top-3 of 128, non-causal 192-wide index rows).

Everything is computed in float64 from exactly dequantized weights, one step
after another, with no blocking or fusion.  The rounding points where the
kernels store a narrower type are applied explicitly:
  R1 boundary activations bf16; R2 MXFP8 quantization of the input of wqkv,
  wq_b, wo_a, wo_b; R3 norms, linear outputs, attention output and router
  logits float32; R4 KV codes e4m3 with a float32 scale; R5 hres bf16;
  R6 MoE input bf16; R7 SwiGLU output bf16; R8 expert outputs and the
  combine float32; R9 outputs bf16.
Where a float32 value decides a code (the KV record), the oracle takes that
decision in float32 arithmetic, as the kernel does.

Readings of points the pages leave open (the residual is a plain pre-norm
residual in place of the mHC seams; no RoPE; scale 1/sqrt(head_dim); K = V =
the dequantized latent record; our own 16-byte-tailed KV record; softmax over
the selected logits; the SwiGLU clamp below) are listed with the design notes.
Parity unpinned: fidelity to the real DeepSeek-V4.1 layer (mHC seams, the true
router and clamp, the 584-byte record), which no page defines.
"""
from __future__ import annotations

import numpy as np

from .cgemv import gemv_fp8b128, gemv_mxfp4, gemv_mxfp8
from .formats import (bf16_encode, bf16_round, bf16_value, e4m3_encode, e4m3_value, f32,
                      mx_e4m3_dequant_act, mx_e4m3_quantize)


# ----------------------------------------------------------------------------- pieces

def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm along the last axis: x / sqrt(mean(x^2) + eps) * gamma, float32 result (R3).
    Used for the attention input, the q and kv latents and the FFN input (eps 1e-6)."""
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return f32(x * r * np.asarray(gamma, dtype=np.float64))


def mxfp8_linear(x: np.ndarray, w: np.ndarray, ws: np.ndarray) -> np.ndarray:
    """y = MXq(x) . W^T for a row-major MXFP8 weight (32x32 E8M0 tiles).  The input is
    quantized per 1x32 block along K straight from float32 (R2); the result is float32
    (R3)."""
    xq, xs = mx_e4m3_quantize(x)
    return f32(gemv_mxfp8(w, ws, mx_e4m3_dequant_act(xq, xs)))


def kv_record(kv: np.ndarray, head_dim: int) -> np.ndarray:
    """One fp8 KV record per row of kv (float32 values): D e4m3 codes, then the float32
    scale s = amax/448, then 12 zero bytes.  Codes are e4m3(kv / s), nearest even with
    saturation; amax = 0 gives s = 0 and zero codes.  The scale and the quotient are
    taken in float32 arithmetic (R4)."""
    kv32 = np.asarray(kv, dtype=np.float32)
    n = kv32.shape[0]
    amax = np.abs(kv32).max(axis=1)
    s = (amax / np.float32(448.0)).astype(np.float32)
    rec = np.zeros((n, head_dim + 16), dtype=np.uint8)
    for i in range(n):
        if s[i] == 0:
            continue
        q = (kv32[i] / s[i]).astype(np.float32)
        rec[i, :head_dim] = e4m3_encode(q.astype(np.float64))
        rec[i, head_dim:head_dim + 4] = np.array([s[i]], dtype=np.float32).view(np.uint8)
    return rec


def record_value(rec: np.ndarray, head_dim: int) -> np.ndarray:
    """Dequantized latent of KV records [n, RECORD] -> float64 [n, D] (codes times scale)."""
    rec = np.asarray(rec, dtype=np.uint8)
    s = rec[:, head_dim:head_dim + 4].copy().view(np.float32).astype(np.float64)
    return e4m3_value(rec[:, :head_dim]) * s


def slot_of(pos: int, req: int, block_table: np.ndarray, B: int) -> int:
    """Physical slot of a request's token position through the block table."""
    return int(block_table[req, pos // B]) * B + pos % B


def key_slots(d, r: int, kv) -> list:
    """Slots a row attends to.  Causal mode: positions [max(0, p-W+1), p] of the row's
    request (the row itself and earlier drafts of the step included).  Index-table mode
    (draft layers): the caller's row of physical slots, -1 entries skipped."""
    p = int(kv.positions[r])
    if d.swa_width > 0:
        row = kv.key_table[r]
        return [int(s) for s in row if s >= 0]
    req = int(kv.row_req[r])
    return [slot_of(t, req, kv.block_table, d.kv_block) for t in range(max(0, p - d.window + 1), p + 1)]


def attention_softmax(q: np.ndarray, kval: np.ndarray, scale: float) -> np.ndarray:
    """Exact attention of query vectors q [H, D] over keys = values kval [n, D]:
    softmax(q . k / sqrt(D)) weighted sum of the same latent vectors (one latent KV head
    shared by all heads)."""
    sc = (q @ kval.T) * scale
    mx = sc.max(axis=1, keepdims=True)
    p = np.exp(sc - mx)
    return (p @ kval) / p.sum(axis=1, keepdims=True)


def attention_split(q: np.ndarray, kval: np.ndarray, scale: float, n_split: int) -> np.ndarray:
    """The same attention computed in n_split chunks of keys, each giving a partial
    (max m_s, sum l_s = sum exp(sc - m_s), output o_s = sum exp(sc - m_s) v), merged by the
    log-sum-exp combine: m = max m_s, l = sum l_s e^(m_s - m), o = sum o_s e^(m_s - m) / l."""
    n = kval.shape[0]
    bounds = np.linspace(0, n, n_split + 1).astype(int)
    parts = []
    for s in range(n_split):
        a, b = bounds[s], bounds[s + 1]
        if a == b:
            continue
        sc = (q @ kval[a:b].T) * scale
        m = sc.max(axis=1)
        p = np.exp(sc - m[:, None])
        parts.append((m, p.sum(axis=1), p @ kval[a:b]))
    m = np.max([pt[0] for pt in parts], axis=0)
    l = sum(pt[1] * np.exp(pt[0] - m) for pt in parts)
    o = sum(pt[2] * np.exp(pt[0] - m)[:, None] for pt in parts)
    return o / l[:, None]


def swiglu_clamp(g: np.ndarray, u: np.ndarray, limit: float) -> np.ndarray:
    """Clamped SwiGLU: gate clamped above at `limit`, up clamped to [-limit, limit],
    z = g' * sigmoid(g') * u'."""
    g = np.minimum(np.asarray(g, dtype=np.float64), limit)
    u = np.clip(np.asarray(u, dtype=np.float64), -limit, limit)
    return g / (1.0 + np.exp(-g)) * u


def router_topk(logits: np.ndarray, k: int):
    """Per row: the k largest float32 logits (ties to the lower expert id), emitted in
    descending order, with weights softmax-renormalized over the selected k:
    w_i = e^(l_i - l_max) / sum_j e^(l_j - l_max).  Returns ids int32 [M, k], w float32."""
    M, E = logits.shape
    ids = np.zeros((M, k), dtype=np.int32)
    w = np.zeros((M, k), dtype=np.float64)
    for m in range(M):
        order = np.lexsort((np.arange(E), -logits[m]))[:k]
        ids[m] = order
        sel = logits[m, order].astype(np.float64)
        e = np.exp(sel - sel.max())
        w[m] = e / e.sum()
    return ids, f32(w)


# ----------------------------------------------------------------------------- halves

def attn_half(d, lw: dict, x_bits: np.ndarray, kv, cache: np.ndarray) -> dict:
    """Attention half of one layer on rows x (bf16 codes).  Writes this step's KV records
    into `cache` (a copy owned by the caller) before any row attends, then returns the
    branch output a (float32) and the intermediates.  Pad rows (position -1) get no KV
    write and a zero branch output."""
    M = x_bits.shape[0]
    qr, D, H = d.q_rank, d.head_dim, d.n_heads
    x = bf16_value(x_bits)
    live = kv.positions >= 0
    xn = rmsnorm(x, lw["attn_norm"], d.norm_eps)
    qkv = mxfp8_linear(xn, lw["wqkv"], lw["wqkv_s"])
    q_lat, kv_lat = qkv[:, :qr], qkv[:, qr:qr + D]
    q_n = rmsnorm(q_lat, lw["q_norm"], d.norm_eps)
    kv_n = rmsnorm(kv_lat, lw["kv_norm"], d.norm_eps)
    recs = kv_record(kv_n, D)
    for r in range(M):
        if live[r]:
            s = slot_of(int(kv.positions[r]), int(kv.row_req[r]), kv.block_table, d.kv_block)
            cache[s // d.kv_block, s % d.kv_block] = recs[r]
    q = mxfp8_linear(q_n, lw["wq_b"], lw["wq_b_s"]).reshape(M, H, D)
    o = np.zeros((M, H, D))
    scale = 1.0 / np.sqrt(D)
    for r in range(M):
        if not live[r]:
            continue
        slots = key_slots(d, r, kv)
        kval = record_value(cache[[s // d.kv_block for s in slots], [s % d.kv_block for s in slots]], D)
        o[r] = attention_softmax(q[r], kval, scale)
    o = f32(o).reshape(M, H * D)
    t = mxfp8_linear(o, lw["wo_a"], lw["wo_a_s"])
    a = mxfp8_linear(t, lw["wo_b"], lw["wo_b_s"])
    a[~live] = 0.0
    return dict(a=a, q=q, o=o, t=t, q_lat=q_lat, kv_n=kv_n, records=recs)


def mxq(v: np.ndarray) -> np.ndarray:
    """MXFP8 quantization per 1x32 block along the last axis, returned as the dequantized
    values (e4m3 code times the block's 2^(X-127)): the activation side of an MXFP8
    linear."""
    return mx_e4m3_dequant_act(*mx_e4m3_quantize(v))


def moe_half(d, lw: dict, u_bits: np.ndarray, live: np.ndarray | None = None) -> dict:
    """MoE on rows u (bf16 codes, already normalized): f32 router logits, top-k with
    renormalized weights, the FP8 shared expert (128x128 f32 block scales, bf16 input),
    the selected MXFP4 experts, and the float32 combine m = shared + sum_j w_j y_j in
    fixed order (shared first, then slots in emission order).  Rows with live False are
    not routed (ids -1, weights 0, m = 0).

    With d.expert_a8 set (the "a8w4 MoE" of the pages' deployments: "Mono decode layer
    for DeepSeek-V4.1-Flash on MI355X", vLLM PR 60397, Test Plan) the routed experts take
    MXFP8 activations: the gate/up input is MXq(u) and the down input MXq(z), each
    quantized per 1x32 block from its bf16 value (u and z stay bf16, R6 and R7).  The
    router and the shared expert keep the bf16 u."""
    M = u_bits.shape[0]
    I, Is = d.inter, d.shared_inter
    a8 = bool(getattr(d, "expert_a8", 0))
    if live is None:
        live = np.ones(M, dtype=bool)
    u = bf16_value(u_bits)
    u_ex = mxq(u) if a8 else u
    logits = f32(u @ np.asarray(lw["w_router"], dtype=np.float64).T)
    ids, w = router_topk(logits, d.top_k)
    ids[~live] = -1
    w[~live] = 0.0
    gu = f32(gemv_fp8b128(lw["sh_w13"], lw["sh_w13_s"], u))
    z_sh = bf16_round(swiglu_clamp(gu[:, :Is], gu[:, Is:], d.swiglu_limit))
    ys = f32(gemv_fp8b128(lw["sh_wd"], lw["sh_wd_s"], z_sh))
    y = np.zeros((M, d.top_k, d.hidden))
    # each selected expert once, on all (row, slot) pairs that chose it
    pairs = {}
    for m in range(M):
        if live[m]:
            for j in range(d.top_k):
                pairs.setdefault(int(ids[m, j]), []).append((m, j))
    for e, pl in sorted(pairs.items()):
        rows = [m for m, _ in pl]
        gu_e = f32(gemv_mxfp4(lw["ex_w13"][e], lw["ex_w13_s"][e], u_ex[rows]))
        z = bf16_round(swiglu_clamp(gu_e[:, :I], gu_e[:, I:], d.swiglu_limit))
        ye = f32(gemv_mxfp4(lw["ex_wd"][e], lw["ex_wd_s"][e], mxq(z) if a8 else z))
        for (m, j), yy in zip(pl, ye):
            y[m, j] = yy
    mo = ys.copy()
    for j in range(d.top_k):
        mo = mo + w[:, j:j + 1] * y[:, j]
    mo = f32(mo)
    mo[~live] = 0.0
    return dict(m=mo, ids=ids, w=w, logits=logits, ys=ys, y=y, z_sh=z_sh, gu_sh=gu,
                n_distinct=len(pairs))


# ----------------------------------------------------------------------------- entry points

def moe_step(d, lw: dict, u_bits: np.ndarray) -> dict:
    """MoE stage on its own: branch output bf16(m) (R9), ids and weights."""
    r = moe_half(d, lw, u_bits)
    r["moe_out"] = bf16_encode(r["m"])
    return r


def attn_step(d, lw: dict, x_bits: np.ndarray, kv, cache: np.ndarray) -> dict:
    """Attention half on its own: branch output bf16(a), no residual add."""
    r = attn_half(d, lw, x_bits, kv, cache)
    r["attn_out"] = bf16_encode(r["a"])
    return r


def layer_step(d, lw: dict, x_bits: np.ndarray, kv, cache: np.ndarray) -> dict:
    """One decode layer, pre-norm residual: hres = bf16(x + Attn(RMSNorm(x))) (R5),
    u = bf16(RMSNorm_ffn(hres)) (R6), out = bf16(f32(hres) + MoE(u)) (R9).
    Pad rows produce zero rows in every output."""
    live = kv.positions >= 0
    at = attn_half(d, lw, x_bits, kv, cache)
    x = bf16_value(x_bits)
    hres_bits = bf16_encode(x + at["a"])
    hres = bf16_value(hres_bits)
    u_bits = bf16_encode(rmsnorm(hres, lw["ffn_norm"], d.norm_eps))
    mo = moe_half(d, lw, u_bits, live)
    out_bits = bf16_encode(hres + mo["m"])
    z = np.uint16(0)
    for arr in (hres_bits, u_bits, out_bits):
        arr[~live] = z
    attn_out = bf16_encode(at["a"])
    moe_out = bf16_encode(mo["m"])
    return dict(out=out_bits, attn_out=attn_out, hres=hres_bits, moe_in=u_bits, moe_out=moe_out,
                ids=mo["ids"], w=mo["w"], logits=mo["logits"], n_distinct=mo["n_distinct"],
                attn=at, moe=mo)


def decode_step(d, layers: list, x_bits: np.ndarray, kv, caches: list, on_layer=None) -> dict:
    """n_layers chained layers (the draft model runs three): layer l's output is layer
    l+1's input; each layer has its own weights and its own cache, the tables are
    shared.  `caches` are updated in place (pass copies).  Returns the last layer's
    outputs and every layer's results.  `on_layer(l)`, when given, is called before
    layer l starts (progress reporting only)."""
    per = []
    x = x_bits
    for l in range(d.n_layers):
        if on_layer is not None:
            on_layer(l)
        r = layer_step(d, layers[l], x, kv, caches[l])
        per.append(r)
        x = r["out"]
    res = dict(per[-1])
    res["layers"] = per
    return res


def topk_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """Per row: gap between the k-th and (k+1)-th largest logit (inf when k = E)."""
    s = -np.sort(-np.asarray(logits, dtype=np.float64), axis=1)
    if k >= s.shape[1]:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]
