"""Seeded synthetic inputs for the decode layer.

This module only draws random numbers and lays them out in the stored formats
the layer reads (e4m3 / e2m1 codes, E8M0 and f32 scales, bf16 activations, a
block-paged KV cache with its tables).  It holds none of the layer's
arithmetic: weight and KV codes are drawn directly (torch's own float8 cast
turns uniform draws into e4m3 codes), never produced by the layer's
quantization rules.  Both the CPU oracle and the HIP path are fed from here.

Shapes follow the workloads the pages describe: DeepSeek-V4.1-Flash decode
steps of up to 48 rows (8 requests x (1 + 5 DSpark drafts)), a sliding window
of 128 over fp8 KV records in blocks of 128, 128 routed experts with top-6
(target) or top-3 (draft, 192-wide non-causal index rows).  Sources: "Mono
decode layer for DeepSeek-V4.1-Flash on MI355X" (vLLM PR 60397), Scope and
Design; "Mono decode for the DSpark draft layers" (vLLM PR 62131), Details.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np
import torch

E4M3_MAX_DRAW = 448.0


@dataclass(frozen=True)
class Dims:
    hidden: int
    n_heads: int
    head_dim: int
    q_rank: int
    o_rank: int
    window: int
    swa_width: int  # 0 = causal window mode; >0 = caller key-table mode
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int
    kv_block: int
    max_rows: int
    n_layers: int = 1
    expert_a8: int = 0  # 1: the routed experts take MXFP8 activations (A8W4); 2: the same on the scaled MX instruction
    norm_eps: float = 1e-6
    swiglu_limit: float = 7.0

    @property
    def record(self) -> int:
        """Bytes of one KV record: head_dim e4m3 codes, f32 scale, 12 pad bytes."""
        return self.head_dim + 16

    def replace(self, **kw) -> "Dims":
        return dataclasses.replace(self, **kw)


# The five workloads, plus a small multi-tile shape for fast parity runs.
BIG = dict(hidden=4096, n_heads=16, head_dim=512, q_rank=1024, o_rank=1024,
           window=128, n_experts=128, inter=2048, shared_inter=2048, kv_block=128)
CONFIGS = {
    # tiny layer, M = 1, top-2 of 8
    "tiny": Dims(hidden=256, n_heads=4, head_dim=64, q_rank=128, o_rank=128, window=16,
                 swa_width=0, n_experts=8, top_k=2, inter=128, shared_inter=128,
                 kv_block=16, max_rows=1),
    # MoE stage only, M = 6, top-3 of 128
    "moe6": Dims(swa_width=0, top_k=3, max_rows=6, **BIG),
    # attention half only, M = 48 (8 requests x 6)
    "attn48": Dims(swa_width=0, top_k=6, max_rows=48, **BIG),
    # full standard layer, top-6 of 128 (M = 48; the M = 6 variant is the same dims)
    "layer48": Dims(swa_width=0, top_k=6, max_rows=48, **BIG),
    # draft shape: three chained layers, 192-wide non-causal index rows, top-3
    "draft": Dims(swa_width=192, top_k=3, max_rows=48, n_layers=3, **BIG),
    # small but multi-tile: several GEMV tiles, split-K chunks, attention splits
    # and expert tasks, with ragged row counts
    "mid": Dims(hidden=512, n_heads=4, head_dim=128, q_rank=256, o_rank=256, window=48,
                swa_width=0, n_experts=16, top_k=4, inter=256, shared_inter=256,
                kv_block=16, max_rows=13),
    "mid_draft": Dims(hidden=512, n_heads=4, head_dim=128, q_rank=256, o_rank=256, window=48,
                      swa_width=64, n_experts=16, top_k=3, inter=256, shared_inter=256,
                      kv_block=16, max_rows=13, n_layers=2),
}
# The same workloads with MXFP8 activations into the MXFP4 experts (A8W4); each draws
# the same weights and inputs as the workload it is named after.
# (_a8mx: the same A8W4 layer on the scaled MX matrix instruction; the same draws.)
for _n in ("moe6", "layer48", "mid"):
    CONFIGS[_n + "_a8"] = CONFIGS[_n].replace(expert_a8=1)
    CONFIGS[_n + "_a8mx"] = CONFIGS[_n].replace(expert_a8=2)


def base_name(name: str) -> str:
    """The workload whose draws a configuration shares (an A8W4 variant's base)."""
    for suffix in ("_a8mx", "_a8"):
        if name.endswith(suffix):
            return name[: -len(suffix)]
    return name


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round f32 draws to bf16 (torch's cast) and return the raw 16-bit codes."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _e4m3_codes(x: np.ndarray) -> np.ndarray:
    """e4m3 codes of draws already inside +-448 (torch's float8_e4m3fn cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def _e8m0_for(rms: float, elem_rms: float, shape, rng) -> np.ndarray:
    """E8M0 bytes whose power of two brings codes of rms `elem_rms` to about `rms`,
    jittered by -1/0/+1 per block so blocks carry distinct, nonzero scales."""
    base = 127 + int(round(np.log2(rms / elem_rms)))
    j = rng.integers(-1, 2, size=shape, dtype=np.int8)
    return (j + np.int8(base - 128)).astype(np.uint8) + np.uint8(128)


def _uniform_rms(a: float) -> float:
    return a / np.sqrt(3.0)


# rms of e2m1 magnitudes drawn uniformly over the 16 codes
_E2M1_CODE_RMS = float(np.sqrt(np.mean(np.array([0, .5, 1, 1.5, 2, 3, 4, 6]) ** 2)))


def gen_mxfp8_weight(n: int, k: int, amp: float, rng) -> tuple[np.ndarray, np.ndarray]:
    """Row-major e4m3 [n, k] with one E8M0 per 32x32 tile [n/32, k/32].
    Values are about U(+-amp): codes from U(+-448), tile scales near amp/448."""
    codes = _e4m3_codes(rng.uniform(-E4M3_MAX_DRAW, E4M3_MAX_DRAW, size=(n, k)).astype(np.float32))
    base = 127 + int(round(np.log2(amp / E4M3_MAX_DRAW)))
    scales = (base + rng.integers(-1, 2, size=(n // 32, k // 32), dtype=np.int8)).astype(np.uint8)
    return codes, scales


def gen_fp8_block_weight(n: int, k: int, amp: float, rng) -> tuple[np.ndarray, np.ndarray]:
    """Row-major e4m3 [n, k] with one f32 scale per 128x128 block [n/128, k/128]."""
    codes = _e4m3_codes(rng.uniform(-E4M3_MAX_DRAW, E4M3_MAX_DRAW, size=(n, k)).astype(np.float32))
    scales = (amp / E4M3_MAX_DRAW * rng.uniform(0.8, 1.25, size=(n // 128, k // 128))).astype(np.float32)
    return codes, scales


def gen_mxfp4_experts(e: int, n: int, k: int, amp: float, rng) -> tuple[np.ndarray, np.ndarray]:
    """e2m1 nibbles [e, n, k/2] (low nibble = even k) with one E8M0 per 32 along k
    [e, n, k/32].  Nibbles are uniform over all 16 codes."""
    packed = rng.integers(0, 256, size=(e, n, k // 2), dtype=np.uint8)
    scales = _e8m0_for(_uniform_rms(amp), _E2M1_CODE_RMS, (e, n, k // 32), rng)
    return packed, scales


def gen_layer_weights(d: Dims, rng, attn_amp: float | None = None, gate_gain: float = 1.0) -> dict:
    """One layer's weights.  Input-side projections are about U(+-1.5/sqrt(K)), the
    projections back into the residual (wo_b, expert and shared down) U(+-0.5/sqrt(K)),
    so both branches stay near 0.3 rms and layer outputs stay below 4.  gate_gain scales
    the routed and shared gate/up weights (large values drive the SwiGLU clamp)."""
    h, qr, orr, H, D = d.hidden, d.q_rank, d.o_rank, d.n_heads, d.head_dim
    E, I, Is = d.n_experts, d.inter, d.shared_inter
    w = {}
    for name, n in (("attn_norm", h), ("q_norm", qr), ("kv_norm", D), ("ffn_norm", h)):
        w[name] = rng.uniform(0.9, 1.1, size=n).astype(np.float32)

    def amp(k):
        return attn_amp if attn_amp is not None else 1.5 / np.sqrt(k)

    w["wqkv"], w["wqkv_s"] = gen_mxfp8_weight(qr + D, h, amp(h), rng)
    w["wq_b"], w["wq_b_s"] = gen_mxfp8_weight(H * D, qr, amp(qr), rng)
    w["wo_a"], w["wo_a_s"] = gen_mxfp8_weight(orr, H * D, amp(H * D), rng)
    w["wo_b"], w["wo_b_s"] = gen_mxfp8_weight(h, orr, amp(orr) / 3.0, rng)
    w["w_router"] = rng.normal(0.0, 0.02, size=(E, h)).astype(np.float32)
    w["sh_w13"], w["sh_w13_s"] = gen_fp8_block_weight(2 * Is, h, gate_gain * 1.5 / np.sqrt(h), rng)
    w["sh_wd"], w["sh_wd_s"] = gen_fp8_block_weight(h, Is, 0.5 / np.sqrt(Is), rng)
    w["ex_w13"], w["ex_w13_s"] = gen_mxfp4_experts(E, 2 * I, h, gate_gain * 1.5 / np.sqrt(h), rng)
    w["ex_wd"], w["ex_wd_s"] = gen_mxfp4_experts(E, h, I, 0.5 / np.sqrt(I), rng)
    return w


@dataclass
class KVState:
    """A block-paged fp8 KV cache and its tables (shared tables across layers)."""
    cache: list  # per layer: uint8 [n_blocks, B, RECORD] (block stride = B*RECORD)
    block_table: np.ndarray  # int32 [n_req, max_blocks]
    row_req: np.ndarray  # int32 [M]
    positions: np.ndarray  # int32 [M], -1 = pad row
    key_table: np.ndarray | None  # int32 [M, swa_width] physical slots or -1
    contexts: np.ndarray  # int32 [n_req] tokens already cached per request
    meta: dict = field(default_factory=dict)


def _random_records(n: int, d: Dims, rng) -> np.ndarray:
    """n KV records: e4m3 codes of N(0,1)*100 (clipped to +-448), f32 scale U(0.008, 0.012),
    12 zero pad bytes."""
    rec = np.zeros((n, d.record), dtype=np.uint8)
    rec[:, : d.head_dim] = _e4m3_codes(np.clip(rng.normal(0, 100.0, size=(n, d.head_dim)), -448, 448).astype(np.float32))
    rec[:, d.head_dim: d.head_dim + 4] = rng.uniform(0.008, 0.012, size=(n, 1)).astype(np.float32).view(np.uint8)
    return rec


def gen_kv(d: Dims, rng, n_req: int, rows_per_req: int, ctx_lo: int, ctx_hi: int,
           n_pad: int = 0, fill_all: bool = False) -> KVState:
    """Paged caches for n_req requests with contexts ~ U[ctx_lo, ctx_hi] already cached,
    and rows_per_req new rows per request at the next positions (1 + drafts).
    Physical blocks are a random permutation.  Records are filled for every position a
    window can reach (all of them when fill_all); other bytes stay zero.  n_pad trailing
    rows are pad rows (position -1)."""
    B, W = d.kv_block, d.window
    ctx = rng.integers(ctx_lo, ctx_hi + 1, size=n_req).astype(np.int32)
    need = ctx + rows_per_req
    nblk_req = (need + B - 1) // B
    max_blocks = int(nblk_req.max())
    total = int(nblk_req.sum())
    perm = rng.permutation(total).astype(np.int32)
    bt = np.full((n_req, max_blocks), -1, dtype=np.int32)
    o = 0
    for r in range(n_req):
        bt[r, : nblk_req[r]] = perm[o: o + nblk_req[r]]
        o += nblk_req[r]
    caches = []
    reach = max(W, d.swa_width) + rows_per_req
    for _ in range(d.n_layers):
        cache = np.zeros((total, B, d.record), dtype=np.uint8)
        for r in range(n_req):
            lo = 0 if fill_all else max(0, int(ctx[r]) - reach)
            pos = np.arange(lo, int(ctx[r]))
            if len(pos) == 0:
                continue
            recs = _random_records(len(pos), d, rng)
            cache[bt[r, pos // B], pos % B] = recs
        caches.append(cache)
    M = n_req * rows_per_req + n_pad
    row_req = np.zeros(M, dtype=np.int32)
    positions = np.full(M, -1, dtype=np.int32)
    for r in range(n_req):
        for j in range(rows_per_req):
            row_req[r * rows_per_req + j] = r
            positions[r * rows_per_req + j] = ctx[r] + j
    key_table = None
    if d.swa_width > 0:
        # Draft rows: the request's W context positions before the block, then every
        # position of the block (non-causal), -1 padded to swa_width.
        key_table = np.full((M, d.swa_width), -1, dtype=np.int32)
        for i in range(n_req * rows_per_req):
            r = row_req[i]
            p0 = int(ctx[r])
            pos = list(range(max(0, p0 - W), p0)) + list(range(p0, p0 + rows_per_req))
            assert len(pos) <= d.swa_width
            key_table[i, : len(pos)] = [int(bt[r, p // B]) * B + p % B for p in pos]
    return KVState(caches, bt, row_req, positions, key_table, ctx)


def gen_x(d: Dims, rng, M: int, truncate: float | None = 2.5) -> np.ndarray:
    """bf16 codes [M, hidden] of N(0,1) draws, re-drawn beyond |x| > truncate."""
    x = rng.normal(0, 1, size=(M, d.hidden))
    if truncate is not None:
        bad = np.abs(x) > truncate
        while bad.any():
            x[bad] = rng.normal(0, 1, size=int(bad.sum()))
            bad = np.abs(x) > truncate
    return _bf16_bits(x.astype(np.float32))


@dataclass
class Case:
    dims: Dims
    layers: list  # per layer weight dicts
    kv: KVState | None
    x: np.ndarray  # bf16 codes [M, hidden] (the MoE input u for MoE-only cases)
    M: int
    seed: int


def make_weights(name: str, weights_seed: int, n_layers: int | None = None, gate_gain: float = 1.0) -> list:
    """The layers' weights of workload `name`, drawn from their own seed."""
    d = CONFIGS[name]
    if n_layers is not None:
        d = d.replace(n_layers=n_layers)
    rng = np.random.default_rng([weights_seed, 0])
    return [gen_layer_weights(d, rng, attn_amp=0.05 if base_name(name) == "tiny" else None, gate_gain=gate_gain)
            for _ in range(d.n_layers)]


def make_case(name: str, seed: int, M: int | None = None, n_pad: int = 0,
              n_req: int | None = None, rows_per_req: int | None = None,
              n_layers: int | None = None, ctx: tuple | None = None,
              gate_gain: float = 1.0, weights_seed: int | None = None,
              layers: list | None = None) -> Case:
    """Draw one workload.  name picks the dims; M, n_req, rows_per_req override the row
    layout (rows = n_req * rows_per_req + n_pad).  Weights come from weights_seed
    (default: seed) unless `layers` passes weights already drawn; activations, caches
    and tables come from seed."""
    d = CONFIGS[name]
    if n_layers is not None:
        d = d.replace(n_layers=n_layers)
    if layers is None:
        layers = make_weights(name, seed if weights_seed is None else weights_seed, n_layers, gate_gain)
    assert len(layers) == d.n_layers
    rng = np.random.default_rng([seed, 1])
    name = base_name(name)
    if name == "moe6":
        M = M or 6
        x = gen_x(d, rng, M, truncate=None)
        return Case(d, layers, None, x, M, seed)
    if name == "tiny":
        kv = gen_kv(d, rng, 1, 1, 16, 63, fill_all=True)
        x = gen_x(d, rng, 1, truncate=None)
        return Case(d, layers, kv, x, 1, seed)
    if name in ("mid", "mid_draft"):
        n_req = n_req or 2
        rows_per_req = rows_per_req or 6
        lo, hi = ctx or (0, 200)
    else:
        if M is not None and n_req is None:
            n_req = max(1, M // 6)
            rows_per_req = rows_per_req or (6 if M >= 6 else M)
        n_req = n_req or 8
        rows_per_req = rows_per_req or 6
        lo, hi = ctx or (1024, 65536)
    kv = gen_kv(d, rng, n_req, rows_per_req, lo, hi, n_pad=n_pad)
    M = n_req * rows_per_req + n_pad
    x = gen_x(d, rng, M)
    return Case(d, layers, kv, x, M, seed)
