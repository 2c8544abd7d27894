"""The decode launch under HIP-graph capture, and a race stress of its replays.

Once a width has run eagerly on a handle (that first call allocates the width's
scratch), a decode step is one kernel launch with its arguments passed by value: no
allocation, no copy, no synchronous call.  A caller can therefore capture it in a HIP
graph.  The grid barrier's counters only ever grow and each launch reads its starting
value on entry, so replays need no reset.  Two widths on one handle use scratch of
their own, and launches on one stream never overlap.

Each test captures launches of two widths alternating on one handle, each width with
its own cache, positions and input buffer.  Every launch writes an output slot and a set
of intermediate taps of its own: attention output, residual, MoE input and output,
expert ids and weights, router logits, every layer's ids.  Between replays the test does
eager work of its own: it fills every buffer with a sentinel, switches the inputs
between two sets, and synchronizes.  After every replay each launch's buffers must equal
the eager launch on the same inputs bit for bit, and at the end the caches must hold what
the eager launches wrote.

  full-size layer (hidden 4096, top-6 of 128), widths 48 and 6:
      a graph of 50 (48, 6) pairs replayed 1000 times = 100,000 launches; the eager
      launches they are compared with are themselves checked against the oracle first,
      at the per-layer parity bars, on both input sets (seeds from tests/golden/seeds.json
      whose top-k gap holds on both)
  two chained draft layers (index-table mode) at small dims, widths 13 and 5:
      a graph of 8 pairs replayed 40 times
"""
import numpy as np
import pytest

from moe_transformer_layer_amd import synth
from parity import Errors, GAP_MIN, check_layer, load_seeds, min_gap

pytestmark = [pytest.mark.gpu]

SENTINEL = 0x7FC1FFFF  # fill of the 32-bit buffers (a NaN; no id); the bf16 ones take -1 (0xFFFF, a NaN)


def _say(msg):
    print(f"[graph] {msg}", flush=True)


@pytest.fixture(scope="module")
def dsl(gpu):
    from moe_transformer_layer_amd import dsl as d
    d.lib()
    return d


class _Side:
    """One width on the shared handle: its own cache, tables, inputs, and for every launch
    in the graph an output slot and a set of intermediate taps of its own."""

    def __init__(self, dsl, torch, name, layers, weights, layout, seed, pairs):
        self.dsl, self.torch = dsl, torch
        case = synth.make_case(name, seed, layers=layers, **layout)
        self.case = case
        d = case.dims
        self.M = M = case.M
        self.dev = dsl.LayerOnDevice(case, weights=weights)
        rng = np.random.default_rng([seed, 77])
        self.inputs = [torch.from_numpy(case.x.view(np.int16)).cuda(),
                       torch.from_numpy(synth.gen_x(d, rng, M).view(np.int16)).cuda()]
        self.x = torch.empty_like(self.inputs[0])
        i16, i32 = torch.int16, torch.int32
        # every buffer as raw integers: bit-for-bit compares, sentinel fills
        self.shapes = dict(out=((M, d.hidden), i16), attn_out=((M, d.hidden), i16), hres=((M, d.hidden), i16),
                           moe_in=((M, d.hidden), i16), moe_out=((M, d.hidden), i16), ids=((M, d.top_k), i32),
                           w=((M, d.top_k), i32), logits=((M, d.n_experts), i32),
                           layer_ids=((d.n_layers, M, d.top_k), i32))
        self.slots = {k: torch.empty((pairs, *shp), dtype=dt, device="cuda") for k, (shp, dt) in self.shapes.items()}
        self.ref = []

    def launch(self, bufs):
        dsl = self.dsl
        taps = dsl.Taps(*(bufs[k].data_ptr() for k in ("attn_out", "hres", "moe_in", "moe_out", "ids", "w",
                                                         "logits", "layer_ids")))
        dsl.dsl_decode_step(self.dev.handle, self.x.data_ptr(), self.M, self.dev.kv_structs,
                            self.dev.positions.data_ptr(), bufs["out"].data_ptr(), taps,
                            self.torch.cuda.current_stream().cuda_stream)

    def slot(self, j):
        return {k: v[j] for k, v in self.slots.items()}

    def select(self, i):
        self.x.copy_(self.inputs[i])

    def mismatches(self, i):
        """Slots whose buffers differ from the eager launch on input set i, per buffer."""
        bad = {}
        for k, v in self.slots.items():
            same = (v == self.ref[i][k]).flatten(1).all(dim=1)
            if not bool(same.all()):
                bad[k] = [j for j in range(v.shape[0]) if not bool(same[j])][:8]
        return bad


def _oracle_check(dsl, side, layers, caches_after):
    """The eager launches the replays are compared with, against the oracle on the same
    inputs, at the per-layer parity bars (one-layer cases): input set i's outputs and the
    cache as that launch left it."""
    from oracle import layer as OL
    case = side.case
    d = case.dims
    live = case.kv.positions >= 0
    er = Errors()
    for i in range(2):
        x = side.inputs[i].cpu().numpy().view(np.uint16)
        caches = [c.copy() for c in case.kv.cache]
        _say(f"oracle: width {side.M}, input set {i}")
        want = OL.decode_step(d, layers, x, case.kv, caches)
        g = min_gap(d, want["layers"], live)
        assert g >= GAP_MIN, f"width {side.M} input set {i}: top-k gap {g} below {GAP_MIN}"
        ref = {k: v.cpu().numpy() for k, v in side.ref[i].items()}
        got = dict(ref)
        for k in ("out", "attn_out", "hres", "moe_in", "moe_out"):
            got[k] = ref[k].view(np.uint16)
        got["w"] = ref["w"].view(np.float32)
        got["logits"] = ref["logits"].view(np.float32)
        check_layer(er, d, layers[0], got, want, live, caches_after[i][0].cpu().numpy(), caches[0],
                    case.kv.cache[0], tag=f"M{side.M}.set{i}")
    er.raise_any(f"eager reference, width {side.M}", _say)


def _stress(dsl, name, layouts, pairs, replays, wseed=5, seeds=None, oracle=False):
    """layouts: one make_case row layout per width (requests x rows per request + pad rows).
    seeds: each width's input seed (default 100, 101, ...).  oracle: check the eager
    launches against the oracle first (one-layer workloads)."""
    import torch
    layers = synth.make_weights(name, wseed)
    weights = dsl.DeviceWeights(synth.CONFIGS[name], layers)
    seeds = seeds or [100 + j for j in range(len(layouts))]
    sides = [_Side(dsl, torch, name, layers, weights, lay, seeds[j], pairs) for j, lay in enumerate(layouts)]
    widths = tuple(s.M for s in sides)
    # eager runs: each width once per input set (the first call allocates the width's scratch)
    caches_after = [[] for _ in sides]
    for i in range(2):
        for j, s in enumerate(sides):
            s.select(i)
            bufs = {k: torch.full(shp, SENTINEL, dtype=dt, device="cuda") if dt == torch.int32
                    else torch.full(shp, -1, dtype=dt, device="cuda") for k, (shp, dt) in s.shapes.items()}
            s.launch(bufs)
            s.ref.append(bufs)
            torch.cuda.synchronize()
            caches_after[j].append([c.clone() for c in s.dev.caches])
    dsl._check(dsl.dsl_layer_health(weights.handle))
    caches_ref = [c[1] for c in caches_after]  # after input set 1
    if oracle:
        for j, s in enumerate(sides):
            _oracle_check(dsl, s, layers, caches_after[j])
    for s in sides:
        assert not torch.equal(s.ref[0]["out"], s.ref[1]["out"])
        for i in range(2):
            for k, v in s.ref[i].items():
                assert not (v == (SENTINEL if v.dtype == torch.int32 else -1)).all(), f"eager launch left {k} unwritten"

    graph = torch.cuda.CUDAGraph()
    capture = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=capture):
        for j in range(pairs):
            for s in sides:
                s.launch(s.slot(j))
    _say(f"{name}: captured {pairs} x {widths}; {replays} replays = {replays * pairs * len(sides)} launches, "
         f"{len(sides[0].slots)} buffers compared per launch")

    bad = []
    for r in range(replays):
        i = r % 2
        for s in sides:
            for v in s.slots.values():
                v.fill_(SENTINEL if v.dtype == torch.int32 else -1)
            s.select(i)
        graph.replay()
        torch.cuda.synchronize()
        for s in sides:
            m = s.mismatches(i)
            if m:
                bad.append((r, s.M, m))
        if bad:
            break
        if (r + 1) % 200 == 0:
            _say(f"{name}: {r + 1} replays bit-exact")
    dsl._check(dsl.dsl_layer_health(weights.handle))
    assert not bad, f"replays that differ from the eager launch (replay, width, buffer: first slots): {bad[:4]}"
    assert (replays - 1) % 2 == 1, "the last replay must use input set 1 for the cache check"
    for s, refs in zip(sides, caches_ref):
        for c, cr in zip(s.dev.caches, refs):
            assert torch.equal(c, cr), f"width {s.M}: cache differs from the eager launches'"
    del graph
    for s in sides:
        s.dev.close()
    weights.close()


def test_graph_draft_small(dsl):
    _stress(dsl, "mid_draft", (dict(n_req=2, rows_per_req=6, n_pad=1), dict(n_req=1, rows_per_req=5)),
            pairs=8, replays=40)


@pytest.mark.timeout(900)
def test_graph_race_stress_full(dsl):
    sd = load_seeds()
    seeds = [sd[k]["seed"] for k in ("stress_m48", "stress_m6")]
    assert all(sd[k]["weights_seed"] == 5 for k in ("stress_m48", "stress_m6"))
    _stress(dsl, "layer48", (dict(M=48), dict(M=6)), pairs=50, replays=1000, seeds=seeds, oracle=True)
