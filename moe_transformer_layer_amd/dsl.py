"""ctypes binding of the C ABI in include/dsl.h (libdsl.so, built in-tree).

Argument marshalling only: every step of the layer runs in the HIP kernels.
The functions keep the C names; `LayerOnDevice` uploads one set of weights,
KV caches and tables (numpy arrays in the stored formats) into device memory
with torch and holds the handle.  There is no CPU fallback: without the built
library every call raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from ctypes import c_float, c_int32, c_int64, c_void_p

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsl.so")

DSL_OK, DSL_EINVAL, DSL_EUNSUPPORTED, DSL_ENOMEM, DSL_EHIP, DSL_EDEVICE = 0, -1, -2, -3, -4, -5
DSL_MAX_ROWS, DSL_MAX_LAYERS = 48, 4


class DslError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dsl error {code}: {msg}")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in ("hidden", "n_heads", "head_dim", "q_rank", "o_rank", "window",
                                       "swa_width", "n_experts", "top_k", "inter", "shared_inter",
                                       "kv_block", "max_rows", "n_layers", "expert_a8")] + \
               [("norm_eps", c_float), ("swiglu_limit", c_float)]


WEIGHT_FIELDS = ("attn_norm", "q_norm", "kv_norm", "ffn_norm", "wqkv", "wqkv_s", "wq_b", "wq_b_s",
                 "wo_a", "wo_a_s", "wo_b", "wo_b_s", "w_router", "sh_w13", "sh_w13_s", "sh_wd",
                 "sh_wd_s", "ex_w13", "ex_w13_s", "ex_wd", "ex_wd_s")


class Weights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in WEIGHT_FIELDS]


class KV(ctypes.Structure):
    _fields_ = [("base", c_void_p), ("block_stride", c_int64), ("n_blocks", c_int64),
                ("block_table", c_void_p), ("max_blocks", c_int32), ("n_req", c_int32),
                ("row_req", c_void_p), ("key_table", c_void_p)]


class Taps(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("attn_out", "hres", "moe_in", "moe_out", "topk_ids", "topk_w",
                                        "logits", "layer_ids")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdsl.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (__graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.dsl_layer_build.argtypes = [P(Dims), P(Weights), P(c_void_p)]
        L.dsl_layer_reserve.argtypes = [c_void_p, c_int32]
        L.dsl_decode_step.argtypes = [c_void_p, c_void_p, c_int32, P(KV), c_void_p, c_void_p, P(Taps), c_void_p]
        L.dsl_decode_step_noalloc.argtypes = [c_void_p, c_void_p, c_int32, P(KV), c_void_p, c_void_p, P(Taps),
                                              c_void_p]
        L.dsl_attn_step.argtypes = [c_void_p, c_void_p, c_int32, P(KV), c_void_p, c_void_p, c_void_p]
        L.dsl_moe_step.argtypes = [c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]
        L.dsl_layer_health.argtypes = [c_void_p]
        L.dsl_layer_grid.argtypes = [c_void_p, P(c_int32), P(c_int32)]
        L.dsl_layer_last_kernel.argtypes = [c_void_p]
        L.dsl_linear_mxfp8.argtypes = [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                       c_void_p]
        L.dsl_linear_mxfp8.restype = c_int32
        L.dsl_linear_workspace_bytes.argtypes = [c_int32, c_int32, c_int32]
        L.dsl_linear_workspace_bytes.restype = c_int64
        L.dsl_layer_set_trace.argtypes = [c_void_p, c_int32]
        L.dsl_layer_read_trace.argtypes = [c_void_p, ctypes.POINTER(ctypes.c_double), c_int32]
        L.dsl_layer_destroy.argtypes = [c_void_p]
        L.dsl_layer_destroy.restype = None
        L.dsl_last_error.restype = ctypes.c_char_p
        for f in ("dsl_layer_build", "dsl_layer_reserve", "dsl_decode_step", "dsl_decode_step_noalloc",
                  "dsl_attn_step", "dsl_moe_step",
                  "dsl_layer_health", "dsl_layer_grid", "dsl_layer_set_trace", "dsl_layer_read_trace",
                  "dsl_layer_last_kernel"):
            getattr(L, f).restype = c_int32
        _lib = L
    return _lib


def _check(rc: int):
    if rc != 0:
        raise DslError(rc, lib().dsl_last_error().decode())


def dims_struct(d) -> Dims:
    return Dims(d.hidden, d.n_heads, d.head_dim, d.q_rank, d.o_rank, d.window, d.swa_width, d.n_experts,
                d.top_k, d.inter, d.shared_inter, d.kv_block, d.max_rows, d.n_layers, d.expert_a8, d.norm_eps,
                d.swiglu_limit)


# --------------------------------------------------------------------------- C calls

def dsl_layer_build(dims: Dims, weights: list) -> c_void_p:
    arr = (Weights * len(weights))(*weights)
    h = c_void_p()
    _check(lib().dsl_layer_build(ctypes.byref(dims), arr, ctypes.byref(h)))
    return h


def dsl_layer_reserve(h, M: int):
    _check(lib().dsl_layer_reserve(h, M))


def dsl_decode_step(h, x: int, M: int, kv: list, positions: int, out: int, taps: Taps | None = None,
                    stream: int = 0):
    arr = (KV * len(kv))(*kv)
    _check(lib().dsl_decode_step(h, x, M, arr, positions, out, ctypes.byref(taps) if taps else None, stream))


def dsl_decode_step_noalloc(h, x: int, M: int, kv: list, positions: int, out: int, taps: Taps | None = None,
                            stream: int = 0):
    arr = (KV * len(kv))(*kv)
    _check(lib().dsl_decode_step_noalloc(h, x, M, arr, positions, out, ctypes.byref(taps) if taps else None,
                                         stream))


def dsl_attn_step(h, x: int, M: int, kv: list, positions: int, out: int, stream: int = 0):
    arr = (KV * len(kv))(*kv)
    _check(lib().dsl_attn_step(h, x, M, arr, positions, out, stream))


def dsl_moe_step(h, u: int, M: int, out: int, ids: int | None, w: int | None, stream: int = 0):
    _check(lib().dsl_moe_step(h, u, M, out, ids, w, stream))


def dsl_layer_health(h) -> int:
    return lib().dsl_layer_health(h)


def dsl_layer_grid(h) -> tuple:
    b, t = c_int32(), c_int32()
    _check(lib().dsl_layer_grid(h, ctypes.byref(b), ctypes.byref(t)))
    return b.value, t.value


def dsl_layer_last_kernel(h) -> int:
    """1 if the handle's most recent step ran the narrow kernel instantiation, 0 if the
    general one, -1 before any step."""
    rc = lib().dsl_layer_last_kernel(h)
    if rc < -1:
        _check(rc)
    return rc


def dsl_linear_workspace_bytes(M: int, N: int, K: int) -> int:
    n = lib().dsl_linear_workspace_bytes(M, N, K)
    if n < 0:
        raise DslError(DSL_EUNSUPPORTED, lib().dsl_last_error().decode())
    return n


def dsl_linear_mxfp8(x: int, M: int, K: int, w: int, w_s: int, N: int, y: int, workspace: int, stream: int = 0):
    _check(lib().dsl_linear_mxfp8(x, M, K, w, w_s, N, y, workspace, stream))


class LinearOnDevice:
    """One MXFP8 weight [N][K] (codes and E8M0 tiles) in device memory, run on bf16 rows."""

    def __init__(self, w: np.ndarray, w_s: np.ndarray, device="cuda:0"):
        import torch
        self.torch = torch
        self.dev = torch.device(device)
        self.N, self.K = w.shape
        self.w = torch.from_numpy(np.ascontiguousarray(w)).to(self.dev)
        self.w_s = torch.from_numpy(np.ascontiguousarray(w_s)).to(self.dev)

    def __call__(self, x_bits: np.ndarray) -> np.ndarray:
        torch = self.torch
        M = x_bits.shape[0]
        x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(self.dev)
        y = torch.empty((M, self.N), dtype=torch.float32, device=self.dev)
        ws = torch.empty(dsl_linear_workspace_bytes(M, self.N, self.K) + 256, dtype=torch.uint8, device=self.dev)
        base = (ws.data_ptr() + 255) & ~255
        dsl_linear_mxfp8(x.data_ptr(), M, self.K, self.w.data_ptr(), self.w_s.data_ptr(), self.N, y.data_ptr(), base,
                         torch.cuda.current_stream(self.dev).cuda_stream)
        torch.cuda.synchronize(self.dev)
        return y.cpu().numpy()


def dsl_layer_set_trace(h, on: bool):
    _check(lib().dsl_layer_set_trace(h, 1 if on else 0))


def dsl_layer_read_trace(h, n_marks: int = 256) -> np.ndarray:
    """Stamps of the last traced launch: [marks, blocks] nanoseconds (-1 = none)."""
    blocks, _ = dsl_layer_grid(h)
    buf = np.zeros(n_marks * blocks, dtype=np.float64)
    cnt = lib().dsl_layer_read_trace(h, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), n_marks)
    if cnt < 0:
        _check(cnt)
    return buf[: cnt * blocks].reshape(cnt, blocks)


def dsl_layer_destroy(h):
    lib().dsl_layer_destroy(h)


def dsl_last_error() -> str:
    return lib().dsl_last_error().decode()


# --------------------------------------------------------------------------- device-side holder

class DeviceWeights:
    """One model's layer weights in device memory (torch tensors) and a handle built on them."""

    def __init__(self, dims, layers: list, device="cuda:0"):
        import torch
        self.dev = torch.device(device)
        self.dims = dims
        self.w_dev = [{k: torch.from_numpy(np.ascontiguousarray(v)).to(self.dev) for k, v in lw.items()}
                      for lw in layers]
        self.handle = dsl_layer_build(dims_struct(dims), [Weights(**{k: t[k].data_ptr() for k in WEIGHT_FIELDS})
                                                          for t in self.w_dev])

    def single(self, l: int) -> "DeviceWeights":
        """A one-layer handle on layer l's tensors (shared, not copied)."""
        sub = DeviceWeights.__new__(DeviceWeights)
        sub.dev, sub.dims = self.dev, dataclasses.replace(self.dims, n_layers=1)
        sub.w_dev = [self.w_dev[l]]
        sub._parent = self
        sub.handle = dsl_layer_build(dims_struct(sub.dims), [Weights(**{k: self.w_dev[l][k].data_ptr()
                                                                         for k in WEIGHT_FIELDS})])
        return sub

    def close(self):
        if self.handle:
            dsl_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class LayerOnDevice:
    """Caches, tables and activations of a synthetic case in device memory, with the weights
    (uploaded here unless a DeviceWeights of the same dims is passed) and the handle."""

    def __init__(self, case, device="cuda:0", weights: DeviceWeights | None = None):
        import torch
        self.torch = torch
        self.dev = torch.device(device)
        self.case = case
        d = case.dims
        self.dims = d
        self._keep = []
        self._owns = weights is None
        self.weights = weights if weights is not None else DeviceWeights(d, case.layers, device)
        self.w_dev = self.weights.w_dev
        self.handle = self.weights.handle
        self.caches = []
        self.kv_structs = []
        if case.kv is not None:
            kvs = case.kv
            self.block_table = self._up(kvs.block_table)
            self.row_req = self._up(kvs.row_req)
            self.positions = self._up(kvs.positions)
            self.key_table = self._up(kvs.key_table) if kvs.key_table is not None else None
            for c in kvs.cache:
                cd = self._up(c)
                self.caches.append(cd)
                self.kv_structs.append(KV(cd.data_ptr(), d.kv_block * d.record, c.shape[0],
                                          self.block_table.data_ptr(), kvs.block_table.shape[1],
                                          kvs.block_table.shape[0], self.row_req.data_ptr(),
                                          self.key_table.data_ptr() if self.key_table is not None else None))

    def _up(self, a: np.ndarray):
        t = self.torch.from_numpy(np.ascontiguousarray(a)).to(self.dev)
        self._keep.append(t)
        return t

    def stream(self) -> int:
        return self.torch.cuda.current_stream(self.dev).cuda_stream

    def new_bf16(self, M: int):
        return self.torch.zeros((M, self.dims.hidden), dtype=self.torch.int16, device=self.dev)

    def decode(self, x_bits: np.ndarray, taps: bool = True, noalloc: bool = False) -> dict:
        """One decode step on x (bf16 codes); returns host copies of the outputs.  noalloc:
        through dsl_decode_step_noalloc."""
        torch = self.torch
        M = x_bits.shape[0]
        x = self._up(x_bits.view(np.int16))
        out = self.new_bf16(M)
        res = {"out": out}
        t = None
        if taps:
            res.update(attn_out=self.new_bf16(M), hres=self.new_bf16(M), moe_in=self.new_bf16(M),
                       moe_out=self.new_bf16(M),
                       ids=torch.zeros((M, self.dims.top_k), dtype=torch.int32, device=self.dev),
                       w=torch.zeros((M, self.dims.top_k), dtype=torch.float32, device=self.dev),
                       logits=torch.zeros((M, self.dims.n_experts), dtype=torch.float32, device=self.dev),
                       layer_ids=torch.zeros((self.dims.n_layers, M, self.dims.top_k), dtype=torch.int32,
                                             device=self.dev))
            t = Taps(res["attn_out"].data_ptr(), res["hres"].data_ptr(), res["moe_in"].data_ptr(),
                     res["moe_out"].data_ptr(), res["ids"].data_ptr(), res["w"].data_ptr(),
                     res["logits"].data_ptr(), res["layer_ids"].data_ptr())
        step = dsl_decode_step_noalloc if noalloc else dsl_decode_step
        step(self.handle, x.data_ptr(), M, self.kv_structs, self.positions.data_ptr(), out.data_ptr(), t,
             self.stream())
        torch.cuda.synchronize(self.dev)
        _check(dsl_layer_health(self.handle))
        return self._host(res)

    def attn(self, x_bits: np.ndarray) -> dict:
        torch = self.torch
        M = x_bits.shape[0]
        x = self._up(x_bits.view(np.int16))
        out = self.new_bf16(M)
        dsl_attn_step(self.handle, x.data_ptr(), M, self.kv_structs[:1], self.positions.data_ptr(),
                      out.data_ptr(), self.stream())
        torch.cuda.synchronize(self.dev)
        _check(dsl_layer_health(self.handle))
        return self._host({"attn_out": out})

    def moe(self, u_bits: np.ndarray) -> dict:
        torch = self.torch
        M = u_bits.shape[0]
        u = self._up(u_bits.view(np.int16))
        out = self.new_bf16(M)
        ids = torch.zeros((M, self.dims.top_k), dtype=torch.int32, device=self.dev)
        w = torch.zeros((M, self.dims.top_k), dtype=torch.float32, device=self.dev)
        dsl_moe_step(self.handle, u.data_ptr(), M, out.data_ptr(), ids.data_ptr(), w.data_ptr(), self.stream())
        torch.cuda.synchronize(self.dev)
        _check(dsl_layer_health(self.handle))
        return self._host({"moe_out": out, "ids": ids, "w": w})

    def caches_host(self) -> list:
        return [c.cpu().numpy() for c in self.caches]

    def _host(self, res: dict) -> dict:
        out = {}
        for k, v in res.items():
            a = v.cpu().numpy()
            out[k] = a.view(np.uint16) if a.dtype == np.int16 else a
        return out

    def close(self):
        if self.handle and self._owns:
            self.weights.close()
        self.handle = None
