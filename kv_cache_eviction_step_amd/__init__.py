"""Python binding of libkve.so, the gfx950 KV-cache eviction step.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/kve.h``.  PyTorch supplies device
memory and streams.  There is no fallback: if the library is missing this
module fails to import.

Calls (same names as the C ABI):
    keyformer_step(layer, new_k, new_v, ctr, budget, n_sink, tau_init, tau_end,
                   anneal_steps, rope_base, seed, evicted=None, stream=None)
    pyramid_step(layer, new_k, new_v, ctr, budget, n_sink, rope_base,
                 evicted=None, stream=None)
    keyformer_step_layers(batch, new_k, new_v, n_sink, tau_init, tau_end,
                          anneal_steps, rope_base, seed, evicted=None, stream=None)
    pyramid_step_layers(batch, new_k, new_v, n_sink, rope_base, evicted=None,
                        stream=None)
    keyformer_step_tokens(layer, new_k[S], new_v[S], ctr, budget, n_sink, tau_init,
                          tau_end, anneal_steps, rope_base, seed, evicted=None, stream=None)
    pyramid_step_tokens(layer, new_k[S], new_v[S], ctr, budget, n_sink, rope_base,
                        evicted=None, stream=None)
    step(batch, new_k, new_v, policy, evicted=None, stream=None, n_tokens=None,
         workspace=None)                     (kve_step / kve_step_ws)
    step_noalloc(batch, new_k, new_v, policy, evicted=None, stream=None, n_tokens=None)
    workspace_size(caches, max_budget, d), workspace(caches, max_budget, d, device)
    pyramid_budgets(n_layers, avg_budget, n_sink, beta) -> list[int]
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

import torch  # noqa: F401  (loads torch's HIP runtime first; libkve binds to it)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkve.so")

KVE_OK, KVE_EINVAL, KVE_ELAUNCH, KVE_ENODEV, KVE_ENOSPACE = 0, -1, -2, -3, -4
NOALLOC_SCRATCH_BYTES = 16 << 20       # KVE_NOALLOC_SCRATCH_BYTES


class KveLayer(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("scores", ctypes.c_void_p), ("gumbel", ctypes.c_void_p),
        ("positions", ctypes.c_void_p),
        ("bh", ctypes.c_int32), ("cap", ctypes.c_int32), ("d", ctypes.c_int32),
        ("hh_base", ctypes.c_int32),
    ]


class Counters(ctypes.Structure):
    """Host counters shared by a layer's caches (n_kept, next_pos, pos)."""
    _fields_ = [("n_kept", ctypes.c_int32), ("next_pos", ctypes.c_int32),
                ("pos", ctypes.c_int32)]

    def copy(self) -> "Counters":
        return Counters(self.n_kept, self.next_pos, self.pos)

    def __repr__(self) -> str:
        return f"Counters(n_kept={self.n_kept}, next_pos={self.next_pos}, pos={self.pos})"


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first "
                      "(python -c 'import __graft_entry__ as g; g.build()')")

_lib = ctypes.CDLL(LIB_PATH)
_lib.keyformer_step.restype = ctypes.c_int
_lib.keyformer_step.argtypes = [
    ctypes.POINTER(KveLayer), ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(Counters),
    ctypes.c_int32, ctypes.c_int32, ctypes.c_double, ctypes.c_double, ctypes.c_int32,
    ctypes.c_double, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
_lib.pyramid_step.restype = ctypes.c_int
_lib.pyramid_step.argtypes = [
    ctypes.POINTER(KveLayer), ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(Counters),
    ctypes.c_int32, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p]
_lib.keyformer_step_layers.restype = ctypes.c_int
_lib.keyformer_step_layers.argtypes = [
    ctypes.c_int32, ctypes.POINTER(KveLayer), ctypes.c_void_p, ctypes.c_void_p,
    ctypes.POINTER(Counters), ctypes.c_void_p, ctypes.c_int32, ctypes.c_double, ctypes.c_double,
    ctypes.c_int32, ctypes.c_double, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
_lib.pyramid_step_layers.restype = ctypes.c_int
_lib.pyramid_step_layers.argtypes = [
    ctypes.c_int32, ctypes.POINTER(KveLayer), ctypes.c_void_p, ctypes.c_void_p,
    ctypes.POINTER(Counters), ctypes.c_void_p, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p,
    ctypes.c_void_p]
_lib.keyformer_step_tokens.restype = ctypes.c_int
_lib.keyformer_step_tokens.argtypes = [
    ctypes.POINTER(KveLayer), ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
    ctypes.POINTER(Counters), ctypes.c_int32, ctypes.c_int32, ctypes.c_double, ctypes.c_double,
    ctypes.c_int32, ctypes.c_double, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
_lib.pyramid_step_tokens.restype = ctypes.c_int
_lib.pyramid_step_tokens.argtypes = [
    ctypes.POINTER(KveLayer), ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
    ctypes.POINTER(Counters), ctypes.c_int32, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p,
    ctypes.c_void_p]
_lib.keyformer_step_layers_tokens.restype = ctypes.c_int
_lib.keyformer_step_layers_tokens.argtypes = [
    ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(KveLayer), ctypes.c_void_p, ctypes.c_void_p,
    ctypes.POINTER(Counters), ctypes.c_void_p, ctypes.c_int32, ctypes.c_double, ctypes.c_double,
    ctypes.c_int32, ctypes.c_double, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
_lib.pyramid_step_layers_tokens.restype = ctypes.c_int
_lib.pyramid_step_layers_tokens.argtypes = [
    ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(KveLayer), ctypes.c_void_p, ctypes.c_void_p,
    ctypes.POINTER(Counters), ctypes.c_void_p, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p,
    ctypes.c_void_p]
class Policy(ctypes.Structure):
    """kve_policy: the eviction rule of kve_step (see policy())."""
    _fields_ = [("n_sink", ctypes.c_int32), ("recent", ctypes.c_int32),
                ("score", ctypes.c_int32), ("gumbel", ctypes.c_int32),
                ("tau_init", ctypes.c_double), ("tau_end", ctypes.c_double),
                ("anneal_steps", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("rope_base", ctypes.c_double), ("seed", ctypes.c_uint64)]


SCORE_CUMULATIVE, SCORE_CURRENT = 0, 1

_lib.kve_step.restype = ctypes.c_int
_lib.kve_step.argtypes = [
    ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(KveLayer), ctypes.c_void_p, ctypes.c_void_p,
    ctypes.POINTER(Counters), ctypes.c_void_p, ctypes.POINTER(Policy), ctypes.c_void_p,
    ctypes.c_void_p]
_lib.kve_step_ws.restype = ctypes.c_int
_lib.kve_step_ws.argtypes = [
    ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(KveLayer), ctypes.c_void_p, ctypes.c_void_p,
    ctypes.POINTER(Counters), ctypes.c_void_p, ctypes.POINTER(Policy), ctypes.c_void_p,
    ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
_lib.kve_step_noalloc.restype = ctypes.c_int
_lib.kve_step_noalloc.argtypes = [
    ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(KveLayer), ctypes.c_void_p, ctypes.c_void_p,
    ctypes.POINTER(Counters), ctypes.c_void_p, ctypes.POINTER(Policy), ctypes.c_void_p,
    ctypes.c_void_p]
_lib.kve_workspace_size.restype = ctypes.c_int64
_lib.kve_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
_lib.kve_kept_indices.restype = ctypes.c_int32
_lib.kve_kept_indices.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                  ctypes.c_void_p]
_lib.kve_fp16_bytes.restype = ctypes.c_int64
_lib.kve_fp16_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32]
_lib.kve_full_fp16_bytes.restype = ctypes.c_int64
_lib.kve_full_fp16_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32]
_lib.pyramid_budgets.restype = ctypes.c_int
_lib.pyramid_budgets.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_double, ctypes.c_void_p]
_lib.kve_strerror.restype = ctypes.c_char_p
_lib.kve_strerror.argtypes = [ctypes.c_int]

EXPORTED = ("keyformer_step", "pyramid_step", "keyformer_step_layers", "pyramid_step_layers",
            "keyformer_step_tokens", "pyramid_step_tokens", "keyformer_step_layers_tokens",
            "pyramid_step_layers_tokens", "kve_step", "kve_step_ws", "kve_workspace_size",
            "kve_step_noalloc",
            "pyramid_budgets", "kve_kept_indices",
            "kve_fp16_bytes", "kve_full_fp16_bytes", "kve_strerror")


def lib() -> ctypes.CDLL:
    return _lib


def strerror(code: int) -> str:
    return _lib.kve_strerror(code).decode()


def _check(rc: int, what: str) -> None:
    if rc == KVE_OK:
        return
    msg = f"{what}: {strerror(rc)} (code {rc})"
    if rc in (KVE_EINVAL, KVE_ENOSPACE):
        raise ValueError(msg)
    raise RuntimeError(msg)


def hip_runtimes_mapped() -> list[str]:
    """Paths of every libamdhip64 mapped into this process (should be one)."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                paths.add(os.path.realpath(line.split()[-1]))
    return sorted(paths)


class Layer:
    """One layer's B*H caches as caller-owned device tensors (the ABI's kve_layer).

    k, v:       fp16 [bh, cap, d]
    scores:     fp32 [bh, cap]
    gumbel:     fp32 [bh, cap] or None (pyramid_step)
    positions:  int32 [bh, cap]
    """

    def __init__(self, k, v, scores, gumbel, positions, hh_base: int = 0):
        bh, cap, d = k.shape
        for t, dt, shp in ((k, torch.float16, (bh, cap, d)), (v, torch.float16, (bh, cap, d)),
                           (scores, torch.float32, (bh, cap)),
                           (positions, torch.int32, (bh, cap))):
            if t.dtype != dt or tuple(t.shape) != shp or not t.is_contiguous():
                raise ValueError(f"layer tensor must be contiguous {dt} {shp}, got "
                                 f"{t.dtype} {tuple(t.shape)}")
            if t.device != k.device:
                raise ValueError("layer tensors must share one device")
        if gumbel is not None and (gumbel.dtype != torch.float32 or
                                   tuple(gumbel.shape) != (bh, cap) or
                                   not gumbel.is_contiguous() or gumbel.device != k.device):
            raise ValueError("gumbel must be contiguous float32 [bh, cap] on the same device")
        self.k, self.v, self.scores, self.gumbel, self.positions = k, v, scores, gumbel, positions
        self.bh, self.cap, self.d, self.hh_base = bh, cap, d, hh_base
        # what the per-call checks compare against (plain ints and tuples are
        # cheaper to compare than torch.device objects)
        self._dev = k.get_device()                # -1 for host tensors
        self._row_shape = (bh, d)

    @classmethod
    def empty(cls, bh: int, cap: int, d: int, device, gumbel: bool = True, hh_base: int = 0):
        z = dict(device=device)
        return cls(torch.zeros((bh, cap, d), dtype=torch.float16, **z),
                   torch.zeros((bh, cap, d), dtype=torch.float16, **z),
                   torch.zeros((bh, cap), dtype=torch.float32, **z),
                   torch.zeros((bh, cap), dtype=torch.float32, **z) if gumbel else None,
                   torch.zeros((bh, cap), dtype=torch.int32, **z), hh_base)

    def get_kv(self, n_kept: int):
        """keyformer_get_kv: views (no copies) of the live rows, keys and values
        [bh, n_kept, d]; zero-row views before the first step."""
        if not 0 <= n_kept <= self.cap:
            raise ValueError(f"n_kept must be in [0, {self.cap}]")
        return self.k[:, :n_kept], self.v[:, :n_kept]

    def c_struct(self) -> KveLayer:
        return KveLayer(self.k.data_ptr(), self.v.data_ptr(), self.scores.data_ptr(),
                        self.gumbel.data_ptr() if self.gumbel is not None else None,
                        self.positions.data_ptr(), self.bh, self.cap, self.d, self.hh_base)


def _rows(t, layer: Layer, name: str):
    if (t.dtype is not torch.float16 or t.shape != layer._row_shape or
            not t.is_contiguous() or t.get_device() != layer._dev):
        raise ValueError(f"{name} must be contiguous float16 [{layer.bh}, {layer.d}] on "
                         f"{layer.k.device}")
    return t.data_ptr()


def _evicted_ptr(evicted, layer: Layer):
    if evicted is None:
        return None
    if (evicted.dtype is not torch.int32 or evicted.shape != (layer.bh,) or
            not evicted.is_contiguous() or evicted.get_device() != layer._dev):
        raise ValueError(f"evicted must be contiguous int32 [{layer.bh}] on {layer.k.device}")
    return evicted.data_ptr()


# torch's query of the current stream's raw handle (no Stream object is
# built: about a tenth of the public call's host time); the public call where
# a build lacks it
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_ptr(stream, layer: Layer):
    """The stream handle, after checking that the layer lives on the current
    device (the library launches there)."""
    dev = layer._dev
    if dev < 0 or dev != torch.cuda.current_device():
        raise ValueError(f"layer tensors are on {layer.k.device}; calls run on the current "
                         "GPU (use torch.cuda.device(...) to select it)")
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(dev)
        return torch.cuda.current_stream(dev).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def keyformer_step(layer: Layer, new_k, new_v, ctr: Counters, budget: int, n_sink: int,
                   tau_init: float, tau_end: float, anneal_steps: int, rope_base: float,
                   seed: int, evicted=None, stream=None, c_layer: KveLayer | None = None) -> None:
    """One token into every cache of `layer` (Keyformer-adapted).  Updates `ctr`."""
    cl = c_layer if c_layer is not None else layer.c_struct()
    rc = _lib.keyformer_step(ctypes.byref(cl), _rows(new_k, layer, "new_k"),
                             _rows(new_v, layer, "new_v"), ctypes.byref(ctr), budget, n_sink,
                             tau_init, tau_end, anneal_steps, rope_base,
                             seed & 0xFFFFFFFFFFFFFFFF, _evicted_ptr(evicted, layer),
                             _stream_ptr(stream, layer))
    _check(rc, "keyformer_step")


def pyramid_step(layer: Layer, new_k, new_v, ctr: Counters, budget: int, n_sink: int,
                 rope_base: float, evicted=None, stream=None,
                 c_layer: KveLayer | None = None) -> None:
    """One token into every cache of `layer` (H2O / PyramidKV-adapted).  Updates `ctr`."""
    cl = c_layer if c_layer is not None else layer.c_struct()
    rc = _lib.pyramid_step(ctypes.byref(cl), _rows(new_k, layer, "new_k"),
                           _rows(new_v, layer, "new_v"), ctypes.byref(ctr), budget, n_sink,
                           rope_base, _evicted_ptr(evicted, layer), _stream_ptr(stream, layer))
    _check(rc, "pyramid_step")


def _blocks_contiguous(t) -> bool:
    """Every t[i] is contiguous (any stride along dimension 0)."""
    expect = 1
    for size, stride in zip(reversed(t.shape[1:]), reversed(t.stride()[1:])):
        if size != 1 and stride != expect:
            return False
        expect *= size
    return t.stride(0) >= 0


class LayerBatch:
    """Several layers stepped together by keyformer_step_layers / pyramid_step_layers.

    Holds the host arrays the batched C calls take: layer descriptors, per-layer
    budgets and per-layer counters (``ctrs[l]``, updated by every call).
    """

    def __init__(self, layers: list[Layer], budgets: list[int],
                 counters: list[Counters] | None = None):
        if not layers or len(layers) != len(budgets):
            raise ValueError("one budget per layer")
        n = len(layers)
        self.layers = layers
        self.n = n
        self.c_layers = (KveLayer * n)(*[x.c_struct() for x in layers])
        self.budgets = (ctypes.c_int32 * n)(*budgets)
        self.ctrs = (Counters * n)()
        for i, c in enumerate(counters or []):
            self.ctrs[i] = c
        self._pk = (ctypes.c_void_p * n)()
        self._pv = (ctypes.c_void_p * n)()
        self._pe = (ctypes.c_void_p * n)()
        # numpy views of the pointer arrays: a whole-batch tensor fills them
        # with one vectorised write instead of a Python loop over the layers
        self._pk_np = np.frombuffer(self._pk, dtype=np.uint64)
        self._pv_np = np.frombuffer(self._pv, dtype=np.uint64)
        self._pe_np = np.frombuffer(self._pe, dtype=np.uint64)
        self._idx = np.arange(n, dtype=np.uint64)
        dev = layers[0].k.device
        if any(x.k.device != dev for x in layers):
            raise ValueError("all layers must be on one device")
        self.device = dev
        self._dev = layers[0]._dev
        self._offsets = {}                        # byte stride -> per-layer offsets
        # (bh, d) of every layer, and the common one when all layers agree
        self._rows = [(x.bh, x.d) for x in layers]
        self._common = self._rows[0] if len(set(self._rows)) == 1 else None

    def _layer_offsets(self, stride_bytes: int):
        """Byte offsets l * stride_bytes of the layers' blocks in a whole-batch
        tensor (kept per stride: a decode loop passes the same layout every call)."""
        offs = self._offsets.get(stride_bytes)
        if offs is None:
            if len(self._offsets) >= 16:
                self._offsets.clear()
            offs = self._idx * np.uint64(stride_bytes)
            self._offsets[stride_bytes] = offs
        return offs

    def _same_rows(self, shape: tuple, tok: tuple, with_d: bool = True) -> bool:
        """shape == tok + (bh_l, d_l) for every layer l (tok + (bh_l,) without d)."""
        def want(rows):
            return tok + (rows if with_d else rows[:1])
        if self._common is not None:
            return shape == want(self._common)
        return all(shape == want(r) for r in self._rows)

    def _fill(self, new_k, new_v, evicted, n_tokens: int | None = None):
        """Pointer arrays for this call.

        One token (n_tokens None): new_k / new_v are a list of [bh_l, d]
        tensors or one [n_layers, bh, d] tensor; evicted is None, a list of
        [bh_l] int32 tensors or one [n_layers, bh] tensor.  S tokens
        (n_tokens S): the same with a token axis after the layer axis:
        [S, bh_l, d] per layer or [n_layers, S, bh, d]; evicted [S, bh_l] per
        layer or [n_layers, S, bh].  A single tensor may have any stride along
        the layer axis (a slice of a longer token axis, say) as long as each
        layer's block is contiguous."""
        n = self.n
        tok = () if n_tokens is None else (n_tokens,)
        for arr, arr_np, src, name in ((self._pk, self._pk_np, new_k, "new_k"),
                                       (self._pv, self._pv_np, new_v, "new_v")):
            if isinstance(src, torch.Tensor):
                L0 = self.layers[0]
                if (src.dtype is not torch.float16 or src.dim() != 3 + len(tok) or
                        src.shape[0] != n or src.get_device() != self._dev or
                        not self._same_rows(tuple(src.shape[1:]), tok) or
                        not (src.is_contiguous() or _blocks_contiguous(src))):
                    raise ValueError(f"{name} must be float16 {[n, *tok, L0.bh, L0.d]} "
                                     "with contiguous per-layer blocks")
                np.add(self._layer_offsets(src.stride(0) * 2), np.uint64(src.data_ptr()),
                       out=arr_np)
            else:
                if len(src) != n:
                    raise ValueError(f"{name}: one tensor per layer")
                for i in range(n):
                    if n_tokens is None:
                        arr[i] = _rows(src[i], self.layers[i], name)
                    else:
                        if src[i].shape[0] != n_tokens:
                            raise ValueError(f"{name}[{i}]: {n_tokens} tokens expected")
                        arr[i] = _tokens(src[i], self.layers[i], name)
        if evicted is None:
            return None
        if isinstance(evicted, torch.Tensor):
            if (evicted.dtype is not torch.int32 or evicted.dim() != 2 + len(tok) or
                    evicted.shape[0] != n or evicted.get_device() != self._dev or
                    not self._same_rows(tuple(evicted.shape[1:]), tok, with_d=False) or
                    not (evicted.is_contiguous() or _blocks_contiguous(evicted))):
                raise ValueError(f"evicted must be int32 {[n, *tok, 'bh']} with contiguous "
                                 "per-layer blocks")
            np.add(self._layer_offsets(evicted.stride(0) * 4), np.uint64(evicted.data_ptr()),
                   out=self._pe_np)
        else:
            if len(evicted) != n:
                raise ValueError("evicted: one tensor (or None) per layer")
            for i in range(n):
                e = evicted[i]
                if e is None:
                    self._pe[i] = None
                elif n_tokens is None:
                    self._pe[i] = _evicted_ptr(e, self.layers[i])
                else:
                    self._pe[i] = _evicted_tokens(e, self.layers[i], n_tokens)
        return self._pe


def keyformer_step_layers(batch: LayerBatch, new_k, new_v, n_sink: int, tau_init: float,
                          tau_end: float, anneal_steps: int, rope_base: float, seed: int,
                          evicted=None, stream=None) -> None:
    """One token into every cache of every layer of `batch`, in one launch."""
    pe = batch._fill(new_k, new_v, evicted)
    rc = _lib.keyformer_step_layers(batch.n, batch.c_layers, batch._pk, batch._pv, batch.ctrs,
                                    batch.budgets, n_sink, tau_init, tau_end, anneal_steps,
                                    rope_base, seed & 0xFFFFFFFFFFFFFFFF, pe,
                                    _stream_ptr(stream, batch.layers[0]))
    _check(rc, "keyformer_step_layers")


def pyramid_step_layers(batch: LayerBatch, new_k, new_v, n_sink: int, rope_base: float,
                        evicted=None, stream=None) -> None:
    """One token into every cache of every layer of `batch` (H2O / PyramidKV), one launch."""
    pe = batch._fill(new_k, new_v, evicted)
    rc = _lib.pyramid_step_layers(batch.n, batch.c_layers, batch._pk, batch._pv, batch.ctrs,
                                  batch.budgets, n_sink, rope_base, pe,
                                  _stream_ptr(stream, batch.layers[0]))
    _check(rc, "pyramid_step_layers")


def _tokens(t, layer: Layer, name: str):
    if (t.dtype is not torch.float16 or t.dim() != 3 or t.shape[1:] != layer._row_shape
            or not t.is_contiguous() or t.get_device() != layer._dev):
        raise ValueError(f"{name} must be contiguous float16 [S, {layer.bh}, {layer.d}] on "
                         f"{layer.k.device}")
    return t.data_ptr()


def _evicted_tokens(evicted, layer: Layer, n: int):
    if evicted is None:
        return None
    if (evicted.dtype is not torch.int32 or evicted.shape != (n, layer.bh) or
            not evicted.is_contiguous() or evicted.get_device() != layer._dev):
        raise ValueError(f"evicted must be contiguous int32 [{n}, {layer.bh}]")
    return evicted.data_ptr()


def keyformer_step_tokens(layer: Layer, new_k, new_v, ctr: Counters, budget: int, n_sink: int,
                          tau_init: float, tau_end: float, anneal_steps: int, rope_base: float,
                          seed: int, evicted=None, stream=None,
                          c_layer: KveLayer | None = None) -> None:
    """new_k.shape[0] consecutive tokens into every cache of `layer`, one launch."""
    n = new_k.shape[0]
    cl = c_layer if c_layer is not None else layer.c_struct()
    pk, pv = _tokens(new_k, layer, "new_k"), _tokens(new_v, layer, "new_v")
    if new_v.shape[0] != n:
        raise ValueError("new_k and new_v must hold the same number of tokens")
    rc = _lib.keyformer_step_tokens(ctypes.byref(cl), n, pk, pv, ctypes.byref(ctr), budget,
                                    n_sink, tau_init, tau_end, anneal_steps, rope_base,
                                    seed & 0xFFFFFFFFFFFFFFFF, _evicted_tokens(evicted, layer, n),
                                    _stream_ptr(stream, layer))
    _check(rc, "keyformer_step_tokens")


def pyramid_step_tokens(layer: Layer, new_k, new_v, ctr: Counters, budget: int, n_sink: int,
                        rope_base: float, evicted=None, stream=None,
                        c_layer: KveLayer | None = None) -> None:
    """new_k.shape[0] consecutive tokens into every cache of `layer` (H2O / PyramidKV)."""
    n = new_k.shape[0]
    cl = c_layer if c_layer is not None else layer.c_struct()
    pk, pv = _tokens(new_k, layer, "new_k"), _tokens(new_v, layer, "new_v")
    if new_v.shape[0] != n:
        raise ValueError("new_k and new_v must hold the same number of tokens")
    rc = _lib.pyramid_step_tokens(ctypes.byref(cl), n, pk, pv, ctypes.byref(ctr), budget, n_sink,
                                  rope_base, _evicted_tokens(evicted, layer, n),
                                  _stream_ptr(stream, layer))
    _check(rc, "pyramid_step_tokens")


def keyformer_step_layers_tokens(batch: LayerBatch, new_k, new_v, n_sink: int, tau_init: float,
                                 tau_end: float, anneal_steps: int, rope_base: float, seed: int,
                                 evicted=None, stream=None, n_tokens: int | None = None) -> None:
    """S consecutive tokens into every cache of every layer of `batch`, one launch.

    new_k / new_v: [n_layers, S, bh, d] or a list of [S, bh_l, d]; evicted:
    None, [n_layers, S, bh] or a list of [S, bh_l] (or None entries)."""
    S = n_tokens if n_tokens is not None else new_k[0].shape[0]
    pe = batch._fill(new_k, new_v, evicted, S)
    rc = _lib.keyformer_step_layers_tokens(batch.n, S, batch.c_layers, batch._pk, batch._pv,
                                           batch.ctrs, batch.budgets, n_sink, tau_init, tau_end,
                                           anneal_steps, rope_base, seed & 0xFFFFFFFFFFFFFFFF,
                                           pe, _stream_ptr(stream, batch.layers[0]))
    _check(rc, "keyformer_step_layers_tokens")


def pyramid_step_layers_tokens(batch: LayerBatch, new_k, new_v, n_sink: int, rope_base: float,
                               evicted=None, stream=None, n_tokens: int | None = None) -> None:
    """S consecutive tokens into every cache of every layer of `batch` (H2O / PyramidKV)."""
    S = n_tokens if n_tokens is not None else new_k[0].shape[0]
    pe = batch._fill(new_k, new_v, evicted, S)
    rc = _lib.pyramid_step_layers_tokens(batch.n, S, batch.c_layers, batch._pk, batch._pv,
                                         batch.ctrs, batch.budgets, n_sink, rope_base, pe,
                                         _stream_ptr(stream, batch.layers[0]))
    _check(rc, "pyramid_step_layers_tokens")


def policy(kind: str, n_sink: int, recent: int = 0, tau_init: float = 0.0, tau_end: float = 0.0,
           anneal_steps: int = 0, rope_base: float = 10000.0, seed: int = 0) -> Policy:
    """The kve_step policy of one method.

    kind: "keyformer" (cumulative score + annealed Gumbel noise), "h2o" or
    "pyramid" (cumulative score, no noise; PyramidKV differs from H2O only in
    the per-layer budgets), "tova" (current-step score, no noise)."""
    if kind not in ("keyformer", "h2o", "pyramid", "tova"):
        raise ValueError(f"unknown method {kind!r}")
    kf = kind == "keyformer"
    return Policy(n_sink, recent, SCORE_CURRENT if kind == "tova" else SCORE_CUMULATIVE,
                  1 if kf else 0, tau_init if kf else 0.0, tau_end if kf else 0.0,
                  anneal_steps if kf else 0, 0, rope_base,
                  (seed & 0xFFFFFFFFFFFFFFFF) if kf else 0)


def step(batch: LayerBatch, new_k, new_v, pol: Policy, evicted=None, stream=None,
         n_tokens: int | None = None, workspace=None) -> None:
    """kve_step over every layer of `batch` (kve_step_ws with a workspace).

    n_tokens None: one token, inputs as keyformer_step_layers; n_tokens S:
    S tokens, inputs as keyformer_step_layers_tokens.  workspace: a tensor
    from workspace() on the layers' device, or None."""
    S = 1 if n_tokens is None else n_tokens
    pe = batch._fill(new_k, new_v, evicted, n_tokens)
    st = _stream_ptr(stream, batch.layers[0])
    if workspace is None:
        rc = _lib.kve_step(batch.n, S, batch.c_layers, batch._pk, batch._pv, batch.ctrs,
                           batch.budgets, ctypes.byref(pol), pe, st)
        _check(rc, "kve_step")
        return
    if (workspace.dtype is not torch.uint8 or workspace.dim() != 1 or
            not workspace.is_contiguous() or workspace.get_device() != batch._dev):
        raise ValueError("workspace must be a contiguous uint8 tensor on the layers' device "
                         "(see workspace())")
    rc = _lib.kve_step_ws(batch.n, S, batch.c_layers, batch._pk, batch._pv, batch.ctrs,
                          batch.budgets, ctypes.byref(pol), pe, workspace.data_ptr(),
                          workspace.numel(), st)
    _check(rc, "kve_step_ws")


def step_noalloc(batch: LayerBatch, new_k, new_v, pol: Policy, evicted=None, stream=None,
                 n_tokens: int | None = None) -> None:
    """kve_step_noalloc: step() with the workspace in the library's fixed device
    buffer (nothing allocated; raises ValueError when the call would need more
    than NOALLOC_SCRATCH_BYTES of it)."""
    S = 1 if n_tokens is None else n_tokens
    pe = batch._fill(new_k, new_v, evicted, n_tokens)
    rc = _lib.kve_step_noalloc(batch.n, S, batch.c_layers, batch._pk, batch._pv, batch.ctrs,
                               batch.budgets, ctypes.byref(pol), pe,
                               _stream_ptr(stream, batch.layers[0]))
    _check(rc, "kve_step_noalloc")


def workspace_size(caches: int, max_budget: int, d: int) -> int:
    """kve_workspace_size: bytes with which kve_step_ws hands over every long
    move of a single-token launch over `caches` caches at budgets <= max_budget."""
    r = _lib.kve_workspace_size(caches, max_budget, d)
    if r < 0:
        raise ValueError("workspace_size: invalid arguments")
    return int(r)


def workspace(caches: int, max_budget: int, d: int, device) -> "torch.Tensor":
    """A zeroed device workspace of workspace_size(caches, max_budget, d) bytes
    for step(..., workspace=...).  Each call leaves it ready for the next;
    reuse it for every call on one stream."""
    n = workspace_size(caches, max_budget, d)
    t = torch.zeros(n + 256, dtype=torch.uint8, device=device)
    off = (-t.data_ptr()) % 256                   # the library wants 256-byte alignment
    return t[off:off + n]


def kept_indices(n_prev: int, evicted) -> list[int]:
    """return_indices: the kept rows after stepping len(evicted) tokens into a
    cache of n_prev rows, as chronological indices into prior + new rows.
    evicted: that cache's evicted outputs (a sequence of ints, or a CPU int32
    array / tensor), in token order."""
    import numpy as np
    ev = np.ascontiguousarray(np.asarray(evicted, dtype=np.int32).reshape(-1))
    out = np.empty(max(n_prev + len(ev), 1), dtype=np.int32)
    n = _lib.kve_kept_indices(n_prev, len(ev), ev.ctypes.data, out.ctypes.data)
    if n < 0:
        raise ValueError("kve_kept_indices: invalid arguments")
    return out[:n].tolist()


def fp16_bytes(n_kept: int, d: int) -> int:
    """K + V payload of n_kept rows in fp16 (keyformer_fp16_bytes), one cache."""
    r = _lib.kve_fp16_bytes(n_kept, d)
    if r < 0:
        raise ValueError("fp16_bytes: invalid arguments")
    return int(r)


def full_fp16_bytes(tokens_seen: int, d: int) -> int:
    """K + V payload had every token been kept (full_keyformer_fp16_bytes)."""
    r = _lib.kve_full_fp16_bytes(tokens_seen, d)
    if r < 0:
        raise ValueError("full_fp16_bytes: invalid arguments")
    return int(r)


def pyramid_budgets(n_layers: int, avg_budget: int, n_sink: int, beta: float) -> list[int]:
    buf = (ctypes.c_int32 * max(n_layers, 1))()
    _check(_lib.pyramid_budgets(n_layers, avg_budget, n_sink, beta, buf), "pyramid_budgets")
    return [int(buf[i]) for i in range(n_layers)]
