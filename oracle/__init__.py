"""CPU oracle of the per-token KV-cache eviction step (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``kve_oracle.c`` (plain C,
single-threaded) through ctypes and shares nothing with the GPU library.

The method follows the VeloxQuant-MLX documentation pages
"veloxquant_mlx.quantizers.keyformer module" (keyformer_update, KeyformerState)
and "PyramidKV -- Layer-Adaptive Budget Attention-Mass Eviction" (How it works,
The budget schedule); the C source cites the section behind every step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kve_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkve_oracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/libkve_oracle.so``."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Cache(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int32), ("cap", ctypes.c_int32),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("s", ctypes.c_void_p), ("g", ctypes.c_void_p),
        ("p", ctypes.c_void_p), ("tid", ctypes.c_void_p),
        ("work", ctypes.c_void_p), ("snew", ctypes.c_void_p),
        ("n", ctypes.c_int32), ("next_pos", ctypes.c_int32), ("pos", ctypes.c_int32),
    ]


class _Params(ctypes.Structure):
    _fields_ = [
        ("budget", ctypes.c_int32), ("n_sink", ctypes.c_int32),
        ("use_gumbel", ctypes.c_int32), ("anneal_steps", ctypes.c_int32),
        ("tau_init", ctypes.c_double), ("tau_end", ctypes.c_double),
        ("rope_base", ctypes.c_double),
        ("seed", ctypes.c_uint64), ("hh", ctypes.c_int64),
        ("recent", ctypes.c_int32), ("current_score", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = os.environ.get("KVE_ORACLE_LIB")      # a planted-mistake build, in tests
        if not path:
            path = _LIB_PATH
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
                build()
        L = ctypes.CDLL(path)
        L.oracle_splitmix64_mix.restype = ctypes.c_uint64
        L.oracle_splitmix64_mix.argtypes = [ctypes.c_uint64]
        L.oracle_splitmix64_next.restype = ctypes.c_uint64
        L.oracle_splitmix64_next.argtypes = [ctypes.POINTER(ctypes.c_uint64)]
        L.oracle_gumbel_uniform.restype = ctypes.c_double
        L.oracle_gumbel_uniform.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64]
        L.oracle_gumbel.restype = ctypes.c_float
        L.oracle_gumbel.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64]
        L.oracle_tau.restype = ctypes.c_float
        L.oracle_tau.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_int32, ctypes.c_int64]
        L.oracle_pyramid_budgets.restype = ctypes.c_int
        L.oracle_pyramid_budgets.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_double, ctypes.c_void_p]
        L.oracle_f16_to_f32.restype = ctypes.c_float
        L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f32_to_f16.restype = ctypes.c_uint16
        L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        L.oracle_rope_rotate.restype = None
        L.oracle_rope_rotate.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                         ctypes.c_double]
        L.oracle_step.restype = ctypes.c_int
        L.oracle_step.argtypes = [ctypes.POINTER(_Cache), ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.POINTER(_Params), ctypes.c_double,
                                  ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double)]
        L.oracle_run.restype = ctypes.c_int
        L.oracle_run.argtypes = [ctypes.POINTER(_Cache), ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_int32, ctypes.POINTER(_Params), ctypes.c_void_p]
        _lib = L
    return _lib


# --------------------------------------------------------------------------
# scalar helpers
# --------------------------------------------------------------------------

def splitmix64_mix(z: int) -> int:
    return int(lib().oracle_splitmix64_mix(ctypes.c_uint64(z & (2**64 - 1))))


def splitmix64_stream(state: int, count: int) -> list[int]:
    st = ctypes.c_uint64(state)
    return [int(lib().oracle_splitmix64_next(ctypes.byref(st))) for _ in range(count)]


def gumbel_uniform(seed: int, hh: int, pos: int) -> float:
    return float(lib().oracle_gumbel_uniform(seed, hh, pos))


def gumbel(seed: int, hh: int, pos: int) -> np.float32:
    return np.float32(lib().oracle_gumbel(seed, hh, pos))


def tau(tau_init: float, tau_end: float, anneal_steps: int, pos: int) -> np.float32:
    return np.float32(lib().oracle_tau(tau_init, tau_end, anneal_steps, pos))


def pyramid_budgets(n_layers: int, avg_budget: int, n_sink: int, beta: float) -> list[int]:
    out = np.zeros(max(n_layers, 1), dtype=np.int32)
    rc = lib().oracle_pyramid_budgets(n_layers, avg_budget, n_sink, beta, out.ctypes.data)
    if rc != 0:
        raise ValueError(f"pyramid_budgets({n_layers}, {avg_budget}, {n_sink}, {beta}) rejected")
    return [int(x) for x in out[:n_layers]]


def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    f = lib().oracle_f16_to_f32
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([f(int(x)) for x in b], dtype=np.float32).reshape(np.shape(bits))


def f32_to_f16(vals: np.ndarray) -> np.ndarray:
    f = lib().oracle_f32_to_f16
    a = np.asarray(vals, dtype=np.float32).ravel()
    return np.array([f(float(x)) for x in a], dtype=np.uint16).reshape(np.shape(vals))


def rope_rotate(row_bits: np.ndarray, delta: int, base: float = 10000.0) -> np.ndarray:
    r = np.ascontiguousarray(np.array(row_bits, dtype=np.uint16))
    lib().oracle_rope_rotate(r.ctypes.data, r.shape[-1], int(delta), float(base))
    return r


# --------------------------------------------------------------------------
# one cache
# --------------------------------------------------------------------------

@dataclass
class Params:
    budget: int
    n_sink: int
    use_gumbel: bool = True
    tau_init: float = 0.0
    tau_end: float = 0.0
    anneal_steps: int = 0
    rope_base: float = 10000.0
    seed: int = 0
    hh: int = 0
    recent: int = 0                  # trailing protected window (0 = off)
    current_score: bool = False      # TOVA-adapted: score = this step's weight

    def c(self) -> _Params:
        return _Params(self.budget, self.n_sink, 1 if self.use_gumbel else 0,
                       self.anneal_steps, self.tau_init, self.tau_end, self.rope_base,
                       self.seed & (2**64 - 1), self.hh, self.recent,
                       1 if self.current_score else 0)


class OracleCache:
    """One (batch, layer, kv-head) cache, backed by numpy arrays."""

    def __init__(self, d: int, cap: int):
        self.d, self.cap = d, cap
        self.k = np.zeros((cap, d), dtype=np.uint16)
        self.v = np.zeros((cap, d), dtype=np.uint16)
        self.s = np.zeros(cap, dtype=np.float32)
        self.g = np.zeros(cap, dtype=np.float32)
        self.p = np.zeros(cap, dtype=np.int32)
        self.tid = np.zeros(cap, dtype=np.int64)
        self._work = np.zeros(2 * cap, dtype=np.float64)
        self._snew = np.zeros(cap + 1, dtype=np.float32)
        self._c = _Cache(d, cap, self.k.ctypes.data, self.v.ctypes.data, self.s.ctypes.data,
                         self.g.ctypes.data, self.p.ctypes.data, self.tid.ctypes.data,
                         self._work.ctypes.data, self._snew.ctypes.data, 0, 0, 0)

    # counters ---------------------------------------------------------
    @property
    def n(self) -> int:
        return int(self._c.n)

    @property
    def next_pos(self) -> int:
        return int(self._c.next_pos)

    @property
    def pos(self) -> int:
        return int(self._c.pos)

    def set_counters(self, n: int, next_pos: int, pos: int) -> None:
        self._c.n, self._c.next_pos, self._c.pos = n, next_pos, pos

    # state copies (used by tests and the margin guard) ------------------
    def snapshot(self) -> dict:
        n = self.n
        return dict(k=self.k[:n].copy(), v=self.v[:n].copy(), s=self.s[:n].copy(),
                    g=self.g[:n].copy(), p=self.p[:n].copy(), tid=self.tid[:n].copy(),
                    n=n, next_pos=self.next_pos, pos=self.pos)

    def load(self, st: dict) -> None:
        n = st["n"]
        self.k[:n], self.v[:n], self.s[:n] = st["k"], st["v"], st["s"]
        self.g[:n], self.p[:n], self.tid[:n] = st["g"], st["p"], st["tid"]
        self.set_counters(n, st["next_pos"], st["pos"])

    # the step ----------------------------------------------------------
    def step(self, k_bits: np.ndarray, v_bits: np.ndarray, prm: Params,
             min_margin_rel: float = -1.0) -> tuple[int, int, float]:
        """Returns (rc, evicted, margin); rc 0 = committed, 1 = rejected by the guard."""
        k = np.ascontiguousarray(k_bits, dtype=np.uint16)
        v = np.ascontiguousarray(v_bits, dtype=np.uint16)
        assert k.shape == (self.d,) and v.shape == (self.d,)
        e = ctypes.c_int32(-1)
        m = ctypes.c_double(0.0)
        p = prm.c()
        rc = lib().oracle_step(ctypes.byref(self._c), k.ctypes.data, v.ctypes.data,
                               ctypes.byref(p), float(min_margin_rel),
                               ctypes.byref(e), ctypes.byref(m))
        if rc < 0:
            raise ValueError("oracle_step rejected its arguments")
        return int(rc), int(e.value), float(m.value)

    def run(self, ks: np.ndarray, vs: np.ndarray, prm: Params) -> np.ndarray:
        ks = np.ascontiguousarray(ks, dtype=np.uint16)
        vs = np.ascontiguousarray(vs, dtype=np.uint16)
        T = ks.shape[0]
        assert ks.shape == (T, self.d) and vs.shape == (T, self.d)
        ev = np.full(T, -1, dtype=np.int32)
        p = prm.c()
        rc = lib().oracle_run(ctypes.byref(self._c), ks.ctypes.data, vs.ctypes.data, T,
                              ctypes.byref(p), ev.ctypes.data)
        if rc != 0:
            raise ValueError("oracle_run rejected its arguments")
        return ev
