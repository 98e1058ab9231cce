"""Seeded synthetic inputs for the ternary bit-plane GEMV workloads.

Input generation only: nothing here packs, validates, multiplies or dequantises.
The CPU oracle and the GPU path are both fed from these arrays, so a parity test
compares two independent computations on identical inputs.

Shapes follow the model the Tritium paper measures ("Tritium: One Weight Format for
Ternary Inference ...", section "The model"): BitNet b1.58 2B4T, 30 layers, hidden
2560, FFN 6912, 20 query heads and 5 key/value heads of dim 128, vocabulary 128256,
seven ternary projections per layer. Zero densities come from the same paper's
introduction (42.19% for that checkpoint) and from the BITCOS essay's survey of 29
ternary checkpoints (29.66% to 51.48%).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_SRC = os.path.join(_HERE, "synth.c")

# ---------------------------------------------------------------------------- shapes

HIDDEN = 2560
FFN = 6912
N_LAYERS = 30
VOCAB = 128256
# (name, rows, cols) of the seven ternary projections in one layer.
PROJECTIONS = (
    ("q_proj", 2560, 2560),
    ("k_proj", 640, 2560),
    ("v_proj", 640, 2560),
    ("o_proj", 2560, 2560),
    ("gate_proj", 6912, 2560),
    ("up_proj", 6912, 2560),
    ("down_proj", 2560, 6912),
)
P_ZERO_2B4T = 0.4219
P_ZERO_SWEEP = (0.2966, 0.4219, 0.5148)
HEAD_STD = 0.02

# ---------------------------------------------------------------------------- build / load


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (OpenMP, strict IEEE: no contraction, no fast-math)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
             "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _SO)
    return _SO


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        u64, i64, vp, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        lib.synth_u64.argtypes = [u64, u64, i64, vp]
        lib.synth_uniform.argtypes = [u64, i64, vp]
        lib.synth_trits.argtypes = [u64, i64, dbl, vp]
        lib.synth_normal_f32.argtypes = [u64, i64, dbl, dbl, vp]
        lib.synth_absmax_codes.argtypes = [vp, i64, vp, vp]
        lib.synth_weight_scale.argtypes = [u64]
        lib.synth_weight_scale.restype = ctypes.c_float
        lib.synth_bf16_from_f32.argtypes = [vp, i64, vp]
        lib.synth_normal_bf16.argtypes = [u64, i64, dbl, dbl, vp]
        for f in ("synth_u64", "synth_uniform", "synth_trits", "synth_normal_f32",
                  "synth_absmax_codes", "synth_bf16_from_f32", "synth_normal_bf16"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ---------------------------------------------------------------------------- draws


def u64(seed: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().synth_u64(seed, start, n, _ptr(out))
    return out


def uniform(seed: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_uniform(seed, n, _ptr(out))
    return out


def trits(seed: int, rows: int, cols: int, p_zero: float = P_ZERO_2B4T) -> np.ndarray:
    """int8[rows, cols] in {-1, 0, +1}, i.i.d., P(0) = p_zero, nonzeros split evenly."""
    out = np.empty((rows, cols), dtype=np.int8)
    _load().synth_trits(seed, rows * cols, float(p_zero), _ptr(out))
    return out


def normal_f32(seed: int, n: int, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _load().synth_normal_f32(seed, n, float(mean), float(std), _ptr(out))
    return out


def absmax_codes(v: np.ndarray) -> tuple[np.ndarray, float]:
    """int8 codes rint(127 v / max|v|) and the float scale max|v| / 127 (the activation recipe)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    q = np.empty(v.shape, dtype=np.int8)
    s = np.zeros(1, dtype=np.float32)
    _load().synth_absmax_codes(_ptr(v), v.size, _ptr(q), _ptr(s))
    return q, float(s[0])


def activation(seed: int, cols: int) -> tuple[np.ndarray, float]:
    """An int8 activation of length cols, absmax-quantised from N(0, 1), and its scale."""
    return absmax_codes(normal_f32(seed, cols))


def weight_scale(seed: int) -> float:
    return float(np.float32(_load().synth_weight_scale(seed)))


def bf16_from_f32(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().synth_bf16_from_f32(_ptr(v), v.size, _ptr(out))
    return out


def normal_bf16(seed: int, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    shape = (shape,) if isinstance(shape, int) else tuple(shape)
    out = np.empty(shape, dtype=np.uint16)
    _load().synth_normal_bf16(seed, int(np.prod(shape)), float(mean), float(std), _ptr(out))
    return out


# ---------------------------------------------------------------------------- workloads

# Roles within one matrix's seed block.
ROLE_W, ROLE_X, ROLE_WSCALE = 0, 1, 2


def seed_of(base: int, layer: int, proj: int, role: int) -> int:
    """Seed rule: base + 16 * (7 * layer + proj) + role (distinct streams per matrix and role)."""
    return (base + 16 * (7 * layer + proj) + role) & 0xFFFFFFFFFFFFFFFF


@dataclass
class TernaryCase:
    """One ternary GEMV input set: W as trits, the int8 activation and both scales."""
    name: str
    w: np.ndarray          # int8 [rows, cols] in {-1, 0, +1}
    x: np.ndarray          # int8 [cols]
    x_scale: float
    w_scale: float

    @property
    def rows(self) -> int:
        return self.w.shape[0]

    @property
    def cols(self) -> int:
        return self.w.shape[1]


def ternary_case(base: int, layer: int, proj: int, rows: int, cols: int,
                 p_zero: float = P_ZERO_2B4T, name: str = "") -> TernaryCase:
    w = trits(seed_of(base, layer, proj, ROLE_W), rows, cols, p_zero)
    x, xs = activation(seed_of(base, layer, proj, ROLE_X), cols)
    ws = weight_scale(seed_of(base, layer, proj, ROLE_WSCALE))
    return TernaryCase(name or f"L{layer}.{proj}", w, x, xs, ws)


def layer_cases(base: int, layer: int, p_zero: float = P_ZERO_2B4T) -> list[TernaryCase]:
    """The seven projections of one layer, one seed block each."""
    return [ternary_case(base, layer, i, r, c, p_zero, f"L{layer}.{n}")
            for i, (n, r, c) in enumerate(PROJECTIONS)]


def decode_step_shapes() -> list[tuple[int, int, str, int, int]]:
    """(layer, proj, name, rows, cols) for all 210 ternary matrices of one decode step."""
    return [(l, i, n, r, c) for l in range(N_LAYERS) for i, (n, r, c) in enumerate(PROJECTIONS)]


def small_batch_x(seed: int, batch: int, cols: int) -> tuple[np.ndarray, np.ndarray]:
    """batch activations int8[batch, cols] (each absmax-quantised on its own) and their scales."""
    xs = np.empty((batch, cols), dtype=np.int8)
    sc = np.empty(batch, dtype=np.float32)
    for t in range(batch):
        xs[t], sc[t] = activation(seed + 1000003 * t, cols)
    return xs, sc


def head_case(seed: int, rows: int = VOCAB, cols: int = HIDDEN) -> tuple[np.ndarray, np.ndarray]:
    """bf16 W [rows, cols] ~ N(0, 0.02) and bf16 x [cols] ~ N(0, 1) as uint16 bit patterns."""
    w = normal_bf16(seed, (rows, cols), 0.0, HEAD_STD)
    x = normal_bf16(seed + 1, cols, 0.0, 1.0)
    return w, x
