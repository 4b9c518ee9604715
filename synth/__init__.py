"""Seeded synthetic inputs for the WKV operators.

This module only draws random numbers and casts them. It holds none of the
operator's arithmetic, so that both the fp64 oracle and the HIP path can be
fed from it without sharing any of the method.

Recipe (the same for every caller):

* Generator: ``numpy.random.Generator(PCG64(seed))``.
* Draw order: omega, u, k, v, then r (Eagle only).  Every draw is float64
  ``standard_normal`` / ``uniform``, scaled, then cast.
* RWKV-4: ``w = exp(omega)`` (the positive decay rate; the per-step factor is
  ``exp(-w)``), then everything is cast to float32 with round-to-nearest-even.
* Eagle: ``w = exp(-exp(omega))`` in (0, 1], cast to float32.  ``r, k, v``
  are cast float64 -> float32 -> bfloat16 with round-to-nearest-even and are
  returned both as raw bf16 bit patterns (uint16) and as the exact float32
  values those bits encode.
* Finch: the Eagle recipe, then a per-token decay w_t = exp(-exp(omega +
  delta_t)) with delta_t ~ N(0, delta_std) [B, T, H, D] drawn after r (a
  synthetic stand-in for the data-dependent correction), cast to float32.
* RWKV-4 backward: the upstream gradient gy ~ N(0, 1) [B, T, C] comes from
  its own generator, ``PCG64(seed + 100000)``, so the forward inputs of a
  seed are unchanged.
* "N(0, s)" means standard deviation ``s``.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = [
    "Wkv4Config", "Wkv4StepConfig", "Wkv5Config",
    "CFG_WKV4_TINY", "CFG_WKV4_169M", "CFG_WKV4_LONG", "CFG_WKV4_DECODE",
    "CFG_WKV5_EAGLE", "CFG_WKV5_DECODE", "Wkv5StepConfig",
    "rng_for", "wkv4_inputs", "wkv4_step_inputs", "wkv5_inputs", "wkv5_step_inputs",
    "wkv4_backward_inputs", "wkv6_inputs", "CFG_WKV6_FINCH",
    "bf16_bits_from_f32", "f32_from_bf16_bits",
]


@dataclasses.dataclass(frozen=True)
class Wkv4Config:
    name: str
    B: int
    T: int
    C: int
    seed: int
    omega_lo: float = -3.0
    omega_hi: float = 1.0
    u_std: float = 0.5
    k_std: float = 1.0
    v_std: float = 1.0


@dataclasses.dataclass(frozen=True)
class Wkv4StepConfig:
    name: str
    B: int
    C: int
    steps: int
    pool: int
    seed: int
    omega_lo: float = -3.0
    omega_hi: float = 1.0
    u_std: float = 0.5


@dataclasses.dataclass(frozen=True)
class Wkv5Config:
    name: str
    B: int
    T: int
    H: int
    D: int
    seed: int
    omega_lo: float = -6.0
    omega_hi: float = 0.0
    u_std: float = 0.5


@dataclasses.dataclass(frozen=True)
class Wkv5StepConfig:
    name: str
    B: int
    H: int
    D: int
    steps: int
    pool: int
    seed: int


# The workloads.  Seeds are 1000 + workload number.
CFG_WKV4_TINY = Wkv4Config("wkv4_fwd_B1_T64_C64", 1, 64, 64, 1001)
CFG_WKV4_169M = Wkv4Config("wkv4_fwd_B8_T1024_C768", 8, 1024, 768, 1002)
CFG_WKV4_LONG = Wkv4Config("wkv4_fwd_B1_T65536_C5120", 1, 65536, 5120, 1003,
                           omega_lo=-5.0, omega_hi=2.0, u_std=1.0, k_std=3.0)
# Decode: 4096 steps for 256 streams at C=4096; per-step k, v come from a
# pre-drawn pool of 64 steps (step t uses pool[t % 64]) so that inputs stay
# resident on the device.
CFG_WKV4_DECODE = Wkv4StepConfig("wkv4_step_B256_C4096_x4096", 256, 4096, 4096, 64, 1004)
CFG_WKV5_EAGLE = Wkv5Config("wkv5_fwd_B4_T4096_H32_D64", 4, 4096, 32, 64, 1005)
# Finch forward at the Eagle workload's shape, with per-token decays.
CFG_WKV6_FINCH = Wkv5Config("wkv6_fwd_B4_T4096_H32_D64", 4, 4096, 32, 64, 1007)
# Eagle decode: 64 streams of 32 heads (a 32 MB fp32 state), 256 steps drawn
# from a pool of 16 tokens (step t uses token t mod 16).
CFG_WKV5_DECODE = Wkv5StepConfig("wkv5_step_B64_H32_D64_x256", 64, 32, 64, 256, 16, 1006)


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs here are finite; NaN handling is not needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = (bits + 0x7FFF + lsb) >> 16
    return rounded.astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value encoded by bf16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def _f32(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x.astype(np.float32))


def wkv4_inputs(B: int, T: int, C: int, seed: int, *, omega_lo=-3.0,
                omega_hi=1.0, u_std=0.5, k_std=1.0, v_std=1.0) -> dict:
    """RWKV-4 forward inputs: w, u [C]; k, v [B, T, C]; all float32."""
    rng = rng_for(seed)
    omega = rng.uniform(omega_lo, omega_hi, size=C)
    u = rng.standard_normal(C) * u_std
    k = rng.standard_normal((B, T, C)) * k_std
    v = rng.standard_normal((B, T, C)) * v_std
    return {"w": _f32(np.exp(omega)), "u": _f32(u), "k": _f32(k), "v": _f32(v)}


def wkv4_inputs_for(cfg: Wkv4Config) -> dict:
    return wkv4_inputs(cfg.B, cfg.T, cfg.C, cfg.seed, omega_lo=cfg.omega_lo,
                       omega_hi=cfg.omega_hi, u_std=cfg.u_std,
                       k_std=cfg.k_std, v_std=cfg.v_std)


def wkv4_backward_inputs(B: int, T: int, C: int, seed: int, **kw) -> dict:
    """Forward inputs of ``wkv4_inputs`` plus an upstream gradient ``gy``."""
    out = wkv4_inputs(B, T, C, seed, **kw)
    out["gy"] = _f32(rng_for(seed + 100000).standard_normal((B, T, C)))
    return out


def wkv4_step_inputs(B: int, C: int, pool: int, seed: int, *, omega_lo=-3.0,
                     omega_hi=1.0, u_std=0.5) -> dict:
    """RWKV-4 decode inputs: w, u [C]; a pool of k, v [pool, B, C]."""
    rng = rng_for(seed)
    omega = rng.uniform(omega_lo, omega_hi, size=C)
    u = rng.standard_normal(C) * u_std
    k = rng.standard_normal((pool, B, C))
    v = rng.standard_normal((pool, B, C))
    return {"w": _f32(np.exp(omega)), "u": _f32(u), "k": _f32(k), "v": _f32(v)}


def wkv5_inputs(B: int, T: int, H: int, D: int, seed: int, *, omega_lo=-6.0,
                omega_hi=0.0, u_std=0.5) -> dict:
    """Eagle inputs.

    Returns ``w, u`` [H, D] float32, and for each of ``r, k, v`` [B, T, H, D]
    both ``<name>_bits`` (uint16 bf16 patterns) and ``<name>`` (float32 values
    of those bits).  r, k, v ~ N(0, 1) / sqrt(D).
    """
    rng = rng_for(seed)
    omega = rng.uniform(omega_lo, omega_hi, size=(H, D))
    u = rng.standard_normal((H, D)) * u_std
    out = {"w": _f32(np.exp(-np.exp(omega))), "u": _f32(u)}
    scale = 1.0 / np.sqrt(D)
    for name in ("k", "v", "r"):
        x = _f32(rng.standard_normal((B, T, H, D)) * scale)
        bits = bf16_bits_from_f32(x)
        out[name + "_bits"] = bits
        out[name] = f32_from_bf16_bits(bits)
    return out


def wkv6_inputs(B: int, T: int, H: int, D: int, seed: int, *, omega_lo=-6.0, omega_hi=0.0,
                u_std=0.5, delta_std=0.5) -> dict:
    """Finch inputs: the Eagle recipe plus ``wt`` [B, T, H, D] float32, the
    per-token decay factors (``w`` stays the static part's factor)."""
    rng = rng_for(seed)
    omega = rng.uniform(omega_lo, omega_hi, size=(H, D))
    u = rng.standard_normal((H, D)) * u_std
    out = {"w": _f32(np.exp(-np.exp(omega))), "u": _f32(u)}
    scale = 1.0 / np.sqrt(D)
    for name in ("k", "v", "r"):
        x = _f32(rng.standard_normal((B, T, H, D)) * scale)
        bits = bf16_bits_from_f32(x)
        out[name + "_bits"] = bits
        out[name] = f32_from_bf16_bits(bits)
    delta = rng.standard_normal((B, T, H, D)) * delta_std
    out["wt"] = _f32(np.exp(-np.exp(omega[None, None] + delta)))
    return out


def wkv5_step_inputs(cfg: Wkv5StepConfig) -> dict:
    """Eagle decode inputs: the forward recipe with T = pool, so that
    ``r[:, t % pool]`` etc. ([B, H, D]) is the token of step t."""
    return wkv5_inputs(cfg.B, cfg.pool, cfg.H, cfg.D, cfg.seed)


def wkv5_inputs_for(cfg: Wkv5Config) -> dict:
    return wkv5_inputs(cfg.B, cfg.T, cfg.H, cfg.D, cfg.seed,
                       omega_lo=cfg.omega_lo, omega_hi=cfg.omega_hi,
                       u_std=cfg.u_std)
