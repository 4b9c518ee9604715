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
    "CFG_WKV5_EAGLE", "CFG_WKV5_EAGLE_WIDE", "CFG_WKV5_DECODE", "Wkv5StepConfig",
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
# The Eagle workload's shape over the wider decay range omega ~ U(-6, 2)
# (w down to exp(-e^2) = 6e-4, |log2 w| up to 10.7): every head has decays
# too fast for the mid-chunk reference.
CFG_WKV5_EAGLE_WIDE = Wkv5Config("wkv5_fwd_B4_T4096_H32_D64_omega-6to2", 4, 4096, 32, 64, 1008,
                                 omega_lo=-6.0, omega_hi=2.0)
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


def dyadic_matrix_inputs(B: int, T: int, H: int, seed: int, *, per_token_decay=False,
                         seams=(), slow_head=None, fast_head=None, growing_head=None) -> dict:
    """Sparse one-hot inputs for bit-exact checks of the matrix-state paths.

    Every nonzero r, k, v, u is +-1/2, +-1 or +-2 and every decay factor is 1,
    1/2 or 1/4 (Eagle w [H, D]; with ``per_token_decay`` a Finch w_t
    [B, T, H, D]), plus (Eagle) 1/16 on some key rows of ``slow_head``, 2^-16
    on some of ``fast_head`` and a factor 2 (a growing row, outside the
    pages' (0, 1)) on one of ``growing_head``, or (Finch) a few factors
    2^-16.  Per (batch, head):

    * each key row i is written by at most one token (k one-hot at i, v
      one-hot at a column j), so every state entry is a single term;
    * a token reads at most one row (r one-hot), so every output sum has at
      most one nonzero term (the read row's entry, or the token's own bonus
      when it reads the row it writes);
    * a row that decays is read only a few decay steps after its write, and
      a write that is still in the final state is either a few steps old or
      old enough to have decayed below 2^-160.

    Every exact result is then a power of two times +-1 inside the normal
    float32 range, or zero: a correct kernel reproduces it bit for bit.
    Writes and reads are placed at chunk edges (0, 31, 32, 63, 64, ...), at
    the ``seams`` given (and one token to either side) and at random.

    Returns the Eagle/Finch input dict (``w`` [H, D] or ``wt`` [B, T, H, D],
    ``u``, and ``r/k/v`` with their ``_bits``).
    """
    D = 64
    rng = rng_for(seed)
    vals = np.array([0.5, 1.0, 2.0])

    def pm(shape=None):
        return rng.choice(vals, size=shape) * rng.choice([-1.0, 1.0], size=shape)

    # Row kinds per (h, i).  reach: decay steps after a write within which it
    # may be read; keep: a write still in the final state must be at most
    # `reach` or at least `gone` steps old.
    if per_token_decay:
        # 0: no decay; 1: w_t in {1/4, 1/2}; 2: w_t in {1/4, 1/2, 1};
        # 3: mostly 1/2 with some 2^-16
        n_kinds = 4
        reach = {0: 10 ** 9, 1: 30, 2: 30, 3: 6}
        gone = {0: None, 1: 160, 2: None, 3: 160}
    else:
        # 0: w = 1; 1: w = 1/2; 2: w = 1/4; 3: w = 1/16 (slow_head only);
        # 4: w = 2^-16 (fast_head only); 5: w = 2 (growing_head only: written
        # only within its reach of the end, read within it)
        n_kinds = 3
        reach = {0: 10 ** 9, 1: 60, 2: 30, 3: 7, 4: 3, 5: 20}
        gone = {0: None, 1: 160, 2: 80, 3: 40, 4: 10, 5: None}
    kind = rng.integers(0, n_kinds, size=(H, D))
    if not per_token_decay:
        if slow_head is not None:
            kind[slow_head, rng.permutation(D)[:8]] = 3
        if fast_head is not None:
            kind[fast_head, rng.permutation(D)[:8]] = 4
        if growing_head is not None:
            kind[growing_head, rng.integers(D)] = 5
    u = pm((H, D))
    r = np.zeros((B, T, H, D))
    k = np.zeros((B, T, H, D))
    v = np.zeros((B, T, H, D))
    if per_token_decay:
        wt = np.ones((B, T, H, D))
        for h in range(H):
            for i in range(D):
                kd = kind[h, i]
                if kd == 1:
                    wt[:, :, h, i] = rng.choice([0.25, 0.5], size=(B, T))
                elif kd == 2:
                    wt[:, :, h, i] = rng.choice([0.25, 0.5, 1.0], size=(B, T))
                elif kd == 3:
                    wt[:, :, h, i] = np.where(rng.random((B, T)) < 0.05, 2.0 ** -16, 0.5)
    else:
        w = np.choose(kind, [1.0, 0.5, 0.25, 0.0625, 2.0 ** -16, 2.0])

    special = set()
    for e in (0, 31, 32, 63, 64, 95, 96, 127, 128, 191, 192, T - 2, T - 1):
        special.add(e)
    for s in seams:
        special.update((s - 1, s, s + 1))
    special = sorted(x for x in special if 0 <= x < T)

    for b in range(B):
        for h in range(H):
            rows = rng.permutation(D)
            n_w = min(D, max(1, T // 3))
            times = list(special) + list(rng.permutation(T))
            writer_t, used = {}, set()
            for t in times:
                if len(writer_t) >= n_w:
                    break
                if t in used:
                    continue
                i = int(rows[len(writer_t)])
                age = T - 1 - t
                kd = int(kind[h, i])
                if age > reach[kd] and (gone[kd] is None or age < gone[kd]):
                    continue  # would leave an unrepresentable entry in the final state
                writer_t[i] = t
                used.add(t)
                k[b, t, h, i] = pm()
                v[b, t, h, rng.integers(D)] = pm()
            # readers: the writer itself (bonus), the next token, the edge of
            # the reach, across the next chunk edge, and rows never written
            reader = {}
            for i, t0 in writer_t.items():
                rc = reach[int(kind[h, i])]
                nxt_edge = (t0 // 32 + 1) * 32
                for t in (t0, t0 + 1, t0 + 1 + min(rc, 10 ** 6), nxt_edge, t0 + 1 + rc // 2):
                    if t0 <= t < T and t - 1 - t0 <= rc and t not in reader:
                        reader[t] = i
                        break
                for t in (t0 + 1, nxt_edge, nxt_edge + 1):
                    if t0 < t < T and t - 1 - t0 <= rc and t not in reader:
                        reader[t] = i
                        break
            unwritten = [i for i in range(D) if i not in writer_t]
            for t in rng.permutation(T)[: max(1, T // 8)]:
                if t not in reader and unwritten:
                    reader[int(t)] = int(rng.choice(unwritten))
            for t, i in reader.items():
                r[b, t, h, i] = pm()

    out = {"u": _f32(u)}
    if per_token_decay:
        out["wt"] = _f32(wt)
        out["w"] = _f32(np.ones((H, D)))
    else:
        out["w"] = _f32(w)
    for name, x in (("r", r), ("k", k), ("v", v)):
        bits = bf16_bits_from_f32(_f32(x))
        out[name + "_bits"] = bits
        out[name] = f32_from_bf16_bits(bits)
    return out
