"""The seeded input generators shared by the oracle tests, the GPU tests and
the bench (`synth/`): deterministic per seed, of the stated shapes, types and
ranges, and with bf16 values rounded to nearest, ties to even."""
import numpy as np
import pytest

import synth


def test_same_seed_same_inputs_other_seed_other_inputs():
    a = synth.wkv4_backward_inputs(2, 50, 7, seed=5)
    b = synth.wkv4_backward_inputs(2, 50, 7, seed=5)
    c = synth.wkv4_backward_inputs(2, 50, 7, seed=6)
    for n in ("w", "u", "k", "v", "gy"):
        assert np.array_equal(a[n], b[n])
        assert not np.array_equal(a[n], c[n])
    e1 = synth.wkv6_inputs(1, 20, 2, 64, seed=9)
    e2 = synth.wkv6_inputs(1, 20, 2, 64, seed=9)
    for n in ("w", "u", "r_bits", "k_bits", "v_bits", "wt"):
        assert np.array_equal(e1[n], e2[n])


def test_wkv4_shapes_types_and_decay_range():
    lo, hi = -5.0, 2.0
    e = synth.wkv4_backward_inputs(3, 40, 9, seed=1, omega_lo=lo, omega_hi=hi)
    assert e["w"].shape == e["u"].shape == (9,)
    for n in ("k", "v", "gy"):
        assert e[n].shape == (3, 40, 9)
    for x in e.values():
        assert x.dtype == np.float32 and x.flags["C_CONTIGUOUS"]
    # w = e^omega, omega ~ U(lo, hi): a positive rate
    assert np.all(e["w"] >= np.float32(np.exp(lo))) and np.all(e["w"] <= np.float32(np.exp(hi)))
    # the gradient has its own generator: not a copy of k or v
    assert not np.array_equal(e["gy"], e["k"]) and not np.array_equal(e["gy"], e["v"])


@pytest.mark.parametrize("gen", ["wkv5", "wkv6"])
def test_matrix_state_shapes_types_and_decay_range(gen):
    B, T, H, D = 2, 30, 3, 64
    make = synth.wkv5_inputs if gen == "wkv5" else synth.wkv6_inputs
    e = make(B, T, H, D, seed=3)
    assert e["w"].shape == e["u"].shape == (H, D)
    for n in ("r", "k", "v"):
        assert e[n].shape == e[n + "_bits"].shape == (B, T, H, D)
        assert e[n + "_bits"].dtype == np.uint16 and e[n].dtype == np.float32
        # the float values are exactly the bf16 patterns the kernels read
        assert np.array_equal(e[n], synth.f32_from_bf16_bits(e[n + "_bits"]))
        # N(0, 1) / sqrt(D): a loose check of the scale
        assert 0.08 < float(np.std(e[n])) < 0.17
    # w = exp(-exp(omega)), omega ~ U(-6, 0): in [e^-1, e^-e^-6]
    assert np.all(e["w"] > 0.36) and np.all(e["w"] <= 1.0)
    if gen == "wkv6":
        assert e["wt"].shape == (B, T, H, D) and e["wt"].dtype == np.float32
        assert np.all(e["wt"] > 0.0) and np.all(e["wt"] <= 1.0)


def test_bf16_rounding_is_nearest_ties_to_even():
    one = 0x3F80
    cases = {
        1.0: one,
        1.0 + 2.0 ** -8: one,           # half way, 0x3F80 is even: down
        1.0 + 3 * 2.0 ** -8: one + 2,   # half way, 0x3F82 is even: up
        1.0 + 2.0 ** -8 + 2.0 ** -20: one + 1,  # above half way: up
        -1.0 - 3 * 2.0 ** -8: 0x8000 | (one + 2),
        0.0: 0x0000,
    }
    x = np.array(list(cases), dtype=np.float32)
    assert list(synth.bf16_bits_from_f32(x)) == list(cases.values())
    # values already in bf16 round-trip unchanged
    b = np.arange(0x3000, 0x4800, 7, dtype=np.uint16)
    assert np.array_equal(synth.bf16_bits_from_f32(synth.f32_from_bf16_bits(b)), b)


def test_named_workloads_have_the_stated_sizes():
    assert (synth.CFG_WKV4_169M.B, synth.CFG_WKV4_169M.T, synth.CFG_WKV4_169M.C) == (8, 1024, 768)
    assert (synth.CFG_WKV4_LONG.B, synth.CFG_WKV4_LONG.T, synth.CFG_WKV4_LONG.C) == (1, 65536, 5120)
    for cfg in (synth.CFG_WKV5_EAGLE, synth.CFG_WKV5_EAGLE_WIDE, synth.CFG_WKV6_FINCH):
        assert (cfg.B, cfg.T, cfg.H, cfg.D) == (4, 4096, 32, 64)
    assert (synth.CFG_WKV5_EAGLE_WIDE.omega_lo, synth.CFG_WKV5_EAGLE_WIDE.omega_hi) == (-6.0, 2.0)
    seeds = [c.seed for c in (synth.CFG_WKV4_TINY, synth.CFG_WKV4_169M, synth.CFG_WKV4_LONG,
                              synth.CFG_WKV4_DECODE, synth.CFG_WKV5_EAGLE, synth.CFG_WKV5_DECODE,
                              synth.CFG_WKV6_FINCH, synth.CFG_WKV5_EAGLE_WIDE)]
    assert len(set(seeds)) == len(seeds)
