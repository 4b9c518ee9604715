"""The error word of the RWKV-4 workspaces (the first 32-bit word).

Bit 1, a tile claim that found a workspace never zero-filled (the rows of
that tile are NaN), is forced from the host with every wait left untouched:
the workspace gets a zero header and ticket counters that hold a later tag
than any call makes, and tiles are claimed (the claim override), so every
claim fails at once and each workgroup writes NaN over the rows its launch
index names and returns before any look-back.

Bit 0, a look-back that reached its spin limit (its tile's rows are NaN), is
forced with the spin-limit override at one poll: on 128 tiles per channel
block the later tiles cannot see an inclusive history within their window in
two polls, so they give up at once.

In the backward, gw and gu (sums over every tile) are NaN in the channels of
a tile that gave up or was never claimed.  Zero-filling the workspace clears the word, and the next call on it
(with the default limit) is right again."""
import numpy as np
import pytest

import linear_attention_sequence_rwkv_amd as rw
import oracle.wkv_oracle as O
import synth
from wkv_testutil import WKV4_TOL, log, to_dev, torch_dev, tuned, wkv4_scaled_err

pytestmark = pytest.mark.gpu

HEADER_BYTES = 128    # error word, epoch, claim count
COUNTER_STRIDE = 128  # one 64-bit ticket counter per (sequence, channel block)
# tag 0xFFFFFFFF (later than any call's), count 5, as a signed 64-bit value
POISON = (0xFFFFFFFF << 32 | 5) - (1 << 64)


def _poisoned(torch, nbytes, B, C, dev):
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    n_ctr = B * ((C + 63) // 64)
    assert HEADER_BYTES + n_ctr * COUNTER_STRIDE <= nbytes
    idx = (HEADER_BYTES + COUNTER_STRIDE * torch.arange(n_ctr, device=dev)) // 8
    ws.view(torch.int64)[idx] = POISON
    return ws


def test_forward_flags_a_workspace_never_zero_filled():
    torch, dev = torch_dev()
    inp = synth.wkv4_inputs(2, 300, 200, seed=91)
    B, T, C = inp["k"].shape
    t = {n: to_dev(inp[n]) for n in ("w", "u", "k", "v")}
    need = rw.rwkv_wkv4_forward_workspace(B, T, C)
    ws = _poisoned(torch, need, B, C, dev)
    with tuned(wkv4_claim=True):
        log(f"wkv4_forward {B}x{T}x{C} on a workspace with foreign ticket counters")
        y = rw.rwkv_wkv4_forward(t["w"], t["u"], t["k"], t["v"], ws=ws)
        torch.cuda.synchronize()
        assert rw.rwkv_wkv4_workspace_error(ws) == 2
        assert torch.isnan(y).all().item()
        log("  zero-filled, again")
        ws.zero_()
        y = rw.rwkv_wkv4_forward(t["w"], t["u"], t["k"], t["v"], ws=ws)
        torch.cuda.synchronize()
        assert rw.rwkv_wkv4_workspace_error(ws) == 0
    y_ref, _ = O.wkv4_recurrent(inp["w"], inp["u"], inp["k"], inp["v"])
    S = O.wkv4_scale(inp["w"], inp["u"], inp["k"], inp["v"])
    assert wkv4_scaled_err(y.cpu().numpy(), y_ref, S) <= WKV4_TOL


def test_backward_flags_a_workspace_never_zero_filled():
    torch, dev = torch_dev()
    e = synth.wkv4_backward_inputs(2, 300, 200, seed=92)
    B, T, C = e["k"].shape
    t = {n: to_dev(e[n]) for n in ("w", "u", "k", "v", "gy")}
    args = (t["w"], t["u"], t["k"], t["v"], t["gy"])
    need = rw.rwkv_wkv4_backward_workspace(B, T, C)
    ws = _poisoned(torch, need, B, C, dev)
    with tuned(wkv4_claim=True):
        log(f"wkv4_backward {B}x{T}x{C} on a workspace with foreign ticket counters")
        gw, gu, gk, gv = rw.rwkv_wkv4_backward(*args, ws=ws)
        torch.cuda.synchronize()
        assert rw.rwkv_wkv4_workspace_error(ws) == 2
        for g in (gw, gu, gk, gv):
            assert torch.isnan(g).all().item()
        log("  zero-filled, again")
        ws.zero_()
        got = rw.rwkv_wkv4_backward(*args, ws=ws)
        torch.cuda.synchronize()
        assert rw.rwkv_wkv4_workspace_error(ws) == 0
        fresh = rw.rwkv_wkv4_backward(*args, ws=torch.zeros_like(ws))
        torch.cuda.synchronize()
    for a, b in zip(got, fresh):
        assert torch.equal(a, b)
        assert torch.isfinite(a).all().item()


def test_forward_look_back_that_gives_up_sets_bit_0():
    torch, dev = torch_dev()
    inp = synth.wkv4_inputs(1, 16384, 256, seed=93)
    B, T, C = inp["k"].shape
    t = {n: to_dev(inp[n]) for n in ("w", "u", "k", "v")}
    ws = torch.zeros(rw.rwkv_wkv4_forward_workspace(B, T, C), dtype=torch.uint8, device=dev)
    with tuned(wkv4_spin=1):
        log(f"wkv4_forward {B}x{T}x{C} with a one-poll look-back limit")
        y = rw.rwkv_wkv4_forward(t["w"], t["u"], t["k"], t["v"], ws=ws)
        torch.cuda.synchronize()
        err = rw.rwkv_wkv4_workspace_error(ws)
        assert err & 1, err
        assert torch.isnan(y).any().item()
    log("  zero-filled, default limit")
    ws.zero_()
    y = rw.rwkv_wkv4_forward(t["w"], t["u"], t["k"], t["v"], ws=ws)
    torch.cuda.synchronize()
    assert rw.rwkv_wkv4_workspace_error(ws) == 0
    y_ref, _ = O.wkv4_recurrent(inp["w"], inp["u"], inp["k"], inp["v"])
    S = O.wkv4_scale(inp["w"], inp["u"], inp["k"], inp["v"])
    assert wkv4_scaled_err(y.cpu().numpy(), y_ref, S) <= WKV4_TOL


def test_backward_look_back_that_gives_up_sets_bit_0():
    torch, dev = torch_dev()
    e = synth.wkv4_backward_inputs(1, 16384, 256, seed=94)
    B, T, C = e["k"].shape
    t = {n: to_dev(e[n]) for n in ("w", "u", "k", "v", "gy")}
    args = (t["w"], t["u"], t["k"], t["v"], t["gy"])
    ws = torch.zeros(rw.rwkv_wkv4_backward_workspace(B, T, C), dtype=torch.uint8, device=dev)
    with tuned(wkv4_spin=1):
        log(f"wkv4_backward {B}x{T}x{C} with a one-poll look-back limit")
        gw, gu, gk, gv = rw.rwkv_wkv4_backward(*args, ws=ws)
        torch.cuda.synchronize()
        err = rw.rwkv_wkv4_workspace_error(ws)
        assert err & 1, err
        assert torch.isnan(gk).any().item()
        # the channels of tiles that gave up
        gave_up = torch.isnan(gk).any(dim=1).any(dim=0)
        assert torch.isnan(gw)[gave_up].all().item() and torch.isnan(gu)[gave_up].all().item()
    log("  zero-filled, default limit")
    ws.zero_()
    got = rw.rwkv_wkv4_backward(*args, ws=ws)
    torch.cuda.synchronize()
    assert rw.rwkv_wkv4_workspace_error(ws) == 0
    fresh = rw.rwkv_wkv4_backward(*args, ws=torch.zeros_like(ws))
    torch.cuda.synchronize()
    for a, b in zip(got, fresh):
        assert torch.equal(a, b)
        assert torch.isfinite(a).all().item()
