"""The no-allocation layout entry point (moe_layout_noalloc), through the C ABI.

Its histogram scratch lives in the library's per-device static array, so it
calls no allocator.  Its handle must equal moe_layout's field for field, bit
for bit, on two calls in a row on one handle (the second with fewer tokens:
the static array keeps the first call's contents), and the row calls on it
must give the same rows.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
import combine_moe_layout_04_amd as M
from combine_moe_layout_04_amd._lib import lib

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
FIELDS = ["num_tokens_per_expert", "num_tokens_per_rank", "is_token_in_rank", "expert_offset",
          "rank_offset", "send_offset", "token_slot", "recv_pos", "recv_token", "recv_k", "status",
          "send_token"]


def say(msg):
    print(msg, flush=True)


def noalloc_layout(h, idx, E, P, ws):
    """moe_layout_noalloc on handle h, straight through ctypes."""
    T, K = idx.shape
    itype = 0 if idx.dtype == torch.int32 else 1
    stream = torch.cuda.current_stream(DEV).cuda_stream
    rc = lib().moe_layout_noalloc(h.ptr, ctypes.c_void_p(idx.data_ptr()), itype, T, K, E, P,
                                  ctypes.c_void_p(ws.data_ptr()), ws.numel(), ctypes.c_void_p(stream))
    assert rc == 0, lib().moe_strerror(rc)
    h.workspace, h.T, h.K, h.E, h.P, h.device = ws, T, K, E, P, DEV
    n = ctypes.c_int64(0)
    assert lib().moe_recv_capacity(h.ptr, ctypes.byref(n)) == 0
    h.R = n.value
    return h


@pytest.mark.parametrize("name,T2,pad", [("qwen3_30b_a3b", 1500, 1), ("deepseek_v3", 777, 1),
                                         ("tiny", 100, 1), ("qwen3_30b_a3b", 2049, 16)])
def test_noalloc_layout_matches_moe_layout(name, T2, pad):
    cfg = W.get_config(name)
    ws = torch.empty(M.moe_workspace_size(cfg.T, cfg.K, cfg.E, cfg.P, pad), dtype=torch.uint8, device=DEV)
    h_na = M.Handle(pad_multiple=pad)
    for T, seed in ((cfg.T, 21), (T2, 22)):   # the second call with a smaller input
        say(f"noalloc layout {name} T={T} pad={pad}")
        c = W.get_config(name, T=T)
        inp = W.layer_inputs(c, seed=seed)
        idx = torch.from_numpy(inp.topk_idx).to(DEV)
        ref = M.moe_layout(idx, c.E, c.P, handle=M.Handle(pad_multiple=pad))
        noalloc_layout(h_na, idx, c.E, c.P, ws)
        n_send = int(ref.field("send_offset")[-1].item())
        for f in FIELDS:
            a, b = h_na.field(f), ref.field(f)
            if f == "send_token":   # rows past send_offset[P] are unspecified
                a, b = a[:n_send], b[:n_send]
            assert torch.equal(a, b), f
        assert h_na.check() == 0
        # the row calls read the no-allocation handle like any other
        x = torch.from_numpy(inp.x.view(np.int16) if c.dtype == "bf16" else inp.x).to(DEV)
        if c.dtype == "bf16":
            x = x.view(torch.bfloat16)
        w = torch.from_numpy(inp.topk_weights).to(DEV)
        r1, s1 = M.moe_dispatch(ref, x, w, recv_scores=True)
        r2, s2 = M.moe_dispatch(h_na, x, w, recv_scores=True)
        rows = int(ref.field("expert_offset")[-1].item())  # rows past the last segment are not written
        iv = torch.int16 if c.dtype == "bf16" else torch.int32
        assert torch.equal(r1[:rows].view(iv), r2[:rows].view(iv))
        assert torch.equal(s1[:rows], s2[:rows])


def test_python_binding_of_the_noalloc_layout():
    """M.moe_layout_noalloc: the same handle as M.moe_layout, and, given a
    workspace, no new tensor from torch's allocator on either call."""
    cfg = W.get_config("qwen3_30b_a3b")
    ws = torch.empty(M.moe_workspace_size(cfg.T, cfg.K, cfg.E, cfg.P), dtype=torch.uint8, device=DEV)
    h = M.Handle()
    for T, seed in ((cfg.T, 31), (1234, 32)):
        say(f"python noalloc layout T={T}")
        c = W.get_config("qwen3_30b_a3b", T=T)
        idx = torch.from_numpy(W.layer_inputs(c, seed=seed, with_rows=False).topk_idx).to(DEV)
        ref = M.moe_layout(idx, c.E, c.P)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated(DEV)
        M.moe_layout_noalloc(idx, c.E, c.P, handle=h, workspace=ws)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated(DEV) == before
        n_send = int(ref.field("send_offset")[-1].item())
        for f in FIELDS:
            a, b = h.field(f), ref.field(f)
            if f == "send_token":
                a, b = a[:n_send], b[:n_send]
            assert torch.equal(a, b), f
        assert h.check() == 0 and h.R == ref.R


def test_noalloc_layout_rejects_what_it_cannot_hold():
    """A shape whose histogram exceeds the static scratch is refused on the
    host (MOE_ERR_SCRATCH), and a short workspace with MOE_ERR_WORKSPACE."""
    L = lib()
    h = M.Handle()
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    T, K, E, P = 1 << 21, 1, 1024, 64      # 2048 tiles x 1089 columns x 4 bytes > the maximum
    fake = ctypes.c_void_p(1 << 20)         # never dereferenced: the call fails before any launch
    assert L.moe_layout_noalloc(h.ptr, fake, 0, T, K, E, P, fake, 1 << 40, stream) == -8
    idx = torch.zeros((64, 2), dtype=torch.int32, device=DEV)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    assert L.moe_layout_noalloc(h.ptr, ctypes.c_void_p(idx.data_ptr()), 0, 64, 2, 8, 2,
                                ctypes.c_void_p(ws.data_ptr()), ws.numel(), stream) == -5
    assert b"static" in L.moe_strerror(-8)
