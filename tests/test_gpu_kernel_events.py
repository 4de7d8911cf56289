"""The measurement hook moe_time_next_kernel: the next kernel a row call
launches records the caller's events around its own execution.  The results
stay bit-exact, the kernel's interval lies inside the call's, and the hook is
one-shot."""
import numpy as np
import pytest
import torch

import workloads as W
import combine_moe_layout_04_amd as M
from bench import HipEvents

from devutil import to_dev

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_kernel_events_bracket_the_kernel():
    cfg = W.get_config("qwen3_30b_a3b", T=2048)
    inp = W.layer_inputs(cfg, seed=21)
    print(f"kernel events: T={cfg.T}", flush=True)
    idx = torch.from_numpy(inp.topk_idx).to(DEV)
    w = torch.from_numpy(inp.topk_weights).to(DEV)
    y = to_dev(inp.y, cfg.dtype, DEV)
    h = M.moe_layout(idx, cfg.E, cfg.P)
    ref = M.moe_combine(h, y, w)
    ev = HipEvents(6)
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    ev.record(0, stream)
    M.moe_time_next_kernel(h, ev.ev[2].value, ev.ev[3].value)
    out = M.moe_combine(h, y, w)
    ev.record(1, stream)
    out2 = M.moe_combine(h, y, w)   # the hook was consumed: no event here
    ev.record(4, stream)
    ev.record(5, stream)
    torch.cuda.synchronize()
    call_ms, kern_ms = ev.elapsed_ms(0, 1), ev.elapsed_ms(2, 3)
    ev.close()
    assert 0 < kern_ms <= call_ms, (kern_ms, call_ms)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(out2.view(torch.int16), ref.view(torch.int16))
    assert h.check() == 0


def test_stop_only_events_time_consecutive_kernels():
    """A stop alone binds to the kernel's completion with no marker.  Stream
    order then fixes the timeline: the second call's kernel, timed by its own
    start and stop, lies between the first call's stop and the third's."""
    cfg = W.get_config("qwen3_30b_a3b", T=2048)
    inp = W.layer_inputs(cfg, seed=22)
    print(f"stop-only events: T={cfg.T}", flush=True)
    idx = torch.from_numpy(inp.topk_idx).to(DEV)
    w = torch.from_numpy(inp.topk_weights).to(DEV)
    y = to_dev(inp.y, cfg.dtype, DEV)
    h = M.moe_layout(idx, cfg.E, cfg.P)
    ref = M.moe_combine(h, y, w)
    ev = HipEvents(4)
    torch.cuda.synchronize()
    M.moe_time_next_kernel(h, None, ev.ev[0].value)
    a = M.moe_combine(h, y, w)
    M.moe_time_next_kernel(h, ev.ev[1].value, ev.ev[2].value)
    b = M.moe_combine(h, y, w)
    M.moe_time_next_kernel(h, None, ev.ev[3].value)
    c = M.moe_combine(h, y, w)
    torch.cuda.synchronize()
    kern_ms = ev.elapsed_ms(1, 2)          # the second kernel
    to_second, to_third = ev.elapsed_ms(0, 2), ev.elapsed_ms(0, 3)
    ev.close()
    assert 0 < kern_ms <= to_second < to_third, (kern_ms, to_second, to_third)
    for t in (a, b, c):
        assert torch.equal(t.view(torch.int16), ref.view(torch.int16))
