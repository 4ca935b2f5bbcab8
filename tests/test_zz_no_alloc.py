"""The plane-at-a-time call with the library's static windows, through the C
ABI, against the same call with caller-owned windows: bit-exact outputs, two
calls in a row (the second on a smaller geometry, so the array holds the
first call's bytes), both modes.  Also the size limit, refused before any
launch with real device buffers."""
import numpy as np
import pytest
import torch

import gpu_helpers as H
from sequence_attention_relayout_amd import ulysses as U
from sequence_attention_relayout_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def bits(t):
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()])


def static_equals_windows(world, b, d, seq, head, dt, seed):
    H.say(f"case: static windows W={world} b={b} d={d} {dt} seq={seq} head={head}")
    probe = U.ulysses_plan_create(world, b, d, seq, head, dt)
    cap = max(U.ulysses_plan_window_bytes(probe, 0), U.ulysses_plan_window_bytes(probe, 1))
    plan = U.ulysses_plan_create(world, b, d, seq, head, dt, cap)
    wl = W.Workload("static windows", world, b, d, seq, head)
    for mode in (0, 1):
        xs = W.make_shards(wl, mode, dt, seed + mode, DEV)
        shapes = [U.ulysses_plan_shape(plan, mode, r, True) for r in range(world)]
        win = [torch.empty(max(1, U.ulysses_plan_window_bytes(plan, mode)), dtype=torch.uint8,
                           device=DEV) for _ in range(world)]
        want = H.Guarded(shapes, dt, DEV)
        U.ulysses_a2a_4d_chunked(plan, mode, xs, want.views, win)
        got = H.Guarded(shapes, dt, DEV)
        U.ulysses_a2a_4d_chunked_static(plan, mode, xs, got.views)
        torch.cuda.synchronize()
        assert want.guards_intact() and got.guards_intact()
        for w, g in zip(want.views, got.views):
            assert torch.equal(bits(w), bits(g))


def test_static_windows_equal_caller_windows_twice():
    # the first call fills most of the 64 MiB array (4 windows of 14.3 MB);
    # the second, smaller one runs over what the first left there
    static_equals_windows(4, 3, 128, [1000] * 4, [14] * 4, "bf16", 600)
    static_equals_windows(3, 2, 64, [37, 250, 9], [3, 1, 5], "fp32", 610)


def test_static_windows_refuse_plans_beyond_the_array():
    """Five windows of 14.3 MB exceed 64 MiB: EWINDOW before any launch."""
    seq, head = [1000] * 5, [14] * 5
    plan = U.ulysses_plan_create(5, 1, 128, seq, head, "bf16", 1 << 30)
    wl = W.Workload("too big", 5, 1, 128, seq, head)
    xs = W.make_shards(wl, 0, "bf16", 620, DEV)
    ys = [torch.empty(U.ulysses_plan_shape(plan, 0, r, True), dtype=torch.bfloat16, device=DEV)
          for r in range(5)]
    with pytest.raises(U.UlyssesError) as e:
        U.ulysses_a2a_4d_chunked_static(plan, 0, xs, ys)
    assert e.value.code == -4 and "static window array" in str(e.value)
