"""Host ABI checks that pass fake, never-dereferenced device addresses.

Run only in a child process with every GPU hidden (test_host_abi.py starts
it): require_no_device() refuses to go on if a device is visible, and every
call below must fail validation before anything is launched.
"""
import pytest

from sequence_attention_relayout_amd import ulysses as U


def require_no_device():
    import torch
    n = torch.cuda.device_count()
    if n != 0:
        raise SystemExit(f"{n} GPU(s) visible: fake-address checks run only with the GPU hidden")


def expect(code, fn, *args):
    with pytest.raises(U.UlyssesError) as e:
        fn(*args)
    assert e.value.code == code, str(e.value)
    return str(e.value)


# Fake, never-dereferenced device addresses: each call below fails
# validation before any launch.
BASE = 1 << 40


def fake(n, stride=1 << 32, off=0):
    return [BASE + off + i * stride for i in range(n)]


def call_errors_before_launch():
    plan = U.ulysses_plan_create(2, 1, 8, [3, 4], [1, 2], "bf16")
    src, dst = fake(2), fake(2, off=1 << 36)
    expect(-1, U.ulysses_a2a_4d, plan, 2, src, dst, 0)                       # bad mode
    expect(-1, U.ulysses_a2a_4d, plan, 0, [src[0], 0], dst, 0)               # null src
    expect(-2, U.ulysses_a2a_4d, plan, 0, [src[0] + 8, src[1]], dst, 0)      # misaligned
    expect(-2, U.ulysses_a2a_4d, plan, 1, src, [dst[0], dst[1] + 4], 0)
    expect(-5, U.ulysses_a2a_4d, plan, 0, src, [dst[0], src[1] + 16], 0)     # dst on a src
    expect(-5, U.ulysses_a2a_4d, plan, 0, src, [dst[0], dst[0] + 16], 0)     # dst on a dst
    msg = expect(-1, U.ulysses_a2a_4d, plan, 0, src, [dst[0], (1 << 64) - 16], 0)
    assert "past the end of the address space" in msg
    # chunked: no cap, window too small for the cap, window overlapping
    expect(-1, U.ulysses_a2a_4d_chunked, plan, 0, src, dst, fake(2, off=1 << 37), 0)
    small = U.ulysses_plan_create(2, 1, 8, [3, 4], [1, 2], "bf16", 64)
    expect(-4, U.ulysses_a2a_4d_chunked, small, 0, src, dst, fake(2, off=1 << 37), 0)
    capped = U.ulysses_plan_create(2, 1, 8, [3, 4], [1, 2], "bf16", 1 << 20)
    expect(-5, U.ulysses_a2a_4d_chunked, capped, 0, src, dst, [src[0], dst[1] + (1 << 30)], 0)
    expect(-5, U.ulysses_a2a_4d_chunked, capped, 1, src, dst,
           [BASE + (1 << 38), BASE + (1 << 38) + 16], 0)
    # fused: bf16 only, power-of-two d/8, non-null tables, eps >= 0
    f32 = U.ulysses_plan_create(2, 1, 8, [3, 4], [1, 2], "fp32")
    g, t = BASE + (1 << 39), BASE + (1 << 39) + (1 << 30)
    expect(-3, U.ulysses_a2a_4d_qknorm_rope, f32, src, dst, fake(2, off=7 << 33),
           fake(2, off=15 << 33), g, g + 64, 1e-6, t, t + (1 << 28), 0)
    d24 = U.ulysses_plan_create(2, 1, 24, [3, 4], [1, 2], "bf16")
    expect(-1, U.ulysses_a2a_4d_qknorm_rope, d24, src, dst, fake(2, off=7 << 33),
           fake(2, off=15 << 33), g, g + 128, 1e-6, t, t + (1 << 28), 0)
    expect(-1, U.ulysses_a2a_4d_qknorm_rope, plan, src, dst, fake(2, off=7 << 33),
           fake(2, off=15 << 33), g, g + 64, -1.0, t, t + (1 << 28), 0)
    expect(-1, U.ulysses_a2a_4d_qknorm_rope, plan, src, dst, fake(2, off=7 << 33),
           fake(2, off=15 << 33), g, g + 64, 1e-6, 0, t + (1 << 28), 0)
    expect(-5, U.ulysses_a2a_4d_qknorm_rope, plan, src, dst, fake(2, off=7 << 33),
           [g, BASE + (15 << 33)], g + 64, g + 128, 1e-6, t, t + (1 << 28), 0)


def binding_checks_tensor_size_and_device():
    """The C ABI takes bare pointers; the Python binding checks what a
    tensor argument can tell it before any pointer is passed: enough bytes
    for the shard the call touches, contiguity, and a HIP device (a host
    tensor's address would fault the GPU).  Host tensors only here, so every
    call fails before reaching the library."""
    import torch
    plan = U.ulysses_plan_create(2, 1, 8, [3, 4], [1, 2], "bf16", 1 << 20)
    assert plan.shard_bytes(0, False) == [3 * 3 * 8 * 2, 4 * 3 * 8 * 2]
    assert plan.shard_bytes(0, True) == [7 * 1 * 8 * 2, 7 * 2 * 8 * 2]
    xs = [torch.zeros(U.ulysses_plan_shape(plan, 0, r, False), dtype=torch.bfloat16)
          for r in range(2)]
    ys = [torch.zeros(U.ulysses_plan_shape(plan, 0, r, True), dtype=torch.bfloat16)
          for r in range(2)]
    with pytest.raises(ValueError, match=r"src\[0\]: is on cpu"):
        U.ulysses_a2a_4d(plan, 0, xs, ys, 0)
    with pytest.raises(ValueError, match=r"src\[0\]: holds 48 bytes, the call uses 144"):
        U.ulysses_a2a_4d(plan, 0, [xs[0][:, :1], xs[1]], ys, 0)
    with pytest.raises(ValueError, match=r"dst\[1\]: device buffers must be contiguous"):
        U.ulysses_a2a_4d(plan, 0, fake(2), [fake(1)[0], ys[1].transpose(1, 2)], 0)
    with pytest.raises(ValueError, match=r"window\[0\]: holds 2 bytes"):
        U.ulysses_a2a_4d_chunked(plan, 0, fake(2), fake(2, off=1 << 36),
                                 [torch.zeros(1, dtype=torch.bfloat16), fake(1)[0]], 0)
    with pytest.raises(ValueError, match=r"rope_cos: holds 4 bytes"):
        U.ulysses_a2a_4d_qknorm_rope(plan, fake(2), fake(2, off=1 << 36), fake(2, off=1 << 37),
                                     fake(2, off=3 << 36), BASE, BASE + 64, 1e-6,
                                     torch.zeros(1), BASE + 128, 0)


def launch_wider_than_grid_x_refused():
    """8 shards of 2^30 16-byte vectors per plane: one pass needs more than
    2^32 threads along x, which one launch cannot hold; the call refuses
    before launching instead of truncating the block count."""
    plan = U.ulysses_plan_create(8, 1, 8, [1 << 27] * 8, [1] * 8, "bf16")
    assert U.ulysses_plan_bytes(plan, 0) == 2 * (1 << 30) * 8 * 16
    src, dst = fake(8, stride=1 << 35), fake(8, stride=1 << 35, off=1 << 39)
    for mode in (0, 1):
        msg = expect(-1, U.ulysses_a2a_4d, plan, mode, src, dst, 0)
        assert "one launch" in msg


def multi_tensor_errors_before_launch():
    plan = U.ulysses_plan_create(2, 1, 8, [3, 4], [1, 2], "bf16")
    lib = U.library()
    import ctypes
    srcs = [fake(2), fake(2, off=1 << 35)]
    dsts = [fake(2, off=1 << 36), fake(2, off=3 << 35)]
    for n in (0, 5):
        arr = (ctypes.c_void_p * 10)(*([BASE] * 10))
        rc = lib.ulysses_a2a_4d_multi(plan.handle, 0, n, arr, arr, None)
        assert rc == -1 and "ntensors" in U.ulysses_last_error()
    # a destination of tensor 1 on a source of tensor 0
    expect(-5, U.ulysses_a2a_4d_multi, plan, 0, srcs, [dsts[0], [srcs[0][1], dsts[1][1]]], 0)
    # two tensors writing the same destination
    expect(-5, U.ulysses_a2a_4d_multi, plan, 1, srcs, [dsts[0], dsts[0]], 0)
    expect(-2, U.ulysses_a2a_4d_multi, plan, 0, [srcs[0], [srcs[1][0] + 4, srcs[1][1]]], dsts, 0)



def chunked_without_windows_errors_before_launch():
    """The plane-at-a-time call without windows (straight into the
    destination) keeps the cap and the overlap checks."""
    src, dst = fake(2), fake(2, off=1 << 36)
    plan = U.ulysses_plan_create(2, 1, 8, [3, 4], [1, 2], "bf16")
    expect(-1, U.ulysses_a2a_4d_chunked, plan, 0, src, dst, None, 0)      # no cap
    small = U.ulysses_plan_create(2, 1, 8, [3, 4], [1, 2], "bf16", 64)
    expect(-4, U.ulysses_a2a_4d_chunked, small, 0, src, dst, None, 0)     # over the cap
    capped = U.ulysses_plan_create(2, 1, 8, [3, 4], [1, 2], "bf16", 1 << 20)
    expect(-5, U.ulysses_a2a_4d_chunked, capped, 0, src, [dst[0], src[1] + 16], None, 0)
    expect(-2, U.ulysses_a2a_4d_chunked, capped, 1, src, [dst[0] + 8, dst[1]], None, 0)
