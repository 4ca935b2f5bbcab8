"""Host-only checks of libulysses.so: no GPU, nothing is launched.

- the library loads and exports every function include/ulysses.h declares;
- the plan (shapes, window bytes, byte counts) agrees with the oracle on
  random geometries and with the value the FastVideo page prints;
- every validation error is returned before anything is enqueued (the
  calls that pass fake device addresses run in a child process with every
  GPU hidden, tests/fake_address_checks.py);
- the library's rotary table equals the oracle's bit for bit;
- the native plan test replays the kernels' index math over every vector.
"""
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from sequence_attention_relayout_amd import build as ulybuild
from sequence_attention_relayout_amd import ulysses as U

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(U.LIB_PATH):
        ulybuild.build()


def header_functions():
    text = open(os.path.join(ROOT, "include", "ulysses.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ulysses_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = header_functions()
    assert len(names) >= 10
    lib = U.library()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ulysses.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", U.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ulysses_\w+)", out))
    assert set(names) <= exported


def test_native_plan_replay_under_sanitizers():
    """The same replay built with AddressSanitizer and UBSan: no out-of-bounds
    access, overflow or other undefined behaviour in the plan."""
    exe = ulybuild.build_plan_test(sanitize=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert res.returncode == 0, res.stderr[-2000:]
    assert res.stdout.startswith("OK")


def test_plain_c_caller_host_paths():
    """include/ulysses.h compiles as strict C99 (-pedantic -Werror) and a C
    program links and drives the host-side calls and error paths."""
    exe = ulybuild.build_c_check()
    res = subprocess.run([exe, "host"], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stderr
    assert res.stdout.startswith("OK")


def test_native_plan_replay():
    exe = ulybuild.build_plan_test()
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr
    assert res.stdout.startswith("OK")


def rand_geom(rng):
    world = int(rng.integers(1, 9))
    seq = [int(v) for v in rng.integers(0, 50, world)]
    head = [int(v) for v in rng.integers(0, 6, world)]
    if sum(seq) == 0:
        seq[0] = 1
    if sum(head) == 0:
        head[-1] = 1
    return world, int(rng.integers(1, 4)), seq, head


@pytest.mark.parametrize("seed", range(30))
def test_plan_agrees_with_oracle(seed):
    rng = np.random.default_rng(seed)
    world, b, seq, head = rand_geom(rng)
    dt = ["bf16", "fp32", "fp8_e4m3", "int8", "fp16", "uint8", "fp8_e5m2"][seed % 7]
    esz = {"bf16": 2, "fp16": 2, "fp32": 4}.get(dt, 1)
    d = (16 // esz) * int(rng.integers(1, 5))
    plan = U.ulysses_plan_create(world, b, d, seq, head, dt)
    for mode in (0, 1):
        for r in range(world):
            for is_dst in (False, True):
                assert U.ulysses_plan_shape(plan, mode, r, is_dst) == \
                    oracle.shape(mode, b, d, seq, head, r, is_dst)
        assert U.ulysses_plan_window_bytes(plan, mode) == \
            oracle.window_bytes(mode, d, esz, seq, head)
        assert U.ulysses_plan_bytes(plan, mode) == 2 * b * sum(seq) * sum(head) * d * esz


def test_fastvideo_plane_bytes(golden):
    g = golden["fastvideo_window"]
    w = g["world"]
    plan = U.ulysses_plan_create(w, 3, g["d"], [g["s_global"] // w] * w,
                                 [g["n_global"] // w] * w, "bf16", g["window_cap_bytes"])
    for mode in (0, 1):
        assert U.ulysses_plan_window_bytes(plan, mode) == g["bytes_per_plane"]


def test_page_limits(golden):
    lim = golden["limits_021"]
    for w in range(lim["world_min"], lim["world_max"] + 1):
        U.ulysses_plan_create(w, 1, 8, [1] * w, [1] * w, "bf16")
    for w in (lim["world_min"] - 1, lim["world_max"] + 1):
        with pytest.raises(U.UlyssesError) as e:
            U.ulysses_plan_create(w, 1, 8, [1] * w, [1] * w, "bf16")
        assert e.value.code == -1
    for dt, m in lim["min_d_multiple"].items():
        U.ulysses_plan_create(1, 1, m, [1], [1], dt)
        if m > 1:
            with pytest.raises(U.UlyssesError) as e:
                U.ulysses_plan_create(1, 1, m // 2, [1], [1], dt)
            assert e.value.code == -2


def expect(code, fn, *args):
    with pytest.raises(U.UlyssesError) as e:
        fn(*args)
    assert e.value.code == code, str(e.value)
    return str(e.value)


def test_plan_errors():
    expect(-1, U.ulysses_plan_create, 2, 0, 8, [1, 1], [1, 1], "bf16")
    expect(-1, U.ulysses_plan_create, 2, 1, 8, [-1, 2], [1, 1], "bf16")
    expect(-1, U.ulysses_plan_create, 2, 1, 8, [0, 0], [1, 1], "bf16")
    expect(-1, U.ulysses_plan_create, 2, 1, 8, [1, 1], [0, 0], "bf16")
    expect(-2, U.ulysses_plan_create, 2, 1, 4, [1, 1], [1, 1], "bf16")
    expect(-3, U.ulysses_plan_create, 2, 1, 8, [1, 1], [1, 1], 17)
    msg = expect(-1, U.ulysses_plan_create, 1, 1, 4096, [1], [33], "fp32")
    assert "512 KiB" in msg
    assert "512 KiB" in U.ulysses_last_error()


# Checks that pass fake device addresses run in a child process with every
# GPU hidden (tests/fake_address_checks.py): each call must fail validation
# before any launch, and even if one did not, no device would be there to
# take it.
FAKE_ADDRESS_CHECKS = ["call_errors_before_launch", "binding_checks_tensor_size_and_device",
                       "launch_wider_than_grid_x_refused", "multi_tensor_errors_before_launch",
                       "chunked_without_windows_errors_before_launch"]


@pytest.mark.parametrize("name", FAKE_ADDRESS_CHECKS)
def test_fake_address_checks_with_gpu_hidden(name):
    import sys
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1",
               PYTHONPATH=os.pathsep.join([ROOT, os.path.join(ROOT, "tests")]))
    code = f"import fake_address_checks as f; f.require_no_device(); f.{name}(); print('OK')"
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip().endswith("OK"), res.stdout + res.stderr


def test_autograd_entry_checks_dtype_and_shape():
    import torch
    from sequence_attention_relayout_amd.autograd import all_to_all_4d
    plan = U.ulysses_plan_create(2, 1, 8, [3, 4], [1, 2], "bf16")
    good = [torch.zeros(U.ulysses_plan_shape(plan, 0, r, False), dtype=torch.bfloat16)
            for r in range(2)]
    with pytest.raises(ValueError, match="2-byte elements"):
        all_to_all_4d(plan, [good[0].float(), good[1]], 0)
    with pytest.raises(ValueError, match="shape"):
        all_to_all_4d(plan, [good[1], good[0]], 0)


def test_rope_table_matches_oracle_bitwise():
    for theta, s, d in [(10000.0, 75600, 128), (500000.0, 1000, 64), (10000.0, 3, 8)]:
        c, sn = U.ulysses_rope_table(theta, s, d)
        oc, osn = oracle.rope_table(theta, s, d)
        assert c.view(np.uint32).tobytes() == oc.view(np.uint32).tobytes()
        assert sn.view(np.uint32).tobytes() == osn.view(np.uint32).tobytes()
    expect(-1, U.ulysses_rope_table, 0.0, 4, 8)
    expect(-1, U.ulysses_rope_table, 10000.0, 4, 7)
