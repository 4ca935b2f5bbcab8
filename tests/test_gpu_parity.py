"""GPU parity: libulysses.so (through its C ABI) against the CPU oracle.

Bar: bit-exact bytes for the pure relayout in every dtype; for the fused
QK RMSNorm + RoPE path at most 1 bf16 ulp (ordinal distance) from the
oracle, every element.  Every element is compared, at medium sizes (several
blocks per shard, ragged tails) and at the full sizes of the timed
workloads (the oracle's threaded loops on the host's cores); only the
shards beyond 4 GiB are checked on sampled elements.  Destination shards
sit between guard bands and are pre-filled with poison.
"""
import os

import numpy as np
import pytest
import torch

import gpu_helpers as H
import oracle
from sequence_attention_relayout_amd import ulysses as U
from sequence_attention_relayout_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EPS = 1e-6
THETA = 10000.0
# host threads for the oracle at full sizes (the same loops; identical results)
NT = max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no HIP device visible")
    U.library()   # fails loudly when the library is not built
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def bits(t):
    """Integer view of the same bytes, for bitwise torch.equal."""
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()])


def dst_shapes(plan, mode):
    return [U.ulysses_plan_shape(plan, mode, r, True) for r in range(plan.world)]


def run_relayout(plan, mode, srcs, dtype_name):
    out = H.Guarded(dst_shapes(plan, mode), dtype_name, DEV)
    U.ulysses_a2a_4d(plan, mode, srcs, out.views)
    torch.cuda.synchronize()
    assert out.guards_intact(), "write outside a destination shard"
    return out


def check_full(mode, b, d, seq, head, srcs, outs, threads=1):
    want = oracle.a2a_4d(mode, b, d, seq, head, [H.to_np(x) for x in srcs], threads=threads)
    for r, (g, w) in enumerate(zip(outs, want)):
        got = H.to_np(g)
        assert got.shape == w.shape
        bad = np.count_nonzero(got != w)
        assert bad == 0, f"mode {mode} rank {r}: {bad} elements differ"


def boundary_rows(mode, b, seq, head):
    """(rank, bi, row) of the rows next to every rank boundary."""
    rows = []
    so = np.concatenate([[0], np.cumsum(seq)])
    for r in range(len(seq)):
        for bi in sorted({0, b - 1}):
            if mode == 0:   # destination rows are global positions
                cand = {int(v) for o in so[1:-1] for v in (o - 1, o)} | {0, int(so[-1]) - 1}
                cand = {c for c in cand if 0 <= c < so[-1]}
            else:
                cand = {0, seq[r] - 1} if seq[r] > 0 else set()
            rows += [(r, bi, c) for c in sorted(cand)]
    return rows


# ---------------------------------------------------------------------------
# the two-rank example and an index-coded twin
# ---------------------------------------------------------------------------

def test_w2_tiny_modes_and_roundtrip():
    wl = W.workloads()["w2_tiny"]
    H.say(f"case: {wl.name}")
    plan = U.ulysses_plan_create(wl.world, wl.b, wl.d, wl.seq_splits, wl.head_splits, "bf16")
    xs = W.make_shards(wl, 0, "bf16", wl.seed, DEV)
    ys = run_relayout(plan, 0, xs, "bf16").views
    check_full(0, wl.b, wl.d, wl.seq_splits, wl.head_splits, xs, ys)
    for y in ys:
        assert tuple(y.shape) == (1, 32, 4, 128)
    zs = run_relayout(plan, 1, ys, "bf16").views
    for x, z in zip(xs, zs):
        assert torch.equal(x.view(torch.int16), z.view(torch.int16))
    fresh = W.make_shards(wl, 1, "bf16", wl.seed + 100, DEV)
    check_full(1, wl.b, wl.d, wl.seq_splits, wl.head_splits, fresh,
               run_relayout(plan, 1, fresh, "bf16").views)


def test_w2_index_coded_twin():
    """int32 codes of each element's own source coordinates, moved as fp32
    bytes: every output decodes to the coordinates the definition names."""
    wl = W.workloads()["w2_tiny"]
    H.say("case: w2 index-coded fp32 twin")
    plan = U.ulysses_plan_create(2, 1, 128, [16, 16], [4, 4], "fp32")
    codes = W.index_coded_shards(wl, 0)
    srcs = [torch.from_numpy(c).to(DEV).view(torch.float32) for c in codes]
    ys = run_relayout(plan, 0, srcs, "fp32").views
    for r, y in enumerate(ys):
        got = y.view(torch.int32).cpu().numpy().astype(np.int64)
        bi, S, h, e = np.indices(got.shape)
        j = S // 16
        want = (j << 27) + ((bi * 16 + S - 16 * j) * 8 + 4 * r + h) * 128 + e
        assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
# random geometries: every dtype, uneven and zero splits, several tiles
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(21))
def test_random_geometries_every_dtype(seed):
    rng = np.random.default_rng(1000 + seed)
    dt = W.DTYPES[seed % len(W.DTYPES)]
    esz = W.ELEM_BYTES[dt]
    world = int(rng.integers(1, 9))
    b = int(rng.integers(1, 4))
    d = (16 // esz) * int(rng.choice([1, 2, 3, 8]))
    seq = [int(v) for v in rng.integers(0, 400, world)]
    head = [int(v) for v in rng.integers(0, 7, world)]
    if seed % 3 == 0 and world > 1:
        seq[int(rng.integers(0, world))] = 0
    seq[0] = max(seq[0], 1) if sum(seq) == 0 else seq[0]
    head[-1] = max(head[-1], 1) if sum(head) == 0 else head[-1]
    H.say(f"case: random seed={seed} dtype={dt} W={world} b={b} d={d} seq={seq} head={head}")
    plan = U.ulysses_plan_create(world, b, d, seq, head, dt)
    wl = W.Workload("random", world, b, d, seq, head)
    for mode in (0, 1):
        xs = W.make_shards(wl, mode, dt, 2000 + seed * 2 + mode, DEV)
        outs = run_relayout(plan, mode, xs, dt).views
        check_full(mode, b, d, seq, head, xs, outs)


def test_many_tiny_random_geometries():
    """300 tiny random geometries in one process (W 1-8, splits 0-40 with
    zeros, head counts 0-12, b 1-3, every dtype and several row widths, a
    third of them with head counts in multiples of 4): both modes, two
    tensors in one launch, the plane-at-a-time call through windows and
    straight into the destination, and the fused call for bf16, every
    element against the oracle."""
    rng = np.random.default_rng(9000)
    for case in range(300):
        dt = W.DTYPES[int(rng.integers(0, len(W.DTYPES)))]
        esz = W.ELEM_BYTES[dt]
        world = int(rng.integers(1, 9))
        b = int(rng.integers(1, 4))
        d = (16 // esz) * int(rng.choice([1, 2, 4, 8]))
        seq = [int(v) for v in rng.integers(0, 41, world)]
        head = [int(v) for v in rng.integers(0, 10, world)]
        if case % 3 == 0:   # row widths in whole multiples of 32 vectors
            d = (16 // esz) * 8
            head = [4 * int(v) for v in rng.integers(0, 4, world)]
        seq[int(rng.integers(0, world))] += 1
        if sum(head) == 0:
            head[int(rng.integers(0, world))] += 4
        plan = U.ulysses_plan_create(world, b, d, seq, head, dt, 1 << 30)
        wl = W.Workload("tiny random", world, b, d, seq, head)
        for mode in (0, 1):
            xs = W.make_shards(wl, mode, dt, 9100 + 2 * case + mode, DEV)
            outs = run_relayout(plan, mode, xs, dt).views
            try:
                check_full(mode, b, d, seq, head, xs, outs)
            except AssertionError:
                H.say(f"failing case {case}: {dt} W={world} b={b} d={d} seq={seq} head={head}")
                raise
            if mode == 0 and case % 2 == 0:   # two tensors in one launch (grid.z = 2)
                xs2 = W.make_shards(wl, 0, dt, 9500 + case, DEV)
                o1 = [torch.empty(s_, dtype=W.torch_dtype(dt), device=DEV)
                      for s_ in dst_shapes(plan, 0)]
                o2 = [torch.empty_like(t) for t in o1]
                U.ulysses_a2a_4d_multi(plan, 0, [xs, xs2], [o1, o2])
                torch.cuda.synchronize()
                check_full(0, b, d, seq, head, xs, o1)
                check_full(0, b, d, seq, head, xs2, o2)
            if mode == 1:
                win = [torch.empty(max(1, U.ulysses_plan_window_bytes(plan, 1)), dtype=torch.uint8,
                                   device=DEV) for _ in range(world)]
                cout = [torch.empty(s_, dtype=W.torch_dtype(dt), device=DEV)
                        for s_ in dst_shapes(plan, 1)]
                U.ulysses_a2a_4d_chunked(plan, 1, xs, cout, win)
                torch.cuda.synchronize()
                check_full(1, b, d, seq, head, xs, cout)
                direct = [torch.empty_like(t) for t in cout]
                U.ulysses_a2a_4d_chunked(plan, 1, xs, direct, None)
                torch.cuda.synchronize()
                check_full(1, b, d, seq, head, xs, direct)
        if dt == "bf16" and (d // 8) & (d // 8 - 1) == 0:
            qs = W.make_shards(wl, 0, "bf16", 9700 + case, DEV)
            ks = W.make_shards(wl, 0, "bf16", 9800 + case, DEV)
            gq, gk = W.make_gamma(d, 9900 + case, DEV), W.make_gamma(d, 9950 + case, DEV)
            tab, (oc, osn) = rope_tables(sum(seq), d)
            qo, ko = run_fused(plan, qs, ks, gq, gk, tab)
            for src, out, g in ((qs, qo, gq), (ks, ko, gk)):
                want = oracle.qknorm_rope_mode0(b, d, seq, head, [H.to_np(x) for x in src],
                                                g.cpu().numpy(), EPS, oc, osn)
                for o, w in zip(out, want):
                    hist = ulp_hist(H.to_np(o), w)
                    assert hist[2] == 0 and hist[3] == 0, f"fused case {case}"
    H.say("  300 cases")


@pytest.mark.parametrize("head", [[6, 6, 6, 6, 4, 4, 4, 4], [4, 4, 4, 4, 2, 2, 2, 2],
                                  [8, 8, 4, 4], [4, 2, 0, 2, 6]])
def test_unequal_head_widths(head):
    """Head splits whose rows differ in width (and a rank without heads):
    destination rows of different lengths in mode 0, pieces of different
    widths within one destination row in mode 1.  Uneven sequence splits,
    two batch planes, every element compared in both modes."""
    world = len(head)
    seq = W.seeded_partition(11, 2001 * world, world)
    H.say(f"case: unequal head widths W={world} seq={seq} head={head}")
    plan = U.ulysses_plan_create(world, 2, 128, seq, head, "bf16")
    wl = W.Workload("unequal widths", world, 2, 128, seq, head)
    for mode in (0, 1):
        xs = W.make_shards(wl, mode, "bf16", 7700 + mode, DEV)
        check_full(mode, 2, 128, seq, head, xs, run_relayout(plan, mode, xs, "bf16").views)


@pytest.mark.parametrize("seed", range(12))
def test_random_medium_geometries(seed):
    """Larger random geometries (up to ~48 MB per tensor): many blocks per
    shard, long and short rows, uneven and zero splits, every dtype; every
    element compared in both modes, plus the fused path for bf16 with
    d = 128, 64 or 256."""
    rng = np.random.default_rng(7000 + seed)
    dt = W.DTYPES[seed % len(W.DTYPES)]
    esz = W.ELEM_BYTES[dt]
    world = int(rng.integers(1, 9))
    b = int(rng.integers(1, 4))
    d = (16 // esz) * int(rng.choice([1, 2, 4, 8, 16]))
    head = [int(v) for v in rng.integers(0, 9, world)]
    head[-1] = max(head[-1], 1)
    row = sum(head) * d * esz
    per_rank = max(1, (48 << 20) // (b * row * world))
    seq = [int(v) for v in rng.integers(0, per_rank + 1, world)]
    if seed % 4 == 1 and world > 1:
        seq[int(rng.integers(0, world))] = 0
    seq[0] = max(seq[0], 1)
    H.say(f"case: random medium seed={seed} dtype={dt} W={world} b={b} d={d} "
          f"seq={seq} head={head}")
    plan = U.ulysses_plan_create(world, b, d, seq, head, dt)
    wl = W.Workload("random medium", world, b, d, seq, head)
    for mode in (0, 1):
        xs = W.make_shards(wl, mode, dt, 7100 + seed * 2 + mode, DEV)
        check_full(mode, b, d, seq, head, xs, run_relayout(plan, mode, xs, dt).views)
    if dt != "bf16":
        return
    fd = [128, 64, 256][seed % 3]
    fseq = [max(1, v // 8) for v in seq]
    fplan = U.ulysses_plan_create(world, b, fd, fseq, head, "bf16")
    fwl = W.Workload("random medium fused", world, b, fd, fseq, head)
    qs = W.make_shards(fwl, 0, "bf16", 7200 + seed, DEV)
    ks = W.make_shards(fwl, 0, "bf16", 7300 + seed, DEV)
    gq, gk = W.make_gamma(fd, 7400 + seed, DEV), W.make_gamma(fd, 7500 + seed, DEV)
    tab, (oc, osn) = rope_tables(sum(fseq), fd)
    qo, ko = run_fused(fplan, qs, ks, gq, gk, tab)
    for src, out, g in ((qs, qo, gq), (ks, ko, gk)):
        want = oracle.qknorm_rope_mode0(b, fd, fseq, head, [H.to_np(x) for x in src],
                                        g.cpu().numpy(), EPS, oc, osn)
        hist = np.zeros(4, np.int64)
        for o, w in zip(out, want):
            hist += ulp_hist(H.to_np(o), w)
        H.say(f"  fused d={fd} ulp histogram (0,1,2,>=3): {hist.tolist()}")
        assert hist[2] == 0 and hist[3] == 0


# ---------------------------------------------------------------------------
# the W=8, 75,600-token video-DiT operand (the timed workload)
# ---------------------------------------------------------------------------

def test_w8_medium_full_compare():
    """The same geometry at 1/10 of the tokens: every element compared."""
    H.say("case: W=8, s=7,560, n=40, d=128, bf16, full compare")
    seq, head = [945] * 8, [5] * 8
    plan = U.ulysses_plan_create(8, 1, 128, seq, head, "bf16")
    wl = W.Workload("w8 medium", 8, 1, 128, seq, head)
    xs = W.make_shards(wl, 0, "bf16", 21, DEV)
    ys = run_relayout(plan, 0, xs, "bf16").views
    check_full(0, 1, 128, seq, head, xs, ys)
    zs = run_relayout(plan, 1, ys, "bf16").views
    check_full(1, 1, 128, seq, head, ys, zs)


def test_w8_wan720p_full_size():
    """The timed geometry: every element of both modes against the oracle,
    and the round trip."""
    wl = W.workloads()["w8_wan720p"]
    H.say(f"case: {wl.name} (every element)")
    plan = U.ulysses_plan_create(wl.world, wl.b, wl.d, wl.seq_splits, wl.head_splits, "bf16")
    xs = W.make_shards(wl, 0, "bf16", wl.seed, DEV)
    ys = run_relayout(plan, 0, xs, "bf16").views
    for y in ys:
        assert tuple(y.shape) == (1, 75600, 5, 128)
    check_full(0, wl.b, wl.d, wl.seq_splits, wl.head_splits, xs, ys, threads=NT)
    zs = run_relayout(plan, 1, ys, "bf16").views
    for x, z in zip(xs, zs):
        assert torch.equal(x.view(torch.int16), z.view(torch.int16))
    del ys, zs
    fresh = W.make_shards(wl, 1, "bf16", wl.seed + 1, DEV)
    outs = run_relayout(plan, 1, fresh, "bf16").views
    check_full(1, wl.b, wl.d, wl.seq_splits, wl.head_splits, fresh, outs, threads=NT)


# ---------------------------------------------------------------------------
# uneven splits, W=7, b=2, four dtypes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["bf16", "fp32", "fp8_e4m3", "int8"])
def test_w7_uneven_medium_full_compare(dt):
    seq = W.seeded_partition(3, 7559, 7)
    head = [6, 6, 6, 6, 6, 5, 5]
    H.say(f"case: W=7 uneven medium {dt} seq={seq}")
    plan = U.ulysses_plan_create(7, 2, 128, seq, head, dt)
    wl = W.Workload("w7 medium", 7, 2, 128, seq, head)
    for mode in (0, 1):
        xs = W.make_shards(wl, mode, dt, 31 + mode, DEV)
        check_full(mode, 2, 128, seq, head, xs, run_relayout(plan, mode, xs, dt).views)


@pytest.mark.parametrize("dt", ["bf16", "fp32", "fp8_e4m3", "int8"])
def test_w7_uneven_full_size(dt):
    """The uneven W=7 workload in each of its dtypes: every element of both
    modes against the oracle, and the round trip."""
    wl = W.workloads()["w7_uneven"]
    H.say(f"case: {wl.name} dtype={dt} seq={wl.seq_splits} (every element)")
    plan = U.ulysses_plan_create(wl.world, wl.b, wl.d, wl.seq_splits, wl.head_splits, dt)
    for mode in (0, 1):
        xs = W.make_shards(wl, mode, dt, 40 + mode, DEV)
        outs = run_relayout(plan, mode, xs, dt).views
        check_full(mode, wl.b, wl.d, wl.seq_splits, wl.head_splits, xs, outs, threads=NT)
        back = run_relayout(plan, 1 - mode, outs, dt).views
        for x, z in zip(xs, back):
            assert torch.equal(bits(x), bits(z))
        del xs, outs, back
        torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# several tensors in one launch
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ntensors,dt,world", [(3, "bf16", 8), (4, "fp8_e4m3", 5), (2, "fp32", 3),
                                                (1, "int8", 4)])
def test_multi_tensor_equals_oracle(ntensors, dt, world):
    rng = np.random.default_rng(ntensors * 10 + world)
    seq = W.seeded_partition(int(rng.integers(0, 100)), 1200, world)
    head = [int(v) for v in rng.integers(1, 6, world)]
    H.say(f"case: multi ntensors={ntensors} {dt} W={world} seq={seq} head={head}")
    plan = U.ulysses_plan_create(world, 2, 128, seq, head, dt)
    wl = W.Workload("multi", world, 2, 128, seq, head)
    for mode in (0, 1):
        xs = [W.make_shards(wl, mode, dt, 120 + 10 * t + mode, DEV) for t in range(ntensors)]
        outs = [H.Guarded(dst_shapes(plan, mode), dt, DEV) for _ in range(ntensors)]
        U.ulysses_a2a_4d_multi(plan, mode, xs, [o.views for o in outs])
        torch.cuda.synchronize()
        for x, o in zip(xs, outs):
            assert o.guards_intact()
            check_full(mode, 2, 128, seq, head, x, o.views)


def test_w8_qkv_multi_full_size():
    """q, k, v of the timed geometry in one launch: every element of each
    against the oracle."""
    wl = W.workloads()["w8_wan720p"]
    H.say("case: w8 75.6k q, k, v in one launch (every element)")
    plan = U.ulysses_plan_create(wl.world, wl.b, wl.d, wl.seq_splits, wl.head_splits, "bf16")
    xs = [W.make_shards(wl, 0, "bf16", 130 + t, DEV) for t in range(3)]
    multi = [H.Guarded(dst_shapes(plan, 0), "bf16", DEV) for _ in range(3)]
    U.ulysses_a2a_4d_multi(plan, 0, xs, [m.views for m in multi])
    torch.cuda.synchronize()
    for x, m in zip(xs, multi):
        assert m.guards_intact()
        check_full(0, wl.b, wl.d, wl.seq_splits, wl.head_splits, x, m.views, threads=NT)


# ---------------------------------------------------------------------------
# autograd: the backward of one mode is the other mode with the same plan
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", [0, 1])
def test_autograd_backward_is_the_inverse_relayout(mode):
    from sequence_attention_relayout_amd.autograd import all_to_all_4d
    seq, head = W.seeded_partition(11, 900, 5), [3, 1, 4, 2, 2]
    H.say(f"case: autograd mode {mode} seq={seq} head={head}")
    plan = U.ulysses_plan_create(5, 2, 64, seq, head, "fp32")
    wl = W.Workload("autograd", 5, 2, 64, seq, head)
    xs = [x.requires_grad_() for x in W.make_shards(wl, mode, "fp32", 140 + mode, DEV)]
    ys = all_to_all_4d(plan, xs, mode)
    check_full(mode, 2, 64, seq, head, [x.detach() for x in xs], [y.detach() for y in ys])
    ws = W.make_shards(wl, 1 - mode, "fp32", 150 + mode, DEV)   # d loss / d y
    loss = sum((y * w).sum() for y, w in zip(ys, ws))
    loss.backward()
    # d loss / d x = the inverse relayout of w, element for element
    want = oracle.a2a_4d(1 - mode, 2, 64, seq, head, [H.to_np(w) for w in ws])
    for x, wnt in zip(xs, want):
        assert np.array_equal(H.to_np(x.grad), wnt)


def test_autograd_round_trip_and_bf16():
    from sequence_attention_relayout_amd.autograd import all_to_all_4d
    wl = W.workloads()["w2_tiny"]
    plan = U.ulysses_plan_create(2, 1, 128, [16, 16], [4, 4], "bf16")
    xs = [x.requires_grad_() for x in W.make_shards(wl, 0, "bf16", 160, DEV)]
    zs = all_to_all_4d(plan, all_to_all_4d(plan, xs, 0), 1)
    for x, z in zip(xs, zs):
        assert torch.equal(bits(x.detach()), bits(z.detach()))
    sum(z.float().sum() for z in zs).backward()
    for x in xs:
        assert torch.equal(x.grad.float(), torch.ones_like(x.grad.float()))


# ---------------------------------------------------------------------------
# plane-at-a-time exchange under a window cap
# ---------------------------------------------------------------------------

def windows(plan, mode):
    nbytes = U.ulysses_plan_window_bytes(plan, mode)
    return [torch.empty(nbytes, dtype=torch.uint8, device=DEV) for _ in range(plan.world)]


def test_chunked_medium_full_compare():
    seq, head = [1500, 1500, 1500, 1500], [14] * 4
    H.say("case: chunked W=4, b=3 planes, s=6,000, n=56, d=128, bf16")
    wl = W.Workload("chunked medium", 4, 3, 128, seq, head)
    plan = U.ulysses_plan_create(4, 3, 128, seq, head, "bf16", 6000 * 14 * 256)
    for mode in (0, 1):
        xs = W.make_shards(wl, mode, "bf16", 50 + mode, DEV)
        out = H.Guarded(dst_shapes(plan, mode), "bf16", DEV)
        U.ulysses_a2a_4d_chunked(plan, mode, xs, out.views, windows(plan, mode))
        torch.cuda.synchronize()
        assert out.guards_intact()
        check_full(mode, 3, 128, seq, head, xs, out.views)
        direct = H.Guarded(dst_shapes(plan, mode), "bf16", DEV)
        U.ulysses_a2a_4d_chunked(plan, mode, xs, direct.views, None)
        torch.cuda.synchronize()
        assert direct.guards_intact()
        check_full(mode, 3, 128, seq, head, xs, direct.views)


@pytest.mark.parametrize("seed", range(12))
def test_random_chunked_every_dtype(seed):
    rng = np.random.default_rng(3000 + seed)
    dt = W.DTYPES[seed % len(W.DTYPES)]
    esz = W.ELEM_BYTES[dt]
    world = int(rng.integers(1, 9))
    b = int(rng.integers(1, 4))
    d = (16 // esz) * int(rng.choice([1, 2, 4]))
    seq = [int(v) for v in rng.integers(0, 300, world)]
    head = [int(v) for v in rng.integers(0, 6, world)]
    seq[0] += 1
    head[-1] += 1
    wl = W.Workload("random chunked", world, b, d, seq, head)
    probe = U.ulysses_plan_create(world, b, d, seq, head, dt)
    cap = max(U.ulysses_plan_window_bytes(probe, 0), U.ulysses_plan_window_bytes(probe, 1))
    cap += int(rng.integers(0, 2)) * 4096          # exactly at the cap, or just above
    plan = U.ulysses_plan_create(world, b, d, seq, head, dt, cap)
    H.say(f"case: random chunked seed={seed} {dt} W={world} b={b} d={d} seq={seq} "
          f"head={head} cap={cap}")
    for mode in (0, 1):
        xs = W.make_shards(wl, mode, dt, 3100 + 2 * seed + mode, DEV)
        out = H.Guarded(dst_shapes(plan, mode), dt, DEV)
        U.ulysses_a2a_4d_chunked(plan, mode, xs, out.views, windows(plan, mode))
        torch.cuda.synchronize()
        assert out.guards_intact()
        check_full(mode, b, d, seq, head, xs, out.views)
        direct = H.Guarded(dst_shapes(plan, mode), dt, DEV)
        U.ulysses_a2a_4d_chunked(plan, mode, xs, direct.views, None)
        torch.cuda.synchronize()
        assert direct.guards_intact()
        check_full(mode, b, d, seq, head, xs, direct.views)


def check_planes(mode, wl, srcs_host, outs):
    """Every element of a batch-plane pack, one plane at a time against the
    oracle (each plane is an independent relayout of batch 1)."""
    outs_host = [H.to_np(o) for o in outs]
    for p in range(wl.b):
        want = oracle.a2a_4d(mode, 1, wl.d, wl.seq_splits, wl.head_splits,
                             [x[p:p + 1] for x in srcs_host], threads=NT)
        for r, (o, w) in enumerate(zip(outs_host, want)):
            bad = np.count_nonzero(o[p:p + 1] != w)
            assert bad == 0, f"mode {mode} plane {p} rank {r}: {bad} elements differ"


def test_w4_qkv_chunked_full_size(golden):
    """The FastVideo geometry (Q, K, V packed as three batch planes, 1 GiB
    window cap): the plane-at-a-time call through the windows, every element
    of every plane against the oracle; the same call writing straight into
    the destination, and the one-pass relayout, equal to it; the mode-1 call
    returns the input."""
    wl = W.workloads()["w4_qkv_chunked"]
    H.say(f"case: {wl.name} (every element)")
    plan = U.ulysses_plan_create(wl.world, wl.b, wl.d, wl.seq_splits, wl.head_splits, "bf16",
                                 wl.window_cap_bytes)
    assert U.ulysses_plan_window_bytes(plan, 0) == golden["fastvideo_window"]["bytes_per_plane"]
    xs = W.make_shards(wl, 0, "bf16", wl.seed, DEV)
    win = windows(plan, 0)
    ys = [torch.empty(s, dtype=torch.bfloat16, device=DEV) for s in dst_shapes(plan, 0)]
    U.ulysses_a2a_4d_chunked(plan, 0, xs, ys, win)
    torch.cuda.synchronize()
    del win
    check_planes(0, wl, [H.to_np(x) for x in xs], ys)
    # the window is invisible in the result: straight into the destination
    # and the one-pass relayout give the same bytes
    for direct_call in (lambda out: U.ulysses_a2a_4d_chunked(plan, 0, xs, out, None),
                        lambda out: U.ulysses_a2a_4d(plan, 0, xs, out)):
        direct = [torch.empty_like(y) for y in ys]
        direct_call(direct)
        torch.cuda.synchronize()
        for y, t in zip(ys, direct):
            assert torch.equal(y.view(torch.int16), t.view(torch.int16))
        del direct
        torch.cuda.empty_cache()
    zs = [torch.empty_like(x) for x in xs]
    U.ulysses_a2a_4d_chunked(plan, 1, ys, zs, windows(plan, 1))
    torch.cuda.synchronize()
    for x, z in zip(xs, zs):
        assert torch.equal(x.view(torch.int16), z.view(torch.int16))


# ---------------------------------------------------------------------------
# fused QK RMSNorm + RoPE on the mode-0 relayout
# ---------------------------------------------------------------------------

def rope_tables(s_global, d):
    c, s = U.ulysses_rope_table(THETA, s_global, d)
    oc, osn = oracle.rope_table(THETA, s_global, d)
    assert c.tobytes() == oc.tobytes() and s.tobytes() == osn.tobytes(), \
        "library and oracle rotary tables differ"
    return (torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV)), (oc, osn)


def ulp_hist(got, want):
    dist = np.abs(H.bf16_key(got) - H.bf16_key(want))
    return np.bincount(np.minimum(dist, 3).ravel(), minlength=4)


def run_fused(plan, qs, ks, gq, gk, tab):
    qo = H.Guarded(dst_shapes(plan, 0), "bf16", DEV)
    ko = H.Guarded(dst_shapes(plan, 0), "bf16", DEV)
    U.ulysses_a2a_4d_qknorm_rope(plan, qs, qo.views, ks, ko.views, gq, gk, EPS, tab[0], tab[1])
    torch.cuda.synchronize()
    assert qo.guards_intact() and ko.guards_intact()
    return qo.views, ko.views


@pytest.mark.parametrize("d,world,seq_total", [(128, 8, 7560), (128, 3, 1001), (64, 5, 777),
                                               (8, 2, 300), (16, 4, 64), (32, 7, 350),
                                               (256, 2, 200), (512, 1, 90)])
def test_fused_medium_full_compare(d, world, seq_total):
    rng = np.random.default_rng(d + world)
    seq = W.seeded_partition(int(rng.integers(0, 1000)), seq_total, world) if world > 1 \
        else [seq_total]
    head = [int(v) for v in rng.integers(1, 7, world)]
    b = 2 if d <= 64 else 1
    H.say(f"case: fused d={d} W={world} b={b} seq={seq} head={head}")
    plan = U.ulysses_plan_create(world, b, d, seq, head, "bf16")
    wl = W.Workload("fused medium", world, b, d, seq, head)
    qs = W.make_shards(wl, 0, "bf16", 60, DEV)
    ks = W.make_shards(wl, 0, "bf16", 61, DEV)
    gq, gk = W.make_gamma(d, 62, DEV), W.make_gamma(d, 63, DEV)
    tab, (oc, osn) = rope_tables(sum(seq), d)
    qo, ko = run_fused(plan, qs, ks, gq, gk, tab)
    for src, out, g in ((qs, qo, gq), (ks, ko, gk)):
        want = oracle.qknorm_rope_mode0(b, d, seq, head, [H.to_np(x) for x in src],
                                        g.cpu().numpy(), EPS, oc, osn)
        hist = np.zeros(4, np.int64)
        for o, w in zip(out, want):
            hist += ulp_hist(H.to_np(o), w)
        H.say(f"  ulp histogram (0,1,2,>=3): {hist.tolist()}")
        assert hist[2] == 0 and hist[3] == 0


def test_relayout_large_planes_one_launch_each():
    """Batch planes that move 64 MiB or more get one launch each (the
    kernel's one-plane form, the shard pointers moved to each plane on the
    host): three fp32 planes of 73.7 MB moved, W=3 uneven, both modes,
    every element against the oracle."""
    world, b, d = 3, 3, 128
    seq, head = W.seeded_partition(11, 6000, world), [4, 3, 5]
    H.say(f"case: relayout fp32 W={world} b={b} seq={seq} head={head} (one launch per plane)")
    plan = U.ulysses_plan_create(world, b, d, seq, head, "fp32")
    assert U.ulysses_plan_bytes(plan, 0) // b >= 64 << 20
    wl = W.Workload("large planes", world, b, d, seq, head)
    for mode in (0, 1):
        xs = W.make_shards(wl, mode, "fp32", 80 + mode, DEV)
        ys = [torch.empty(U.ulysses_plan_shape(plan, mode, r, True), dtype=torch.float32,
                          device=DEV) for r in range(world)]
        U.ulysses_a2a_4d(plan, mode, xs, ys)
        torch.cuda.synchronize()
        check_full(mode, b, d, seq, head, xs, ys, threads=NT)


def test_fused_large_planes_one_launch_each():
    """The fused pass with planes of q and k that move 64 MiB or more: one
    launch per plane.  Three planes, W=3 uneven, every element of q and k
    against the oracle."""
    world, b, d = 3, 3, 128
    seq, head = W.seeded_partition(12, 6000, world), [4, 3, 5]
    H.say(f"case: fused W={world} b={b} seq={seq} head={head} (one launch per plane)")
    plan = U.ulysses_plan_create(world, b, d, seq, head, "bf16")
    assert 2 * U.ulysses_plan_bytes(plan, 0) // b >= 64 << 20
    wl = W.Workload("fused large planes", world, b, d, seq, head)
    qs = W.make_shards(wl, 0, "bf16", 82, DEV)
    ks = W.make_shards(wl, 0, "bf16", 83, DEV)
    gq, gk = W.make_gamma(d, 84, DEV), W.make_gamma(d, 85, DEV)
    tab, (oc, osn) = rope_tables(sum(seq), d)
    qo, ko = run_fused(plan, qs, ks, gq, gk, tab)
    for src, out, g in ((qs, qo, gq), (ks, ko, gk)):
        want = oracle.qknorm_rope_mode0(b, d, seq, head, [H.to_np(x) for x in src],
                                        g.cpu().numpy(), EPS, oc, osn, threads=NT)
        hist = np.zeros(4, np.int64)
        for o, w in zip(out, want):
            hist += ulp_hist(H.to_np(o), w)
        H.say(f"  ulp histogram (0,1,2,>=3): {hist.tolist()}")
        assert hist[2] == 0 and hist[3] == 0


@pytest.mark.parametrize("world,heads", [(2, [12, 9]), (1, [20]), (3, [17, 0, 8])])
def test_fused_many_heads_full_compare(world, heads):
    """Many heads per rank (and a rank with none): with d = 128 a block of
    the fused pass spans many head rows of one destination row, or several
    destination rows when the rows are short."""
    seq = W.seeded_partition(7, 300, world) if world > 1 else [300]
    H.say(f"case: fused many heads W={world} seq={seq} head={heads}")
    plan = U.ulysses_plan_create(world, 2, 128, seq, heads, "bf16")
    wl = W.Workload("fused heads", world, 2, 128, seq, heads)
    qs = W.make_shards(wl, 0, "bf16", 64, DEV)
    ks = W.make_shards(wl, 0, "bf16", 65, DEV)
    gq, gk = W.make_gamma(128, 66, DEV), W.make_gamma(128, 67, DEV)
    tab, (oc, osn) = rope_tables(sum(seq), 128)
    qo, ko = run_fused(plan, qs, ks, gq, gk, tab)
    for src, out, g in ((qs, qo, gq), (ks, ko, gk)):
        want = oracle.qknorm_rope_mode0(2, 128, seq, heads, [H.to_np(x) for x in src],
                                        g.cpu().numpy(), EPS, oc, osn)
        hist = np.zeros(4, np.int64)
        for o, w in zip(out, want):
            hist += ulp_hist(H.to_np(o), w)
        H.say(f"  ulp histogram (0,1,2,>=3): {hist.tolist()}")
        assert hist[2] == 0 and hist[3] == 0


@pytest.mark.parametrize("d", [32, 128])
def test_fused_sum_order_reaches_the_output(d):
    """A row whose fp32 sum of squares depends on the summation order:
    partial sums 2, 1, 3 and 2^24 give 2^24 + 8 under the fixed
    adjacent-pairing order (pinned on the CPU), 2^24 + 4 with the halves
    paired first and 2^24 + 6 in one chain.  Element 0 holds 1 and its gain
    is chosen so that its bf16 output differs between those three sums (the
    row sits at position 0, where the rotation is the identity); the GPU's
    row must equal the oracle's bit for bit."""
    H.say(f"case: fused summation order d={d}")
    row = np.zeros(d)
    row[[0, 1, 8, 16, 17, 18]] = 1.0
    row[24] = 4096.0
    g0 = np.float32(1.2512479)
    f32 = np.float32

    def out0(ss):   # bf16 bits of element 0 for a given sum of squares
        inv = f32(1) / np.sqrt(f32(f32(ss) / f32(d)) + f32(EPS))
        return H.to_np(torch.tensor([(f32(1) * inv) * g0], dtype=torch.float32)
                       .to(torch.bfloat16))[0]
    assert out0(2 ** 24 + 8) != out0(2 ** 24 + 4) and out0(2 ** 24 + 8) != out0(2 ** 24 + 6)
    x = torch.tensor(row, dtype=torch.float32).to(torch.bfloat16).reshape(1, 1, 1, d)
    gamma = np.ones(d, np.float32)
    gamma[0] = g0
    plan = U.ulysses_plan_create(1, 1, d, [1], [1], "bf16")
    qs, ks = [x.to(DEV)], [x.to(DEV)]
    g = torch.from_numpy(gamma).to(DEV)
    tab, (oc, osn) = rope_tables(1, d)
    qo, ko = run_fused(plan, qs, ks, g, g, tab)
    want = oracle.qknorm_rope_mode0(1, d, [1], [1], [H.to_np(x)], gamma, EPS, oc, osn)[0]
    assert want.reshape(-1)[0] == out0(2 ** 24 + 8)
    for o in (qo[0], ko[0]):
        assert np.array_equal(H.to_np(o), want)


def run_one_row(d, x, gamma, cos_row, sin_row, eps):
    """One bf16 row (W = 1, b = 1, one head, position 0) through the fused
    call with an explicit one-row rotary table; returns (gpu bits, oracle
    bits)."""
    row = np.zeros(d)
    row[:len(x)] = x
    xt = torch.tensor(row, dtype=torch.float32).to(torch.bfloat16).reshape(1, 1, 1, d)
    g = np.ones(d, np.float32)
    g[:len(gamma)] = gamma
    c = np.ones((1, d // 2), np.float32)
    s_ = np.zeros((1, d // 2), np.float32)
    c[0, :len(cos_row)] = cos_row
    s_[0, :len(sin_row)] = sin_row
    plan = U.ulysses_plan_create(1, 1, d, [1], [1], "bf16")
    gd = torch.from_numpy(g).to(DEV)
    tab = (torch.from_numpy(c).to(DEV), torch.from_numpy(s_).to(DEV))
    qo = H.Guarded(dst_shapes(plan, 0), "bf16", DEV)
    ko = H.Guarded(dst_shapes(plan, 0), "bf16", DEV)
    U.ulysses_a2a_4d_qknorm_rope(plan, [xt.to(DEV)], qo.views, [xt.to(DEV)], ko.views, gd, gd,
                                 eps, tab[0], tab[1])
    torch.cuda.synchronize()
    assert qo.guards_intact() and ko.guards_intact()
    want = oracle.qknorm_rope_mode0(1, d, [1], [1], [H.to_np(xt)], g, eps, c, s_)[0].reshape(d)
    got_q, got_k = H.to_np(qo.views[0]).reshape(d), H.to_np(ko.views[0]).reshape(d)
    assert np.array_equal(got_q, got_k)
    return got_q, want


@pytest.mark.parametrize("d", [8, 128])
def test_fused_rounding_rows_reach_the_output(d):
    """The rows that pin the fused row's rounding steps on the CPU, through
    the GPU: four rotation pairs whose outputs change if any product is
    contracted into its add or subtract (expected bf16 0, 2, 0, 2, -2, 0,
    -2, 0), and one element whose output changes if the gain is folded into
    inv first (0x4061 at d = 8, 0x415E at d = 128, worked out by hand in
    exact arithmetic on the CPU).  The GPU must give the oracle's bits."""
    H.say(f"case: fused rounding rows d={d}")
    e11, e12 = 2.0 ** -11, 2.0 ** -12
    x = [0.5] * 8 + ([4.0, 3.0, 2.0, 1.0] if d == 128 else [])
    gamma = [1 + e12, 1, 1, 1 + e12, 1 + e12, 1, 1, 1 + e12]
    cos_row = [1 + e12, 1 + e11, -(1 + e11), -(1 + e12)]
    sin_row = [1 + e11, 1 + e12, 1 + e12, 1 + e11]
    got, want = run_one_row(d, x, gamma, cos_row, sin_row, 0.0)
    assert [int(v) for v in want[:8]] == [0x0000, 0x4000, 0x0000, 0x4000,
                                          0xC000, 0x0000, 0xC000, 0x0000]
    assert np.array_equal(got, want)
    g0 = float(np.uint32({8: 0x3F9EBED7, 128: 0x3F9D54CD}[d]).view(np.float32))
    got, want = run_one_row(d, [1.5], [g0], [], [], 0.0)
    assert int(want[0]) == {8: 0x4061, 128: 0x415E}[d]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("seed", range(10))
def test_random_fused(seed):
    rng = np.random.default_rng(4000 + seed)
    d = int(8 << int(rng.integers(0, 7)))          # 8 .. 512
    world = int(rng.integers(1, 9))
    b = int(rng.integers(1, 3))
    seq = [int(v) for v in rng.integers(0, 80, world)]
    head = [int(v) for v in rng.integers(0, 13, world)]
    seq[-1] += 1
    head[0] += 1
    H.say(f"case: random fused seed={seed} d={d} W={world} b={b} seq={seq} head={head}")
    plan = U.ulysses_plan_create(world, b, d, seq, head, "bf16")
    wl = W.Workload("random fused", world, b, d, seq, head)
    qs = W.make_shards(wl, 0, "bf16", 4100 + seed, DEV)
    ks = W.make_shards(wl, 0, "bf16", 4200 + seed, DEV)
    gq, gk = W.make_gamma(d, 4300 + seed, DEV), W.make_gamma(d, 4400 + seed, DEV)
    tab, (oc, osn) = rope_tables(sum(seq), d)
    qo, ko = run_fused(plan, qs, ks, gq, gk, tab)
    for src, out, g in ((qs, qo, gq), (ks, ko, gk)):
        want = oracle.qknorm_rope_mode0(b, d, seq, head, [H.to_np(x) for x in src],
                                        g.cpu().numpy(), EPS, oc, osn)
        hist = np.zeros(4, np.int64)
        for o, w in zip(out, want):
            hist += ulp_hist(H.to_np(o), w)
        H.say(f"  ulp histogram (0,1,2,>=3): {hist.tolist()}")
        assert hist[2] == 0 and hist[3] == 0


def test_w8_fused_full_size():
    """The fused workload: every element of q and k against the oracle's
    fused row operation (at most 1 bf16 ulp; the histogram is reported), and
    every element of v through the plain relayout."""
    wl = W.workloads()["w8_fused_qknorm_rope"]
    H.say(f"case: {wl.name} (every element)")
    plan = U.ulysses_plan_create(wl.world, wl.b, wl.d, wl.seq_splits, wl.head_splits, "bf16")
    qs = W.make_shards(wl, 0, "bf16", 70, DEV)
    ks = W.make_shards(wl, 0, "bf16", 71, DEV)
    gq, gk = W.make_gamma(wl.d, 73, DEV), W.make_gamma(wl.d, 74, DEV)
    tab, (oc, osn) = rope_tables(wl.s_global, wl.d)
    qo, ko = run_fused(plan, qs, ks, gq, gk, tab)
    for name, src, out, g in (("q", qs, qo, gq), ("k", ks, ko, gk)):
        want = oracle.qknorm_rope_mode0(wl.b, wl.d, wl.seq_splits, wl.head_splits,
                                        [H.to_np(x) for x in src], g.cpu().numpy(), EPS, oc, osn,
                                        threads=NT)
        hist = np.zeros(4, np.int64)
        for o, w in zip(out, want):
            hist += ulp_hist(H.to_np(o), w)
        H.say(f"  {name}: ulp histogram (0,1,2,>=3): {hist.tolist()}")
        assert hist[2] == 0 and hist[3] == 0
        del want
    del qs, ks, qo, ko
    torch.cuda.empty_cache()
    vs = W.make_shards(wl, 0, "bf16", 72, DEV)
    vo = run_relayout(plan, 0, vs, "bf16").views
    check_full(0, wl.b, wl.d, wl.seq_splits, wl.head_splits, vs, vo, threads=NT)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

def gather_device(outs, coords):
    """Values of device shards at coords (n x 5), gathered on the device."""
    got = np.empty(len(coords), dtype=H.to_np(outs[0][:0]).dtype)
    for r, o in enumerate(outs):
        sel = coords[:, 0] == r
        if sel.any():
            idx = [torch.from_numpy(coords[sel, i]).to(DEV) for i in range(1, 5)]
            got[sel] = H.to_np(o[idx[0], idx[1], idx[2], idx[3]])
    return got


def test_shards_beyond_4_gib():
    """Shards of 4.5-4.9 GB: byte offsets past 2^32 inside one shard, for both
    modes of the relayout and for the fused pass (d = 128).  Sampled
    elements and rows,
    including the last rows of every shard, against the oracle."""
    seq, head, d = [2_200_000, 2_300_000], [4, 4], 256
    H.say(f"case: relayout uint8 W=2 seq={seq} head={head} d={d} (shards > 4 GiB)")
    plan = U.ulysses_plan_create(2, 1, d, seq, head, "uint8")
    wl = W.Workload("beyond 4 GiB", 2, 1, d, seq, head)
    rng = np.random.default_rng(90)
    for mode in (0, 1):
        xs = W.make_shards(wl, mode, "uint8", 91 + mode, DEV)
        assert max(x.numel() for x in xs) > (1 << 32)
        ys = [torch.empty(s_, dtype=torch.uint8, device=DEV) for s_ in dst_shapes(plan, mode)]
        U.ulysses_a2a_4d(plan, mode, xs, ys)
        torch.cuda.synchronize()
        rows = boundary_rows(mode, 1, seq, head)
        rows += [(r, 0, y.shape[1] - 1 - i) for r, y in enumerate(ys) for i in range(3)]
        coords = H.sample_coords(rng, [tuple(y.shape) for y in ys], 200_000, rows)
        host = [H.to_np(x) for x in xs]
        want = oracle.a2a_4d_sample(mode, 1, d, seq, head, host, coords)
        bad = np.count_nonzero(gather_device(ys, coords) != want)
        H.say(f"  mode {mode}: {len(coords)} sampled elements, {bad} differ")
        assert bad == 0
        del xs, ys, host
        torch.cuda.empty_cache()

    seq, head = [1_100_000, 1_200_000], [8, 8]
    H.say(f"case: fused d=128 W=2 seq={seq} head={head} (shards > 4 GiB)")
    plan = U.ulysses_plan_create(2, 1, 128, seq, head, "bf16")
    wl = W.Workload("fused beyond 4 GiB", 2, 1, 128, seq, head)
    qs = W.make_shards(wl, 0, "bf16", 93, DEV)
    ks = W.make_shards(wl, 0, "bf16", 94, DEV)
    assert max(x.numel() * 2 for x in qs) > (1 << 32)
    gq, gk = W.make_gamma(128, 95, DEV), W.make_gamma(128, 96, DEV)
    c, s = U.ulysses_rope_table(THETA, sum(seq), 128)
    tc, ts = torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV)
    qo = [torch.empty(s_, dtype=torch.bfloat16, device=DEV) for s_ in dst_shapes(plan, 0)]
    ko = [torch.empty_like(t) for t in qo]
    U.ulysses_a2a_4d_qknorm_rope(plan, qs, qo, ks, ko, gq, gk, EPS, tc, ts)
    torch.cuda.synchronize()
    s_global = sum(seq)
    picks = {int(v) for v in rng.integers(0, s_global, 1500)}
    picks |= {0, seq[0] - 1, seq[0], s_global - 2, s_global - 1}
    rows = np.array([(r, 0, S, h) for r in range(2) for S in sorted(picks)
                     for h in range(head[r])], dtype=np.int64)
    host = [H.to_np(x) for x in qs]
    want = oracle.qknorm_rope_mode0_sample(1, 128, seq, head, host, gq.cpu().numpy(), EPS,
                                           c, s, rows)
    got = np.empty_like(want)
    for r in range(2):
        sel = rows[:, 0] == r
        idx = torch.from_numpy(rows[sel, 2]).to(DEV), torch.from_numpy(rows[sel, 3]).to(DEV)
        got[sel] = H.to_np(qo[r][0][idx[0], idx[1]])
    hist = ulp_hist(got, want)
    H.say(f"  q: {len(rows)} rows, ulp histogram (0,1,2,>=3): {hist.tolist()}")
    assert hist[2] == 0 and hist[3] == 0
    del qs, ks, qo, ko, host
    torch.cuda.empty_cache()


def test_world_one_is_a_copy():
    H.say("case: W=1 identity, b=3")
    plan = U.ulysses_plan_create(1, 3, 64, [333], [7], "fp16")
    wl = W.Workload("w1", 1, 3, 64, [333], [7])
    for mode in (0, 1):
        xs = W.make_shards(wl, mode, "fp16", 80 + mode, DEV)
        out = run_relayout(plan, mode, xs, "fp16").views
        assert torch.equal(out[0].view(torch.int16), xs[0].view(torch.int16))


def test_empty_shards_and_null_pointers():
    """Zero splits give empty shards, whose pointers may be null."""
    seq, head = [0, 40, 0, 17, 3], [2, 0, 3, 1, 0]
    H.say(f"case: empty shards seq={seq} head={head}")
    plan = U.ulysses_plan_create(5, 2, 32, seq, head, "bf16")
    wl = W.Workload("empty", 5, 2, 32, seq, head)
    for mode in (0, 1):
        xs = W.make_shards(wl, mode, "bf16", 90 + mode, DEV)
        srcs = [x if x.numel() else 0 for x in xs]
        out = H.Guarded(dst_shapes(plan, mode), "bf16", DEV)
        dsts = [v if v.numel() else 0 for v in out.views]
        U.ulysses_a2a_4d(plan, mode, srcs, dsts)
        torch.cuda.synchronize()
        assert out.guards_intact()
        check_full(mode, 2, 32, seq, head, xs, out.views)


def test_longest_rows_and_single_vector_rows():
    """Rows at the 512 KiB limit (32,768 vectors) and rows of one 16-byte
    vector (d*esz = 16, one head per rank)."""
    cases = [(2, 1, 2048, "fp32", [3, 2], [40, 24]),
             (3, 2, 8, "bf16", [50, 1, 77], [1, 1, 1]),
             (4, 1, 16, "uint8", [9, 0, 33, 5], [1, 1, 1, 1])]
    for world, b, d, dt, seq, head in cases:
        H.say(f"case: rows W={world} b={b} d={d} {dt} seq={seq} head={head}")
        plan = U.ulysses_plan_create(world, b, d, seq, head, dt)
        wl = W.Workload("rows", world, b, d, seq, head)
        for mode in (0, 1):
            xs = W.make_shards(wl, mode, dt, 100 + mode, DEV)
            check_full(mode, b, d, seq, head, xs, run_relayout(plan, mode, xs, dt).views)


def test_more_batch_planes_than_one_launch():
    """70,000 batch planes: more than grid.y of one launch holds, so the
    library splits the planes over launches (relayout, plane-at-a-time,
    both fused kernels)."""
    b = 70_000
    H.say(f"case: b={b} planes")
    seq, head = [2, 1], [1, 2]
    plan = U.ulysses_plan_create(2, b, 8, seq, head, "bf16", 1 << 20)
    wl = W.Workload("planes", 2, b, 8, seq, head)
    for mode in (0, 1):
        xs = W.make_shards(wl, mode, "bf16", 170 + mode, DEV)
        check_full(mode, b, 8, seq, head, xs, run_relayout(plan, mode, xs, "bf16").views)
    xs = W.make_shards(wl, 0, "bf16", 172, DEV)
    out = [torch.empty(s_, dtype=torch.bfloat16, device=DEV) for s_ in dst_shapes(plan, 0)]
    U.ulysses_a2a_4d_chunked(plan, 0, xs, out, windows(plan, 0))
    torch.cuda.synchronize()
    check_full(0, b, 8, seq, head, xs, out)
    for d in (8, 128):
        plan_f = U.ulysses_plan_create(2, b, d, seq, head, "bf16")
        wlf = W.Workload("planes fused", 2, b, d, seq, head)
        qs = W.make_shards(wlf, 0, "bf16", 173, DEV)
        ks = W.make_shards(wlf, 0, "bf16", 174, DEV)
        gq, gk = W.make_gamma(d, 175, DEV), W.make_gamma(d, 176, DEV)
        tab, (oc, osn) = rope_tables(sum(seq), d)
        qo, ko = run_fused(plan_f, qs, ks, gq, gk, tab)
        for src, o, g in ((qs, qo, gq), (ks, ko, gk)):
            want = oracle.qknorm_rope_mode0(b, d, seq, head, [H.to_np(x) for x in src],
                                            g.cpu().numpy(), EPS, oc, osn)
            hist = np.zeros(4, np.int64)
            for oo, w in zip(o, want):
                hist += ulp_hist(H.to_np(oo), w)
            H.say(f"  d={d} ulp histogram (0,1,2,>=3): {hist.tolist()}")
            assert hist[2] == 0 and hist[3] == 0


def test_graph_capture_replays_match_eager():
    """The calls only enqueue kernels (no allocation, synchronisation or
    memset), so they can be captured in a HIP graph: capture mode 0, mode 1
    and the fused call once, replay three times with eager work and
    synchronisations in between, and compare every replay with the eager
    results."""
    H.say("case: graph capture of mode 0 + mode 1 + fused, 3 replays")
    seq, head = [40, 25, 31], [2, 3, 1]
    plan = U.ulysses_plan_create(3, 2, 128, seq, head, "bf16")
    wl = W.Workload("graph", 3, 2, 128, seq, head)
    xs = W.make_shards(wl, 0, "bf16", 180, DEV)
    ks = W.make_shards(wl, 0, "bf16", 181, DEV)
    gq, gk = W.make_gamma(128, 182, DEV), W.make_gamma(128, 183, DEV)
    tab, _ = rope_tables(sum(seq), 128)
    shp0, shp1 = dst_shapes(plan, 0), dst_shapes(plan, 1)
    ys = [torch.empty(sh, dtype=torch.bfloat16, device=DEV) for sh in shp0]
    zs = [torch.empty(sh, dtype=torch.bfloat16, device=DEV) for sh in shp1]
    qo = [torch.empty(sh, dtype=torch.bfloat16, device=DEV) for sh in shp0]
    ko = [torch.empty(sh, dtype=torch.bfloat16, device=DEV) for sh in shp0]

    def work():
        U.ulysses_a2a_4d(plan, 0, xs, ys)
        U.ulysses_a2a_4d(plan, 1, ys, zs)
        U.ulysses_a2a_4d_qknorm_rope(plan, xs, qo, ks, ko, gq, gk, EPS, tab[0], tab[1])

    work()
    torch.cuda.synchronize()
    eager = [bits(t).clone() for t in ys + zs + qo + ko]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    for rep in range(3):
        for t in ys + zs + qo + ko:
            t.zero_()               # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for e, t in zip(eager, ys + zs + qo + ko):
            assert torch.equal(e, bits(t)), f"replay {rep} differs"
    for x, z in zip(xs, zs):
        assert torch.equal(bits(x), bits(z))


def test_plain_c_caller_round_trip():
    """A C99 program (tests/native/abi_c_check.c, built by build()) calls the
    ABI with hipMalloc'ed shards: mode 1 after mode 0 returns its input."""
    import subprocess
    from sequence_attention_relayout_amd import build as ulybuild
    H.say("case: plain C caller, W=3 uneven bf16 round trip")
    if not os.path.exists(ulybuild.C_CHECK):
        pytest.fail(f"{ulybuild.C_CHECK} is not built (run __graft_entry__.build())")
    res = subprocess.run([ulybuild.C_CHECK, "gpu"], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("OK gpu")


def test_fp8_bit_patterns_survive():
    """Every fp8 byte pattern, NaNs included, crosses unchanged."""
    H.say("case: fp8 e5m2 all 256 patterns")
    plan = U.ulysses_plan_create(2, 1, 16, [16, 16], [1, 1], "fp8_e5m2")
    raw = torch.arange(256, dtype=torch.uint8, device=DEV)
    xs = [raw[:256].clone().view(1, 16, 1, 16).repeat(1, 1, 2, 1).contiguous()
          .view(torch.float8_e5m2) for _ in range(2)]
    ys = run_relayout(plan, 0, xs, "fp8_e5m2").views
    check_full(0, 1, 16, [16, 16], [1, 1], xs, ys)


def test_repeated_calls_reuse_the_plan():
    H.say("case: one plan, many calls on two streams")
    seq, head = [100, 200, 300], [3, 2, 1]
    plan = U.ulysses_plan_create(3, 2, 64, seq, head, "bf16")
    wl = W.Workload("reuse", 3, 2, 64, seq, head)
    xs = W.make_shards(wl, 0, "bf16", 110, DEV)
    first = run_relayout(plan, 0, xs, "bf16").views
    side = torch.cuda.Stream()
    outs = [torch.empty_like(f) for f in first]
    with torch.cuda.stream(side):
        for _ in range(5):
            U.ulysses_a2a_4d(plan, 0, xs, outs, side)
    side.synchronize()
    for a, b_ in zip(first, outs):
        assert torch.equal(a.view(torch.int16), b_.view(torch.int16))
