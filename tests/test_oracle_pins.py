"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test checks the oracle against something the pages or mathematics fix:
values the pages print (tests/golden), a library routine that computes the
same permutation (numpy slicing and concatenation, the reshape/transpose of
the permute + all_to_all_single + permute baseline), brute-force decoding of
index-coded inputs, invariants (identity at one rank, mode 1 inverts mode 0,
every element moved exactly once), closed forms of the rotary table, torch's
own float -> bfloat16 conversion, a float64 evaluation of RMSNorm and of
RoPE written as a complex multiplication, and rows worked by hand in exact
rational arithmetic whose bf16 outputs depend on each rounding step the fused
row fixes (summation order, rotation products rounded one by one, the gain
applied after the norm).
"""
import math

import numpy as np
import pytest
import torch

import oracle

# ---------------------------------------------------------------------------
# helpers (library-routine forms, not the oracle's loops)
# ---------------------------------------------------------------------------


def offsets(splits):
    return np.concatenate([[0], np.cumsum(splits)]).astype(np.int64)


def concat_mode0(xs, seq_splits, head_splits):
    """mode 0 for every r: the head block of r sliced out of every source
    shard and concatenated along the sequence axis in rank order."""
    ho = offsets(head_splits)
    return [np.concatenate([x[:, :, ho[r]:ho[r + 1], :] for x in xs], axis=1)
            for r in range(len(xs))]


def concat_mode1(ys, seq_splits, head_splits):
    """mode 1 for every r: the sequence block of r sliced out of every
    source shard and concatenated along the head axis in rank order."""
    so = offsets(seq_splits)
    return [np.concatenate([y[:, so[r]:so[r + 1], :, :] for y in ys], axis=2)
            for r in range(len(ys))]


def random_splits(rng, total, world, allow_zero=True):
    lo = 0 if allow_zero else 1
    while True:
        cuts = np.sort(rng.integers(0, total + 1, world - 1))
        parts = np.diff(np.concatenate([[0], cuts, [total]]))
        if parts.min() >= lo:
            return [int(p) for p in parts]


def random_geometry(rng, max_world=8, allow_zero=True):
    world = int(rng.integers(1, max_world + 1))
    b = int(rng.integers(1, 4))
    d = int(rng.choice([8, 16, 32]))
    s_global = int(rng.integers(world if not allow_zero else 1, 40))
    n_global = int(rng.integers(world if not allow_zero else 1, 20))
    if not allow_zero:
        s_global = max(s_global, world)
        n_global = max(n_global, world)
    return (world, b, d, random_splits(rng, s_global, world, allow_zero),
            random_splits(rng, n_global, world, allow_zero))


def rand_shards(rng, mode, b, d, seq, head, dtype):
    xs = []
    for r in range(len(seq)):
        shp = oracle.shape(mode, b, d, seq, head, r, False)
        raw = rng.integers(0, 256, size=int(np.prod(shp)) * np.dtype(dtype).itemsize,
                           dtype=np.uint8)
        xs.append(raw.view(dtype).reshape(shp))
    return xs


# ---------------------------------------------------------------------------
# shapes and window bytes: values printed on the pages
# ---------------------------------------------------------------------------


def test_quickstart_010_shapes(golden):
    g = golden["quickstart_010"]
    for ws in g["world_sizes"]:
        seq = [g["s_local"]] * ws
        head = [g["n_local"]] * ws
        for r in range(ws):
            assert oracle.shape(0, g["b"], g["d"], seq, head, r, False) == \
                (g["b"], g["s_local"], g["n_local"] * ws, g["d"])
            assert oracle.shape(0, g["b"], g["d"], seq, head, r, True) == \
                (g["b"], g["s_local"] * ws, g["n_local"], g["d"])
    # the launched example itself, with data: output shape as asserted there
    ws = g["launched_world"]
    seq, head = [g["s_local"]] * ws, [g["n_local"]] * ws
    rng = np.random.default_rng(0)
    xs = rand_shards(rng, 0, g["b"], g["d"], seq, head, np.uint16)
    for y in oracle.a2a_4d(0, g["b"], g["d"], seq, head, xs):
        assert y.shape == (g["b"], g["s_local"] * ws, g["n_local"], g["d"])


def test_quickstart_021_roundtrip_shapes(golden):
    g = golden["quickstart_021"]
    ws = g["world"]
    seq, head = [g["s_local"]] * ws, [g["heads"]] * ws
    assert oracle.shape(0, g["b"], g["d"], seq, head, 0, False) == tuple(g["x_shape"])
    assert oracle.shape(0, g["b"], g["d"], seq, head, 0, True) == tuple(g["y_shape"])
    assert oracle.shape(1, g["b"], g["d"], seq, head, 0, False) == tuple(g["y_shape"])
    assert oracle.shape(1, g["b"], g["d"], seq, head, 0, True) == tuple(g["x_shape"])
    # the round trip with data at a reduced d (shape logic is independent of d)
    rng = np.random.default_rng(1)
    d = 8
    xs = rand_shards(rng, 0, g["b"], d, seq, head, np.uint16)
    ys = oracle.a2a_4d(0, g["b"], d, seq, head, xs)
    zs = oracle.a2a_4d(1, g["b"], d, seq, head, ys)
    for x, z in zip(xs, zs):
        assert np.array_equal(x, z)


def test_fastvideo_window_bytes(golden):
    g = golden["fastvideo_window"]
    seq = [g["s_global"] // g["world"]] * g["world"]
    head = [g["n_global"] // g["world"]] * g["world"]
    wb0 = oracle.window_bytes(0, g["d"], g["elem_bytes"], seq, head)
    wb1 = oracle.window_bytes(1, g["d"], g["elem_bytes"], seq, head)
    assert wb0 == g["bytes_per_plane"]
    assert wb1 == g["bytes_per_plane"]
    assert wb0 <= g["window_cap_bytes"]


def test_window_bytes_uneven_is_largest_rank():
    seq, head = [3, 10, 1], [2, 1, 4]
    # mode 0 destination of r: s_global * H_r * d * esz; mode 1: S_r * n_global
    assert oracle.window_bytes(0, 8, 2, seq, head) == 14 * 4 * 8 * 2
    assert oracle.window_bytes(1, 8, 2, seq, head) == 10 * 7 * 8 * 2


# ---------------------------------------------------------------------------
# the permutation: library routines, brute force, invariants
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("seed", range(40))
def test_modes_match_numpy_concatenation(seed):
    rng = np.random.default_rng(100 + seed)
    world, b, d, seq, head = random_geometry(rng)
    dtype = [np.uint8, np.uint16, np.uint32][seed % 3]
    xs = rand_shards(rng, 0, b, d, seq, head, dtype)
    got = oracle.a2a_4d(0, b, d, seq, head, xs)
    for g, w in zip(got, concat_mode0(xs, seq, head)):
        assert g.shape == w.shape and np.array_equal(g, w)
    ys = rand_shards(rng, 1, b, d, seq, head, dtype)
    got = oracle.a2a_4d(1, b, d, seq, head, ys)
    for g, w in zip(got, concat_mode1(ys, seq, head)):
        assert g.shape == w.shape and np.array_equal(g, w)


@pytest.mark.parametrize("world", [1, 2, 3, 4, 5, 7, 8])
def test_even_splits_equal_permute_all_to_all_permute(world):
    """Even splits: the baseline's reshape/transpose form."""
    rng = np.random.default_rng(world)
    b, s_local, n_local, d = 2, 5, 3, 16
    seq, head = [s_local] * world, [n_local] * world
    xs = rand_shards(rng, 0, b, d, seq, head, np.uint16)
    X = np.stack(xs)                                    # (Wj, b, s_local, n, d)
    X = X.reshape(world, b, s_local, world, n_local, d)  # split heads by dst rank
    Y = X.transpose(3, 1, 0, 2, 4, 5)                   # (Wr, b, Wj, s_local, n_local, d)
    Y = Y.reshape(world, b, world * s_local, n_local, d)
    got = oracle.a2a_4d(0, b, d, seq, head, xs)
    for r in range(world):
        assert np.array_equal(got[r], Y[r])
    # mode 1 is the transposed exchange
    back = oracle.a2a_4d(1, b, d, seq, head, got)
    Z = np.stack(got).reshape(world, b, world, s_local, n_local, d)
    Z = Z.transpose(2, 1, 3, 0, 4, 5).reshape(world, b, s_local, world * n_local, d)
    for r in range(world):
        assert np.array_equal(back[r], Z[r])


@pytest.mark.parametrize("seed", range(12))
def test_index_coded_brute_force(seed):
    """Every output element decodes to the source coordinates the
    definition names: mode 0 row S of rank r comes from the rank j whose
    sequence range holds S, at local row S - seq_off_j and head
    head_off_r + h."""
    rng = np.random.default_rng(200 + seed)
    world, b, d, seq, head = random_geometry(rng, allow_zero=(seed % 2 == 0))
    so, ho = offsets(seq), offsets(head)
    n_global = int(ho[-1])
    codes = []
    for j in range(world):
        shp = (b, seq[j], n_global, d)
        bi, s, h, e = np.indices(shp)
        codes.append(((((j * 4 + bi) * 64 + s) * 64 + h) * 64 + e).astype(np.int64))
    got = oracle.a2a_4d(0, b, d, seq, head, codes)
    for r in range(world):
        bi, S, h, e = np.indices(got[r].shape)
        j = np.searchsorted(so, S, side="right") - 1
        want = (((j * 4 + bi) * 64 + (S - so[j])) * 64 + (ho[r] + h)) * 64 + e
        assert np.array_equal(got[r], want)


@pytest.mark.parametrize("seed", range(20))
def test_roundtrip_and_moved_once(seed):
    rng = np.random.default_rng(300 + seed)
    world, b, d, seq, head = random_geometry(rng)
    xs = rand_shards(rng, 0, b, d, seq, head, np.uint16)
    ys = oracle.a2a_4d(0, b, d, seq, head, xs)
    # every element moved exactly once: the multiset of values is unchanged
    a = np.sort(np.concatenate([x.ravel() for x in xs]))
    c = np.sort(np.concatenate([y.ravel() for y in ys]))
    assert np.array_equal(a, c)
    zs = oracle.a2a_4d(1, b, d, seq, head, ys)
    for x, z in zip(xs, zs):
        assert np.array_equal(x, z)


@pytest.mark.parametrize("threads", [2, 5, 8])
def test_threaded_loops_equal_single_thread(threads):
    """The threaded entry points hand destination rows to threads and must
    give the single-threaded result exactly, for the relayout and the fused
    row operation."""
    rng = np.random.default_rng(500 + threads)
    for _ in range(4):
        world, b, d, seq, head = random_geometry(rng)
        for mode in (0, 1):
            xs = rand_shards(rng, mode, b, d, seq, head, np.uint16)
            one = oracle.a2a_4d(mode, b, d, seq, head, xs)
            many = oracle.a2a_4d(mode, b, d, seq, head, xs, threads=threads)
            for a, c in zip(one, many):
                assert np.array_equal(a, c)
    b, d, seq, head = 2, 64, [40, 3, 21], [2, 1, 3]
    xs = [torch_bf16_bits(rng.standard_normal((b, S, 6, d))) for S in seq]
    gamma = (rng.random(d) + 0.5).astype(np.float32)
    c, s = oracle.rope_table(10000.0, 64, d)
    one = oracle.qknorm_rope_mode0(b, d, seq, head, xs, gamma, 1e-6, c, s)
    many = oracle.qknorm_rope_mode0(b, d, seq, head, xs, gamma, 1e-6, c, s, threads=threads)
    for a, m in zip(one, many):
        assert np.array_equal(a, m)


def test_world_one_is_identity():
    rng = np.random.default_rng(7)
    for mode in (0, 1):
        xs = rand_shards(rng, mode, 3, 16, [11], [6], np.uint32)
        got = oracle.a2a_4d(mode, 3, 16, [11], [6], xs)
        assert np.array_equal(got[0], xs[0])


def test_zero_splits_give_empty_pieces():
    rng = np.random.default_rng(8)
    seq, head = [0, 5, 0, 3], [2, 0, 3, 1]
    xs = rand_shards(rng, 0, 2, 8, seq, head, np.uint16)
    got = oracle.a2a_4d(0, 2, 8, seq, head, xs)
    assert got[1].shape == (2, 8, 0, 8)
    for g, w in zip(got, concat_mode0(xs, seq, head)):
        assert np.array_equal(g, w)


def test_bytes_are_copied_not_converted():
    """NaN payloads, -0 and every fp8 / int8 pattern survive unchanged."""
    seq, head = [3, 2], [1, 1]
    pat = np.array([0x7FC1, 0xFFFF, 0x8000, 0x7F81, 0x0001, 0xFF80], dtype=np.uint16)
    xs = [np.resize(pat, (1, s, 2, 8)).astype(np.uint16) for s in seq]
    got = oracle.a2a_4d(0, 1, 8, seq, head, xs)
    for g, w in zip(got, concat_mode0(xs, seq, head)):
        assert g.tobytes() == w.tobytes()


@pytest.mark.parametrize("mode", [0, 1])
def test_sample_equals_full(mode):
    rng = np.random.default_rng(9 + mode)
    world, b, d, seq, head = 5, 2, 16, [4, 0, 7, 2, 9], [3, 1, 0, 2, 2]
    xs = rand_shards(rng, mode, b, d, seq, head, np.uint16)
    full = oracle.a2a_4d(mode, b, d, seq, head, xs)
    coords = []
    for _ in range(500):
        r = int(rng.integers(0, world))
        shp = full[r].shape
        if 0 in shp:
            continue
        coords.append([r] + [int(rng.integers(0, n)) for n in shp])
    coords = np.array(coords)
    got = oracle.a2a_4d_sample(mode, b, d, seq, head, xs, coords)
    want = np.array([full[c[0]][tuple(c[1:])] for c in coords])
    assert np.array_equal(got, want)


def test_invalid_arguments_raise():
    with pytest.raises(ValueError):
        oracle.shape(2, 1, 8, [1], [1], 0, False)
    with pytest.raises(ValueError):
        oracle.window_bytes(0, 8, 2, [-1, 2], [1, 1])
    with pytest.raises(ValueError):
        oracle.a2a_4d_sample(0, 1, 8, [2, 2], [1, 1],
                             [np.zeros((1, 2, 2, 8), np.uint16)] * 2, [[0, 0, 4, 0, 0]])


# ---------------------------------------------------------------------------
# bfloat16 rounding and the rotary table
# ---------------------------------------------------------------------------


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # exact ties (dropped half == 0x8000) with even and odd kept lsb
    ties = (rng.integers(0, 2 ** 16, size=20_000, dtype=np.uint64).astype(np.uint32) << 16) \
        | np.uint32(0x8000)
    bits = np.concatenate([bits, ties, np.array([0, 0x80000000, 0x7F7FFFFF, 0x00000001,
                                                 0x7F800000, 0xFF800000], np.uint32)])
    f = bits.view(np.float32)
    finite = np.isfinite(f) | np.isinf(f)
    got = oracle.f32_to_bf16(f)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got[finite], want[finite])
    nan = ~finite
    assert np.all(np.isnan(oracle.bf16_to_f32(got[nan])))
    # widening is exact
    assert np.array_equal(oracle.bf16_to_f32(want).view(np.uint32), want.astype(np.uint32) << 16)


def test_rope_table_closed_forms():
    theta, d, s_global = 10000.0, 128, 400
    c, s = oracle.rope_table(theta, s_global, d)
    assert c.shape == (s_global, d // 2) and c.dtype == np.float32
    # position 0: no rotation
    assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)
    # pair 0 has frequency theta^0 = 1: the angle is S itself
    for S in range(s_global):
        assert c[S, 0] == np.float32(math.cos(S)) and s[S, 0] == np.float32(math.sin(S))
    # pair d/4 has frequency theta^(-1/2) = 1/100: position 100 is angle 1
    assert c[100, 32] == np.float32(math.cos(1.0)) and s[100, 32] == np.float32(math.sin(1.0))
    # position 1 gives the frequencies: a geometric progression theta^(-2p/d)
    w = np.arctan2(s[1].astype(np.float64), c[1].astype(np.float64))
    p = np.arange(d // 2)
    assert np.allclose(w, theta ** (-2.0 * p / d), rtol=2e-7, atol=0)
    # angles grow linearly with S: angle addition S -> S+1
    c64, s64 = c.astype(np.float64), s.astype(np.float64)
    nxt_c = c64[:-1] * c64[1] - s64[:-1] * s64[1]
    nxt_s = s64[:-1] * c64[1] + c64[:-1] * s64[1]
    assert np.max(np.abs(nxt_c - c64[1:])) < 1e-6
    assert np.max(np.abs(nxt_s - s64[1:])) < 1e-6
    assert np.max(np.abs(c64 ** 2 + s64 ** 2 - 1.0)) < 2e-7


def test_rope_table_other_d_and_theta():
    c, s = oracle.rope_table(500000.0, 10, 64)
    w = np.arctan2(s[1].astype(np.float64), c[1].astype(np.float64))
    assert np.allclose(w, 500000.0 ** (-2.0 * np.arange(32) / 64), rtol=2e-7, atol=0)


# ---------------------------------------------------------------------------
# fused RMSNorm + RoPE
# ---------------------------------------------------------------------------


def bf16_key(u):
    """Monotone integer key of a bf16 bit pattern (+0 and -0 coincide)."""
    u = u.astype(np.int32)
    mag = u & 0x7FFF
    return np.where(u & 0x8000, -mag, mag)


def torch_bf16_bits(x64):
    return torch.from_numpy(np.asarray(x64, dtype=np.float64)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def shadow_fused(xs_bits, seq, head, gamma, eps, c, s, b, d):
    """float64 RMSNorm (textbook) and RoPE as a complex multiplication at the
    global position, over the whole sequence at once; returns the
    destination shards in float64 before rounding."""
    so, ho = offsets(seq), offsets(head)
    full = np.concatenate([oracle.bf16_to_f32(x).astype(np.float64) for x in xs_bits], axis=1)
    rms = np.sqrt(np.mean(full ** 2, axis=-1, keepdims=True) + float(np.float32(eps)))
    y = full / rms * gamma.astype(np.float64)
    z = y[..., 0::2] + 1j * y[..., 1::2]
    rot = c.astype(np.float64) + 1j * s.astype(np.float64)      # [S, d/2]
    z = z * rot[None, :, None, :]
    out = np.empty_like(y)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return [out[:, :, ho[r]:ho[r + 1], :] for r in range(len(seq))], np.abs(y).max()


@pytest.mark.parametrize("seed", range(4))
def test_fused_matches_float64_shadow(seed):
    rng = np.random.default_rng(400 + seed)
    world = [1, 3, 4, 7][seed]
    b, d = 2, [128, 64, 128, 32][seed]
    seq = random_splits(rng, 60, world, allow_zero=False)
    head = random_splits(rng, 2 * world + 1, world, allow_zero=False)
    xs = [torch_bf16_bits(rng.standard_normal((b, S, sum(head), d)) * 3.0) for S in seq]
    gamma = (rng.random(d) + 0.5).astype(np.float32)
    c, s = oracle.rope_table(10000.0, sum(seq), d)
    got = oracle.qknorm_rope_mode0(b, d, seq, head, xs, gamma, 1e-6, c, s)
    shadow, ymax = shadow_fused(xs, seq, head, gamma, 1e-6, c, s, b, d)
    for g, w in zip(got, shadow):
        gf = oracle.bf16_to_f32(g).astype(np.float64)
        # absolute error: fp32 rounding of the row ops plus one bf16 rounding
        assert np.all(np.abs(gf - w) <= np.abs(w) * 2.0 ** -8 + ymax * 1e-6)
        # away from cancellation the result is the correctly rounded one or
        # its neighbour
        big = np.abs(w) > ymax * 1e-3
        dist = np.abs(bf16_key(g) - bf16_key(torch_bf16_bits(w)))
        assert dist[big].max() <= 1


def test_fused_one_hot_closed_form():
    """A row that is 2 at element k and 0 elsewhere: ss = 4, the mean square
    is 4/d, and only the pair holding k is non-zero after RoPE, rotated by
    the angle S * w_p (counter-clockwise: +sin goes to the odd element)."""
    d, seq, head, b = 128, [5, 6], [1, 1], 1
    xs = [np.zeros((b, S, 2, d), np.uint16) for S in seq]
    k = 37                                 # odd element: pair p = 18, second slot
    xs[1][0, 2, 0, k] = torch_bf16_bits(2.0)
    gamma = np.linspace(0.5, 1.5, d).astype(np.float32)
    c, s = oracle.rope_table(10000.0, 11, d)
    got = oracle.qknorm_rope_mode0(b, d, seq, head, xs, gamma, 1e-6, c, s)
    S = 5 + 2                              # global position of rank 1's row 2
    inv = 1.0 / math.sqrt(4.0 / d + float(np.float32(1e-6)))
    yk = 2.0 * inv * float(gamma[k])
    p = k // 2
    want = np.zeros(d)
    want[2 * p] = -yk * float(s[S, p])     # o[2p]   = y[2p] c - y[2p+1] s
    want[2 * p + 1] = yk * float(c[S, p])  # o[2p+1] = y[2p] s + y[2p+1] c
    row = got[0][0, S, 0]
    assert np.abs(bf16_key(row) - bf16_key(torch_bf16_bits(want))).max() <= 1
    # every other destination row is zero (the zero row stays zero: eps > 0)
    mask = np.ones(got[0].shape[:3], bool)
    mask[0, S, 0] = False
    assert np.all(oracle.bf16_to_f32(got[0][mask]) == 0.0)
    assert np.all(oracle.bf16_to_f32(got[1]) == 0.0)


@pytest.mark.parametrize("d", [32, 128])
def test_sum_of_squares_order(d):
    """The order of the fp32 sum of squares, pinned by a row whose partial
    sums round differently under other orders.  Ones at elements 0, 1 (first
    group of 8: partial 2), 8 (partial 1), 16, 17, 18 (partial 3) and 4096 at
    element 24 (partial 2^24); every partial is exact.  The adjacent-pairing
    tree adds (2 + 1) = 3 and (3 + 2^24) = 2^24 + 3, a tie between 2^24 + 2 and
    2^24 + 4 that goes to the even 2^24 + 4; then 3 + 2^24 + 4 = 2^24 + 7, a
    tie that goes to the even 2^24 + 8 (zero partials beyond the fourth add
    nothing).  Pairing the halves first (2 + 3, 1 + 2^24) gives 2^24 + 4, and a
    single chain over the row gives 2^24 + 6."""
    row = np.zeros(d, np.float64)
    row[[0, 1, 8, 16, 17, 18]] = 1.0
    row[24] = 4096.0
    ss = oracle.row_sum_of_squares(d, torch_bf16_bits(row))
    assert ss == np.float32(2 ** 24 + 8)
    with pytest.raises(ValueError):
        oracle.row_sum_of_squares(24, np.zeros(24, np.uint16))


def test_fused_position_is_global():
    """W ranks give the same rows as one rank holding the whole sequence:
    RoPE uses the global position seq_off_j + s, not the local s."""
    rng = np.random.default_rng(12)
    b, d, seq, head = 2, 64, [4, 9, 3], [2, 1, 3]
    xs = [torch_bf16_bits(rng.standard_normal((b, S, 6, d))) for S in seq]
    gamma = (rng.random(d) + 0.5).astype(np.float32)
    c, s = oracle.rope_table(10000.0, 16, d)
    got = oracle.qknorm_rope_mode0(b, d, seq, head, xs, gamma, 1e-6, c, s)
    whole = oracle.qknorm_rope_mode0(b, d, [16], [6], [np.concatenate(xs, axis=1)],
                                     gamma, 1e-6, c, s)[0]
    ho = offsets(head)
    for r in range(3):
        assert np.array_equal(got[r], whole[:, :, ho[r]:ho[r + 1], :])


def test_fused_sample_equals_full():
    rng = np.random.default_rng(13)
    b, d, seq, head = 1, 128, [7, 5], [2, 3]
    xs = [torch_bf16_bits(rng.standard_normal((b, S, 5, d))) for S in seq]
    gamma = (rng.random(d) + 0.5).astype(np.float32)
    c, s = oracle.rope_table(10000.0, 12, d)
    full = oracle.qknorm_rope_mode0(b, d, seq, head, xs, gamma, 1e-6, c, s)
    rows = [[r, 0, S, h] for r in range(2) for S in range(12) for h in range(head[r])]
    got = oracle.qknorm_rope_mode0_sample(b, d, seq, head, xs, gamma, 1e-6, c, s, rows)
    for (r, bi, S, h), g in zip(rows, got):
        assert np.array_equal(g, full[r][bi, S, h])


def test_fused_rejects_unsupported_d():
    with pytest.raises(ValueError):
        oracle.qknorm_rope_mode0(1, 24, [1], [1], [np.zeros((1, 1, 1, 24), np.uint16)],
                                 np.ones(24, np.float32), 1e-6,
                                 np.ones((1, 12), np.float32), np.zeros((1, 12), np.float32))


# ---------------------------------------------------------------------------
# the fused row's remaining rounding steps, pinned by hand-worked rows
# ---------------------------------------------------------------------------
#
# Exact rational arithmetic with IEEE binary32 rounding (nearest, ties to
# even), written here from the format's definition, so that the expected bits
# below are derived independently of the oracle's C code.

from fractions import Fraction as Q


def f32_round(q):
    """The binary32 value nearest to the rational q (ties to even; normal
    range only, which every value below stays in)."""
    if q == 0:
        return Q(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    scaled = a * 2 ** 23                     # in [2^23, 2^24)
    lo = scaled.numerator // scaled.denominator
    rem = scaled - lo
    if rem > Q(1, 2) or (rem == Q(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * Q(lo) * Q(2) ** (e - 23)


def f32_sqrt(q):
    """Correctly rounded binary32 square root of a positive rational: the
    candidate r whose rounding interval [r - ulp/2, r + ulp/2] holds sqrt(q)."""
    r = f32_round(Q(math.sqrt(float(q))))
    for _ in range(4):
        ulp = Q(2) ** (math.frexp(float(r))[1] - 24)
        lo, hi = r - ulp / 2, r + ulp / 2
        if lo * lo <= q <= hi * hi:
            return r
        r = r + ulp if hi * hi < q else r - ulp
    raise AssertionError("no correctly rounded candidate")


def f32_bits(q):
    return int(np.float32(float(q)).view(np.uint32))


def bf16_bits(q):
    """bf16 (nearest, ties to even) of a binary32 value given exactly."""
    u = f32_bits(q)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16) & 0xFFFF


def fused_one_row(d, x, gamma, cos_row, sin_row, eps):
    """The oracle's fused output of one row (W = 1, b = 1, one head, position
    0, tables of one row given explicitly)."""
    row = np.zeros(d, np.float64)
    row[:len(x)] = x
    g = np.ones(d, np.float32)
    g[:len(gamma)] = gamma
    c = np.ones((1, d // 2), np.float32)
    s = np.zeros((1, d // 2), np.float32)
    c[0, :len(cos_row)] = cos_row
    s[0, :len(sin_row)] = sin_row
    xs = [torch_bf16_bits(row).reshape(1, 1, 1, d)]
    return oracle.qknorm_rope_mode0(1, d, [1], [1], xs, g, eps, c, s)[0].reshape(d)


E11, E12 = Q(1, 2 ** 11), Q(1, 2 ** 12)
# Rows whose rotation outputs depend on each product being rounded on its
# own: y = (x * inv) * gamma with x = 1/2 and inv = 2 exactly, so y = gamma.
ROTATION_Y = [1 + E12, 1, 1, 1 + E12, 1 + E12, 1, 1, 1 + E12]
ROTATION_COS = [1 + E12, 1 + E11, -(1 + E11), -(1 + E12)]
ROTATION_SIN = [1 + E11, 1 + E12, 1 + E12, 1 + E11]


def rotation_row(d):
    """Elements 0..7 are 1/2 (sum of squares 2); for d = 128, elements 8..11
    hold 4, 3, 2, 1 (a second partial of 30), so the mean square is 1/4 at
    both d and inv = 1/sqrt(1/4 + 0) = 2 exactly."""
    x = [0.5] * 8 + ([4.0, 3.0, 2.0, 1.0] if d == 128 else [])
    return x, [float(v) for v in ROTATION_Y]


@pytest.mark.parametrize("d", [8, 128])
def test_rotation_products_rounded_separately(d):
    """Each rotation product is rounded before the add or subtract (no fused
    multiply-add), worked by hand for four pairs at position 0 with an
    explicit table row:
      pair 0: y = (1 + 2^-12, 1), cos 1 + 2^-12, sin 1 + 2^-11.
        y0*cos = 1 + 2^-11 + 2^-24, a tie that goes to the even 1 + 2^-11, and
        y1*sin = 1 + 2^-11, so o0 = +0; contracting y0*cos into the subtract
        would leave 2^-24 (bf16 0x3380).  o1 = (1 + 2^-11 + 2^-12 + 2^-23) +
        (1 + 2^-12) = 2 + 2^-10 + 2^-23, a tie to 2 + 2^-10, bf16 2.0.
      pair 1: y = (1, 1 + 2^-12), cos 1 + 2^-11, sin 1 + 2^-12: the second
        product of o2 is the rounded one, o2 = +0 (a contraction of it:
        -2^-24), o3 = 2.0.
      pair 2: y = (1 + 2^-12, 1), cos -(1 + 2^-11), sin 1 + 2^-12: o4 =
        -(2 + 2^-10 + 2^-23) -> -2.0; o5 = (1 + 2^-11) - (1 + 2^-11) = +0 (a
        contraction of y4*sin: 2^-24).
      pair 3: y = (1, 1 + 2^-12), cos -(1 + 2^-12), sin 1 + 2^-11: o6 = -2.0,
        o7 = +0 (a contraction of y7*cos: -2^-24).
    At d = 128 elements 8..11 (4, 3, 2, 1, gain 1, identity rotation) come
    out as 2x."""
    x, gamma = rotation_row(d)
    out = fused_one_row(d, x, gamma, [float(v) for v in ROTATION_COS],
                        [float(v) for v in ROTATION_SIN], 0.0)
    # the hand derivation, step by step in exact arithmetic
    y = ROTATION_Y
    want = []
    for p in range(4):
        c, s = ROTATION_COS[p], ROTATION_SIN[p]
        a, b = f32_round(y[2 * p] * c), f32_round(y[2 * p + 1] * s)
        e, f = f32_round(y[2 * p] * s), f32_round(y[2 * p + 1] * c)
        want += [bf16_bits(f32_round(a - b)), bf16_bits(f32_round(e + f))]
    assert want == [0x0000, 0x4000, 0x0000, 0x4000, 0xC000, 0x0000, 0xC000, 0x0000]
    # each contraction would change one output
    contracted = [bf16_bits(f32_round(y[0] * ROTATION_COS[0] - f32_round(y[1] * ROTATION_SIN[0]))),
                  bf16_bits(f32_round(f32_round(y[2] * ROTATION_COS[1]) - y[3] * ROTATION_SIN[1])),
                  bf16_bits(f32_round(y[4] * ROTATION_SIN[2] + f32_round(y[5] * ROTATION_COS[2]))),
                  bf16_bits(f32_round(f32_round(y[6] * ROTATION_SIN[3]) + y[7] * ROTATION_COS[3]))]
    assert contracted == [0x3380, 0xB380, 0x3380, 0xB380]
    if d == 128:
        want += [0x4100, 0x40C0, 0x4080, 0x4000]      # 8, 6, 4, 2
    want += [0] * (d - len(want))
    assert [int(v) for v in out] == want


# (x * inv) * gamma against x * (inv * gamma): one non-zero element x0 = 1.5,
# eps = 0, identity rotation.  The gains were found by a search over random
# binary32 values in [0.5, 1.5) for a row whose bf16 output depends on the
# order of the two products.
GAIN_ORDER = {8: (0x3F9EBED7, 0x3FF15BF0, 0x4061, 0x4060),
              128: (0x3F9D54CD, 0x40F15BF0, 0x415E, 0x415F)}


@pytest.mark.parametrize("d", [8, 128])
def test_gain_applied_after_the_norm(d):
    """y = (x * inv) * gamma, two products rounded in that order.  With one
    non-zero element x0 = 1.5 and eps = 0: ss = 2.25, ms = 2.25 / d, inv =
    1 / sqrt(ms) with both steps correctly rounded (0x3FF15BF0 at d = 8,
    0x40F15BF0 at d = 128, four times it).  For the gain listed, the bf16
    output of element 0 is 0x4061 (d = 8) or 0x415E (d = 128) in this order,
    and 0x4060 or 0x415F with the gain folded into inv first."""
    g_bits, inv_bits, want0, other0 = GAIN_ORDER[d]
    g0 = Q(float(np.uint32(g_bits).view(np.float32)))
    x0 = Q(3, 2)
    ms = f32_round(x0 * x0 / d)
    inv = f32_round(1 / f32_sqrt(ms))
    assert f32_bits(inv) == inv_bits
    assert bf16_bits(f32_round(f32_round(x0 * inv) * g0)) == want0
    assert bf16_bits(f32_round(x0 * f32_round(inv * g0))) == other0
    out = fused_one_row(d, [1.5], [float(g0)], [], [], 0.0)
    assert int(out[0]) == want0
    assert np.all(out[1:] == 0)
