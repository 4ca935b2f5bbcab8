"""Helpers of the GPU parity tests: guarded destination buffers, host byte
views, coordinate sampling.  Torch is used for device memory only."""
import numpy as np
import torch

from sequence_attention_relayout_amd import workloads as W

GUARD = 4096
GUARD_BYTE = 0xA5
POISON_BYTE = 0x5A


def say(msg):
    print(msg, flush=True)


def to_np(t):
    """Host numpy copy of a tensor as unsigned integers of the element size
    (bitwise: bf16 -> uint16, fp32 -> uint32, 1-byte types -> uint8)."""
    t = t.detach().contiguous().cpu()
    iv = {1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()]
    npv = {1: np.uint8, 2: np.uint16, 4: np.uint32}[t.element_size()]
    return t.view(iv).numpy().view(npv)


class Guarded:
    """Destination shards carved out of larger byte buffers: GUARD bytes of
    0xA5 on both sides (any write outside the shard shows there) and the
    shard itself pre-filled with 0x5A (a vector left unwritten shows in
    the comparison)."""

    def __init__(self, shapes, dtype_name, device):
        esz = W.ELEM_BYTES[dtype_name]
        self.raw, self.views, self.nbytes = [], [], []
        for shp in shapes:
            n = int(np.prod(shp)) * esz
            raw = torch.full((n + 2 * GUARD,), GUARD_BYTE, dtype=torch.uint8, device=device)
            raw[GUARD:GUARD + n].fill_(POISON_BYTE)
            self.raw.append(raw)
            self.nbytes.append(n)
            self.views.append(raw[GUARD:GUARD + n].view(W.torch_dtype(dtype_name)).view(shp))

    def guards_intact(self):
        for raw, n in zip(self.raw, self.nbytes):
            head = raw[:GUARD]
            tail = raw[GUARD + n:]
            if not (bool((head == GUARD_BYTE).all()) and bool((tail == GUARD_BYTE).all())):
                return False
        return True


def sample_coords(rng, shapes, n, boundary_rows=()):
    """n uniform coordinates (rank, bi, s, h, e) over the destination shards,
    weighted by shard size, plus every element of the listed (rank, bi, s)
    rows."""
    sizes = np.array([int(np.prod(s)) for s in shapes], dtype=np.float64)
    ranks = rng.choice(len(shapes), size=n, p=sizes / sizes.sum())
    out = []
    for r in range(len(shapes)):
        k = int((ranks == r).sum())
        if k == 0 or sizes[r] == 0:
            continue
        cols = [rng.integers(0, dim, size=k) for dim in shapes[r]]
        out.append(np.stack([np.full(k, r)] + cols, axis=1))
    for (r, bi, s) in boundary_rows:
        _, _, nh, d = shapes[r]
        h, e = np.meshgrid(np.arange(nh), np.arange(d), indexing="ij")
        m = h.size
        out.append(np.stack([np.full(m, r), np.full(m, bi), np.full(m, s), h.ravel(),
                             e.ravel()], axis=1))
    return np.concatenate(out).astype(np.int64)


def gather(host_shards, coords):
    """Values of host shards at coords (n x 5)."""
    out = np.empty(len(coords), dtype=host_shards[0].dtype)
    for r in range(len(host_shards)):
        sel = coords[:, 0] == r
        if sel.any():
            c = coords[sel]
            out[sel] = host_shards[r][c[:, 1], c[:, 2], c[:, 3], c[:, 4]]
    return out


def bf16_key(u):
    """Monotone integer key of bf16 bit patterns; +0 and -0 coincide."""
    u = u.astype(np.int32)
    mag = u & 0x7FFF
    return np.where(u & 0x8000, -mag, mag)
