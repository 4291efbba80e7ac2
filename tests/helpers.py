"""Shared test helpers: semiring names, vector makers and the parity checks."""
import numpy as np

import oracle

ORC_SEMIRING = {"plus_times": oracle.PLUS_TIMES, "boolean": oracle.BOOLEAN_F32,
                "boolean_u32": oracle.BOOLEAN_U32, "tropical": oracle.TROPICAL}
ORC_DIR = {"right": oracle.RIGHT, "left": oracle.LEFT}
ALL_SEMIRINGS = ("plus_times", "boolean", "boolean_u32", "tropical")


def make_x(rng, semiring, n, batch):
    """Input vectors of the semiring's domain; plus-times values are k*2^-24."""
    size = n * batch
    if semiring == "boolean_u32":
        w = rng.integers(0, 2**32, size=size, dtype=np.uint64).astype(np.uint32)
        w[rng.random(size) < 0.3] = 0
        return w
    if semiring == "tropical":
        x = (rng.integers(0, 100 * 2**16, size=size) / 2**16).astype(np.float32)
        x[rng.random(size) < 0.5] = np.inf
        return x
    if semiring == "boolean":
        x = rng.integers(0, 3, size=size).astype(np.float32)
        x[rng.random(size) < 0.1] = -0.0
        return x
    return (rng.integers(0, 2**24, size=size) / 2**24).astype(np.float32)


def to_device(x, device):
    import torch
    if x.dtype == np.uint32:
        return torch.from_numpy(x.view(np.int32)).to(device)
    return torch.from_numpy(x).to(device)


def from_device(y, semiring):
    a = y.cpu().numpy()
    return a.view(np.uint32) if semiring == "boolean_u32" else a


def check_parity(got, ref, semiring, what=""):
    """Bit-exact for Boolean and tropical; plus-times within relative 1e-5 of
    the fp64 oracle, or absolute 1e-6 where the oracle's value is below 0.1."""
    got = np.asarray(got).reshape(-1)
    ref = np.asarray(ref).reshape(-1)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    if semiring == "plus_times":
        g = got.astype(np.float64)
        err = np.abs(g - ref)
        ok = (err <= 1e-5 * np.abs(ref)) | ((np.abs(ref) < 0.1) & (err <= 1e-6))
        if not ok.all():
            bad = np.nonzero(~ok)[0][:5]
            raise AssertionError(f"{what}: {int((~ok).sum())} entries out of tolerance, e.g. "
                                 f"{[(int(i), float(g[i]), float(ref[i])) for i in bad]}")
    else:
        gb = got.astype(np.float32 if semiring != "boolean_u32" else np.uint32).view(np.uint32)
        rb = ref.astype(np.float32 if semiring != "boolean_u32" else np.uint32).view(np.uint32)
        if not np.array_equal(gb, rb):
            bad = np.nonzero(gb != rb)[0][:5]
            raise AssertionError(f"{what}: {int((gb != rb).sum())} entries differ, e.g. "
                                 f"{[(int(i), int(gb[i]), int(rb[i])) for i in bad]}")
