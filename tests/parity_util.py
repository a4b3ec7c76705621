"""Helpers shared by the GPU parity tests: seeded adversarial inputs and
bit-level comparison.  No quantization arithmetic here."""
import numpy as np


def adversarial_f32(rng, n, block):
    """n values (n a multiple of block) mixing the cases the quantizer must
    get right bit for bit: ordinary blocks, heavy tails, exact ties, all-zero
    and constant blocks, a lone nonzero element, absmax in the last slot,
    tiny (fp32-subnormal) and huge magnitudes."""
    nb = n // block
    x = np.empty((nb, block), np.float64)
    for b in range(nb):
        kind = b % 11
        if kind == 0:
            x[b] = rng.standard_normal(block) * 0.02
        elif kind == 1:
            x[b] = rng.standard_t(3, block) * 1e-3
        elif kind == 2:
            # exact ties (k + 1/2) * s for s = absmax / 7 or / 127 representable
            s = float(np.float32(rng.uniform(0.5, 2)))
            q = 7 if b % 2 else 127
            x[b] = (rng.integers(-q, q, block) + 0.5) * s
            x[b, rng.integers(block)] = q * s
        elif kind == 3:
            x[b] = 0.0
        elif kind == 4:
            x[b] = rng.standard_normal() * 1e-2
        elif kind == 5:
            x[b] = 0.0
            x[b, rng.integers(block)] = rng.standard_normal()
        elif kind == 6:
            x[b] = rng.standard_normal(block)
            x[b, -1] = 50.0
        elif kind == 7:
            x[b] = rng.standard_normal(block) * 1e-41      # fp32 subnormals, s underflows
        elif kind == 8:
            x[b] = rng.standard_normal(block) * 3e-39      # subnormal scale, nonzero
        elif kind == 9:
            x[b] = rng.standard_normal(block) * 1e37       # near the top of fp32
            x[b, 0] = 3.3e38
        else:
            x[b] = rng.integers(-300, 300, block) / 8.0
    return x.ravel().astype(np.float32)


def as_dtype(x32, dtype):
    """fp32 values rounded into a storage type, as numpy arrays (bf16 as uint16 bits)."""
    import torch
    if dtype == "f16":                       # keep values finite in fp16
        x32 = np.clip(x32, -65504.0, 65504.0).astype(np.float32)
    t = torch.from_numpy(np.ascontiguousarray(x32))
    if dtype == "f32":
        return x32.copy()
    if dtype == "f16":
        return t.to(torch.float16).numpy()
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_device(a, dtype=None):
    """numpy -> CUDA tensor (bf16 given as uint16 bits when dtype == 'bf16')."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.cuda()


def from_device(t):
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view({1: np.uint8, 2: np.uint16, 4: np.uint32}[a.dtype.itemsize])


def assert_bits_equal(got, want, what):
    g, w = bits(got), bits(want)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    bad = np.nonzero(g != w)[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {g.size} differ; first at {bad[:8].tolist()}: "
                           f"got {g[bad[:8]].tolist()} want {w[bad[:8]].tolist()}")


def nan_mask(a, dtype):
    """Positions holding a NaN, for fp32 / fp16 arrays or bf16 bit patterns."""
    if dtype == "bf16":
        b = np.ascontiguousarray(a).view(np.uint16)
        return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)
    return np.isnan(a)


def assert_equal_nan_aware(got, want, dtype, what):
    """Bit equality, except that where the expected value is a NaN the result
    must be a NaN of any sign and payload (the definition fixes neither)."""
    wn = nan_mask(want, dtype)
    gn = nan_mask(got, dtype)
    assert np.array_equal(gn, wn), (f"{what}: NaN positions differ: "
                                    f"{np.nonzero(gn != wn)[0][:8].tolist()}")
    keep = ~wn
    assert_bits_equal(np.ascontiguousarray(got)[keep], np.ascontiguousarray(want)[keep], what)
