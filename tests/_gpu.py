"""Helpers for the GPU parity tests: device transfers, sampling and logging."""

import sys

import numpy as np
import pytest
import torch

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def note(msg):
    """Print a progress line that names the case, flushed before the GPU step."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    """uint16 bf16 bit patterns (numpy) -> bf16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host_bits(t):
    """bf16 tensor -> uint16 numpy bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def host(t):
    return t.detach().contiguous().cpu().numpy()


def sample_indices(n, k, seed, group=1):
    """k sorted distinct indices in [0, n) (multiples of `group` kept whole), incl. first and last."""
    rng = np.random.default_rng(seed)
    units = n // group
    k_units = min(units, max(2, k // group))
    pick = set(rng.choice(units, size=k_units, replace=False).tolist()) | {0, units - 1}
    idx = np.concatenate([np.arange(u * group, u * group + group) for u in sorted(pick)])
    return idx


def assert_bytes_equal(got, want, what, x_bits=None):
    """Bit-exact comparison of codes/scales with a report of the first differences."""
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    if bad.size:
        lines = [f"{what}: {len(bad)} of {got.size} differ"]
        for idx in bad[:8]:
            t = tuple(idx)
            extra = f" input bits {x_bits[t]:04x}" if x_bits is not None and x_bits.shape == got.shape else ""
            lines.append(f"  {t}: gpu={got[t]!r} want={want[t]!r}{extra}")
        raise AssertionError("\n".join(lines))


def one_per_tile(n, seed, group=1, band=256):
    """Indices with one `group`-wide unit inside every `band`-wide band of [0, n), plus the last unit."""
    rng = np.random.default_rng(seed)
    units = []
    for t in range((n + band - 1) // band):
        lo, hi = band * t // group, min(band * t + band, n) // group
        units.append(int(rng.integers(lo, hi)))
    units = sorted(set(units) | {n // group - 1})
    return np.concatenate([np.arange(u * group, u * group + group) for u in units])


_weight_cache = {}


def oracle_weight(w):
    """oracle.quant.quantize_weight_128x128 of a device bf16 weight: (codes, scales).

    The 128x128 blocks are independent, so 128-row bands are quantized in
    threads and stacked. The last result is cached by the weight's bytes.
    """
    import hashlib
    from concurrent.futures import ThreadPoolExecutor
    from oracle import quant
    bits = host_bits(w)
    key = hashlib.sha256(bits.tobytes()).hexdigest()
    if key not in _weight_cache:
        bands = [bits[r:r + 128] for r in range(0, bits.shape[0], 128)]
        with ThreadPoolExecutor(max_workers=16) as ex:
            parts = list(ex.map(quant.quantize_weight_128x128, bands))
        _weight_cache.clear()
        _weight_cache[key] = (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))
    return _weight_cache[key]
