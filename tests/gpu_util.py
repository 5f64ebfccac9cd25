"""Helpers of the GPU parity tests: moving bf16 bit patterns to and from the device and
the error measures of the parity bar (max abs error <= 1e-2, relative L2 <= 5e-3)."""
from __future__ import annotations

import sys

import numpy as np

MAX_ABS = 1e-2
REL_L2 = 5e-3


def to_dev(bits, device="cuda"):
    import torch
    arr = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).view(np.int16)
    return torch.from_numpy(arr).view(torch.bfloat16).to(device)


def i32_dev(x, device="cuda"):
    import torch
    return torch.as_tensor(np.asarray(x, dtype=np.int32)).to(device)


def bits_of(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64_of(t) -> np.ndarray:
    return (bits_of(t).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def errors(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), "non-finite output"
    max_abs = float(np.max(np.abs(got - want))) if got.size else 0.0
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    return max_abs, rel


def assert_parity(got, want, what: str):
    max_abs, rel = errors(got, want)
    print(f"[parity] {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)
    assert max_abs <= MAX_ABS, f"{what}: max abs error {max_abs:.3e} > {MAX_ABS}"
    assert rel <= REL_L2, f"{what}: relative L2 error {rel:.3e} > {REL_L2}"


def assert_cached_keys_close(got_bits, want_bits, what: str):
    """Cached (rotated) keys: the GPU rotates in fp32 with hardware sin/cos (absolute error
    ~1e-7 per element for N(0,1) inputs) and rounds to bf16; the oracle rounds the exact
    fp64 rotation.  Allowed: one bf16 step, plus 1e-5 absolute for values near zero where
    a bf16 step is smaller than the fp32 error.  Differences must also be rare."""
    got = (np.asarray(got_bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    want = (np.asarray(want_bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    ulp = np.ldexp(1.0, np.frexp(want)[1] - 8)
    d = np.abs(got - want)
    bad = d > ulp + 1e-5
    frac = float(np.mean(np.asarray(got_bits) != np.asarray(want_bits)))
    worst = int(np.argmax(d - ulp))
    print(f"[cache] {what}: differing={frac:.2e} worst |d|={d.flat[worst]:.3e} at value "
          f"{want.flat[worst]:.4e} (step {ulp.flat[worst]:.2e})", flush=True)
    assert not bad.any(), f"{what}: {int(bad.sum())} cached keys beyond one bf16 step + 1e-5"
    assert frac < 1e-3, f"{what}: {frac:.2e} of cached keys differ"


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()
