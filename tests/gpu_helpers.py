"""Comparison helpers shared by the GPU parity tests (no arithmetic of the path)."""

import sys

import numpy as np
import torch

# fused-layer tolerance: relative Frobenius error and max-abs error against the oracle
REL_FROB_TOL = 1e-2
MAX_ABS_FRAC = 0.05


def say(*a):
    """Name the case on stdout before a GPU step (flushed)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def assert_close_to_oracle(got, ref, what=""):
    g = got.float().cpu().numpy().astype(np.float64) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    nr = np.linalg.norm(r)
    rel = np.linalg.norm(g - r) / nr if nr > 0 else np.linalg.norm(g)
    mx = np.max(np.abs(g - r)) if g.size else 0.0
    lim = MAX_ABS_FRAC * (np.max(np.abs(r)) if r.size else 0.0)
    assert rel <= REL_FROB_TOL, f"{what}: relative Frobenius error {rel:.3e} > {REL_FROB_TOL}"
    assert mx <= lim, f"{what}: max abs error {mx:.3e} > {lim:.3e}"
    return rel, mx


def e4m3_ordinal(codes):
    """Signed ordinal of e4m3 codes: adjacent representable values differ by 1, +0 == -0."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = c & 0x7F
    return np.where(c >> 7, -mag, mag)


def dev_experts(t):
    """Per-expert host view of a device tensor (the oracle indexes weights by expert)."""
    class _V:
        def __len__(self):
            return t.shape[0]

        def __getitem__(self, e):
            return t[e].cpu().numpy()
    return _V()
