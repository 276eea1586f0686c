"""Helpers shared by the GPU parity tests: host <-> device marshalling of the
seeded inputs, and the GEMM acceptance check against the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np

# GEMM acceptance: relative Frobenius error and per-element error against the
# exact (fp64) result computed from the same codes and scales.
TOL_FRO = 5e-3
TOL_MAX = 1e-2


def say(*a) -> None:
    """Name the case before a GPU step, flushed, so a fault still shows it."""
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def dev_bf16(bits: np.ndarray, dev="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def dev_u8(a: np.ndarray, dev="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def host_u8(t) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def host_f32(t) -> np.ndarray:
    return t.contiguous().cpu().numpy().astype(np.float32)


def host_bf16_as_f64(t) -> np.ndarray:
    import torch
    return t.float().contiguous().cpu().numpy().astype(np.float64)


def gemm_errors(y: np.ndarray, ref: np.ndarray) -> dict:
    err = y - ref
    nref = float(np.linalg.norm(ref))
    mref = float(np.abs(ref).max()) if ref.size else 0.0
    out = {
        "rel_fro": float(np.linalg.norm(err)) / nref if nref > 0 else float(np.linalg.norm(err)),
        "max_abs": float(np.abs(err).max()) if err.size else 0.0,
        "max_ref": mref,
    }
    out["max_rel"] = out["max_abs"] / mref if mref > 0 else out["max_abs"]
    ny = float(np.linalg.norm(y))
    out["cosine"] = float(np.dot(y.ravel(), ref.ravel()) / (ny * nref)) if ny > 0 and nref > 0 else 1.0
    return out


def assert_gemm_close(y: np.ndarray, ref: np.ndarray, what: str = "") -> dict:
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    e = gemm_errors(y, ref)
    if e["max_ref"] == 0.0:
        assert e["max_abs"] == 0.0, (what, e)
        return e
    assert e["rel_fro"] <= TOL_FRO, (what, e)
    assert e["max_abs"] <= TOL_MAX * e["max_ref"], (what, e)
    return e


def rows_every_tile(m: int, seed: int, tile: int = 256, per_tile: int = 2,
                    min_total: int = 64) -> np.ndarray:
    """Seeded output rows to compare on a full-size GEMM: at least `per_tile`
    rows in every band of `tile` rows (more per band when that is needed to
    reach `min_total`), plus the first and last row.  With every column of
    those rows compared, every tile x tile output tile is checked."""
    bands = (m + tile - 1) // tile
    per = max(per_tile, -(-min_total // bands))
    rng = np.random.default_rng(seed)
    picks = [0, m - 1]
    for b in range(bands):
        lo, hi = b * tile, min(m, (b + 1) * tile)
        picks.extend(rng.choice(np.arange(lo, hi), size=min(per, hi - lo), replace=False).tolist())
    return np.unique(np.asarray(picks, dtype=np.int64))
