"""Helpers for the GPU parity tests: host arrays to device tensors and the parity
metric (per token row: max |gpu - oracle| / max |oracle|)."""
import numpy as np
import torch

TOL = 1e-2  # max relative error of the FFN output, per token row


def to_dev(arrays, device="cuda"):
    out = {}
    for k, v in arrays.items():
        if v.dtype == np.uint16:
            v = v.view(np.int16)
        out[k] = torch.from_numpy(np.ascontiguousarray(v)).to(device)
    return out


def bf16_out_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def row_rel_err(got, ref):
    num = np.max(np.abs(got - ref), axis=1)
    den = np.max(np.abs(ref), axis=1)
    return num / np.where(den > 0, den, 1.0)


def report(name, got, ref):
    e = row_rel_err(got, ref)
    norm = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    print(f"[parity] {name}: rows={got.shape[0]} max_row_rel={e.max():.3e} "
          f"mean_row_rel={e.mean():.3e} normwise={norm:.3e}", flush=True)
    return e


def tile_cover_rows(topk_ids, E, n_min, seed, chunk=128):
    """Token rows to compare at full size: for every expert, its routed pairs in the align
    order (ascending flat index t * k + s) are cut into pieces of `chunk` rows, the pieces
    the prefill kernels' row tiles are made of (tiles of 128 or 256 rows); the tokens of
    the first and the last pair of every piece are taken, so every row tile and every
    expert's ragged last tile holds a checked row. Seeded random rows top the set up to at
    least n_min. Returns sorted unique token indices."""
    ids = np.asarray(topk_ids)
    T, k = ids.shape
    flat = ids.reshape(-1)
    rows = set()
    for e in range(E):
        pairs = np.flatnonzero(flat == e)
        for s in range(0, pairs.size, chunk):
            piece = pairs[s:s + chunk]
            rows.add(int(piece[0]) // k)
            rows.add(int(piece[-1]) // k)
    rng = np.random.default_rng(seed)
    order = rng.permutation(T)
    i = 0
    while len(rows) < min(n_min, T):
        rows.add(int(order[i]))
        i += 1
    return np.array(sorted(rows), dtype=np.int64)
