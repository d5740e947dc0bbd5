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
