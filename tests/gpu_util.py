"""Helpers of the GPU parity tests: move a workload to the device, run the
library through its binding, read results back, compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads as W

TOL = {"f32": 1e-4, "bf16": 2e-2}          # max|err| <= tol * (1 + |ref|)
DELTA_L2 = {"f32": 1e-5, "bf16": 1e-2}      # ||d_gpu - d_ref|| / ||d_ref|| with add = 0


def to_dev(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def from_dev(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy in the workload's storage (float32, or bf16 bits as uint16)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    return W.to_f32(a).astype(np.float64)


class DevCase:
    """A workload's arrays on the device."""

    def __init__(self, c: W.Case, device="cuda"):
        self.c = c
        self.token_slot = torch.from_numpy(c.token_slot).to(device)
        self.x = to_dev(c.x, c.dtype, device)
        self.A = [to_dev(a, c.dtype, device) for a in c.A]
        self.B = [to_dev(b, c.dtype, device) for b in c.B]
        self.y0 = to_dev(c.y0, c.dtype, device)
        self.slot_scale = (None if c.slot_scale is None
                           else torch.from_numpy(np.asarray(c.slot_scale, np.float32)).to(device))

    def apply(self, L, mode="auto", add=True, y=None, meta=None, workspace=None, stream=None):
        """lora_apply on this case; the apply workspace used (a fresh,
        zero-filled one unless given) is kept in self.ws."""
        meta = meta or L.lora_prepare_meta(self.token_slot, self.c.num_slots, stream=stream)
        y = self.y0.clone() if y is None else y
        if workspace is None:
            workspace = L.apply_workspace(L.lora_apply_workspace_bytes(
                meta.num_tokens, meta.num_slots, self.c.d_in, len(self.A), self.c.r_max, self.x.dtype, mode))
        self.ws = workspace
        L.lora_apply(meta, self.x, self.A, self.B, self.c.offsets, y, scale=self.c.scale,
                     slot_scale=self.slot_scale, add=add, mode=mode, workspace=workspace, stream=stream)
        return y, meta


def oracle_rows(c: W.Case, rows, add=True, return_u=False):
    return oracle.lora_rows(c.x, c.token_slot, c.num_slots, c.A, c.B, c.offsets, c.scale, c.y0,
                            add=add, rows=np.asarray(rows, np.int64), slot_scale=c.slot_scale,
                            return_u=return_u)


def check_rows(c: W.Case, y_rows: np.ndarray, ref: np.ndarray, what=""):
    """The spec gate: max|err| <= tol * (1 + |ref|), element by element."""
    got = as_f64(y_rows)
    tol = TOL[c.dtype]
    err = np.abs(got - ref)
    bound = tol * (1.0 + np.abs(ref))
    bad = err > bound
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; first at "
                             f"({i},{j}) got {got[i, j]!r} ref {ref[i, j]!r} (tol {tol})")
    return float(np.max(err / (1.0 + np.abs(ref)))) if err.size else 0.0


def sample_rows(c: W.Case, k_random=96, seed=0):
    """Rows to check on a full-size workload: first and last token of every
    segment (including the no-adapter one), the first and last rows of the
    batch, and random others."""
    order = np.argsort(c.token_slot, kind="stable")
    keys = c.token_slot[order]
    rows = {0, c.T - 1}
    for k in np.unique(keys):
        idx = order[keys == k]
        rows.update([int(idx[0]), int(idx[-1])])
    rng = np.random.Generator(np.random.PCG64(seed))
    rows.update(rng.integers(0, c.T, min(k_random, c.T)).tolist())
    return np.array(sorted(rows), np.int64)
