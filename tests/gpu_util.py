"""Helpers shared by the GPU parity tests (test infrastructure only)."""
from __future__ import annotations

import numpy as np
import torch

# attention tolerance against the fp64 oracle on the same bf16-cast inputs
ATTN_MAX_ABS = 2e-2
ATTN_REL_L2 = 5e-3


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def np64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy().astype(np.float64) if t.is_floating_point() else t.numpy()


class AttnErr:
    """Accumulates max-abs and relative-L2 error over many rows."""

    def __init__(self):
        self.max_abs = 0.0
        self.num = 0.0
        self.den = 0.0
        self.worst_row = None

    def add(self, got: np.ndarray, want: np.ndarray, tag=None):
        d = np.abs(got - want)
        m = float(d.max()) if d.size else 0.0
        if m > self.max_abs:
            self.max_abs, self.worst_row = m, tag
        self.num += float((d ** 2).sum())
        self.den += float((want ** 2).sum())

    @property
    def rel_l2(self):
        return (self.num ** 0.5) / max(self.den ** 0.5, 1e-300)

    def check(self):
        assert self.max_abs <= ATTN_MAX_ABS, f"max-abs {self.max_abs:.3e} (row {self.worst_row})"
        assert self.rel_l2 <= ATTN_REL_L2, f"rel-L2 {self.rel_l2:.3e}"


def topk_certificate(S: torch.Tensor, J: torch.Tensor, p: torch.Tensor, k: int, keys=None, valid=None):
    """O(n) check that J is the exact top-k of each row of S (ties: lowest key).

    S int32 [R, n] candidate scores; J int32 [R, k]; p int32 [R].  Flat rows:
    candidate c is key c, valid for c <= p.  With ``keys`` (int64 [R, n]) and
    ``valid`` (bool [R, n]) candidates are arbitrary keys (two-stage slots).
    Checks: count = min(k, #candidates), J ascending, unique, every entry a
    candidate, -1 padding after, and min over J of (S, -key) > max over the
    other candidates.  Raises AssertionError naming the first bad row.
    """
    R, n = S.shape
    dv = S.device
    if keys is None:
        keys = torch.arange(n, device=dv, dtype=torch.int64).unsqueeze(0).expand(R, n)
        valid = keys <= p.to(torch.int64).unsqueeze(1)
    n_cand = valid.sum(1)
    want_cnt = torch.clamp(n_cand, max=k)
    Jl = J.to(torch.int64)
    sel_pos = Jl >= 0
    cnt = sel_pos.sum(1)
    bad = cnt != want_cnt
    assert not bool(bad.any()), f"count mismatch in row {int(bad.nonzero()[0])}"
    # padding only at the end and strictly ascending before it
    ar = torch.arange(k, device=dv).unsqueeze(0)
    assert bool((sel_pos == (ar < cnt.unsqueeze(1))).all()), "-1 padding not at the end"
    if k > 1:
        inc = (Jl[:, 1:] > Jl[:, :-1]) | ~sel_pos[:, 1:]
        assert bool(inc.all()), "J not strictly ascending"
    # membership: position of each J entry among the candidate keys (keys ascending per row)
    big = torch.iinfo(torch.int64).max
    kk = torch.where(valid, keys, torch.full_like(keys, big))
    kk_sorted, order = torch.sort(kk, dim=1)
    pos = torch.searchsorted(kk_sorted, torch.where(sel_pos, Jl, torch.zeros_like(Jl)))
    pos = torch.clamp(pos, max=n - 1)
    found = torch.gather(kk_sorted, 1, pos) == Jl
    assert bool((found | ~sel_pos).all()), "J lists a key that is not a candidate"
    slot = torch.gather(order, 1, pos)
    packed = S.to(torch.int64) * (1 << 32) + ((1 << 31) - 1 - keys)   # larger = better
    # scatter_add: padded entries point at slot 0 but add nothing
    hits = torch.zeros((R, n), dtype=torch.int32, device=dv)
    hits.scatter_add_(1, torch.where(sel_pos, slot, torch.zeros_like(slot)), sel_pos.to(torch.int32))
    selected = hits > 0
    lo = torch.where(selected, packed, torch.full_like(packed, big)).min(1).values
    other = valid & ~selected
    hi = torch.where(other, packed, torch.full_like(packed, -big - 1)).max(1).values
    ok = (lo > hi) | (cnt == 0) | (other.sum(1) == 0)
    assert bool(ok.all()), f"top-k certificate fails in row {int((~ok).nonzero()[0])}"
