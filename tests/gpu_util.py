"""Helpers shared by the GPU parity tests (no attention arithmetic here)."""
import sys

import torch

# The parity bar on bf16 N(0,1) inputs against the fp64 oracle.
MAX_ABS = 1.5e-2
MEAN_ABS = 2e-3


def say(*a):
    """Name the case on stdout before a GPU step (a crash then names it)."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def compare(out, ref, what="", max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    """Element-wise comparison of a bf16 device result with an fp64 reference."""
    o = out.detach().to("cpu", torch.float64)
    assert o.shape == ref.shape, (o.shape, ref.shape)
    assert torch.isfinite(o).all(), "%s: non-finite output" % what
    err = (o - ref).abs()
    mx = err.max().item() if err.numel() else 0.0
    mean = err.mean().item() if err.numel() else 0.0
    say("  %s: max_abs %.3e mean_abs %.3e over %d values" % (what, mx, mean, err.numel()))
    assert mx <= max_abs, "%s: max-abs %.4e > %.1e" % (what, mx, max_abs)
    assert mean <= mean_abs, "%s: mean-abs %.4e > %.1e" % (what, mean, mean_abs)
    return mx, mean


def sample_rows(Lq, head=32, tail=32, every=127):
    """A stratified row subset: the first and last rows and a regular stride."""
    rows = set(range(min(head, Lq))) | set(range(max(0, Lq - tail), Lq))
    rows |= set(range(0, Lq, every))
    return sorted(rows)
