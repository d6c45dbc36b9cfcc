"""Helpers for the GPU parity tests (all run through the C ABI)."""
import numpy as np
import torch


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)) if isinstance(a, np.ndarray) else a
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a bf16 / fp32 tensor as unsigned ints (for bitwise compares)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.numpy()


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def same_values(a, b):
    """Bitwise equality except that +0 and -0 compare equal."""
    a = np.asarray(a)
    b = np.asarray(b)
    return a.shape == b.shape and bool(np.all((a == b) | (np.isnan(a) & np.isnan(b))))


def report(name, got, want):
    from tests.helpers import cosine, rel_l2
    r, c = rel_l2(got, want), cosine(got, want)
    print(f"{name}: rel_l2={r:.3e} cos={c:.7f}", flush=True)
    return r, c


def elementwise(name, got, want, atol_frac, rtol, frac=0.999, hard=10.0):
    """Element-wise bound |got - want| <= atol + rtol |want| with atol =
    atol_frac * rms(want): it must hold on at least `frac` of the elements and
    within `hard` times the bound on every element, so a wrong tile anywhere
    (a ragged edge included) fails even when the global norms pass."""
    g = np.asarray(got, np.float64).reshape(-1)
    w = np.asarray(want, np.float64).reshape(-1)
    scale = float(np.sqrt(np.mean(w * w))) if w.size else 0.0
    bound = atol_frac * scale + rtol * np.abs(w)
    err = np.abs(g - w)
    ok = float(np.mean(err <= bound)) if w.size else 1.0
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if w.size else 0.0
    print(f"{name}: {ok * 100:.4f}% within {atol_frac:g} rms + {rtol:g} |ref|, worst {worst:.3g} x bound",
          flush=True)
    assert ok >= frac and worst <= hard, (name, ok, worst)
