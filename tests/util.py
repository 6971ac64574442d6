"""Shared test helpers: host<->device transfer and the parity criteria."""
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    """Function names declared in include/*.h."""
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def dev(a, torch_dtype=None):
    """numpy -> cuda tensor; uint16 arrays are bf16 bit patterns."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    t = torch.from_numpy(a).cuda()
    return t if torch_dtype is None else t.to(torch_dtype)


def host(t):
    """cuda tensor -> numpy; bf16 comes back as float32 values."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (at least the smallest normal spacing)."""
    a = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def check_bf16_attention(got, ref, what=""):
    """bf16 attention bar: max-abs <= 2e-2 and relative L2 <= 1e-2."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err.max() <= 2e-2, f"{what}: max-abs {err.max():.3e}"
    assert rel <= 1e-2, f"{what}: rel-L2 {rel:.3e}"
    return err.max(), rel


def check_f32(got, ref, tol=1e-5, what=""):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    assert err.max() <= tol, f"{what}: max-abs {err.max():.3e}"
    return err.max()


def report_margin(what, max_abs, rel_l2):
    """Prints the measured error of a parity comparison beside its bar."""
    line = f"[margin] {what}: max-abs {max_abs:.3e}"
    if rel_l2 is not None:
        line += f" (bar 2e-2), rel-L2 {rel_l2:.3e} (bar 1e-2)"
    print(line, flush=True)
