import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def to_np(t):
    """torch tensor (any dtype, any device) -> float64 numpy on the host."""
    import torch
    if isinstance(t, torch.Tensor):
        if t.dtype in (torch.bfloat16, torch.float16):
            t = t.float()
        return t.detach().cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def read_golden_pictures(path):
    panels = {}
    cur = None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("["):
            parts = line.strip("[]").split()
            cur = parts[0]
            panels[cur] = {"attrs": dict(p.split("=") for p in parts[1:]), "rows": []}
        else:
            panels[cur]["rows"].append([int(x) for x in line.split()])
    return panels
