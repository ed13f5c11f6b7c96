"""Shared helpers of the GPU tests: the device harness of the package (upload a
generated workload, run the library) and the comparison against the oracle's output.

Nothing here computes attention; expected values always come from `oracle/`.
"""
from __future__ import annotations

import numpy as np
import torch

from paged_kv_scaled_amd import binding as B
from paged_kv_scaled_amd import workloads as wl

# Bars for bf16/fp16 outputs against the fp64 oracle (max-abs, relative L2).
MAX_ABS, REL_L2 = 2e-2, 1e-2
# fp32 inputs run on the fp32 vector path: far tighter.
MAX_ABS_F32, REL_L2_F32 = 1e-5, 1e-6

from paged_kv_scaled_amd.harness import (TORCH_DT, INT_DT, Dev, as_f64, bits_of,  # noqa: E402,F401
                                         to_dev)


def compare(got: np.ndarray, want: np.ndarray, dtype: str, what: str = ""):
    """max-abs and relative-L2 against the oracle, with the bar for the dtype."""
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    diff = got - want
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    nrm = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(diff) / nrm) if nrm > 0 else float(np.linalg.norm(diff))
    ma, rl = (MAX_ABS_F32, REL_L2_F32) if dtype == "f32" else (MAX_ABS, REL_L2)
    assert max_abs <= ma and rel <= rl, f"{what}: max_abs {max_abs:.3e} (bar {ma}), rel_l2 {rel:.3e} (bar {rl})"
    return max_abs, rel
