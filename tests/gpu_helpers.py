"""Helpers for the GPU tests: move a seeded workload to the device, run the
HIP path through the binding, compare with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import rank_specialized_amd as rs

TORCH_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32}

# Tolerances on max |y_gpu - y_ref| relative to max |y_ref| over one call.
TOL = {"bf16": 2e-2, "fp32": 1e-5}


def device():
    assert torch.cuda.is_available(), "GPU tests need an MI355X visible to torch"
    rs.load_library()  # fail loudly if the HIP library is missing
    return torch.device("cuda", 0)


def note(msg: str) -> None:
    """Name the case on stdout before a GPU step."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: torch.dtype, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(dtype).contiguous()


def upload_factors(wl, dev):
    dt = TORCH_DTYPE[wl.dtype]
    A = [to_dev(a, dt, dev) for a in wl.module.A]
    B = [to_dev(b, dt, dev) for b in wl.module.B]
    return A, B


def pack(wl, dev, pad_to: int = 0):
    A, B = upload_factors(wl, dev)
    store = rs.lora_pack_retained(A, B, wl.module.scales, pad_to=pad_to)
    del A, B
    return store


def inputs(wl, dev):
    dt = TORCH_DTYPE[wl.dtype]
    x = to_dev(wl.x, dt, dev)
    ids = torch.from_numpy(wl.ids.astype(np.int32)).to(dev)
    if wl.y0 is None:
        y = torch.zeros(wl.T, wl.module.d_out, dtype=dt, device=dev)
    else:
        y = to_dev(wl.y0, dt, dev)
    return x, ids, y


def y_host(y: torch.Tensor) -> np.ndarray:
    return y.float().cpu().numpy().astype(np.float64)


def rel_err(y, ref) -> float:
    scale = np.abs(ref).max()
    return float(np.abs(y - ref).max() / scale) if scale > 0 else float(np.abs(y - ref).max())


def hbits(y: torch.Tensor) -> np.ndarray:
    """Raw bits of a bf16/f32 device tensor (for bitwise comparisons)."""
    if y.dtype == torch.bfloat16:
        return y.view(torch.int16).cpu().numpy()
    return y.view(torch.int32).cpu().numpy()


def chunks_of(d_in, r, e, T=0, n=0):
    """Partial sums of an h value (the shrink's chunks of d_in) - restated:
    8 waves x 8 K steps of 64 bytes per chunk (2048 bf16, 1024 float32
    values), times the smallest multiple that keeps them at most 8; an input
    of up to two such units goes in one chunk when the call can hold 1024
    sub-tiles or more; the same for every rank r."""
    unit = 8 * 8 * 4 * (16 // e)
    units = -(-d_in // unit)
    mult = max(1, -(-units // 8))
    max_sub = (T + 15 * min(n, T)) // 16 if T > 0 else 0
    if units <= 2 and max_sub >= 1024:
        mult = units
    return max(1, -(-d_in // (mult * unit)))


def ws_offsets(T, n, d_in, r_max, e):
    """(metadata offset, plan offset, S) in an apply's workspace - the layout
    restated: 16 bytes of metadata per possible sub-tile of <= 16 tokens, the
    float32 partial sums of S chunks at row stride r_max rounded up to 8,
    then the plan; each part 256-byte aligned."""
    up = lambda v: -(-v // 256) * 256
    max_sub = (T + 15 * min(n, T)) // 16 if T > 0 else 0
    S = chunks_of(d_in, r_max, e, T, n)
    ldp = -(-max(r_max, 1) // 8) * 8
    part = up(16 * max_sub)
    return 0, part + up(S * T * ldp * 4), S
