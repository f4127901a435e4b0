"""Moves generated workload arrays into torch tensors (plumbing only, no arithmetic)."""
from __future__ import annotations

import numpy as np
import torch


def tensor(a: np.ndarray, dtype: str | None = None, device="cuda") -> torch.Tensor:
    """numpy storage array -> torch tensor; dtype "bf16" reinterprets uint16 bits as
    bfloat16, "fp8" keeps uint8 codes, None keeps the numpy dtype (uint32 -> int32 bits)."""
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    elif a.dtype == np.uint32:
        t = torch.from_numpy(a.view(np.int32))
    elif a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """torch tensor -> numpy storage array (bf16 back to uint16 bit patterns)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def batch_tensors(b, device="cuda") -> dict:
    """Device tensors for one workloads.Batch (pool, pair metadata, remote arrivals)."""
    d = dict(pool=tensor(b.pool, b.act, device), slot=tensor(b.slot, device=device),
             expert=tensor(b.expert, device=device), tok=tensor(b.tok, device=device),
             kslot=tensor(b.kslot, device=device), w=tensor(b.w, device=device), gen=tensor(b.gen, device=device))
    if b.remote is not None and b.remote.m > 0:
        r = b.remote
        d.update(r_rows=tensor(r.rows, r.dtype, device), r_idx=tensor(r.row_idx, device=device),
                 r_tok=tensor(r.tok, device=device), r_kslot=tensor(r.kslot, device=device),
                 r_w=tensor(r.w, device=device), r_gen=tensor(r.gen, device=device))
    return d


def weight_tensors(wts, device="cuda") -> dict:
    dt = "bf16" if wts.dtype == "bf16" else None
    d = dict(wg=tensor(wts.wg, dt, device), wu=tensor(wts.wu, dt, device), wd=tensor(wts.wd, dt, device))
    if wts.dtype == "fp8":
        d.update(s_gate=tensor(wts.sg, device=device), s_up=tensor(wts.su, device=device),
                 s_down=tensor(wts.sd, device=device))
    return d


def device_layer_weights(seed: int, layer: int, E: int, H: int, I: int, sigma: float, device="cuda") -> dict:
    """One layer's bf16 expert weights drawn on the device with torch's seeded generator
    (wg, wu: [E][I][H], wd: [E][H][I]); the same (seed, layer) gives the same tensors."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000 + int(layer))
    out = {}
    for name, shape in (("wg", (E, I, H)), ("wu", (E, I, H)), ("wd", (E, H, I))):
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        out[name] = (t * sigma).to(torch.bfloat16)
    return out
