"""Shared helpers for the GPU parity tests (run the HIP path, compare with the oracle)."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from workloads.device import tensor, to_numpy_bits

TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}


def row_rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of ||gpu_r - ref_r||_inf / ||ref_r||_inf (rows with a zero reference
    must match to 1e-30 absolute)."""
    gpu = np.asarray(gpu, np.float64).reshape(len(ref), -1)
    ref = np.asarray(ref, np.float64).reshape(len(ref), -1)
    worst = 0.0
    for g, r in zip(gpu, ref):
        den = np.abs(r).max()
        num = np.abs(g - r).max()
        if den == 0:
            assert num <= 1e-30, "nonzero output where the reference row is zero"
            continue
        worst = max(worst, num / den)
    return worst


def decode_tensor(t: torch.Tensor) -> np.ndarray:
    a = to_numpy_bits(t)
    if a.dtype == np.uint16:
        return O.decode_bf16(a)
    return a.astype(np.float64)


def dev(a, dtype=None):
    return tensor(a, dtype, "cuda")


def sync_err(t: torch.Tensor) -> int:
    torch.cuda.synchronize()
    return int(t.item()) & 0xFFFFFFFF


class HipEvents:
    """Raw hipEvent_t handles through the HIP runtime (for the library's event arguments)."""

    def __init__(self):
        import ctypes as C
        self.C = C
        self.hip = C.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [C.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self) -> int:
        e = self.C.c_void_p()
        assert self.hip.hipEventCreate(self.C.byref(e)) == 0
        return e.value

    def record(self, ev: int, stream: int) -> None:
        assert self.hip.hipEventRecord(self.C.c_void_p(ev), self.C.c_void_p(stream)) == 0

    def ms(self, a: int, b: int) -> float:
        assert self.hip.hipEventSynchronize(self.C.c_void_p(b)) == 0
        out = self.C.c_float()
        assert self.hip.hipEventElapsedTime(self.C.byref(out), self.C.c_void_p(a), self.C.c_void_p(b)) == 0
        return float(out.value)

    def destroy(self, ev: int) -> None:
        self.hip.hipEventDestroy(self.C.c_void_p(ev))


def elem_rel_err(gpu: np.ndarray, ref: np.ndarray, frac: float = 0.1) -> float:
    """Reported beside row_rel_err: max over the elements whose reference is at least
    `frac` of its row's largest magnitude of |gpu - ref| / |ref| (elementwise relative error
    away from the near-zero entries, where it is ill-posed)."""
    gpu = np.asarray(gpu, np.float64).reshape(len(ref), -1)
    ref = np.asarray(ref, np.float64).reshape(len(ref), -1)
    big = np.abs(ref) >= frac * np.abs(ref).max(axis=1, keepdims=True)
    big &= ref != 0
    if not big.any():
        return 0.0
    return float((np.abs(gpu - ref)[big] / np.abs(ref)[big]).max())
