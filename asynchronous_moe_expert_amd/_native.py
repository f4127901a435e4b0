"""ctypes binding of libmoestep.so.  Argument marshalling only: every step of the path runs
in the library's HIP kernels.  Tensors are torch device tensors (plumbing for device
memory and streams); each function takes the same name as the C call it wraps."""
from __future__ import annotations

import ctypes as C
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoestep.so")

MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2

ERR_SLOT_RANGE = 1 << 0
ERR_EXPERT_NONLOCAL = 1 << 1
ERR_TOKEN_RANGE = 1 << 2
ERR_KSLOT_RANGE = 1 << 3
ERR_ROW_RANGE = 1 << 4
ERR_STALE_GEN = 1 << 5
ERR_DUPLICATE = 1 << 6

_p = C.c_void_p
_i32 = C.c_int32
_i64 = C.c_int64


class AssembleArgs(C.Structure):
    _fields_ = [("n", _i32), ("slot", _p), ("expert", _p), ("expert_base", _i32), ("E_loc", _i32),
                ("pool", _p), ("P", _i64), ("pool_pitch", _i64), ("H", _i32), ("act_dtype", _i32),
                ("perm", _p), ("pos", _p), ("counts", _p), ("offsets", _p), ("xb", _p), ("err", _p),
                ("row_slot", _p)]


class PackArgs(C.Structure):
    _fields_ = [("E_loc", _i32), ("H", _i32), ("I", _i32), ("w_dtype", _i32), ("wg", _p), ("wu", _p), ("wd", _p),
                ("w_gu", _p), ("w_d", _p)]


class FfnArgs(C.Structure):
    _fields_ = [("n", _i32), ("E_loc", _i32), ("H", _i32), ("I", _i32), ("act_dtype", _i32), ("w_dtype", _i32),
                ("xb", _p), ("offsets", _p), ("w_gu", _p), ("w_d", _p), ("s_gate", _p), ("s_up", _p),
                ("s_down", _p), ("y", _p), ("workspace", _p), ("workspace_bytes", C.c_size_t), ("ev_mid", _p),
                ("perm", _p), ("slot", _p), ("pool", _p), ("P", _i64), ("pool_pitch", _i64), ("row_slot", _p),
                ("plan", _p), ("ev_gu_start", _p), ("ev_gu_stop", _p), ("index", _p)]


class StateC(C.Structure):
    _fields_ = [("acc", _p), ("mask", _p), ("head", _p), ("tgen", _p), ("rflag", _p), ("T_cap", _i32), ("H", _i32)]


class CombineArgs(C.Structure):
    _fields_ = [("m", _i32), ("K", _i32), ("rows", _p), ("row_dtype", _i32), ("row_pitch", _i64),
                ("n_rows", _i64), ("row_idx", _p), ("tok", _p), ("kslot", _p), ("w", _p), ("gen", _p),
                ("state", StateC), ("out", _p), ("out_dtype", _i32), ("out_pitch", _i64), ("rel_list", _p),
                ("rel_count", _p), ("err", _p), ("workspace", _p), ("workspace_bytes", C.c_size_t)]


_STRUCTS = [AssembleArgs, PackArgs, FfnArgs, StateC, CombineArgs]
EXPORTS = ["moe_assemble", "moe_pack_ffn_weights", "moe_ffn_workspace_size", "moe_expert_ffn_grouped",
           "moe_state_reset", "moe_combine_release", "moe_combine_plan", "moe_combine_apply",
           "moe_combine_workspace_size", "moe_strerror", "moe_version", "moe_struct_size",
           "moe_combine_release_noalloc", "moe_combine_noalloc_max_arrivals"]


class MoeError(RuntimeError):
    pass


_lib = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Loads the HIP library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise MoeError(f"libmoestep.so not found at {path}; build it with "
                       "`python -m asynchronous_moe_expert_amd.build` (no CPU fallback exists)")
    lib = C.CDLL(path)
    for name, args in [("moe_assemble", [C.POINTER(AssembleArgs), _p]),
                       ("moe_pack_ffn_weights", [C.POINTER(PackArgs), _p]),
                       ("moe_expert_ffn_grouped", [C.POINTER(FfnArgs), _p]),
                       ("moe_state_reset", [C.POINTER(StateC), C.c_uint32, _p]),
                       ("moe_combine_release", [C.POINTER(CombineArgs), _p]),
                       ("moe_combine_plan", [C.POINTER(CombineArgs), _p]),
                       ("moe_combine_apply", [C.POINTER(CombineArgs), _p]),
                       ("moe_combine_release_noalloc", [C.POINTER(CombineArgs), _p]),
                       ("moe_version", []), ("moe_strerror", [C.c_int])]:
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = C.c_int
    lib.moe_strerror.restype = C.c_char_p
    lib.moe_ffn_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32]
    lib.moe_ffn_workspace_size.restype = C.c_size_t
    lib.moe_combine_workspace_size.argtypes = [_i32]
    lib.moe_combine_workspace_size.restype = C.c_size_t
    lib.moe_combine_noalloc_max_arrivals.argtypes = []
    lib.moe_combine_noalloc_max_arrivals.restype = C.c_size_t
    lib.moe_struct_size.argtypes = [C.c_int]
    lib.moe_struct_size.restype = C.c_size_t
    for k, s in enumerate(_STRUCTS):
        if lib.moe_struct_size(k) != C.sizeof(s):
            raise MoeError(f"struct layout mismatch for {s.__name__}: library {lib.moe_struct_size(k)} "
                           f"vs binding {C.sizeof(s)}")
    _lib = lib
    return lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise MoeError(f"{what}: {load().moe_strerror(rc).decode()} ({rc})")


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MOE_FP8_E4M3
    raise MoeError(f"unsupported dtype {t.dtype}")


def moe_version() -> int:
    return load().moe_version()


def moe_strerror(rc: int) -> str:
    return load().moe_strerror(rc).decode()


def moe_ffn_workspace_size(n_max: int, E_loc: int, H: int, I: int, act_dtype: int) -> int:
    return load().moe_ffn_workspace_size(n_max, E_loc, H, I, act_dtype)


def assemble_args(slot, expert, expert_base: int, E_loc: int, pool, perm, pos, counts, offsets, xb, err,
                  n: int | None = None, row_slot=None, H: int | None = None) -> AssembleArgs:
    """The moe_assemble argument struct (for moe_assemble, or as moe_ffn_args.index)."""
    if H is None:
        H = pool.shape[1] if xb is None else xb.shape[1]
    return AssembleArgs(int(slot.numel() if n is None else n), _ptr(slot), _ptr(expert), expert_base, E_loc,
                        _ptr(pool), pool.shape[0], pool.stride(0), H, dtype_code(pool), _ptr(perm),
                        _ptr(pos), _ptr(counts), _ptr(offsets), _ptr(xb), _ptr(err), _ptr(row_slot))


def moe_assemble(slot, expert, expert_base: int, E_loc: int, pool, perm, pos, counts, offsets, xb, err,
                 n: int | None = None, stream=None, row_slot=None) -> None:
    """pool: [P][pitch] (f32 or bf16); xb: [>= n][H] of the same dtype (or None);
    row_slot: optional [>= n] int32 output, the pool slot of each batch row."""
    a = assemble_args(slot, expert, expert_base, E_loc, pool, perm, pos, counts, offsets, xb, err, n=n,
                      row_slot=row_slot)
    _check(load().moe_assemble(C.byref(a), _stream(stream)), "moe_assemble")


def moe_pack_ffn_weights(wg, wu, wd, w_gu, w_d, w_dtype: int, stream=None) -> None:
    E, I, H = wg.shape
    a = PackArgs(E, H, I, w_dtype, _ptr(wg), _ptr(wu), _ptr(wd), _ptr(w_gu), _ptr(w_d))
    _check(load().moe_pack_ffn_weights(C.byref(a), _stream(stream)), "moe_pack_ffn_weights")


def moe_expert_ffn_grouped(n: int, E_loc: int, H: int, I: int, act_dtype: int, w_dtype: int, xb, offsets, w_gu,
                           w_d, y, workspace, s_gate=None, s_up=None, s_down=None, ev_mid: int | None = None,
                           stream=None, gather=None, plan: "CombineArgs | None" = None,
                           ev_gu: tuple[int, int] | None = None, index: "AssembleArgs | None" = None) -> None:
    """gather=(perm, slot, pool) or (perm, slot, pool, row_slot): read batch rows from the pool
    (gather-on-load; with row_slot, pool row row_slot[r] and perm/slot unused); xb may be None.
    plan: the arguments (combine_args) of a moe_combine_plan call that this call enqueues as
    well, inside the gate/up launch where it fits.  ev_gu: (start, stop) hipEvent_t handles
    that the weight-streaming gate/up kernel records around itself.  index: the arguments
    (assemble_args, xb None) of a moe_assemble call that this call does as well, inside the
    gate/up launch where it fits; offsets and gather are then taken from it."""
    perm = slot = pool = row_slot = None
    P = pitch = 0
    if gather is not None:
        perm, slot, pool = gather[:3]
        row_slot = gather[3] if len(gather) > 3 else None
        P, pitch = pool.shape[0], pool.stride(0)
    a = FfnArgs(n, E_loc, H, I, act_dtype, w_dtype, _ptr(xb), _ptr(offsets), _ptr(w_gu), _ptr(w_d),
                _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(y), _ptr(workspace),
                workspace.numel() * workspace.element_size(), ev_mid, _ptr(perm), _ptr(slot), _ptr(pool), P, pitch,
                _ptr(row_slot), None if plan is None else C.addressof(plan), *(ev_gu or (None, None)),
                None if index is None else C.addressof(index))
    _check(load().moe_expert_ffn_grouped(C.byref(a), _stream(stream)), "moe_expert_ffn_grouped")


class CombineState:
    """Device tensors of the per-token combine state (allocated here with torch)."""

    def __init__(self, T_cap: int, H: int, device="cuda"):
        self.T_cap, self.H = T_cap, H
        self.acc = torch.empty((T_cap, H), dtype=torch.float32, device=device)
        self.mask = torch.empty(T_cap, dtype=torch.int32, device=device)
        self.head = torch.empty(T_cap, dtype=torch.int32, device=device)
        self.tgen = torch.empty(T_cap, dtype=torch.int32, device=device)
        self.rflag = torch.empty((T_cap + 15) // 16 * 16, dtype=torch.uint8, device=device)

    def c(self) -> StateC:
        return StateC(_ptr(self.acc), _ptr(self.mask), _ptr(self.head), _ptr(self.tgen), _ptr(self.rflag),
                      self.T_cap, self.H)


def moe_state_reset(state: CombineState, gen0: int = 0, stream=None) -> None:
    s = state.c()
    _check(load().moe_state_reset(C.byref(s), gen0, _stream(stream)), "moe_state_reset")


def moe_combine_workspace_size(m_max: int) -> int:
    return load().moe_combine_workspace_size(m_max)


def moe_combine_noalloc_max_arrivals() -> int:
    return load().moe_combine_noalloc_max_arrivals()


def _combine_args(rows, row_idx, tok, kslot, w, gen, K, state, out, rel_list, rel_count, err, workspace, m, n_rows):
    return CombineArgs(int(tok.numel() if m is None else m), K, _ptr(rows), dtype_code(rows), rows.stride(0),
                       rows.shape[0] if n_rows is None else n_rows, _ptr(row_idx), _ptr(tok), _ptr(kslot), _ptr(w),
                       _ptr(gen), state.c(), _ptr(out), dtype_code(out), out.stride(0), _ptr(rel_list),
                       _ptr(rel_count), _ptr(err), _ptr(workspace),
                       0 if workspace is None else workspace.numel() * workspace.element_size())


def combine_args(rows, row_idx, tok, kslot, w, gen, K: int, state: CombineState, out, rel_list, rel_count, err,
                 workspace, m: int | None = None, n_rows: int | None = None) -> CombineArgs:
    """The argument struct of a combine call (for moe_expert_ffn_grouped's plan)."""
    return _combine_args(rows, row_idx, tok, kslot, w, gen, K, state, out, rel_list, rel_count, err, workspace, m,
                         n_rows)


def moe_combine_release(rows, row_idx, tok, kslot, w, gen, K: int, state: CombineState, out, rel_list, rel_count,
                        err, workspace, m: int | None = None, n_rows: int | None = None, stream=None,
                        part: str = "release") -> None:
    """rows: [n_rows][pitch] f32/bf16 result rows; out: [T_cap][pitch] f32/bf16.
    part = "plan" / "apply" calls moe_combine_plan / moe_combine_apply instead; part =
    "noalloc" calls moe_combine_release_noalloc (the library's static scratch; workspace
    may be None)."""
    a = _combine_args(rows, row_idx, tok, kslot, w, gen, K, state, out, rel_list, rel_count, err, workspace, m,
                      n_rows)
    combine_call(a, part, stream)


def combine_call(a: CombineArgs, part: str = "release", stream=None) -> None:
    """moe_combine_release / _plan / _apply on an argument struct from combine_args."""
    fn = {"release": "moe_combine_release", "plan": "moe_combine_plan", "apply": "moe_combine_apply",
          "noalloc": "moe_combine_release_noalloc"}[part]
    _check(getattr(load(), fn)(C.byref(a), _stream(stream)), fn)
