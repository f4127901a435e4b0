"""One rank's expert step as three C-ABI calls on one stream, with the buffers they need.

torch only allocates device memory here; every stage runs in libmoestep's kernels:
  moe_assemble -> moe_expert_ffn_grouped -> moe_combine_release
The local results are combined straight from the FFN output: arrival i of the combine is
queue entry i, whose result row is pos[i] (the batch row moe_assemble gave it).

With gather_on_load (the default) moe_assemble only builds the index (perm, pos, counts,
offsets) and the FFN reads each batch row straight from the token pool through
slot[perm[r]]; the contiguous batch is never written out.

With fuse_plan (the default) run() hands the first half of the combine (moe_combine_plan)
to moe_expert_ffn_grouped, which runs it in a spare workgroup of the gate/up launch when the
batch takes the weight-streaming kernels (every decode step) and launches it before the FFN
otherwise; moe_combine_apply follows the FFN.

With overlap, run() puts the first half of the combine (moe_combine_plan: it reads only
the arrival metadata and the token state) on a side stream, where it runs while the FFN
streams the expert weights; moe_combine_apply then waits for it on the main stream.  The
side stream has the default priority.  Off by default: on the decode step the two
cross-stream event waits cost more than the ~8 us plan kernel they hide (97.5 us per step
in order, 101 us overlapped).
"""
from __future__ import annotations

import torch

from . import _native as N

_TORCH = {N.MOE_F32: torch.float32, N.MOE_BF16: torch.bfloat16, N.MOE_FP8_E4M3: torch.uint8}


class ExpertStep:
    def __init__(self, E_loc: int, H: int, I: int, K: int, act_dtype: int, w_dtype: int, n_max: int, T_cap: int,
                 device="cuda", gather_on_load: bool = True, overlap: bool = False, fuse_plan: bool = True,
                 fuse_index: bool = True):
        self.E_loc, self.H, self.I, self.K = E_loc, H, I, K
        self.act_dtype, self.w_dtype, self.n_max, self.T_cap = act_dtype, w_dtype, n_max, T_cap
        dev = torch.device(device)
        adt = _TORCH[act_dtype]
        nm = max(n_max, 1)
        self.perm = torch.empty(nm, dtype=torch.int32, device=dev)
        self.pos = torch.empty(nm, dtype=torch.int32, device=dev)
        self.row_slot = torch.empty(nm, dtype=torch.int32, device=dev)  # pool slot of each batch row
        self.counts = torch.empty(E_loc, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(E_loc + 1, dtype=torch.int32, device=dev)
        self.xb = torch.empty((nm, H), dtype=adt, device=dev)
        self.y = torch.empty((nm, H), dtype=adt, device=dev)
        ws = N.moe_ffn_workspace_size(nm, E_loc, H, I, act_dtype)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.rel_list = torch.empty(max(T_cap, 1), dtype=torch.int32, device=dev)
        self.rel_count = torch.zeros(1, dtype=torch.int32, device=dev)
        self.state = N.CombineState(T_cap, H, device=dev)
        self.cmb_ws_m = max(n_max, 1)
        self.cmb_ws = torch.empty(N.moe_combine_workspace_size(self.cmb_ws_m), dtype=torch.uint8, device=dev)
        self.out = torch.empty((T_cap, H), dtype=adt, device=dev)
        self.w_gu = self.w_d = None
        self.gather_on_load = gather_on_load
        self._gather = None  # (perm, slot, pool, row_slot) of the last assemble when gathering on load
        self.fuse_plan = fuse_plan
        self.fuse_index = fuse_index and gather_on_load  # the queue index derived in the FFN call
        self.side = torch.cuda.Stream(device=dev) if overlap else None
        self._ev_asm = torch.cuda.Event() if overlap else None
        self._ev_plan = torch.cuda.Event() if overlap else None
        self.s_gate = self.s_up = self.s_down = None
        N.moe_state_reset(self.state, 0)

    def load_weights(self, wg, wu, wd, s_gate=None, s_up=None, s_down=None, stream=None) -> None:
        """wg, wu: [E][I][H], wd: [E][H][I] device tensors in the weight dtype (row-major);
        fp8 weights come as uint8 codes with fp32 row scales."""
        self.w_gu = torch.empty(self.E_loc * 2 * self.I * self.H, dtype=wg.dtype, device=wg.device)
        self.w_d = torch.empty(self.E_loc * self.H * self.I, dtype=wg.dtype, device=wg.device)
        N.moe_pack_ffn_weights(wg, wu, wd, self.w_gu, self.w_d, self.w_dtype, stream=stream)
        self.s_gate, self.s_up, self.s_down = s_gate, s_up, s_down

    def assemble(self, slot, expert, expert_base: int, pool, n: int | None = None, stream=None) -> None:
        xb = None if self.gather_on_load else self.xb
        rs = self.row_slot if self.gather_on_load else None
        N.moe_assemble(slot, expert, expert_base, self.E_loc, pool, self.perm, self.pos, self.counts, self.offsets,
                       xb, self.err, n=n, stream=stream, row_slot=rs)
        self._gather = (self.perm, slot, pool, rs) if self.gather_on_load else None

    def ffn(self, n: int, ev_mid: int | None = None, stream=None, plan=None, ev_gu=None, index=None) -> None:
        N.moe_expert_ffn_grouped(n, self.E_loc, self.H, self.I, self.act_dtype, self.w_dtype, self.xb, self.offsets,
                                 self.w_gu, self.w_d, self.y, self.workspace, self.s_gate, self.s_up, self.s_down,
                                 ev_mid=ev_mid, stream=stream, gather=self._gather, plan=plan, ev_gu=ev_gu,
                                 index=index)

    def index_args(self, slot, expert, expert_base: int, pool, n: int):
        """The moe_assemble arguments (index only) of this step's queue, for ffn(index=...): the
        FFN call then derives the queue index itself (inside its gate/up launch for decode-sized
        queues) and gathers the rows through it."""
        self._gather = (self.perm, slot, pool, self.row_slot)
        return N.assemble_args(slot, expert, expert_base, self.E_loc, pool, self.perm, self.pos, self.counts,
                               self.offsets, None, self.err, n=n, row_slot=self.row_slot, H=self.H)

    def _combine_room(self, m: int) -> None:
        if m > self.cmb_ws_m:  # plumbing: grow the caller-owned scratch (outside any timed loop)
            self.cmb_ws_m = m
            self.cmb_ws = torch.empty(N.moe_combine_workspace_size(m), dtype=torch.uint8, device=self.cmb_ws.device)
        if m > self.rel_list.numel():
            self.rel_list = torch.empty(m, dtype=torch.int32, device=self.rel_list.device)

    def local_combine_args(self, tok, kslot, w, gen, n: int):
        """Arguments of the combine of this step's local results (rows y[pos[i]])."""
        self._combine_room(n)
        return N.combine_args(self.y, self.pos, tok, kslot, w, gen, self.K, self.state, self.out, self.rel_list,
                              self.rel_count, self.err, self.cmb_ws, m=n, n_rows=n)

    def combine(self, rows, row_idx, tok, kslot, w, gen, m: int | None = None, n_rows: int | None = None,
                stream=None, part: str = "release") -> None:
        m = int(tok.numel() if m is None else m)
        self._combine_room(m)
        N.moe_combine_release(rows, row_idx, tok, kslot, w, gen, self.K, self.state, self.out, self.rel_list,
                              self.rel_count, self.err, self.cmb_ws, m=m, n_rows=n_rows, stream=stream, part=part)

    def run(self, slot, expert, expert_base: int, pool, tok, kslot, w, gen, n: int | None = None,
            ev_mid: int | None = None, stream=None) -> None:
        """The whole step on one batch: assemble, FFN, combine of the local results."""
        n = int(slot.numel() if n is None else n)
        if self.side is None and self.fuse_plan:
            # the queue index and the combine plan ride in the FFN call (inside the gate/up
            # launch where they fit); the plan's argument struct then drives the apply
            index = self.index_args(slot, expert, expert_base, pool, n) if self.fuse_index else None
            if index is None:
                self.assemble(slot, expert, expert_base, pool, n=n, stream=stream)
            plan = self.local_combine_args(tok, kslot, w, gen, n)
            self.ffn(n, ev_mid=ev_mid, stream=stream, plan=plan, index=index)
            N.combine_call(plan, "apply", stream)
            return
        self.assemble(slot, expert, expert_base, pool, n=n, stream=stream)
        if self.side is None:
            self.ffn(n, ev_mid=ev_mid, stream=stream)
            self.combine(self.y, self.pos, tok, kslot, w, gen, m=n, n_rows=n, stream=stream)
            return
        main = torch.cuda.current_stream() if stream is None else stream
        self._ev_asm.record(main)
        self.side.wait_event(self._ev_asm)
        for t in (tok, kslot, w, gen):
            t.record_stream(self.side)  # the allocator keeps them until the side stream is done
        self.combine(self.y, self.pos, tok, kslot, w, gen, m=n, n_rows=n, stream=self.side, part="plan")
        self._ev_plan.record(self.side)
        self.ffn(n, ev_mid=ev_mid, stream=main)
        main.wait_event(self._ev_plan)
        self.combine(self.y, self.pos, tok, kslot, w, gen, m=n, n_rows=n, stream=main, part="apply")


class SharedExpert:
    """A shared expert at the home rank ([SEP] section 3: models with a shared expert run
    it locally on the home rank after attention, before the routed experts' results come
    back).  Every home token goes through the same dense SwiGLU; its result joins the
    token's combine as one more position, `kslot` (K of the routed top-K), with weight 1,
    so the released row is y = sum_j w_j E_j(x) + E_shared(x) and a token is released only
    once its routed results and its shared result have all arrived.

    The three calls are the step's own: moe_assemble (one local expert), the grouped FFN
    (a single group) and moe_combine_release into the routed step's combine state."""

    def __init__(self, H: int, I: int, act_dtype: int, w_dtype: int, n_max: int, device="cuda"):
        self.step = ExpertStep(1, H, I, 1, act_dtype, w_dtype, n_max, 1, device=device)
        self.n_max = n_max
        dev = torch.device(device)
        self._zero = torch.zeros(max(n_max, 1), dtype=torch.int32, device=dev)
        self._one = torch.ones(max(n_max, 1), dtype=torch.float32, device=dev)
        self._kslots: dict[int, torch.Tensor] = {}  # kslot -> constant [n_max] tensor, never written again
        self._dev = dev
        torch.cuda.synchronize(dev)  # the constants above are complete before any stream reads them

    def load_weights(self, wg, wu, wd, s_gate=None, s_up=None, s_down=None, stream=None) -> None:
        """wg, wu: [1][I][H], wd: [1][H][I] (one expert)."""
        self.step.load_weights(wg, wu, wd, s_gate, s_up, s_down, stream=stream)

    def run(self, owner: ExpertStep, slot, pool, tok, gen, kslot: int, n: int | None = None, stream=None) -> None:
        """Shared-expert results of the n home tokens at pool rows `slot` (state indices
        `tok`, generations `gen`) into `owner`'s combine state at position `kslot`."""
        n = int(slot.numel() if n is None else n)
        s = self.step
        s.assemble(slot, self._zero[:n], 0, pool, n=n, stream=stream)
        s.ffn(n, stream=stream)
        ks = self._kslots.get(kslot)
        if ks is None:
            # one-time setup per position: filled and synchronised before any combine reads it,
            # and never written again, so calls on any stream may share it
            ks = torch.full((max(self.n_max, 1),), kslot, dtype=torch.int32, device=self._dev)
            torch.cuda.synchronize(self._dev)
            self._kslots[kslot] = ks
        owner.combine(s.y, s.pos, tok, ks[:n], self._one[:n], gen, m=n, n_rows=n, stream=stream)
