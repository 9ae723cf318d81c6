"""MI355X (gfx950) MoE expert layer: thin Python binding of libmoe_mi355x.so.

Every function here marshals torch tensors (device memory) into the C ABI
declared in ``include/moe_mi355x.h`` and calls it on the current HIP stream;
all arithmetic runs in the library's HIP kernels.  There is no fallback: if
the library is missing the import of a compute function raises.

Functions keep the C names without the ``moe_`` prefix.  Outputs not passed
in are allocated with torch (device memory is the only thing torch provides
here).
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "moe_mi355x.h")

MOE_OK = 0
DT_F32, DT_BF16 = 0, 1
_DT = {torch.float32: DT_F32, torch.bfloat16: DT_BF16}


class MoEError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


_lib = None


def lib():
    """The loaded library (ctypes); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m mixture_experts_expert_router_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                            ctypes.c_size_t)
        L.moe_status_string.argtypes = [i32]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_version.restype = i32
        L.moe_route_topk.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i32,
                                     vp, vp, vp]
        L.moe_permute_workspace_bytes.argtypes = [i64, i64, i64]
        L.moe_permute_workspace_bytes.restype = sz
        L.moe_permute.argtypes = [vp, vp, vp, i64, i64, i64, i32, i64, i64,
                                  i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_grouped_ffn_workspace_bytes.argtypes = [i64, i64, i64, i64, i32]
        L.moe_grouped_ffn_workspace_bytes.restype = sz
        L.moe_grouped_gate_up.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp,
                                          vp, i32, vp, vp, sz, vp]
        L.moe_grouped_down.argtypes = [vp, vp, i64, i64, i64, i64, vp, i32,
                                       vp, vp, sz, vp]
        L.moe_grouped_ffn.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp, vp,
                                      vp, i32, vp, vp, vp, sz, vp]
        L.moe_unpermute_combine.argtypes = [vp, vp, vp, i64, i64, i64, i32,
                                            vp, vp]
        L.moe_grouped_ffn_loop.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64,
                                           vp, vp, vp, i32, vp, vp, vp, sz, vp]
        L.moe_grouped_ffn_gather.argtypes = [vp, vp, i64, i64, vp, vp, i64,
                                             i64, i64, i64, vp, vp, vp, i32,
                                             vp, vp, vp, sz, vp]
        L.moe_grouped_ffn_fused.argtypes = [vp, vp, i64, i64, vp, vp, i64, i64,
                                            i64, i64, vp, vp, vp, i32, vp, vp,
                                            vp, sz, vp]
        L.moe_eplb_plan.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp, vp]
        L.moe_permute_replicated_workspace_bytes.argtypes = [i64, i64, i64, i64]
        L.moe_permute_replicated_workspace_bytes.restype = sz
        L.moe_permute_replicated.argtypes = [vp, vp, vp, i64, i64, i64, i32,
                                             i64, i64, vp, vp, vp, vp, i64, i64, vp,
                                             vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_grouped_ffn_slots.argtypes = [vp, vp, vp, i64, vp, i64, i64, i64,
                                            i64, vp, vp, vp, i32, vp, vp, vp,
                                            sz, vp]
        L.moe_debug_sync.argtypes = [vp]
        L.moe_read_device_error.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_int32)]
        L.moe_permute_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, i32, i64,
                                          i64, i64, vp, vp, vp, vp, vp, vp, vp]
        L.moe_mxfp8_quantize.argtypes = [vp, i64, i64, i64, i32, i32, vp, i64,
                                         i64, vp, i64, vp, i64, vp, vp]
        L.moe_grouped_mlp_mxfp8_fwd_workspace_bytes.argtypes = [i64, i64, i64, i64]
        L.moe_grouped_mlp_mxfp8_fwd_workspace_bytes.restype = sz
        L.moe_grouped_mlp_mxfp8_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64,
                                                i64, vp, vp, vp, vp, vp, vp,
                                                vp, vp, vp, vp, sz, vp]
        L.moe_grouped_mlp_mxfp8_fwd_down.argtypes = [vp, i64, i64, i64, i64, vp,
                                                     vp, vp, vp, sz, vp]
        L.moe_grouped_mlp_mxfp8_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64]
        L.moe_grouped_mlp_mxfp8_bwd_workspace_bytes.restype = sz
        L.moe_grouped_mlp_mxfp8_bwd.argtypes = [vp, vp, vp, vp, vp, i64,
                                                i64, i64, i64, vp, vp, vp, vp,
                                                vp, vp, vp, vp, vp, vp, vp, i32,
                                                vp, sz, vp]
        L.moe_grouped_gate_up_gather.argtypes = [vp, vp, i64, i64, vp, vp, i64,
                                                 i64, i64, i64, vp, vp, i32, vp,
                                                 vp, sz, vp]
        L.moe_grouped_linear_mxfp8_workspace_bytes.argtypes = [i64, i64, i64]
        L.moe_grouped_linear_mxfp8_workspace_bytes.restype = sz
        L.moe_grouped_linear_mxfp8.argtypes = [vp, vp, i64, i64, i64, i64, vp,
                                               vp, vp, vp, sz, vp]
        L.moe_grouped_mlp_mxfp8_bwd_down_workspace_bytes.argtypes = [i64, i64, i64, i64]
        L.moe_grouped_mlp_mxfp8_bwd_down_workspace_bytes.restype = sz
        L.moe_grouped_mlp_mxfp8_bwd_down.argtypes = [vp, vp, vp, vp, i64,
                                                     i64, i64, i64, vp, vp, vp,
                                                     vp, vp, i32, vp, sz, vp]
        L.moe_grouped_mlp_mxfp8_bwd_gate_up_workspace_bytes.argtypes = [i64, i64, i64, i64]
        L.moe_grouped_mlp_mxfp8_bwd_gate_up_workspace_bytes.restype = sz
        L.moe_grouped_mlp_mxfp8_bwd_gate_up.argtypes = [vp, vp, vp, i64, i64,
                                                        i64, i64, vp, vp, vp,
                                                        vp, vp, vp, vp, i32, vp,
                                                        sz, vp]
        L.moe_mxfp8_workspace_view.argtypes = [i32, i32, i64, i64, i64, i64,
                                                ctypes.POINTER(MxView)]
        for name in declared_functions():
            getattr(L, name).restype = getattr(L, name).restype or i32
        _lib = L
    return _lib


def declared_functions(header: str = HEADER):
    """Names of the functions include/moe_mi355x.h declares."""
    text = open(header, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def version() -> int:
    return lib().moe_version()


def _p(t):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != MOE_OK:
        raise MoEError(name, st)


def _dt(t):
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def route_topk(k, logits=None, x=None, w_router=None, bias=None,
               topk_idx=None, topk_w=None, stream=None, T=None, E=None):
    """Router GEMM (when x and w_router are given) + softmax/top-k.

    Returns (topk_idx [T,k] int32, topk_w [T,k] fp32, logits [T,E] fp32).
    """
    if x is not None:
        T, H = x.shape
        E = w_router.shape[0]
        dtype = _dt(x)
        if logits is None:
            logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    else:
        T, E = logits.shape
        H = 0
        dtype = DT_F32
    dev = logits.device
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _call("moe_route_topk", _p(x), _p(w_router), _p(bias), _p(logits), T, H,
          E, k, dtype, _p(topk_idx), _p(topk_w), _stream(stream))
    return topk_idx, topk_w, logits


class PermuteOut:
    """Outputs of permute (capacity-sized; rows < offsets[n_local] valid)."""

    def __init__(self, T, k, H, n_local, dtype, device, with_x=True):
        F = T * k
        self.x_perm = (torch.empty((F, H), dtype=dtype, device=device)
                       if with_x else None)
        self.s_perm = torch.empty(F, dtype=torch.float32, device=device)
        self.row_src = torch.empty(F, dtype=torch.int32, device=device)
        self.inv = torch.empty((T, k), dtype=torch.int32, device=device)
        self.counts = torch.empty(n_local, dtype=torch.int32, device=device)
        self.offsets = torch.empty(n_local + 1, dtype=torch.int32,
                                   device=device)
        ws = lib().moe_permute_workspace_bytes(T, k, n_local)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8,
                                     device=device)


def permute(topk_idx, x, e_begin, n_local, topk_w=None, out=None,
            stream=None, *, E):
    """Local dispatch of the slots routed to experts [e_begin, e_begin +
    n_local) of the layer's E experts.  Indices outside [0, E) are dropped
    and flagged in out.workspace's error word (see read_device_error)."""
    T, k = topk_idx.shape
    H = x.shape[1] if x is not None else 0
    dtype = x.dtype if x is not None else torch.bfloat16
    if out is None:
        out = PermuteOut(T, k, max(H, 1), n_local, dtype, topk_idx.device,
                         with_x=x is not None)
    _call("moe_permute", _p(topk_idx), _p(topk_w), _p(x), T, k, H,
          _DT[dtype], E, e_begin, n_local, _p(out.x_perm),
          _p(out.s_perm) if topk_w is not None else None, _p(out.row_src),
          _p(out.inv), _p(out.counts), _p(out.offsets), _p(out.workspace),
          out.workspace.numel(), _stream(stream))
    return out


def permute_noalloc(topk_idx, x, e_begin, n_local, out, topk_w=None,
                    stream=None, *, E):
    """permute into caller-provided outputs `out` (a PermuteOut; its
    workspace is not used): the library allocates nothing and takes its
    scratch from a static per-GPU array."""
    T, k = topk_idx.shape
    H = x.shape[1] if x is not None else 0
    dtype = x.dtype if x is not None else torch.bfloat16
    _call("moe_permute_noalloc", _p(topk_idx), _p(topk_w), _p(x), T, k, H,
          _DT[dtype], E, e_begin, n_local, _p(out.x_perm),
          _p(out.s_perm) if topk_w is not None else None, _p(out.row_src),
          _p(out.inv), _p(out.counts), _p(out.offsets), _stream(stream))
    return out


def ffn_workspace(R_cap, n_local, H, I, dtype, device):
    n = lib().moe_grouped_ffn_workspace_bytes(R_cap, n_local, H, I,
                                              _DT[dtype])
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def grouped_gate_up(x_perm, offsets, s_perm, w_gate, w_up, a=None,
                    workspace=None, stream=None):
    R_cap, H = x_perm.shape
    n_local, I, _ = w_gate.shape
    if a is None:
        a = torch.empty((R_cap, I), dtype=x_perm.dtype, device=x_perm.device)
    if workspace is None:
        workspace = ffn_workspace(R_cap, n_local, H, I, x_perm.dtype,
                                  x_perm.device)
    _call("moe_grouped_gate_up", _p(x_perm), _p(offsets), _p(s_perm),
          n_local, R_cap, H, I, _p(w_gate), _p(w_up), _dt(x_perm), _p(a),
          _p(workspace), workspace.numel(), _stream(stream))
    return a


def grouped_gate_up_gather(x, row_src, k, offsets, s_perm, w_gate, w_up,
                           a=None, workspace=None, stream=None):
    """grouped_gate_up with permuted row r read as x[row_src[r] // k]."""
    T, H = x.shape
    R_cap = row_src.shape[0]
    n_local, I, _ = w_gate.shape
    if a is None:
        a = torch.empty((R_cap, I), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = ffn_workspace(R_cap, n_local, H, I, x.dtype, x.device)
    _call("moe_grouped_gate_up_gather", _p(x), _p(row_src), T, k, _p(offsets),
          _p(s_perm), n_local, R_cap, H, I, _p(w_gate), _p(w_up), _dt(x),
          _p(a), _p(workspace), workspace.numel(), _stream(stream))
    return a


def grouped_down(a, offsets, w_down, y=None, workspace=None, stream=None):
    R_cap, I = a.shape
    n_local, H, _ = w_down.shape
    if y is None:
        y = torch.empty((R_cap, H), dtype=a.dtype, device=a.device)
    if workspace is None:
        workspace = ffn_workspace(R_cap, n_local, H, I, a.dtype, a.device)
    _call("moe_grouped_down", _p(a), _p(offsets), n_local, R_cap, H, I,
          _p(w_down), _dt(a), _p(y), _p(workspace), workspace.numel(),
          _stream(stream))
    return y


def grouped_ffn(x_perm, offsets, s_perm, w_gate, w_up, w_down, a=None,
                y=None, workspace=None, stream=None):
    R_cap, H = x_perm.shape
    n_local, I, _ = w_gate.shape
    if a is None:
        a = torch.empty((R_cap, I), dtype=x_perm.dtype, device=x_perm.device)
    if y is None:
        y = torch.empty((R_cap, H), dtype=x_perm.dtype, device=x_perm.device)
    if workspace is None:
        workspace = ffn_workspace(R_cap, n_local, H, I, x_perm.dtype,
                                  x_perm.device)
    _call("moe_grouped_ffn", _p(x_perm), _p(offsets), _p(s_perm), n_local,
          R_cap, H, I, _p(w_gate), _p(w_up), _p(w_down), _dt(x_perm), _p(a),
          _p(y), _p(workspace), workspace.numel(), _stream(stream))
    return a, y


def grouped_ffn_gather(x, row_src, k, offsets, s_perm, w_gate, w_up, w_down,
                       a=None, y=None, workspace=None, stream=None):
    """grouped_ffn with permuted row r of the gate/up input read as
    x[row_src[r] // k] (R_cap = row_src.shape[0])."""
    T, H = x.shape
    R_cap = row_src.shape[0]
    n_local, I, _ = w_gate.shape
    if a is None:
        a = torch.empty((R_cap, I), dtype=x.dtype, device=x.device)
    if y is None:
        y = torch.empty((R_cap, H), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = ffn_workspace(R_cap, n_local, H, I, x.dtype, x.device)
    _call("moe_grouped_ffn_gather", _p(x), _p(row_src), T, k, _p(offsets),
          _p(s_perm), n_local, R_cap, H, I, _p(w_gate), _p(w_up), _p(w_down),
          _dt(x), _p(a), _p(y), _p(workspace), workspace.numel(),
          _stream(stream))
    return a, y


def grouped_ffn_loop(x_perm, offsets, host_counts, s_perm, w_gate, w_up,
                     w_down, a=None, y=None, workspace=None, stream=None):
    """grouped_ffn issued expert by expert (one set of launches per expert
    with rows); host_counts: the per-expert row counts as a host sequence."""
    R_cap, H = x_perm.shape
    n_local, I, _ = w_gate.shape
    hc = (ctypes.c_int32 * n_local)(*[int(c) for c in host_counts])
    if a is None:
        a = torch.empty((R_cap, I), dtype=x_perm.dtype, device=x_perm.device)
    if y is None:
        y = torch.empty((R_cap, H), dtype=x_perm.dtype, device=x_perm.device)
    if workspace is None:
        workspace = ffn_workspace(R_cap, n_local, H, I, x_perm.dtype,
                                  x_perm.device)
    _call("moe_grouped_ffn_loop", _p(x_perm), _p(offsets), hc, _p(s_perm),
          n_local, R_cap, H, I, _p(w_gate), _p(w_up), _p(w_down),
          _dt(x_perm), _p(a), _p(y), _p(workspace), workspace.numel(),
          _stream(stream))
    return a, y


def grouped_ffn_fused(x, offsets, s_perm, w_gate, w_up, w_down, row_src=None,
                      k=1, a=None, y=None, workspace=None, stream=None):
    """grouped_ffn in one persistent launch (decode-sized shares).  With
    row_src, x holds the token rows and permuted row r is x[row_src[r] // k]
    (R_cap = row_src.shape[0]); without it x is x_perm [R_cap, H]."""
    T, H = x.shape
    R_cap = row_src.shape[0] if row_src is not None else T
    n_local, I, _ = w_gate.shape
    if a is None:
        a = torch.empty((R_cap, I), dtype=x.dtype, device=x.device)
    if y is None:
        y = torch.empty((R_cap, H), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = ffn_workspace(R_cap, n_local, H, I, x.dtype, x.device)
    _call("moe_grouped_ffn_fused", _p(x), _p(row_src), T, k, _p(offsets),
          _p(s_perm), n_local, R_cap, H, I, _p(w_gate), _p(w_up), _p(w_down),
          _dt(x), _p(a), _p(y), _p(workspace), workspace.numel(),
          _stream(stream))
    return a, y


# ---------------------------------------------------------------- EPLB


def eplb_plan(counts, n_slots, n_ranks, stream=None):
    """Placement of len(counts) experts on n_slots slots over n_ranks ranks
    from observed per-expert loads (device int32 [E]).  Returns a dict of
    device int32 tensors: rep, rep_first, rep_slot, slot_expert, slot_copy."""
    E = counts.numel()
    dev = counts.device
    plan = dict(rep=torch.empty(E, dtype=torch.int32, device=dev),
                rep_first=torch.empty(E + 1, dtype=torch.int32, device=dev),
                rep_slot=torch.empty(n_slots, dtype=torch.int32, device=dev),
                slot_expert=torch.empty(n_slots, dtype=torch.int32, device=dev),
                slot_copy=torch.empty(n_slots, dtype=torch.int32, device=dev))
    _call("moe_eplb_plan", _p(counts), E, n_slots, n_ranks, _p(plan["rep"]),
          _p(plan["rep_first"]), _p(plan["rep_slot"]), _p(plan["slot_expert"]),
          _p(plan["slot_copy"]), _stream(stream))
    return plan


def permute_replicated(topk_idx, x, plan, s_begin, n_slots, topk_w=None,
                       out=None, stream=None, *, E):
    """Dispatch of the current routing to the slots [s_begin, s_begin +
    n_slots) of a plan (the rows of an expert's copies split evenly).
    Returns a PermuteOut whose counts/offsets index the local slots."""
    T, k = topk_idx.shape
    H = x.shape[1] if x is not None else 0
    dtype = x.dtype if x is not None else torch.bfloat16
    dev = topk_idx.device
    if out is None:
        out = PermuteOut(T, k, max(H, 1), n_slots, dtype, dev,
                         with_x=x is not None)
        nb = lib().moe_permute_replicated_workspace_bytes(T, k, E, n_slots)
        out.workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    _call("moe_permute_replicated", _p(topk_idx), _p(topk_w), _p(x), T, k, H,
          _DT[dtype], E, plan["rep_slot"].numel(), _p(plan["rep_first"]),
          _p(plan["rep_slot"]),
          _p(plan["slot_expert"]), _p(plan["slot_copy"]), s_begin, n_slots,
          _p(out.x_perm), _p(out.s_perm) if topk_w is not None else None,
          _p(out.row_src), _p(out.inv), _p(out.counts), _p(out.offsets),
          _p(out.workspace), out.workspace.numel(), _stream(stream))
    return out


def grouped_ffn_slots(x_perm, offsets, s_perm, slot_expert, w_gate, w_up,
                      w_down, a=None, y=None, workspace=None, stream=None):
    """grouped_ffn over slots; slot g uses the weights of expert
    slot_expert[g] (device int32) of the stacked [n_experts, ...] weights."""
    R_cap, H = x_perm.shape
    n_slots = slot_expert.numel()
    n_experts, I, _ = w_gate.shape
    if a is None:
        a = torch.empty((R_cap, I), dtype=x_perm.dtype, device=x_perm.device)
    if y is None:
        y = torch.empty((R_cap, H), dtype=x_perm.dtype, device=x_perm.device)
    if workspace is None:
        workspace = ffn_workspace(R_cap, n_slots, H, I, x_perm.dtype,
                                  x_perm.device)
    _call("moe_grouped_ffn_slots", _p(x_perm), _p(offsets), _p(s_perm),
          n_slots, _p(slot_expert), n_experts, R_cap, H, I, _p(w_gate),
          _p(w_up), _p(w_down), _dt(x_perm), _p(a), _p(y), _p(workspace),
          workspace.numel(), _stream(stream))
    return a, y


def unpermute_combine(y, inv, topk_w=None, out=None, stream=None):
    T, k = inv.shape
    H = y.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=y.dtype, device=y.device)
    _call("moe_unpermute_combine", _p(y), _p(inv), _p(topk_w), T, k, H,
          _dt(y), _p(out), _stream(stream))
    return out


def debug_sync(stream=None):
    _call("moe_debug_sync", _stream(stream))


DEVERR_EXPERT_INDEX = 1
DEVERR_ROWS = 2
DEVERR_WAIT = 4


def read_device_error(workspace, stream=None) -> int:
    """The device error word of a workspace a call used (0 = no error, else
    an OR of DEVERR_* bits).  Synchronises the stream."""
    v = ctypes.c_int32(-1)
    _call("moe_read_device_error", _p(workspace), _stream(stream),
          ctypes.byref(v))
    return int(v.value)


# ---------------------------------------------------------------- MXFP8

# MX element formats (moe_mx_format): E4M3 for every operand by default, E5M2
# as the option for the backward's gradient operands.
MX_FORMATS = {"e4m3": 0, "e5m2": 1}


def _mxf(fmt):
    try:
        return MX_FORMATS[fmt]
    except KeyError:
        raise ValueError(f"unknown MX element format {fmt!r}") from None


def mxfp8_quantize(x, axis=0, seg_offsets=None, align=32, stream=None,
                   codes=None, scales=None, fmt="e4m3"):
    """MX-quantise a bf16 matrix [rows, cols] (elements of format fmt).

    axis 0 -> (codes [rows, cols] u8, scales [rows, cols/32] u8).
    axis 1 -> (codesT [cols, P] u8, scalesT [cols, P/32] u8, pad_offsets or
    None) with rows padded per segment to a multiple of `align`.  Without
    segments P is rows rounded up to `align` (the transposed stacked weights
    the backward reads have exactly that pitch); with segments P is a
    capacity rounded up to 512 and the used width is pad_offsets[-1].
    """
    rows, cols = x.shape
    dev = x.device
    ld_in = x.stride(0)
    if axis == 0:
        if codes is None:
            codes = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        if scales is None:
            scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
        assert codes.shape == (rows, cols) and scales.shape == (rows, cols // 32)
        _call("moe_mxfp8_quantize", _p(x), rows, cols, ld_in, 0, _mxf(fmt),
              None, 0, 32, _p(codes), cols, _p(scales), cols // 32, None,
              _stream(stream))
        return codes, scales
    nseg = 0 if seg_offsets is None else seg_offsets.numel() - 1
    if seg_offsets is None:
        cap = (rows + align - 1) // align * align    # exact padded width
    else:
        cap = (rows + (align - 1) * nseg + 511) // 512 * 512
    codes = torch.zeros((cols, cap), dtype=torch.uint8, device=dev)
    scales = torch.zeros((cols, cap // 32), dtype=torch.uint8, device=dev)
    pad = (torch.empty(nseg + 1, dtype=torch.int32, device=dev)
           if seg_offsets is not None else None)
    _call("moe_mxfp8_quantize", _p(x), rows, cols, ld_in, 1, _mxf(fmt),
          _p(seg_offsets), nseg, align, _p(codes), cap, _p(scales), cap // 32,
          _p(pad), _stream(stream))
    return codes, scales, pad


class MxView(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("codes", "scales", "ld_codes", "ld_scales", "rows", "cols",
                 "pad")]


MXCALL_FWD, MXCALL_BWD_DOWN, MXCALL_BWD = 0, 1, 2
MXT_A_ROWS, MXT_A_COLS, MXT_DGU_ROWS, MXT_DG_COLS, MXT_DU_COLS = 0, 1, 2, 3, 4


def mxfp8_workspace_view(workspace, call, tensor, R_cap, n_local, H, I):
    """The MX codes a call left in its workspace, as views of it: (codes
    [rows, cols] u8, scales [rows, cols/32] u8, pad int32 [n_local+1] or
    None) -- see moe_mxfp8_workspace_view."""
    v = MxView()
    _call("moe_mxfp8_workspace_view", call, tensor, R_cap, n_local, H, I,
          ctypes.byref(v))

    def part(off, rows, ld, cols):
        return workspace[off:off + rows * ld].view(rows, ld)[:, :cols]

    codes = part(v.codes, v.rows, v.ld_codes, v.cols)
    scales = part(v.scales, v.rows, v.ld_scales, v.cols // 32)
    pad = (workspace[v.pad:v.pad + 4 * (n_local + 1)].view(torch.int32)
           if v.pad >= 0 else None)
    return codes, scales, pad


class MxWeights:
    """Stacked expert weights quantised for the MXFP8 grouped MLP:
    row-wise copies for the forward, transposed column-wise copies for the
    data gradients of the backward."""

    def __init__(self, w_gate, w_up, w_down, stream=None):
        n, I, H = w_gate.shape
        self.n_local, self.I, self.H = n, I, H
        g2, u2 = w_gate.reshape(n * I, H), w_up.reshape(n * I, H)
        d2 = w_down.reshape(n * H, I)
        self.wg, self.wgs = mxfp8_quantize(g2, 0, stream=stream)
        self.wu, self.wus = mxfp8_quantize(u2, 0, stream=stream)
        self.wd, self.wds = mxfp8_quantize(d2, 0, stream=stream)
        self.wgt, self.wgts, _ = mxfp8_quantize(g2, 1, stream=stream)
        self.wut, self.wuts, _ = mxfp8_quantize(u2, 1, stream=stream)
        self.wdt, self.wdts, _ = mxfp8_quantize(d2, 1, stream=stream)


def mxfp8_mlp_fwd(xq, xs, offsets, s_perm, mw, a=None, gu=None, y=None,
                  workspace=None, stream=None, down=True):
    """down=False stops after a (y is returned as None)."""
    R_cap = xq.shape[0]
    H, I, n = mw.H, mw.I, mw.n_local
    dev = xq.device
    if a is None:
        a = torch.empty((R_cap, I), dtype=torch.bfloat16, device=dev)
    if gu is None:
        gu = torch.empty((R_cap, 2 * I), dtype=torch.float32, device=dev)
    if not down:
        y = None
    elif y is None:
        y = torch.empty((R_cap, H), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        nb = lib().moe_grouped_mlp_mxfp8_fwd_workspace_bytes(R_cap, n, H, I)
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    _call("moe_grouped_mlp_mxfp8_fwd", _p(xq), _p(xs), _p(offsets),
          _p(s_perm), n, R_cap, H, I, _p(mw.wg), _p(mw.wgs), _p(mw.wu),
          _p(mw.wus), _p(mw.wd), _p(mw.wds), _p(a), _p(gu), _p(y),
          _p(workspace), workspace.numel(), _stream(stream))
    return a, gu, y


def mxfp8_mlp_bwd(dy, x_perm, gu, offsets, s_perm, mw, dx=None, ds=None,
                  dw_gate=None, dw_up=None, dw_down=None, workspace=None,
                  stream=None, grad_format="e4m3"):
    R_cap, H = dy.shape
    I, n = mw.I, mw.n_local
    dev = dy.device
    bf = torch.bfloat16
    if dx is None:
        dx = torch.empty((R_cap, H), dtype=bf, device=dev)
    if ds is None:
        ds = torch.empty(R_cap, dtype=torch.float32, device=dev)
    if dw_gate is None:
        dw_gate = torch.empty((n, I, H), dtype=bf, device=dev)
    if dw_up is None:
        dw_up = torch.empty((n, I, H), dtype=bf, device=dev)
    if dw_down is None:
        dw_down = torch.empty((n, H, I), dtype=bf, device=dev)
    if workspace is None:
        nb = lib().moe_grouped_mlp_mxfp8_bwd_workspace_bytes(R_cap, n, H, I)
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    _call("moe_grouped_mlp_mxfp8_bwd", _p(dy), _p(x_perm), _p(gu),
          _p(offsets), _p(s_perm), n, R_cap, H, I, _p(mw.wdt), _p(mw.wdts),
          _p(mw.wgt), _p(mw.wgts), _p(mw.wut), _p(mw.wuts), _p(dx), _p(ds),
          _p(dw_gate), _p(dw_up), _p(dw_down), _mxf(grad_format),
          _p(workspace), workspace.numel(), _stream(stream))
    return dict(dx=dx, ds=ds, dw_gate=dw_gate, dw_up=dw_up, dw_down=dw_down)


def mxfp8_mlp_fwd_down(offsets, mw, workspace, R_cap, y=None, stream=None):
    """The down projection of mxfp8_mlp_fwd(..., down=False) called with
    `workspace`: reads the MX(a) that call left there."""
    if y is None:
        y = torch.empty((R_cap, mw.H), dtype=torch.bfloat16, device=workspace.device)
    _call("moe_grouped_mlp_mxfp8_fwd_down", _p(offsets), mw.n_local, R_cap,
          mw.H, mw.I, _p(mw.wd), _p(mw.wds), _p(y), _p(workspace),
          workspace.numel(), _stream(stream))
    return y


def grouped_linear_mxfp8(x, offsets, n_local, w, w_scales, y=None,
                         workspace=None, stream=None):
    """y = MX(x) MX(W_e)^T per expert segment; w codes [n_local*N, K]."""
    R_cap, K = x.shape
    N = w.shape[0] // n_local
    dev = x.device
    if y is None:
        y = torch.empty((R_cap, N), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        nb = lib().moe_grouped_linear_mxfp8_workspace_bytes(R_cap, n_local, K)
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    _call("moe_grouped_linear_mxfp8", _p(x), _p(offsets), n_local, R_cap, K,
          N, _p(w), _p(w_scales), _p(y), _p(workspace), workspace.numel(),
          _stream(stream))
    return y


def mxfp8_mlp_bwd_down(dy, gu, offsets, s_perm, mw, dgu=None, ds=None,
                       dw_down=None, workspace=None, stream=None,
                       grad_format="e4m3"):
    R_cap, H = dy.shape
    I, n = mw.I, mw.n_local
    dev = dy.device
    if dgu is None:
        dgu = torch.empty((R_cap, 2 * I), dtype=torch.bfloat16, device=dev)
    if ds is None:
        ds = torch.empty(R_cap, dtype=torch.float32, device=dev)
    if dw_down is None:
        dw_down = torch.empty((n, H, I), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        nb = lib().moe_grouped_mlp_mxfp8_bwd_down_workspace_bytes(R_cap, n, H, I)
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    _call("moe_grouped_mlp_mxfp8_bwd_down", _p(dy), _p(gu), _p(offsets),
          _p(s_perm), n, R_cap, H, I, _p(mw.wdt), _p(mw.wdts), _p(dgu), _p(ds),
          _p(dw_down), _mxf(grad_format), _p(workspace), workspace.numel(),
          _stream(stream))
    return dict(dgu=dgu, ds=ds, dw_down=dw_down)


def mxfp8_mlp_bwd_gate_up(dgu, x_perm, offsets, mw, dx=None, dw_gate=None,
                          dw_up=None, workspace=None, stream=None,
                          grad_format="e4m3"):
    R_cap, H = x_perm.shape
    I, n = mw.I, mw.n_local
    dev = x_perm.device
    bf = torch.bfloat16
    if dx is None:
        dx = torch.empty((R_cap, H), dtype=bf, device=dev)
    if dw_gate is None:
        dw_gate = torch.empty((n, I, H), dtype=bf, device=dev)
    if dw_up is None:
        dw_up = torch.empty((n, I, H), dtype=bf, device=dev)
    if workspace is None:
        nb = lib().moe_grouped_mlp_mxfp8_bwd_gate_up_workspace_bytes(R_cap, n, H, I)
        workspace = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    _call("moe_grouped_mlp_mxfp8_bwd_gate_up", _p(dgu), _p(x_perm),
          _p(offsets), n, R_cap, H, I, _p(mw.wgt), _p(mw.wgts), _p(mw.wut),
          _p(mw.wuts), _p(dx), _p(dw_gate), _p(dw_up), _mxf(grad_format),
          _p(workspace), workspace.numel(), _stream(stream))
    return dict(dx=dx, dw_gate=dw_gate, dw_up=dw_up)
