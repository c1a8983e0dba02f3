"""Python binding of the MoE layer's C ABI, over torch tensors.

The functions carry the C names and argument order of include/moe.h.  Tensors
must be contiguous device tensors; ``None`` passes NULL.  The stream defaults to
torch's current stream.  PyTorch supplies device memory and the stream only:
every step runs in the library's HIP kernels.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import torch

from ._lib import MOE_BF16, MOE_F32, MoeShape, MoeWScales, check, lib

TORCH_DTYPE = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16}


def make_shape(T: int, d: int, d_e: int, E: int, k: int, capacity: int = -1, renormalize: bool = True,
               d_e_shared: int = 0, dtype: int = MOE_BF16, scoring: int = 0, n_group: int = 1,
               topk_group: int = 1, wfmt: int = 0, afmt: int = 0) -> MoeShape:
    return MoeShape(T, d, d_e, E, k, capacity, int(bool(renormalize)), d_e_shared, dtype, scoring, n_group,
                    topk_group, wfmt, afmt)


def moe_mxfp8_quantize(x, codes, scales, stream=None) -> None:
    """MXFP8 rows of x [rows, K] (bf16) into codes [rows, K] and scales [rows, K/32] (uint8)."""
    rows, K = x.shape
    check("moe_mxfp8_quantize", lib().moe_mxfp8_quantize(rows, K, _ptr(x), _ptr(codes), _ptr(scales),
                                                         _stream(stream)))


def _scales(sc):
    """(gate, up, down) row-scale tensors -> MoeWScales pointer, or NULL."""
    if sc is None:
        return None
    g, u, d = sc
    return C.pointer(MoeWScales(_ptr(g), _ptr(u), _ptr(d)))


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor or None")
    if not t.is_cuda:
        raise ValueError("tensor must live in device memory")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return C.c_void_p(stream.cuda_stream)
    return C.c_void_p(int(stream))


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


# ------------------------------------------------------------------ host-only helpers

def moe_capacity(T: int, k: int, E: int, C_factor: float) -> int:
    cap = C.c_int32(0)
    check("moe_capacity", lib().moe_capacity(T, k, E, float(C_factor), C.byref(cap)))
    return cap.value


def moe_workspace_bytes(shape: MoeShape) -> int:
    n = C.c_size_t(0)
    check("moe_workspace_bytes", lib().moe_workspace_bytes(C.byref(shape), C.byref(n)))
    return n.value


def moe_status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


# ------------------------------------------------------------------ device calls

def moe_route(shape, x, w_r, b_r, idx, gate, counts, f, P, aux, ws, stream=None) -> None:
    check("moe_route", lib().moe_route(C.byref(shape), _ptr(x), _ptr(w_r), _ptr(b_r), _ptr(idx), _ptr(gate),
                                       _ptr(counts), _ptr(f), _ptr(P), _ptr(aux), _ptr(ws), _nbytes(ws),
                                       _stream(stream)))


def moe_permute(shape, x, idx, kept, offsets, row_token, row_of, x_perm, ws, stream=None) -> None:
    check("moe_permute", lib().moe_permute(C.byref(shape), _ptr(x), _ptr(idx), _ptr(kept), _ptr(offsets),
                                           _ptr(row_token), _ptr(row_of), _ptr(x_perm), _ptr(ws), _nbytes(ws),
                                           _stream(stream)))


def moe_expert_ffn(shape, x_perm, offsets, w_gate, w_up, w_down, scales, o, ws, stream=None) -> None:
    """scales: None, or the (gate, up, down) scale tensors of quantised weights."""
    check("moe_expert_ffn", lib().moe_expert_ffn(C.byref(shape), _ptr(x_perm), _ptr(offsets), _ptr(w_gate),
                                                 _ptr(w_up), _ptr(w_down), _scales(scales), _ptr(o), _ptr(ws),
                                                 _nbytes(ws), _stream(stream)))


def moe_combine(shape, o, row_of, gate, shared_out, y, stream=None) -> None:
    check("moe_combine", lib().moe_combine(C.byref(shape), _ptr(o), _ptr(row_of), _ptr(gate), _ptr(shared_out),
                                           _ptr(y), _stream(stream)))


def moe_forward(shape, x, w_r, b_r, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, scales, shared_scales, y, idx,
                gate, counts, kept, f, P, aux, offsets, row_token, row_of, ws, stream=None, stage_events=None) -> None:
    """scales / shared_scales: None, or (gate, up, down) row-scale tensors of FP8 weights.
    stage_events: None, or a ctypes array of MOE_NUM_STAGES + 1 hipEvent_t handles."""
    check("moe_forward", lib().moe_forward(
        C.byref(shape), _ptr(x), _ptr(w_r), _ptr(b_r), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(ws_gate),
        _ptr(ws_up), _ptr(ws_down), _scales(scales), _scales(shared_scales), _ptr(y), _ptr(idx), _ptr(gate),
        _ptr(counts), _ptr(kept), _ptr(f), _ptr(P),
        _ptr(aux), _ptr(offsets), _ptr(row_token), _ptr(row_of), _ptr(ws), _nbytes(ws), _stream(stream),
        stage_events))


def moe_forward_noalloc(shape, x, w_r, b_r, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, scales, shared_scales, y,
                        idx, gate, counts, kept, f, P, aux, offsets, row_token, row_of, stream=None,
                        stage_events=None) -> None:
    """moe_forward without a workspace: the library's static per-GPU scratch is used (calls that
    overlap on one GPU race)."""
    check("moe_forward_noalloc", lib().moe_forward_noalloc(
        C.byref(shape), _ptr(x), _ptr(w_r), _ptr(b_r), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(ws_gate),
        _ptr(ws_up), _ptr(ws_down), _scales(scales), _scales(shared_scales), _ptr(y), _ptr(idx), _ptr(gate),
        _ptr(counts), _ptr(kept), _ptr(f), _ptr(P),
        _ptr(aux), _ptr(offsets), _ptr(row_token), _ptr(row_of), _stream(stream), stage_events))


# ------------------------------------------------------------------ convenience

@dataclass
class ForwardOutputs:
    y: torch.Tensor
    idx: torch.Tensor
    gate: torch.Tensor
    counts: torch.Tensor
    kept: torch.Tensor
    f: torch.Tensor
    P: torch.Tensor
    aux: torch.Tensor
    offsets: torch.Tensor
    row_token: torch.Tensor
    row_of: torch.Tensor
    ws: torch.Tensor


def alloc_forward(shape: MoeShape, device="cuda") -> ForwardOutputs:
    """Output tensors and workspace for moe_forward (allocated by torch)."""
    T, d, E, k = shape.T, shape.d, shape.E, shape.k
    i32, f32 = torch.int32, torch.float32
    return ForwardOutputs(
        y=torch.empty((T, d), dtype=f32, device=device),
        idx=torch.empty((T, k), dtype=i32, device=device),
        gate=torch.empty((T, k), dtype=f32, device=device),
        counts=torch.empty(E, dtype=i32, device=device),
        kept=torch.empty(E, dtype=i32, device=device),
        f=torch.empty(E, dtype=f32, device=device),
        P=torch.empty(E, dtype=f32, device=device),
        aux=torch.empty(1, dtype=f32, device=device),
        offsets=torch.empty(E + 1, dtype=i32, device=device),
        row_token=torch.empty(max(T * k, 1), dtype=i32, device=device),
        row_of=torch.empty((T, k), dtype=i32, device=device),
        ws=torch.empty(max(moe_workspace_bytes(shape), 1), dtype=torch.uint8, device=device),
    )


def forward(shape: MoeShape, x, w_r, b_r, w_gate, w_up, w_down, shared=None, out: ForwardOutputs | None = None,
            stream=None, stage_events=None, scales=None, shared_scales=None) -> ForwardOutputs:
    """Run the whole layer; returns the outputs (allocating them unless `out` is given).
    scales / shared_scales: (gate, up, down) row scales when the weights are FP8 codes."""
    out = out or alloc_forward(shape, x.device)
    sg, su, sd = shared if shared is not None else (None, None, None)
    moe_forward(shape, x, w_r, b_r, w_gate, w_up, w_down, sg, su, sd, scales, shared_scales, out.y, out.idx,
                out.gate, out.counts, out.kept, out.f, out.P, out.aux, out.offsets, out.row_token, out.row_of, out.ws,
                stream, stage_events)
    return out


# ------------------------------------------------------------------ backward

def moe_backward_workspace_bytes(shape: MoeShape) -> int:
    n = C.c_size_t(0)
    check("moe_backward_workspace_bytes", lib().moe_backward_workspace_bytes(C.byref(shape), C.byref(n)))
    return int(n.value)


def moe_backward(shape, x, w_r, b_r, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, idx, gate, counts, offsets,
                 row_token, row_of, dy, d_aux, dx, dw_r, db_r, dw_gate, dw_up, dw_down, dws_gate, dws_up, dws_down,
                 dgate, ws, stream=None, stage_events=None) -> None:
    """stage_events: None, or a ctypes array of MOE_NUM_BSTAGES + 1 hipEvent_t handles."""
    check("moe_backward", lib().moe_backward(
        C.byref(shape), _ptr(x), _ptr(w_r), _ptr(b_r), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(ws_gate),
        _ptr(ws_up), _ptr(ws_down), _ptr(idx), _ptr(gate), _ptr(counts), _ptr(offsets), _ptr(row_token),
        _ptr(row_of), _ptr(dy), C.c_float(d_aux), _ptr(dx), _ptr(dw_r), _ptr(db_r), _ptr(dw_gate), _ptr(dw_up),
        _ptr(dw_down), _ptr(dws_gate), _ptr(dws_up), _ptr(dws_down), _ptr(dgate), _ptr(ws), _nbytes(ws),
        _stream(stream), stage_events))


@dataclass
class BackwardOutputs:
    dx: torch.Tensor
    dw_r: torch.Tensor
    db_r: torch.Tensor | None
    dw_gate: torch.Tensor
    dw_up: torch.Tensor
    dw_down: torch.Tensor
    dshared: tuple | None
    dgate: torch.Tensor
    ws: torch.Tensor


def alloc_backward(shape: MoeShape, bias: bool, device="cuda") -> BackwardOutputs:
    """Gradient tensors (fp32) and workspace for moe_backward (allocated by torch)."""
    T, d, de, E, k, des = shape.T, shape.d, shape.d_e, shape.E, shape.k, shape.d_e_shared
    f32 = torch.float32
    dshared = None
    if des > 0:
        dshared = (torch.empty((des, d), dtype=f32, device=device), torch.empty((des, d), dtype=f32, device=device),
                   torch.empty((d, des), dtype=f32, device=device))
    return BackwardOutputs(
        dx=torch.empty((T, d), dtype=f32, device=device),
        dw_r=torch.empty((E, d), dtype=f32, device=device),
        db_r=torch.empty(E, dtype=f32, device=device) if bias else None,
        dw_gate=torch.empty((E, de, d), dtype=f32, device=device),
        dw_up=torch.empty((E, de, d), dtype=f32, device=device),
        dw_down=torch.empty((E, d, de), dtype=f32, device=device),
        dshared=dshared,
        dgate=torch.empty((T, k), dtype=f32, device=device),
        ws=torch.empty(max(moe_backward_workspace_bytes(shape), 1), dtype=torch.uint8, device=device),
    )


def backward(shape: MoeShape, x, w_r, b_r, w_gate, w_up, w_down, fwd: ForwardOutputs, dy, d_aux: float = 0.0,
             shared=None, out: BackwardOutputs | None = None, stream=None, stage_events=None) -> BackwardOutputs:
    """Gradients of sum(dy * y) + d_aux * aux for the layer call that produced `fwd`."""
    out = out or alloc_backward(shape, b_r is not None, x.device)
    sg, su, sd = shared if shared is not None else (None, None, None)
    dsg, dsu, dsd = out.dshared if out.dshared is not None else (None, None, None)
    moe_backward(shape, x, w_r, b_r, w_gate, w_up, w_down, sg, su, sd, fwd.idx, fwd.gate, fwd.counts, fwd.offsets,
                 fwd.row_token, fwd.row_of, dy, d_aux, out.dx, out.dw_r, out.db_r, out.dw_gate, out.dw_up,
                 out.dw_down, dsg, dsu, dsd, out.dgate, out.ws, stream, stage_events)
    return out
