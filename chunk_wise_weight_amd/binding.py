"""Python binding of libttt.so: the C ABI's entry points under the same names.

Argument marshalling only: tensors are turned into device pointers and sizes,
and torch's current HIP stream is passed along. Every step of the
computation runs in the library's HIP kernels; there is no fallback path, and
a missing or unloadable library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Tuple

import torch  # loads the HIP runtime the library binds to (same libamdhip64 soname)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libttt.so")

TTT_F32, TTT_BF16 = 0, 1
ERRORS = {-1: "TTT_E_NULL", -2: "TTT_E_SHAPE", -3: "TTT_E_DTYPE", -4: "TTT_E_NOMEM", -5: "TTT_E_HIP",
          -6: "TTT_E_NODEV", -7: "TTT_E_ARG"}
EXPORTS = ("ttt_init", "ttt_forward_chunked", "ttt_forward_docs", "ttt_reset", "ttt_destroy", "ttt_last_error",
           "ttt_set_group_chunks", "ttt_set_clip", "ttt_set_target_conv", "ttt_plan", "ttt_set_profiling", "ttt_phase_times",
           "ttt_workspace_bytes", "ttt_set_output_f32", "ttt_state_delta", "ttt_forward_chunked_noalloc")

_lib = None


class TTTError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where}: {ERRORS.get(code, code)}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libttt.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m chunk_wise_weight_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.ttt_init.argtypes = [ctypes.POINTER(vp), vp, vp, vp, i32, i32, i32, f32, i32, i32, vp]
    L.ttt_init.restype = i32
    L.ttt_forward_chunked.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp, vp]
    L.ttt_forward_chunked.restype = i32
    L.ttt_reset.argtypes = [vp, i32, vp]
    L.ttt_reset.restype = i32
    L.ttt_destroy.argtypes = [vp]
    L.ttt_destroy.restype = None
    L.ttt_last_error.argtypes = []
    L.ttt_last_error.restype = ctypes.c_char_p
    L.ttt_set_group_chunks.argtypes = [vp, i32]
    L.ttt_set_group_chunks.restype = i32
    L.ttt_set_clip.argtypes = [vp, f32]
    L.ttt_set_clip.restype = i32
    L.ttt_set_target_conv.argtypes = [vp, vp, i32, vp, vp]
    L.ttt_set_target_conv.restype = i32
    ip = ctypes.POINTER(i32)
    L.ttt_forward_docs.argtypes = [vp, vp, vp, vp, i32, i32, i32, ip, ip, vp, vp, vp]
    L.ttt_forward_docs.restype = i32
    L.ttt_plan.argtypes = [i32, i32, i32, ip, ip, ip, ip]
    L.ttt_plan.restype = i32
    L.ttt_set_profiling.argtypes = [vp, i32]
    L.ttt_set_profiling.restype = i32
    L.ttt_phase_times.argtypes = [vp, ctypes.POINTER(f32), i32]
    L.ttt_phase_times.restype = i32
    L.ttt_workspace_bytes.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t)]
    L.ttt_workspace_bytes.restype = i32
    L.ttt_set_output_f32.argtypes = [vp, i32]
    L.ttt_set_output_f32.restype = i32
    L.ttt_state_delta.argtypes = [vp, vp, i32, vp]
    L.ttt_state_delta.restype = i32
    L.ttt_forward_chunked_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp, vp]
    L.ttt_forward_chunked_noalloc.restype = i32
    _lib = L
    return L


def ttt_last_error() -> str:
    return lib().ttt_last_error().decode()


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise TTTError(rc, where, ttt_last_error())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


class Handle:
    """An initialised layer (library handle) and the shapes it was made with."""

    def __init__(self, ptr: ctypes.c_void_p, d: int, f: int, C: int, eta: float, dtype: torch.dtype,
                 max_batch: int):
        self._ptr = ptr
        self.d, self.f, self.C, self.eta, self.dtype, self.max_batch = d, f, C, eta, dtype, max_batch
        self.y_dtype = dtype  # the dtype forward calls write y in

    @property
    def ptr(self) -> ctypes.c_void_p:
        if not self._ptr:
            raise RuntimeError("handle already destroyed")
        return self._ptr

    def __del__(self):
        try:
            ttt_destroy(self)
        except Exception:
            pass


def ttt_init(W_up: torch.Tensor, W_gate: torch.Tensor, W_down0: torch.Tensor, C: int, eta: float,
             max_batch: int = 1, stream=None) -> Handle:
    """W_up, W_gate [f][d]; W_down0 [d][f]; float32 or bfloat16 (all the same)."""
    dt = W_up.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise ValueError("weights must be float32 or bfloat16")
    for t, n in ((W_up, "W_up"), (W_gate, "W_gate"), (W_down0, "W_down0")):
        _dev(t, n, dt)
        if t.dim() != 2:
            raise ValueError(f"{n} must be 2-D")
    f, d = W_up.shape
    h = ctypes.c_void_p()
    _check(lib().ttt_init(ctypes.byref(h), _ptr(W_up), _ptr(W_gate), _ptr(W_down0), d, f, int(C), float(eta),
                          TTT_BF16 if dt == torch.bfloat16 else TTT_F32, int(max_batch), _stream(stream)),
           "ttt_init")
    if tuple(W_gate.shape) != (f, d) or tuple(W_down0.shape) != (d, f):
        ttt_destroy(Handle(h, d, f, C, eta, dt, max_batch))
        raise ValueError("shapes must be W_up, W_gate [f][d] and W_down0 [d][f]")
    return Handle(h, d, f, int(C), float(eta), dt, int(max_batch))


def _forward_args(h, x, ids, E_tgt, y, W_final, want_W_final):
    _dev(x, "x", h.dtype)
    _dev(ids, "ids", torch.int32)
    _dev(E_tgt, "E_tgt", h.dtype)
    if x.dim() != 3 or ids.dim() != 2 or E_tgt.dim() != 2:
        raise ValueError("x must be [B][T][d], ids [B][T+1], E_tgt [vocab][d]")
    B, T, d = x.shape
    if tuple(ids.shape) != (B, T + 1) or d != h.d or E_tgt.shape[1] != h.d:
        raise ValueError("shape mismatch among x, ids, E_tgt and the handle")
    if y is None:
        y = torch.empty((B, T, d), dtype=h.y_dtype, device=x.device)
    else:
        _dev(y, "y", h.y_dtype)
        if tuple(y.shape) != (B, T, d):
            raise ValueError("y must be [B][T][d]")
    if W_final is None and want_W_final:
        W_final = torch.empty((B, h.d, h.f), dtype=torch.float32, device=x.device)
    if W_final is not None:
        _dev(W_final, "W_final", torch.float32)
        if tuple(W_final.shape) != (B, h.d, h.f):
            raise ValueError("W_final must be [B][d][f]")
    return B, T, y, W_final



def ttt_forward_chunked(h: Handle, x: torch.Tensor, ids: torch.Tensor, E_tgt: torch.Tensor,
                        y: Optional[torch.Tensor] = None, W_final: Optional[torch.Tensor] = None,
                        want_W_final: bool = False, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """x [B][T][d], ids [B][T+1] int32, E_tgt [vocab][d] -> (y [B][T][d], W_final [B][d][f] fp32 or None)."""
    B, T, y, W_final = _forward_args(h, x, ids, E_tgt, y, W_final, want_W_final)
    _check(lib().ttt_forward_chunked(h.ptr, _ptr(x), _ptr(ids), _ptr(E_tgt), int(E_tgt.shape[0]), int(B), int(T),
                                     _ptr(y), _ptr(W_final), _stream(stream)), "ttt_forward_chunked")
    return y, W_final


NOALLOC_WORKSPACE_BYTES = 64 << 20  # TTT_NOALLOC_WORKSPACE_BYTES in include/ttt.h


def ttt_forward_chunked_noalloc(h: Handle, x: torch.Tensor, ids: torch.Tensor, E_tgt: torch.Tensor,
                                y: torch.Tensor, W_final: Optional[torch.Tensor] = None,
                                stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """ttt_forward_chunked with the library's fixed workspace: the call allocates nothing on the device.
    y (and W_final, if wanted) must be given."""
    if y is None:
        raise ValueError("y must be given (the call allocates nothing)")
    B, T, y, W_final = _forward_args(h, x, ids, E_tgt, y, W_final, False)
    _check(lib().ttt_forward_chunked_noalloc(h.ptr, _ptr(x), _ptr(ids), _ptr(E_tgt), int(E_tgt.shape[0]), int(B),
                                             int(T), _ptr(y), _ptr(W_final), _stream(stream)),
           "ttt_forward_chunked_noalloc")
    return y, W_final


def ttt_forward_docs(h: Handle, x: torch.Tensor, ids: torch.Tensor, E_tgt: torch.Tensor, doc_starts,
                     y: Optional[torch.Tensor] = None, W_final: Optional[torch.Tensor] = None,
                     want_W_final: bool = False, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Packed documents: doc_starts[b] lists the positions in (0, T) where a new
    document starts in sequence b (the state returns to W_down0 there)."""
    B, T, y, W_final = _forward_args(h, x, ids, E_tgt, y, W_final, want_W_final)
    if len(doc_starts) != B:
        raise ValueError("doc_starts needs one list per sequence")
    counts = (ctypes.c_int32 * max(B, 1))(*[len(s) for s in doc_starts])
    flat = [int(p) for s in doc_starts for p in s]
    starts = (ctypes.c_int32 * max(len(flat), 1))(*flat)
    _check(lib().ttt_forward_docs(h.ptr, _ptr(x), _ptr(ids), _ptr(E_tgt), int(E_tgt.shape[0]), int(B), int(T),
                                  starts, counts, _ptr(y), _ptr(W_final), _stream(stream)), "ttt_forward_docs")
    return y, W_final

def ttt_reset(h: Handle, b: int = -1, stream=None) -> None:
    _check(lib().ttt_reset(h.ptr, int(b), _stream(stream)), "ttt_reset")


def ttt_destroy(h: Handle) -> None:
    if h._ptr:
        lib().ttt_destroy(h._ptr)
        h._ptr = None


def ttt_set_group_chunks(h: Handle, G: int) -> None:
    _check(lib().ttt_set_group_chunks(h.ptr, int(G)), "ttt_set_group_chunks")


def ttt_set_clip(h: Handle, tau: float) -> None:
    """Frobenius clipping of each chunk update at threshold tau (0 or inf: off)."""
    _check(lib().ttt_set_clip(h.ptr, float(tau)), "ttt_set_clip")


def ttt_set_target_conv(h: Handle, conv_w=None, W_target=None, stream=None) -> None:
    """The general target Conv1D(X0) W_target: conv_w [K][d], W_target [d][d]
    (device tensors of the handle's dtype). conv_w None restores the next-token target."""
    if conv_w is None:
        _check(lib().ttt_set_target_conv(h.ptr, None, 0, None, _stream(stream)), "ttt_set_target_conv")
        return
    cw = conv_w.contiguous()
    wt = W_target.contiguous()
    _dev(cw, "conv_w", h.dtype)
    _dev(wt, "W_target", h.dtype)
    if cw.dim() != 2 or cw.shape[1] != h.d or tuple(wt.shape) != (h.d, h.d):
        raise ValueError("shapes must be conv_w [K][d] and W_target [d][d]")
    _check(lib().ttt_set_target_conv(h.ptr, _ptr(cw), int(cw.shape[0]), _ptr(wt), _stream(stream)),
           "ttt_set_target_conv")


def ttt_plan(T: int, C: int, G: int = 0) -> Dict[str, int]:
    """Host-only: the group layout a call with T tokens and chunk C uses."""
    g, L, n, tp = (ctypes.c_int() for _ in range(4))
    _check(lib().ttt_plan(int(T), int(C), int(G), ctypes.byref(g), ctypes.byref(L), ctypes.byref(n),
                          ctypes.byref(tp)), "ttt_plan")
    return {"G": g.value, "L": L.value, "ngroups": n.value, "T_pad": tp.value}


def ttt_state_delta(h: Handle, B: Optional[int] = None, out: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """D = W - W_down0 of sequences 0 .. B-1 (the change since each last reset), [B][d][f] float32."""
    B = h.max_batch if B is None else int(B)
    if out is None:
        out = torch.empty((B, h.d, h.f), dtype=torch.float32, device="cuda")
    _dev(out, "out", torch.float32)
    if tuple(out.shape) != (B, h.d, h.f):
        raise ValueError("out must be [B][d][f]")
    _check(lib().ttt_state_delta(h.ptr, _ptr(out), B, _stream(stream)), "ttt_state_delta")
    return out


def ttt_set_output_f32(h: Handle, on: bool = True) -> None:
    """On a bfloat16 handle, later forward calls write y as float32 (no final rounding to bf16)."""
    _check(lib().ttt_set_output_f32(h.ptr, 1 if on else 0), "ttt_set_output_f32")
    h.y_dtype = torch.float32 if (on or h.dtype == torch.float32) else h.dtype


def ttt_set_profiling(h: Handle, on: bool = True) -> None:
    _check(lib().ttt_set_profiling(h.ptr, 1 if on else 0), "ttt_set_profiling")


PHASES = ("gather", "up_gate_swiglu", "clip_factors", "update_snapshots", "group_scores", "output", "final_copy")


def ttt_phase_times(h: Handle) -> List[float]:
    """Milliseconds per phase, the mean per forward call over the profiled calls since the previous read
    (waits for them)."""
    buf = (ctypes.c_float * len(PHASES))()
    _check(lib().ttt_phase_times(h.ptr, buf, len(PHASES)), "ttt_phase_times")
    return list(buf)


def ttt_workspace_bytes(h: Handle) -> int:
    n = ctypes.c_size_t()
    _check(lib().ttt_workspace_bytes(h.ptr, ctypes.byref(n)), "ttt_workspace_bytes")
    return n.value
