"""Python binding of libswitch_moe.so, the Switch FFN layer forward on MI355X.

Argument marshalling only: every function takes torch tensors (device memory
and the current HIP stream come from PyTorch), passes their pointers and sizes
to the C entry point of the same name and raises SwitchError on a non-zero
status.  All computation happens in the library's HIP kernels.  There is no
fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libswitch_moe.so")

_lib = None

SWITCH_OK, SWITCH_E_INVALID, SWITCH_E_UNSUPPORTED, SWITCH_E_WORKSPACE, SWITCH_E_HIP = range(5)

# Every symbol include/switch_moe.h declares.
EXPORTS = [
    "switch_capacity", "switch_route_workspace_bytes", "switch_dispatch_workspace_bytes",
    "switch_expert_ffn_workspace_bytes", "switch_aux_loss_workspace_bytes", "switch_workspace_bytes",
    "switch_status_string", "switch_last_error", "switch_route", "switch_dispatch", "switch_expert_ffn",
    "switch_combine", "switch_aux_loss", "switch_layer_fwd", "switch_stream_copy", "switch_profile_enable",
    "switch_profile_collect", "switch_kernel_name", "switch_router_z_loss",
    "switch_route_ex", "switch_dispatch_ex", "switch_dispatch_workspace_bytes_ex", "switch_combine_ex",
    "switch_aux_loss_ex", "switch_workspace_bytes_ex", "switch_layer_bwd", "switch_layer_bwd_workspace_bytes",
    "switch_layer_bwd_workspace_bytes_ex", "switch_build_source_hash", "switch_dispatch_noalloc",
    "switch_dispatch_noalloc_max_scratch_bytes", "switch_ffn_gemm1_token_tile",
]


class SwitchError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


class LayerArgs(ctypes.Structure):
    """Mirror of switch_layer_args."""
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "x", "w_r", "b_r", "w1", "w2", "out", "expert", "gate", "position", "keep", "counts", "accepted",
        "f", "P", "loss", "logits", "lse", "prob_sum", "dlogits", "slot_token", "buf", "y", "z_loss")] + [
        ("T", ctypes.c_int64), ("d", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("E", ctypes.c_int32),
        ("C", ctypes.c_int32), ("alpha", ctypes.c_float), ("z_beta", ctypes.c_float), ("residual", ctypes.c_int32),
        ("k", ctypes.c_int32), ("priority", ctypes.c_int32), ("group", ctypes.c_int64),
        ("slot", ctypes.c_void_p), ("accepted_total", ctypes.c_void_p), ("h", ctypes.c_void_p)]


class LayerBwdArgs(ctypes.Structure):
    """Mirror of switch_layer_bwd_args."""
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "x", "w_r", "w1", "w2", "expert", "gate", "position", "keep", "accepted", "f", "logits", "lse", "buf", "h",
        "y", "dout", "dx", "dw_r", "db_r", "dw1", "dw2", "dz", "dgate")] + [
        ("T", ctypes.c_int64), ("d", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("E", ctypes.c_int32),
        ("C", ctypes.c_int32), ("alpha", ctypes.c_float), ("z_beta", ctypes.c_float),
        ("k", ctypes.c_int32), ("group", ctypes.c_int64), ("slot", ctypes.c_void_p),
        ("accepted_total", ctypes.c_void_p), ("dx_branch_only", ctypes.c_int32)]


class StaleLibraryError(RuntimeError):
    """The built library does not match the sources beside it."""


_HASH_TAG = b"switch-source-hash:"


def library_hash(path: str = LIB_PATH) -> Optional[str]:
    """The source hash embedded in a built library (read from the file, not
    loaded, so a rebuild in the same process is seen), or None."""
    if not os.path.exists(path):
        return None
    with open(path, "rb") as fh:
        data = fh.read()
    i = data.find(_HASH_TAG)
    if i < 0:
        return None
    j = data.find(b"\0", i)
    return data[i + len(_HASH_TAG):j].decode(errors="replace")


def library_current(path: str = LIB_PATH) -> bool:
    """True when the library exists and was built from the current sources."""
    from .build import source_hash
    return library_hash(path) == source_hash()


def lib():
    """Loads the library once; raises if it has not been built, or if it was
    built from sources other than the ones beside it (a stale build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m sparse_mixture_experts_order_amd.build")
        from .build import source_hash
        built, want = library_hash(), source_hash()
        if built != want:
            raise StaleLibraryError(f"{LIB_PATH} was built from other sources (library {built}, sources {want}): "
                                    "rebuild it with python -m sparse_mixture_experts_order_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        L.switch_build_source_hash.restype = ctypes.c_char_p
        if L.switch_build_source_hash().decode() != want:   # the loader kept an older copy of this path
            raise StaleLibraryError(f"{LIB_PATH}: the loaded copy predates a rebuild in this process; "
                                    "start a new process")
        P, I64, I32, SZ, F32, F64 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t,
                                      ctypes.c_float, ctypes.c_double)
        sig = {
            "switch_capacity": (I32, [I64, I32, F64, ctypes.POINTER(ctypes.c_int32)]),
            "switch_route_workspace_bytes": (SZ, [I64, I32, I32]),
            "switch_dispatch_workspace_bytes": (SZ, [I64, I32]),
            "switch_expert_ffn_workspace_bytes": (SZ, [I32, I32, I32]),
            "switch_aux_loss_workspace_bytes": (SZ, [I64, I32]),
            "switch_workspace_bytes": (SZ, [I64, I32, I32, I32, I32]),
            "switch_status_string": (ctypes.c_char_p, [I32]),
            "switch_last_error": (ctypes.c_char_p, []),
            "switch_route": (I32, [P, P, P, P, I64, I32, I32, P, P, P, P, P, P, SZ, P]),
            "switch_dispatch": (I32, [P, P, I64, I32, I32, I32, P, P, P, P, P, P, P, SZ, P]),
            "switch_expert_ffn": (I32, [P, P, P, P, I32, I32, I32, I32, P, P, SZ, P]),
            "switch_combine": (I32, [P, P, P, P, P, P, I64, I32, I32, I32, P, P]),
            "switch_aux_loss": (I32, [P, P, P, P, I64, I32, F32, P, P, P, P, P, SZ, P]),
            "switch_layer_fwd": (I32, [ctypes.POINTER(LayerArgs), P, SZ, P]),
            "switch_stream_copy": (I32, [P, P, SZ, P]),
            "switch_profile_enable": (None, [I32]),
            "switch_profile_collect": (I32, [I32, P, P]),
            "switch_kernel_name": (ctypes.c_char_p, [I32]),
            "switch_ffn_gemm1_token_tile": (I32, [I32, I32, I64, I32]),
            "switch_router_z_loss": (I32, [P, P, I64, I32, F32, P, P, I32, P]),
            "switch_route_ex": (I32, [P, P, P, P, I64, I32, I32, I32, I64, P, P, P, P, P, P, SZ, P]),
            "switch_dispatch_workspace_bytes_ex": (SZ, [I64, I32, I32, I64]),
            "switch_dispatch_ex": (I32, [P, P, I64, I32, I32, I32, I64, I32, I32, P, P, P, P, P, P, P, P, P, SZ, P]),
            "switch_combine_ex": (I32, [P, P, P, P, P, P, I64, I32, I32, I32, I32, P, P]),
            "switch_aux_loss_ex": (I32, [P, P, P, P, I64, I32, I32, I64, F32, P, P, P, P, P]),
            "switch_workspace_bytes_ex": (SZ, [I64, I32, I32, I32, I32, I32, I64]),
            "switch_layer_bwd_workspace_bytes": (SZ, [I64, I32, I32, I32, I32]),
            "switch_layer_bwd_workspace_bytes_ex": (SZ, [I64, I32, I32, I32, I32, I32, I64]),
            "switch_layer_bwd": (I32, [ctypes.POINTER(LayerBwdArgs), P, SZ, P]),
            "switch_build_source_hash": (ctypes.c_char_p, []),
            "switch_dispatch_noalloc": (I32, [P, P, I64, I32, I32, I32, P, P, P, P, P, P, P]),
            "switch_dispatch_noalloc_max_scratch_bytes": (SZ, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int, where: str):
    if status != SWITCH_OK:
        raise SwitchError(status, where, lib().switch_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch
    if stream is not None:
        return stream.cuda_stream
    return torch.cuda.current_stream().cuda_stream


def _ws(ws):
    if ws is None:
        return None, 0
    if isinstance(ws, tuple):
        return ws
    return ws.data_ptr(), ws.numel() * ws.element_size()


# ------------------------------------------------------------ host helpers
def switch_capacity(T: int, E: int, c: float) -> int:
    out = ctypes.c_int32(0)
    _check(lib().switch_capacity(T, E, c, ctypes.byref(out)), "switch_capacity")
    return out.value


def switch_ffn_gemm1_token_tile(E: int, rows: int, assignments: int, d_ff: int) -> int:
    return lib().switch_ffn_gemm1_token_tile(E, rows, assignments, d_ff)


def switch_route_workspace_bytes(T, d, E):
    return lib().switch_route_workspace_bytes(T, d, E)


def switch_dispatch_workspace_bytes(T, E):
    return lib().switch_dispatch_workspace_bytes(T, E)


def switch_expert_ffn_workspace_bytes(E, C, d_ff):
    return lib().switch_expert_ffn_workspace_bytes(E, C, d_ff)


def switch_aux_loss_workspace_bytes(T, E):
    return lib().switch_aux_loss_workspace_bytes(T, E)


def switch_workspace_bytes(T, d, d_ff, E, C):
    return lib().switch_workspace_bytes(T, d, d_ff, E, C)


def switch_dispatch_workspace_bytes_ex(T, E, k, group):
    return lib().switch_dispatch_workspace_bytes_ex(T, E, k, group)


def switch_workspace_bytes_ex(T, d, d_ff, E, C, k, group):
    return lib().switch_workspace_bytes_ex(T, d, d_ff, E, C, k, group)


# ------------------------------------------------------------ device calls
# Tensors: bf16 arrays are torch.bfloat16, int32 arrays torch.int32, keep is
# torch.uint8, floats torch.float32; all contiguous on the current device.
def switch_route(x, w_r, b_r, logits_in, T, d, E, logits_out, expert, gate, lse, prob_sum, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib().switch_route(_ptr(x), _ptr(w_r), _ptr(b_r), _ptr(logits_in), T, d, E, _ptr(logits_out),
                              _ptr(expert), _ptr(gate), _ptr(lse), _ptr(prob_sum), wp, wn, _stream(stream)),
           "switch_route")


def switch_dispatch(x, expert, T, d, E, C, position, keep, counts, accepted, slot_token, buf, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib().switch_dispatch(_ptr(x), _ptr(expert), T, d, E, C, _ptr(position), _ptr(keep), _ptr(counts),
                                 _ptr(accepted), _ptr(slot_token), _ptr(buf), wp, wn, _stream(stream)),
           "switch_dispatch")


def switch_dispatch_noalloc(x, expert, T, d, E, C, position, keep, counts, accepted, slot_token, buf, stream=None):
    _check(lib().switch_dispatch_noalloc(_ptr(x), _ptr(expert), T, d, E, C, _ptr(position), _ptr(keep),
                                         _ptr(counts), _ptr(accepted), _ptr(slot_token), _ptr(buf), _stream(stream)),
           "switch_dispatch_noalloc")


def switch_dispatch_noalloc_max_scratch_bytes():
    return lib().switch_dispatch_noalloc_max_scratch_bytes()


def switch_expert_ffn(buf, accepted, w1, w2, E, C, d, d_ff, y, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib().switch_expert_ffn(_ptr(buf), _ptr(accepted), _ptr(w1), _ptr(w2), E, C, d, d_ff, _ptr(y), wp, wn,
                                   _stream(stream)), "switch_expert_ffn")


def switch_combine(y, expert, position, keep, gate, residual, T, d, E, C, out, stream=None):
    _check(lib().switch_combine(_ptr(y), _ptr(expert), _ptr(position), _ptr(keep), _ptr(gate), _ptr(residual),
                                T, d, E, C, _ptr(out), _stream(stream)), "switch_combine")


def switch_aux_loss(counts, prob_sum, logits, lse, T, E, alpha, f, P, loss, dlogits, ws=None, stream=None):
    wp, wn = _ws(ws)
    _check(lib().switch_aux_loss(_ptr(counts), _ptr(prob_sum), _ptr(logits), _ptr(lse), T, E, alpha, _ptr(f),
                                 _ptr(P), _ptr(loss), _ptr(dlogits), wp, wn, _stream(stream)), "switch_aux_loss")


def switch_router_z_loss(lse, logits, T, E, beta, z_loss, dlogits=None, accumulate=False, stream=None):
    _check(lib().switch_router_z_loss(_ptr(lse), _ptr(logits), T, E, beta, _ptr(z_loss), _ptr(dlogits),
                                      1 if accumulate else 0, _stream(stream)), "switch_router_z_loss")


def switch_route_ex(x, w_r, b_r, logits_in, T, d, E, k, group, logits_out, expert, gate, lse, prob_sum, ws,
                    stream=None):
    wp, wn = _ws(ws)
    _check(lib().switch_route_ex(_ptr(x), _ptr(w_r), _ptr(b_r), _ptr(logits_in), T, d, E, k, group, _ptr(logits_out),
                                 _ptr(expert), _ptr(gate), _ptr(lse), _ptr(prob_sum), wp, wn, _stream(stream)),
           "switch_route_ex")


def switch_dispatch_ex(x, expert, T, d, E, k, group, C, priority, position, keep, slot, counts, accepted,
                       accepted_total, slot_token, buf, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib().switch_dispatch_ex(_ptr(x), _ptr(expert), T, d, E, k, group, C, priority, _ptr(position), _ptr(keep),
                                    _ptr(slot), _ptr(counts), _ptr(accepted), _ptr(accepted_total), _ptr(slot_token),
                                    _ptr(buf), wp, wn, _stream(stream)), "switch_dispatch_ex")


def switch_combine_ex(y, expert, slot, keep, gate, residual, T, d, E, k, rows, out, stream=None):
    _check(lib().switch_combine_ex(_ptr(y), _ptr(expert), _ptr(slot), _ptr(keep), _ptr(gate), _ptr(residual),
                                   T, d, E, k, rows, _ptr(out), _stream(stream)), "switch_combine_ex")


def switch_aux_loss_ex(counts, prob_sum, logits, lse, T, E, k, group, alpha, f, P, loss, dlogits, stream=None):
    _check(lib().switch_aux_loss_ex(_ptr(counts), _ptr(prob_sum), _ptr(logits), _ptr(lse), T, E, k, group, alpha,
                                    _ptr(f), _ptr(P), _ptr(loss), _ptr(dlogits), _stream(stream)),
           "switch_aux_loss_ex")


def switch_layer_fwd(args: LayerArgs, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib().switch_layer_fwd(ctypes.byref(args), wp, wn, _stream(stream)), "switch_layer_fwd")


def switch_layer_bwd_workspace_bytes(T, d, d_ff, E, C):
    return lib().switch_layer_bwd_workspace_bytes(T, d, d_ff, E, C)


def switch_layer_bwd_workspace_bytes_ex(T, d, d_ff, E, C, k, group):
    return lib().switch_layer_bwd_workspace_bytes_ex(T, d, d_ff, E, C, k, group)


def switch_layer_bwd(args: LayerBwdArgs, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib().switch_layer_bwd(ctypes.byref(args), wp, wn, _stream(stream)), "switch_layer_bwd")


def make_layer_bwd_args(fwd: dict, x, w_r, w1, w2, dout, grads: dict, T, d, d_ff, E, C, alpha,
                        z_beta=0.0, k=1, group=0, dx_branch_only=False) -> LayerBwdArgs:
    """fwd: the forward's tensors (expert, gate, position, keep, accepted, f,
    logits, lse, buf, h, y, and with several groups slot and accepted_total);
    grads: dx, dw_r, db_r, dw1, dw2 and optionally dz, dgate.  C is the
    capacity of one routing group."""
    a = LayerBwdArgs()
    for name, v in (("x", x), ("w_r", w_r), ("w1", w1), ("w2", w2), ("dout", dout)):
        setattr(a, name, _ptr(v))
    for name in ("expert", "gate", "position", "keep", "accepted", "f", "logits", "lse", "buf", "h", "y", "slot",
                 "accepted_total"):
        setattr(a, name, _ptr(fwd.get(name)))
    for name in ("dx", "dw_r", "db_r", "dw1", "dw2", "dz", "dgate"):
        setattr(a, name, _ptr(grads.get(name)))
    a.T, a.d, a.d_ff, a.E, a.C, a.alpha, a.z_beta = T, d, d_ff, E, C, alpha, z_beta
    a.k, a.group = k, group
    a.dx_branch_only = 1 if dx_branch_only else 0
    return a


def layer_bwd_tensors(T, d, d_ff, E, C, device="cuda", inspect=False, k=1, group=0):
    """Gradient tensors of switch_layer_bwd (plus its workspace); C is the
    capacity of one routing group."""
    import torch
    dev = torch.device(device)
    g = {
        "dx": torch.empty((T, d), dtype=torch.bfloat16, device=dev),
        "dw_r": torch.empty((d, E), dtype=torch.float32, device=dev),
        "db_r": torch.empty(E, dtype=torch.float32, device=dev),
        "dw1": torch.empty((E, d_ff, d), dtype=torch.float32, device=dev),
        "dw2": torch.empty((E, d, d_ff), dtype=torch.float32, device=dev),
    }
    if inspect:
        g["dz"] = torch.empty((T, E), dtype=torch.float32, device=dev)
        g["dgate"] = torch.empty((T,) if k == 1 else (T, k), dtype=torch.float32, device=dev)
    g["ws"] = torch.empty(max(256, switch_layer_bwd_workspace_bytes_ex(T, d, d_ff, E, C, k, group)),
                          dtype=torch.uint8, device=dev)
    return g


def switch_stream_copy(dst, src, nbytes: int, stream=None):
    _check(lib().switch_stream_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream)), "switch_stream_copy")


def switch_profile_enable(on: bool):
    lib().switch_profile_enable(1 if on else 0)


def switch_profile_collect(max_records: int = 1 << 16):
    """[(kernel name, milliseconds)] for launches made while profiling was on."""
    ids = (ctypes.c_int32 * max_records)()
    ms = (ctypes.c_float * max_records)()
    n = lib().switch_profile_collect(max_records, ctypes.cast(ids, ctypes.c_void_p), ctypes.cast(ms, ctypes.c_void_p))
    if n < 0:
        raise SwitchError(SWITCH_E_HIP, "switch_profile_collect", "HIP event error")
    return [(lib().switch_kernel_name(ids[i]).decode(), ms[i]) for i in range(n)]


# ------------------------------------------------------------ allocation helpers
def layer_tensors(T, d, d_ff, E, C, device="cuda", logits=False, dlogits=False, inspect=False, z_loss=False,
                  k=1, group=0, for_backward=False):
    """Output tensors of switch_layer_fwd (plus a workspace), allocated with torch.
    With k choices the per-choice arrays are [T, k]; with several routing groups
    of `group` tokens the per-expert statistics are [T // group, E], C is the
    capacity of one group and the buffer has (T // group) * C rows per expert."""
    import torch
    dev = torch.device(device)
    ng = 1 if group in (0, T) else T // group
    rows = ng * C
    kk = () if k == 1 else (k,)
    o = {
        "out": torch.empty((T, d), dtype=torch.bfloat16, device=dev),
        "expert": torch.empty((T,) + kk, dtype=torch.int32, device=dev),
        "gate": torch.empty((T,) + kk, dtype=torch.float32, device=dev),
        "position": torch.empty((T,) + kk, dtype=torch.int32, device=dev),
        "keep": torch.empty((T,) + kk, dtype=torch.uint8, device=dev),
        "counts": torch.empty((ng, E) if ng != 1 else E, dtype=torch.int32, device=dev),
        "accepted": torch.empty((ng, E) if ng != 1 else E, dtype=torch.int32, device=dev),
        "f": torch.empty((ng, E) if ng != 1 else E, dtype=torch.float32, device=dev),
        "P": torch.empty((ng, E) if ng != 1 else E, dtype=torch.float32, device=dev),
        "loss": torch.empty(1, dtype=torch.float32, device=dev),
        "lse": torch.empty(T, dtype=torch.float32, device=dev),
        "prob_sum": torch.empty((ng, E) if ng != 1 else E, dtype=torch.float32, device=dev),
    }
    if ng != 1:
        o["slot"] = torch.empty((T,) + kk, dtype=torch.int32, device=dev)
        o["accepted_total"] = torch.empty(E, dtype=torch.int32, device=dev)
    if for_backward:   # what switch_layer_bwd reads besides the inputs
        logits = inspect = True
        o["h"] = torch.empty((E, rows, d_ff), dtype=torch.bfloat16, device=dev)
    if logits or dlogits:
        o["logits"] = torch.empty((T, E), dtype=torch.float32, device=dev)
    if dlogits:
        o["dlogits"] = torch.empty((T, E), dtype=torch.float32, device=dev)
    if z_loss:
        o["z_loss"] = torch.empty(1, dtype=torch.float32, device=dev)
    if inspect:
        o["slot_token"] = torch.empty((E, rows), dtype=torch.int32, device=dev)
        o["buf"] = torch.empty((E, rows, d), dtype=torch.bfloat16, device=dev)
        o["y"] = torch.empty((E, rows, d), dtype=torch.float32, device=dev)
    nbytes = switch_workspace_bytes_ex(T, d, d_ff, E, C, k, group)
    o["ws"] = torch.empty(max(256, nbytes), dtype=torch.uint8, device=dev)
    return o


def make_layer_args(x, w_r, b_r, w1, w2, t: dict, T, d, d_ff, E, C, alpha, residual=True, z_beta=0.0,
                    k=1, group=0, priority=0) -> LayerArgs:
    a = LayerArgs()
    for name, v in (("x", x), ("w_r", w_r), ("b_r", b_r), ("w1", w1), ("w2", w2)):
        setattr(a, name, _ptr(v))
    for name in ("out", "expert", "gate", "position", "keep", "counts", "accepted", "f", "P", "loss", "logits",
                 "lse", "prob_sum", "dlogits", "slot_token", "buf", "y", "z_loss", "slot", "accepted_total", "h"):
        setattr(a, name, _ptr(t.get(name)))
    a.T, a.d, a.d_ff, a.E, a.C, a.alpha, a.residual = T, d, d_ff, E, C, alpha, 1 if residual else 0
    a.z_beta = z_beta
    a.k, a.group, a.priority = k, group, priority
    return a
