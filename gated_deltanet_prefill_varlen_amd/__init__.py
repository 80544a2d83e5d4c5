"""Python binding of libgdn (packed gated-delta-rule prefill, checkpoints,
decode, short conv and checkpoint copy on MI355X / gfx950).

Argument marshalling only: every function here passes torch tensor data
pointers, sizes and the current HIP stream to the C entry point of the same
name in ``libgdn.so`` and raises ``GdnError`` on a non-OK status.  All compute
runs in the library's HIP kernels; there is no other implementation behind
these names, and importing fails loudly when the library is not built.

torch is imported before the library is loaded so that the process holds a
single HIP runtime (torch's), which makes torch streams, events and device
pointers valid handles for libgdn.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = [
    "GdnError", "gdn_shape", "make_shape", "load", "GDN_BF16", "GDN_F32", "GDN_QK_L2NORM",
    "gdn_status_string", "gdn_plan_checkpoints", "gdn_prefill_packed", "gdn_prefill_conv_packed",
    "gdn_decode_step", "gdn_decode_tokens",
    "gdn_conv1d_silu_packed", "gdn_snapshot_copy", "LIB_PATH", "EXPORTED",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")
GDN_BF16, GDN_F32 = 0, 1
GDN_QK_L2NORM = 1
STATUS = {0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_SHAPE", 3: "GDN_ERR_UNSUPPORTED",
          4: "GDN_ERR_SEQLENS", 5: "GDN_ERR_CKPT", 6: "GDN_ERR_CAPACITY", 7: "GDN_ERR_HIP"}
EXPORTED = ("gdn_status_string", "gdn_plan_checkpoints", "gdn_conv1d_silu_packed",
            "gdn_prefill_packed", "gdn_prefill_conv_packed", "gdn_decode_step",
            "gdn_decode_tokens", "gdn_snapshot_copy")


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {gdn_status_string(status)}")


class gdn_shape(ctypes.Structure):
    _fields_ = [
        ("num_qk_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
        ("head_k_dim", ctypes.c_int32), ("head_v_dim", ctypes.c_int32),
        ("chunk", ctypes.c_int32), ("io_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("scale", ctypes.c_float), ("l2_eps", ctypes.c_float), ("reserved", ctypes.c_int32),
        ("q_tok_stride", ctypes.c_int64), ("k_tok_stride", ctypes.c_int64),
        ("v_tok_stride", ctypes.c_int64),
    ]


def make_shape(Hqk: int, Hv: int, dk: int, dv: int, chunk: int = 64, io_dtype: int = GDN_BF16,
               l2norm: bool = True, scale: float = 1.0, l2_eps: float = 1e-6,
               q_tok_stride: int = 0, k_tok_stride: int = 0, v_tok_stride: int = 0) -> gdn_shape:
    return gdn_shape(Hqk, Hv, dk, dv, chunk, io_dtype, GDN_QK_L2NORM if l2norm else 0,
                     scale, l2_eps, 0, q_tok_stride, k_tok_stride, v_tok_stride)


_lib: Optional[ctypes.CDLL] = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SP = ctypes.POINTER(gdn_shape)


def load() -> ctypes.CDLL:
    """Load libgdn.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libgdn.so is not built ({LIB_PATH}); run __graft_entry__.build() "
                           "or python gated_deltanet_prefill_varlen_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [_I32]
    lib.gdn_plan_checkpoints.restype = _I32
    lib.gdn_plan_checkpoints.argtypes = [_P, _I32, _P, _I32, _I32, _P, _I32, _P]
    lib.gdn_prefill_packed.restype = _I32
    lib.gdn_prefill_packed.argtypes = [_SP, _P, _P, _I32, _I32, _P, _P, _P, _P, _P, _P,
                                       _P, _P, _I32, _P, _P, _P, _P]
    lib.gdn_prefill_conv_packed.restype = _I32
    lib.gdn_prefill_conv_packed.argtypes = [_SP, _P, _P, _I32, _I32, _P, _I64, _P, _P, _P, _P, _P,
                                            _P, _P, _P, _I32, _P, _P, _P, _P, _P]
    lib.gdn_decode_step.restype = _I32
    lib.gdn_decode_step.argtypes = [_SP, _I32, _P, _P, _P, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _P]
    lib.gdn_decode_tokens.restype = _I32
    lib.gdn_decode_tokens.argtypes = [_SP, _I32, _I32, _P, _P, _P, _P, _P, _P, _I64, _P, _P, _P, _P,
                                      _P, _P, _P]
    lib.gdn_conv1d_silu_packed.restype = _I32
    lib.gdn_conv1d_silu_packed.argtypes = [_SP, _P, _P, _I32, _I32, _P, _I64, _P, _P, _P, _I64,
                                           _P, _P, _P, _I32, _P, _P]
    lib.gdn_snapshot_copy.restype = _I32
    lib.gdn_snapshot_copy.argtypes = [_P, _I32, _I64, _P, _I64, _P, _P, _P, _P, _P]
    _lib = lib
    return lib


def gdn_status_string(status: int) -> str:
    return load().gdn_status_string(int(status)).decode()


# ------------------------------------------------------------ marshalling --

def _dev(t) -> Optional[int]:
    """Device pointer of a tensor (None passes NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("device arguments must be torch tensors")
    if not t.is_cuda:
        raise ValueError("device argument is not on the GPU")
    return t.data_ptr()


def _host_i32(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


def _host_i64(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a), dtype=np.int64)


def _hp(a: Optional[np.ndarray]) -> Optional[int]:
    return None if a is None else a.ctypes.data


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream or None
    return int(stream) or None


def _event(ev) -> Optional[int]:
    if ev is None:
        return None
    if isinstance(ev, torch.cuda.Event):
        return ev.cuda_event or None
    return int(ev) or None


def _record_target(ev) -> Optional[int]:
    """Handle of an event the library records.  torch makes an event's HIP
    handle only at its first record, and a null handle would leave the event
    unrecorded (a later wait on it would not wait), so a fresh torch event is
    recorded once on the current stream first; the library's own record after
    its work is the one every later wait sees."""
    if isinstance(ev, torch.cuda.Event) and not ev.cuda_event:
        ev.record()
    return _event(ev)


def _check(status: int, where: str) -> None:
    if status != 0:
        raise GdnError(status, where)


# -------------------------------------------------------------- functions --

def gdn_plan_checkpoints(cu_seqlens_host, block: int, tail: int = 16,
                         p0_host=None) -> np.ndarray:
    """Checkpoint positions (int32 global offsets) for a pack; host only."""
    lib = load()
    cu = _host_i32(cu_seqlens_host)
    p0 = _host_i32(p0_host)
    n = ctypes.c_int32(0)
    st = lib.gdn_plan_checkpoints(_hp(cu), len(cu) - 1, _hp(p0), block, tail, None, 0,
                                  ctypes.byref(n))
    if st not in (0, 6):
        _check(st, "gdn_plan_checkpoints")
    out = np.zeros(max(n.value, 1), dtype=np.int32)
    _check(lib.gdn_plan_checkpoints(_hp(cu), len(cu) - 1, _hp(p0), block, tail, _hp(out),
                                    n.value, ctypes.byref(n)), "gdn_plan_checkpoints")
    return out[:n.value]


def gdn_prefill_packed(shape: gdn_shape, cu_seqlens, cu_seqlens_host, q, k, v, g, beta,
                       init_state, ckpt_positions, ckpt_positions_host, out, final_state,
                       ckpt_buf, stream=None) -> None:
    cu_h = _host_i32(cu_seqlens_host)
    ck_h = _host_i32(ckpt_positions_host)
    n_ckpt = 0 if ck_h is None else len(ck_h)
    n_tokens = int(cu_h[-1]) if len(cu_h) else 0
    _check(load().gdn_prefill_packed(
        ctypes.byref(shape), _dev(cu_seqlens), _hp(cu_h), len(cu_h) - 1, n_tokens,
        _dev(q), _dev(k), _dev(v), _dev(g), _dev(beta), _dev(init_state),
        _dev(ckpt_positions), _hp(ck_h), n_ckpt, _dev(out), _dev(final_state), _dev(ckpt_buf),
        _stream(stream)), "gdn_prefill_packed")


def gdn_prefill_conv_packed(shape: gdn_shape, cu_seqlens, cu_seqlens_host, x, conv_weight, g,
                            beta, init_state, ckpt_positions, ckpt_positions_host, out,
                            final_state, ckpt_buf, conv_state_in=None, conv_state_out=None,
                            conv_ckpt=None, x_tok_stride: int = 0, stream=None) -> None:
    """The packed prefill reading pre-conv rows x (the short conv fused into
    the scan's loads)."""
    cu_h = _host_i32(cu_seqlens_host)
    ck_h = _host_i32(ckpt_positions_host)
    n_ckpt = 0 if ck_h is None else len(ck_h)
    n_tokens = int(cu_h[-1]) if len(cu_h) else 0
    _check(load().gdn_prefill_conv_packed(
        ctypes.byref(shape), _dev(cu_seqlens), _hp(cu_h), len(cu_h) - 1, n_tokens,
        _dev(x), x_tok_stride, _dev(conv_weight), _dev(conv_state_in), _dev(conv_state_out),
        _dev(g), _dev(beta), _dev(init_state), _dev(ckpt_positions), _hp(ck_h), n_ckpt,
        _dev(conv_ckpt), _dev(out), _dev(final_state), _dev(ckpt_buf), _stream(stream)),
        "gdn_prefill_conv_packed")


def gdn_decode_step(shape: gdn_shape, q, k, v, g, beta, state, slot=None, slot_host=None,
                    out=None, conv_w=None, conv_state=None, stream=None) -> None:
    """One token per sequence; with conv_w and conv_state, q, k, v are the
    conv's inputs and the slots' conv windows move on by one token."""
    sl_h = _host_i32(slot_host)
    _check(load().gdn_decode_step(
        ctypes.byref(shape), int(q.shape[0]), _dev(q), _dev(k), _dev(v), _dev(g), _dev(beta),
        _dev(state), int(state.shape[0]), _dev(slot), _hp(sl_h), _dev(out), _dev(conv_w),
        _dev(conv_state), _stream(stream)), "gdn_decode_step")


def gdn_decode_tokens(shape: gdn_shape, n_tok: int, q, k, v, g, beta, state, slot=None,
                      slot_host=None, out=None, snapshots=None, conv_w=None, conv_state=None,
                      stream=None) -> None:
    """n_tok tokens per sequence (rows b * n_tok + i), states kept per token."""
    sl_h = _host_i32(slot_host)
    batch = int(q.shape[0]) // int(n_tok)
    _check(load().gdn_decode_tokens(
        ctypes.byref(shape), batch, int(n_tok), _dev(q), _dev(k), _dev(v), _dev(g), _dev(beta),
        _dev(state), int(state.shape[0]), _dev(slot), _hp(sl_h), _dev(out), _dev(snapshots),
        _dev(conv_w), _dev(conv_state), _stream(stream)), "gdn_decode_tokens")


def gdn_conv1d_silu_packed(shape: gdn_shape, cu_seqlens, cu_seqlens_host, x, weight, y,
                           conv_state_in=None, conv_state_out=None, ckpt_positions=None,
                           ckpt_positions_host=None, conv_ckpt=None, x_tok_stride: int = 0,
                           y_tok_stride: int = 0, stream=None) -> None:
    cu_h = _host_i32(cu_seqlens_host)
    ck_h = _host_i32(ckpt_positions_host)
    n_ckpt = 0 if ck_h is None else len(ck_h)
    _check(load().gdn_conv1d_silu_packed(
        ctypes.byref(shape), _dev(cu_seqlens), _hp(cu_h), len(cu_h) - 1, int(cu_h[-1]),
        _dev(x), x_tok_stride, _dev(weight), _dev(conv_state_in), _dev(y), y_tok_stride,
        _dev(conv_state_out), _dev(ckpt_positions), _hp(ck_h), n_ckpt, _dev(conv_ckpt),
        _stream(stream)), "gdn_conv1d_silu_packed")


def gdn_snapshot_copy(ckpt_buf, n: int, bytes_each: int, dst_pool, dst_slot, dst_slot_host,
                      pool_slots: int, wait_event=None, copy_stream=None, done_event=None) -> None:
    """Copy n checkpoint items of bytes_each bytes into pool slots.  dst_pool is
    a device tensor, or an int device address of mapped pinned host memory.
    copy_stream first waits for wait_event; done_event is recorded on
    copy_stream after the copy."""
    sl_h = _host_i64(dst_slot_host)
    dst = dst_pool if isinstance(dst_pool, int) else _dev(dst_pool)
    _check(load().gdn_snapshot_copy(
        _dev(ckpt_buf), int(n), int(bytes_each), dst, int(pool_slots), _dev(dst_slot), _hp(sl_h),
        _event(wait_event), _stream(copy_stream), _record_target(done_event)), "gdn_snapshot_copy")
