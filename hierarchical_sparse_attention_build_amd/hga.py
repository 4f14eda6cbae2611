"""ctypes binding of ``libhga.so`` (declared in ``include/hga.h``).

Argument marshalling only: every step of the method runs in the library's HIP
kernels.  Functions take torch tensors (device memory) and pass their data
pointers plus the current HIP stream; they raise ``HGAError`` when the library
returns an error.  There is no fallback: if the library is missing, the first
call raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_char_p, c_double, c_int32, c_int64, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhga.so")

HGA_BF16, HGA_F32 = 0, 1
OP_ROUTE, OP_ATTEND, OP_PREFILL, OP_DECODE, OP_DECODE_OFFLOAD, OP_PREFILL_BACKWARD = range(6)
STATUS = {0: "HGA_OK", -1: "HGA_ERR_ARG", -2: "HGA_ERR_SHAPE", -3: "HGA_ERR_ALIGN",
          -4: "HGA_ERR_WORKSPACE", -5: "HGA_ERR_UNSUPPORTED", -6: "HGA_ERR_HIP"}

EXPORTS = ("hga_workspace_size", "hga_build_summaries", "hga_route", "hga_attend", "hga_prefill",
           "hga_prefill_backward", "hga_decode", "hga_decode_static", "hga_decode_offload",
           "hga_decode_offload_warm", "hga_last_error", "hga_version")


class HGAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class HGAParams(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("chunk_size", c_int32), ("group_size", c_int32),
                ("n_sink", c_int32), ("n_local", c_int32), ("top_k", c_int32), ("top_g", c_int32),
                ("rope_base", c_double), ("hf_threshold", c_double), ("qkv_dtype", c_int32),
                ("out_dtype", c_int32)]


class HGAWarm(ctypes.Structure):
    """``hga_warm``: the warm tier's device buffers (see ``warm_state``)."""
    _fields_ = [("K", c_void_p), ("V", c_void_p), ("tags", c_void_p), ("stamps", c_void_p),
                ("clock", c_void_p), ("hits", c_void_p), ("misses", c_void_p), ("slots", c_int32)]


_lib = None


def lib():
    """The loaded library (loads it on first use; raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise HGAError(-6, f"{LIB_PATH} not found: build it with "
                               "`python -m hierarchical_sparse_attention_build_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(HGAParams)
        vp, i32, i64, sz = c_void_p, c_int32, c_int64, c_size_t
        sig = {
            "hga_workspace_size": (sz, [P, i32, i64, i64]),
            "hga_build_summaries": (i32, [P, vp, i64, i32, i32, i32, vp, vp, vp, vp]),
            "hga_route": (i32, [P, vp, i64, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp]),
            "hga_attend": (i32, [P, vp, i64, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp]),
            "hga_prefill": (i32, [P, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, sz, vp]),
            "hga_prefill_backward": (i32, [P, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, sz, vp]),
            "hga_decode": (i32, [P, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "hga_decode_static": (i32, [P, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp]),
            "hga_decode_offload": (i32, [P, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp,
                                         sz, vp, sz, vp, vp]),
            "hga_decode_offload_warm": (i32, [P, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp,
                                              ctypes.POINTER(HGAWarm), vp, sz, vp, vp]),
            "hga_last_error": (c_char_p, []),
            "hga_version": (c_char_p, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def params(batch, n_q_heads, n_kv_heads, head_dim, chunk_size, group_size, n_sink, n_local,
           top_k, top_g, rope_base=10000.0, hf_threshold=1.0, qkv_dtype=HGA_BF16,
           out_dtype=HGA_F32) -> HGAParams:
    return HGAParams(batch, n_q_heads, n_kv_heads, head_dim, chunk_size, group_size, n_sink,
                     n_local, top_k, top_g, float(rope_base), float(hf_threshold), qkv_dtype,
                     out_dtype)


def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream):
    if stream is not None:
        return c_void_p(stream)
    import torch
    return c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int):
    if status != 0:
        raise HGAError(status, lib().hga_last_error().decode())


def last_error() -> str:
    return lib().hga_last_error().decode()


def version() -> str:
    return lib().hga_version().decode()


def workspace_size(p: HGAParams, op: int, nq: int, n_cap: int) -> int:
    n = lib().hga_workspace_size(ctypes.byref(p), op, nq, n_cap)
    if n == 0 and last_error():
        raise HGAError(-1, last_error())
    return n


def workspace(p: HGAParams, op: int, nq: int, n_cap: int, device="cuda"):
    """A zero-filled workspace tensor of the size the library asks for."""
    import torch
    return torch.zeros(max(16, workspace_size(p, op, nq, n_cap)), dtype=torch.uint8, device=device)


def build_summaries(p, K, n_cap, chunk_begin, chunk_end, chunk_sum, group_sum, k_is_rotated=True,
                    K_rot_out=None, stream=None):
    _check(lib().hga_build_summaries(ctypes.byref(p), _ptr(K), n_cap, chunk_begin, chunk_end,
                                     1 if k_is_rotated else 0, _ptr(K_rot_out), _ptr(chunk_sum),
                                     _ptr(group_sum), _stream(stream)))


def route(p, Q, nq, q_pos, chunk_sum, group_sum, n_cap, chunk_idx, group_idx, ws,
          scores_out=None, stream=None):
    _check(lib().hga_route(ctypes.byref(p), _ptr(Q), nq, _ptr(q_pos), _ptr(chunk_sum),
                           _ptr(group_sum), n_cap, _ptr(chunk_idx), _ptr(group_idx),
                           _ptr(scores_out), _ptr(ws), _nbytes(ws), _stream(stream)))


def attend(p, Q, nq, q_pos, K, V, n_cap, group_idx, O, ws, lse_out=None, stream=None):
    _check(lib().hga_attend(ctypes.byref(p), _ptr(Q), nq, _ptr(q_pos), _ptr(K), _ptr(V), n_cap,
                            _ptr(group_idx), _ptr(O), _ptr(lse_out), _ptr(ws), _nbytes(ws),
                            _stream(stream)))


def prefill(p, Q, K, V, n, chunk_sum, group_sum, O, ws, chunk_idx=None, group_idx=None,
            stream=None):
    _check(lib().hga_prefill(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), n, _ptr(chunk_sum),
                             _ptr(group_sum), _ptr(O), _ptr(chunk_idx), _ptr(group_idx),
                             _ptr(ws), _nbytes(ws), _stream(stream)))


def prefill_backward(p, Q, K, V, n, group_idx, dO, dQ, dK, dV, ws, stream=None):
    """hga_prefill_backward: dQ, dK, dV (float32) of the prefill attention for dO."""
    _check(lib().hga_prefill_backward(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), n, _ptr(group_idx),
                                      _ptr(dO), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(ws), _nbytes(ws),
                                      _stream(stream)))


def decode(p, Q, K, V, n_cap, seq_len, chunk_sum, group_sum, O, ws, chunk_idx=None,
           group_idx=None, stream=None):
    _check(lib().hga_decode(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), n_cap, _ptr(seq_len),
                            _ptr(chunk_sum), _ptr(group_sum), _ptr(O), _ptr(chunk_idx),
                            _ptr(group_idx), _ptr(ws), _nbytes(ws), _stream(stream)))


def decode_static(p, Q, K, V, n_cap, seq_len, chunk_sum, group_sum, O, chunk_idx=None,
                  group_idx=None, stream=None):
    """``hga_decode_static``: hga_decode with the library's static device scratch
    (no workspace argument)."""
    _check(lib().hga_decode_static(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), n_cap, _ptr(seq_len),
                                   _ptr(chunk_sum), _ptr(group_sum), _ptr(O), _ptr(chunk_idx),
                                   _ptr(group_idx), _stream(stream)))


def decode_offload(p, Q, K_host, V_host, K_hot, V_hot, n_cap, seq_len, chunk_sum, group_sum, O,
                   staging, ws, chunk_idx=None, group_idx=None, stream=None, copy_stream=None):
    if copy_stream is None:
        raise HGAError(-1, "decode_offload needs a copy stream")
    _check(lib().hga_decode_offload(ctypes.byref(p), _ptr(Q), _ptr(K_host), _ptr(V_host),
                                    _ptr(K_hot), _ptr(V_hot), n_cap, _ptr(seq_len),
                                    _ptr(chunk_sum), _ptr(group_sum), _ptr(O), _ptr(chunk_idx),
                                    _ptr(group_idx), _ptr(staging), _nbytes(staging), _ptr(ws),
                                    _nbytes(ws), _stream(stream), c_void_p(copy_stream)))


def warm_state(p, slots: int, device="cuda"):
    """Fresh warm-tier buffers for ``slots`` groups per (b, kv head): K and V
    rows, tags (-1), stamps (0), clock (0) and the per-step hit and miss counts."""
    import torch
    B, H, G, d = p.batch, p.n_kv_heads, p.group_size, p.head_dim
    dt = torch.bfloat16 if p.qkv_dtype == HGA_BF16 else torch.float32
    i32 = dict(dtype=torch.int32, device=device)
    return {"K": torch.zeros((B, H, slots, G, d), dtype=dt, device=device),
            "V": torch.zeros((B, H, slots, G, d), dtype=dt, device=device),
            "tags": torch.full((B, H, slots), -1, **i32), "stamps": torch.zeros((B, H, slots), **i32),
            "clock": torch.zeros((B, H), **i32), "hits": torch.zeros((B, H), **i32),
            "misses": torch.zeros((B, H), **i32), "slots": slots}


def decode_offload_warm(p, Q, K_host, V_host, K_hot, V_hot, n_cap, seq_len, chunk_sum, group_sum, O,
                        warm, ws, chunk_idx=None, group_idx=None, stream=None, copy_stream=None):
    """hga_decode_offload_warm; ``warm`` is a dict from ``warm_state``.  The
    library does not use ``copy_stream`` for the warm tier (it may be None)."""
    w = HGAWarm(_ptr(warm["K"]), _ptr(warm["V"]), _ptr(warm["tags"]), _ptr(warm["stamps"]),
                _ptr(warm["clock"]), _ptr(warm.get("hits")), _ptr(warm.get("misses")), warm["slots"])
    _check(lib().hga_decode_offload_warm(ctypes.byref(p), _ptr(Q), _ptr(K_host), _ptr(V_host),
                                         _ptr(K_hot), _ptr(V_hot), n_cap, _ptr(seq_len),
                                         _ptr(chunk_sum), _ptr(group_sum), _ptr(O), _ptr(chunk_idx),
                                         _ptr(group_idx), ctypes.byref(w), _ptr(ws), _nbytes(ws),
                                         _stream(stream), c_void_p(copy_stream)))


def hot_slot(c: int, n_sink: int, n_local: int) -> int:
    """Slot of chunk c in the hot-window buffer of decode_offload (layout of hga.h)."""
    return c if c < n_sink else n_sink + (c - n_sink) % (n_local + 1)
