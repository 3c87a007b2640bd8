"""ctypes binding of libmoelb.so.

Argument marshalling only: each function takes PyTorch tensors (device memory
and the current stream are all PyTorch supplies), passes their data pointers
and sizes to the C entry point of the same name, and raises ``MoelbError`` on a
non-zero status.  Every computation runs in the HIP library.  There is no CPU
fallback: if the library cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoelb.so")

MOELB_OK, MOELB_EINVAL, MOELB_ELAUNCH, MOELB_EWORKSPACE = 0, 1, 2, 3
MOELB_F32, MOELB_BF16 = 0, 1
MOELB_FFN_SCHEDULE, MOELB_FFN_GATE_UP, MOELB_FFN_DOWN, MOELB_FFN_ALL = 1, 2, 4, 7
MOELB_FFN_PACKED_WEIGHTS = 8

# name -> (restype, argtypes)
_P, _I, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "moelb_version": (_I, []),
    "moelb_status_string": (ctypes.c_char_p, [_I]),
    "moelb_gate_topk": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moelb_histogram": (_I, [_P, _I, _I, _I, _I, _P, _P, _P]),
    "moelb_plan": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "moelb_split": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P]),
    "moelb_split_variant": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "moelb_split_schedule": (_I, [_P, _P, _I, _I, _I, _P, _P]),
    "moelb_split_scheduled": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "moelb_split_stale": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P]),
    "moelb_plan_swaps": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P]),
    "moelb_permute_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "moelb_permute": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _SZ, _P, _P, _P, _P, _P]),
    "moelb_permute_noalloc": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moelb_permute_local": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P, _P, _P, _P, _P]),
    "moelb_permute_remote": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _SZ, _P, _P, _P, _P, _P]),
    "moelb_grouped_ffn_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "moelb_grouped_ffn": (_I, [_P, _I, _I, _P, _I, _I, _I, _I, _P, _I, _I, _I, _I, _P, _P, _P, _SZ, _P, _P]),
    "moelb_grouped_ffn_stages": (_I, [_I, _P, _I, _I, _P, _I, _I, _I, _I, _P, _I, _I, _I, _I, _P, _P, _P, _SZ, _P,
                                      _P]),
    "moelb_combine": (_I, [_P, _I, _P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "moelb_pack_weights": (_I, [_P, _I, _I, _I, _I, _P, _P]),
}


class MoelbError(RuntimeError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoelb.so (built in-tree by ``routed_expert_ffn_gate_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoelbError(f"{LIB_PATH} is missing: run `python -m routed_expert_ffn_gate_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def _check(status: int, name: str) -> None:
    if status != MOELB_OK:
        msg = lib().moelb_status_string(status).decode()
        raise MoelbError(f"{name} failed with status {status} ({msg})")


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise MoelbError("tensors passed to libmoelb must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOELB_BF16
    if t.dtype == torch.float32:
        return MOELB_F32
    raise MoelbError(f"unsupported dtype {t.dtype}")


def moelb_version() -> int:
    return lib().moelb_version()


def moelb_gate_topk(h, w_cur, b_cur, w_next, b_next, idx, wts, gap=None, idx_next=None, stream=None):
    T, d = h.shape
    E = w_cur.shape[0]
    k = idx.shape[1]
    _check(lib().moelb_gate_topk(_p(h), T, d, E, k, dtype_code(h), _p(w_cur), _p(b_cur), _p(w_next), _p(b_next),
                                 _p(idx), _p(wts), _p(gap), _p(idx_next), _stream(stream)), "moelb_gate_topk")


def moelb_histogram(idx, G, counts, expert_total=None, stream=None):
    T, k = idx.shape
    E = counts.shape[1]
    _check(lib().moelb_histogram(_p(idx), T, k, E, G, _p(counts), _p(expert_total), _stream(stream)),
           "moelb_histogram")


def moelb_plan(counts, home, L, replica, plan_load=None, stream=None):
    G, E = counts.shape
    N = replica.shape[1]
    _check(lib().moelb_plan(_p(counts), _p(home), G, E, N, L, _p(replica), _p(plan_load), _stream(stream)),
           "moelb_plan")


def moelb_split(counts, home, replica, host_count, load, passes=12, eps=0, stream=None):
    G, E = counts.shape
    N = replica.shape[1]
    _check(lib().moelb_split(_p(counts), _p(home), _p(replica), G, E, N, passes, eps, _p(host_count), _p(load),
                             _stream(stream)), "moelb_split")


MOELB_SPLIT_RELIEF, MOELB_SPLIT_NO_REVERSE, MOELB_SPLIT_JACOBI, MOELB_SPLIT_LIBRA_GREEDY = 0, 1, 2, 3
MOELB_SPLIT_WATER_FILL, MOELB_SPLIT_PROPORTIONAL = 4, 5


def moelb_split_variant(counts, home, replica, host_count, load, variant, passes=12, eps=0, stream=None):
    G, E = counts.shape
    N = replica.shape[1]
    _check(lib().moelb_split_variant(_p(counts), _p(home), _p(replica), G, E, N, passes, eps, variant,
                                     _p(host_count), _p(load), _stream(stream)), "moelb_split_variant")


MOELB_SPLIT_SCHEDULE_INTS = 2 + 3 * 64 * 8


def _check_schedule(schedule, name):
    if schedule is not None and schedule.numel() < MOELB_SPLIT_SCHEDULE_INTS:
        raise MoelbError(f"{name}: the schedule holds {schedule.numel()} int32, not MOELB_SPLIT_SCHEDULE_INTS")


def moelb_split_schedule(home, replica, schedule, G, stream=None):
    _check_schedule(schedule, "moelb_split_schedule")
    E = home.shape[0]
    N = replica.shape[1]
    _check(lib().moelb_split_schedule(_p(home), _p(replica), G, E, N, _p(schedule), _stream(stream)),
           "moelb_split_schedule")


def moelb_split_scheduled(counts, home, replica, schedule, host_count, load, variant=0, passes=12, eps=0,
                          stream=None):
    _check_schedule(schedule, "moelb_split_scheduled")
    G, E = counts.shape
    N = replica.shape[1]
    _check(lib().moelb_split_scheduled(_p(counts), _p(home), _p(replica), _p(schedule), G, E, N, passes, eps, variant,
                                       _p(host_count), _p(load), _stream(stream)), "moelb_split_scheduled")


def moelb_split_stale(counts, home, replica, host_count_prev, host_count, load, stream=None):
    G, E = counts.shape
    N = replica.shape[1]
    _check(lib().moelb_split_stale(_p(counts), _p(home), _p(replica), G, E, N, _p(host_count_prev), _p(host_count),
                                   _p(load), _stream(stream)), "moelb_split_stale")


def moelb_plan_swaps(counts, home, home_out, load, tau=0, gamma=(0, 1), max_swaps_per_rank=1 << 30, swaps=None,
                     n_swaps=None, stream=None):
    G, E = counts.shape
    _check(lib().moelb_plan_swaps(_p(counts), _p(home), G, E, tau, gamma[0], gamma[1], max_swaps_per_rank,
                                  _p(home_out), _p(swaps), _p(n_swaps), _p(load), _stream(stream)),
           "moelb_plan_swaps")


def moelb_permute_workspace_bytes(T, k, E, G) -> int:
    return int(lib().moelb_permute_workspace_bytes(T, k, E, G))


def moelb_permute(h, idx, G, home, replica, host_count, ws, group_off, perm, pos, x_perm=None, d=None, dtype=None,
                  stream=None):
    T, k = idx.shape
    E = home.shape[0]
    N = replica.shape[1]
    if h is not None:
        d, dtype = h.shape[1], dtype_code(h)
    _check(lib().moelb_permute(_p(h), _p(idx), T, d, k, E, G, N, dtype, _p(home), _p(replica), _p(host_count),
                               _p(ws), ws.numel() * ws.element_size(), _p(group_off), _p(perm), _p(pos), _p(x_perm),
                               _stream(stream)), "moelb_permute")


def moelb_permute_noalloc(h, idx, G, home, replica, host_count, group_off, perm, pos, x_perm=None, d=None,
                          dtype=None, stream=None):
    T, k = idx.shape
    E = home.shape[0]
    N = replica.shape[1]
    if h is not None:
        d, dtype = h.shape[1], dtype_code(h)
    _check(lib().moelb_permute_noalloc(_p(h), _p(idx), T, d, k, E, G, N, dtype, _p(home), _p(replica),
                                       _p(host_count), _p(group_off), _p(perm), _p(pos), _p(x_perm), _stream(stream)),
           "moelb_permute_noalloc")


def moelb_permute_local(h, idx, G, home, replica, ws, group_off, perm, pos, x_perm=None, d=None, dtype=None,
                        stream=None):
    T, k = idx.shape
    E = home.shape[0]
    N = replica.shape[1]
    if h is not None:
        d, dtype = h.shape[1], dtype_code(h)
    _check(lib().moelb_permute_local(_p(h), _p(idx), T, d, k, E, G, N, dtype, _p(home), _p(replica), _p(ws),
                                     ws.numel() * ws.element_size(), _p(group_off), _p(perm), _p(pos), _p(x_perm),
                                     _stream(stream)), "moelb_permute_local")


def moelb_permute_remote(h, idx, G, home, replica, host_count, ws, group_off, perm, pos, x_perm=None, d=None,
                         dtype=None, stream=None):
    T, k = idx.shape
    E = home.shape[0]
    N = replica.shape[1]
    if h is not None:
        d, dtype = h.shape[1], dtype_code(h)
    _check(lib().moelb_permute_remote(_p(h), _p(idx), T, d, k, E, G, N, dtype, _p(home), _p(replica),
                                      _p(host_count), _p(ws), ws.numel() * ws.element_size(), _p(group_off),
                                      _p(perm), _p(pos), _p(x_perm), _stream(stream)), "moelb_permute_remote")


def moelb_pack_weights(w, packed, stream=None):
    """w [E, rows, K] (or [rows, K]: one expert) bf16 -> packed (same shape and
    dtype, the packed layout)."""
    E, rows, K = (1, *w.shape) if w.dim() == 2 else w.shape
    _check(lib().moelb_pack_weights(_p(w), E, rows, K, dtype_code(w), _p(packed), _stream(stream)),
           "moelb_pack_weights")


def moelb_grouped_ffn_workspace_bytes(rows, num_groups, E, d, inter, dtype) -> int:
    return int(lib().moelb_grouped_ffn_workspace_bytes(rows, num_groups, E, d, inter, dtype))


def moelb_grouped_ffn(x, rows, group_off, E, w13, w2, ws, y, G=1, rank=-1, gather=None, gather_k=1, stream=None):
    rows_x, d = x.shape
    inter = w2.shape[-1]
    num_groups = group_off.numel() - 1
    _check(lib().moelb_grouped_ffn(_p(x), rows_x, rows, _p(group_off), num_groups, E, G, rank, _p(gather), gather_k,
                                   d, inter, dtype_code(x), _p(w13), _p(w2), _p(ws), ws.numel() * ws.element_size(),
                                   _p(y), _stream(stream)), "moelb_grouped_ffn")


def moelb_grouped_ffn_stages(stages, x, rows, group_off, E, w13, w2, ws, y, G=1, rank=-1, gather=None, gather_k=1,
                             stream=None):
    rows_x, d = x.shape
    inter = w2.shape[-1]
    num_groups = group_off.numel() - 1
    _check(lib().moelb_grouped_ffn_stages(stages, _p(x), rows_x, rows, _p(group_off), num_groups, E, G, rank,
                                          _p(gather), gather_k, d, inter, dtype_code(x), _p(w13), _p(w2), _p(ws),
                                          ws.numel() * ws.element_size(), _p(y), _stream(stream)),
           "moelb_grouped_ffn_stages")


def moelb_combine(y, pos, wts, out, shared=None, stream=None):
    T, d = out.shape
    k = wts.shape[1]
    _check(lib().moelb_combine(_p(y), y.shape[0], _p(pos), _p(wts), T, k, d, dtype_code(out), _p(shared), _p(out),
                               _stream(stream)), "moelb_combine")
