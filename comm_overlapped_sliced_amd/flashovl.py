"""ctypes binding of libflashovl (argument marshalling only).

Every entry point of ``include/flashovl.h`` is exposed under the same name without the ``fo_``
prefix. Tensors are torch device tensors (torch provides device memory and streams only); the
computation runs entirely in the library's HIP kernels and its DMA transfers. If the library is
missing this module raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libflashovl.so")

FO_OK, FO_ERR_INVALID_ARG, FO_ERR_UNSUPPORTED, FO_ERR_HIP, FO_ERR_TIMEOUT = range(5)
BF16, F32 = 0, 1
ORDER_FLASH, ORDER_NATURAL = 0, 1
ARR_DEFAULT, ARR_NONE, ARR_EAGER, ARR_LOCKSTEP = 0, 1, 2, 3
TILE_AUTO, TILE_256x256, TILE_256x128, TILE_128x256, TILE_128x128, TILE_64x64 = range(6)
EPI_NONE, EPI_SWIGLU = 0, 1
MAX_P = 32
MAX_GROUPS = 8

EXPORTS = ("fo_opts_init", "fo_ag_gemm", "fo_gemm_rs", "fo_gemm_rs_noalloc", "fo_gemm_ref",
           "fo_swiglu", "fo_attn",
           "fo_attn_ref",
           "fo_transfer_ref", "fo_check", "fo_slice_order", "fo_tile_info", "fo_tile_order",
           "fo_attn_schedule",
           "fo_status_str", "fo_last_error", "fo_version")


class FoError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {_status_name(status)}: {detail}")


class Opts(ctypes.Structure):
    _fields_ = [("order", ctypes.c_int32), ("arrival", ctypes.c_int32),
                ("tile", ctypes.c_int32), ("spin_timeout_us", ctypes.c_uint32),
                ("links", ctypes.c_int32), ("row_groups", ctypes.c_int32),
                ("kernel_events", ctypes.c_void_p * 2), ("epilogue", ctypes.c_int32),
                ("k_chunks", ctypes.c_int32), ("engines_per_link", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_lib = None


def load():
    """Open libflashovl.so (after torch, so that both use the same HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    try:
        import torch  # noqa: F401  (load torch's HIP runtime first so there is only one)
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    op = ctypes.POINTER(Opts)
    lib.fo_opts_init.argtypes = [op]
    lib.fo_opts_init.restype = None
    lib.fo_ag_gemm.argtypes = [vp, vp, vp, vp, vp, i32, i32, i64, i64, i64, i32, i32, vp, op]
    lib.fo_gemm_rs.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i64, i64, i64, i32, vp, op]
    lib.fo_gemm_rs_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i64, i64, i64, i32, vp, op]
    lib.fo_gemm_ref.argtypes = [vp, vp, vp, i64, i64, i64, i32, i32, i32, vp]
    lib.fo_swiglu.argtypes = [vp, vp, i64, i64, vp]
    lib.fo_attn.argtypes = [vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, i32, i32, vp, op]
    lib.fo_attn_ref.argtypes = [vp, vp, i64, i32, i32, i32, i32, vp]
    lib.fo_transfer_ref.argtypes = [i32, vp, vp, i32, i32, i64, vp, op]
    lib.fo_check.argtypes = [vp]
    lib.fo_slice_order.argtypes = [i32, i32, i32, i32, ctypes.POINTER(i32)]
    lib.fo_tile_info.argtypes = [i32, i64, i64, i64, i32, i32, i32, ctypes.POINTER(i32),
                                 ctypes.POINTER(i32), ctypes.POINTER(i64)]
    lib.fo_attn_schedule.argtypes = [i32, i64, i32, i32, ctypes.POINTER(i32), i64,
                                     ctypes.POINTER(i64), ctypes.POINTER(i32)]
    lib.fo_tile_order.argtypes = [i32, i32, i64, i64, i64, i32, i32, op, ctypes.POINTER(i32), i64,
                                  ctypes.POINTER(i64)]
    lib.fo_status_str.argtypes = [i32]
    lib.fo_status_str.restype = ctypes.c_char_p
    lib.fo_last_error.argtypes = []
    lib.fo_last_error.restype = ctypes.c_char_p
    lib.fo_version.argtypes = []
    for f in ("fo_ag_gemm", "fo_gemm_rs", "fo_gemm_rs_noalloc", "fo_gemm_ref", "fo_swiglu",
              "fo_attn", "fo_attn_ref",
              "fo_transfer_ref", "fo_check",
              "fo_slice_order", "fo_tile_info", "fo_tile_order", "fo_attn_schedule",
              "fo_version"):
        getattr(lib, f).restype = ctypes.c_int32
    _lib = lib
    return lib


def _status_name(s: int) -> str:
    try:
        return load().fo_status_str(s).decode()
    except Exception:  # noqa: BLE001
        return str(s)


def _raise_on(status: int, where: str) -> None:
    if status != FO_OK:
        raise FoError(status, where, load().fo_last_error().decode())


_default_engines_per_link = 0


def set_default_engines_per_link(n: int) -> None:
    """The engines_per_link that opts() fills in when none is given (0: the library's)."""
    global _default_engines_per_link
    _default_engines_per_link = int(n)


def opts(order=ORDER_FLASH, arrival=ARR_DEFAULT, tile=TILE_AUTO, spin_timeout_us=0, links=0,
         row_groups=0, kernel_events=None, epilogue=EPI_NONE, k_chunks=0,
         engines_per_link=None) -> Opts:
    o = Opts()
    load().fo_opts_init(ctypes.byref(o))
    o.order, o.arrival, o.tile, o.links = order, arrival, tile, links
    o.row_groups, o.epilogue, o.k_chunks = row_groups, epilogue, k_chunks
    o.engines_per_link = (_default_engines_per_link if engines_per_link is None
                          else engines_per_link)
    if spin_timeout_us:
        o.spin_timeout_us = spin_timeout_us
    if kernel_events is not None:
        o.kernel_events[0] = _event(kernel_events[0])
        o.kernel_events[1] = _event(kernel_events[1])
    return o


def _event(e) -> int | None:
    """hipEvent_t of a torch.cuda.Event (or a raw handle)."""
    if e is None or isinstance(e, int):
        return e
    return e.cuda_event


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s) -> int | None:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _dt(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr_array(ptrs):
    arr = (ctypes.c_void_p * len(ptrs))()
    for i, p in enumerate(ptrs):
        arr[i] = _ptr(p)
    return arr


def ag_gemm(x_local, x_peer, x_recv, w, y, P: int, rank: int, compute_stream=None,
            o: Opts | None = None, raw: bool = False):
    """Flash-AG (fo_ag_gemm). x_local [m, K], x_peer list of P tensors (or None), x_recv
    [P*m, K], w [K, N], y [P*m, N] ([P*m, N/2] with the SwiGLU epilogue). With o.k_chunks = c > 1
    every X slice holds its m*K values in the K-block layout (c blocks [m, K/c] one after
    another; the shapes passed stay [m, K]). Returns the status when raw=True, else raises on
    error."""
    m, K = x_local.shape
    N = w.shape[1]
    peers = None if x_peer is None else _ptr_array(x_peer)
    st = load().fo_ag_gemm(_ptr(x_local), ctypes.cast(peers, ctypes.c_void_p) if peers else None,
                           _ptr(x_recv), _ptr(w), _ptr(y), P, rank, m, K, N, _dt(x_local),
                           _dt(y), _stream(compute_stream),
                           ctypes.byref(o) if o is not None else None)
    if raw:
        return st
    _raise_on(st, "fo_ag_gemm")
    return st


def gemm_rs(x_shard, w, send_buf, out, peer_partial, recv_buf, P: int, rank: int,
            compute_stream=None, o: Opts | None = None, raw: bool = False):
    """Flash-RS (fo_gemm_rs). x_shard [P*m, K], w [K, N], send_buf [P*m, N] fp32, out [m, N]
    fp32, peer_partial list of P fp32 [m, N] tensors (or None), recv_buf [P*m, N] fp32."""
    M, K = x_shard.shape
    N = w.shape[1]
    m = M // P
    peers = None if peer_partial is None else _ptr_array(peer_partial)
    st = load().fo_gemm_rs(_ptr(x_shard), _ptr(w), _ptr(send_buf), _ptr(out),
                           ctypes.cast(peers, ctypes.c_void_p) if peers else None,
                           _ptr(recv_buf), P, rank, m, K, N, _dt(x_shard),
                           _stream(compute_stream),
                           ctypes.byref(o) if o is not None else None)
    if raw:
        return st
    _raise_on(st, "fo_gemm_rs")
    return st


def gemm_rs_noalloc(x_shard, w, send_buf, out, recv_buf, P: int, rank: int, compute_stream=None,
                    o: Opts | None = None, raw: bool = False):
    """Flash-RS with the partials resident in recv_buf, allocating nothing (fo_gemm_rs_noalloc);
    the tensors as for gemm_rs."""
    M, K = x_shard.shape
    N = w.shape[1]
    m = M // P
    st = load().fo_gemm_rs_noalloc(_ptr(x_shard), _ptr(w), _ptr(send_buf), _ptr(out),
                                   _ptr(recv_buf), P, rank, m, K, N, _dt(x_shard),
                                   _stream(compute_stream),
                                   ctypes.byref(o) if o is not None else None)
    if raw:
        return st
    _raise_on(st, "fo_gemm_rs_noalloc")
    return st


def gemm_ref(a, b, c, tile: int = TILE_AUTO, stream=None, raw: bool = False):
    """Monolithic C = A . B (fo_gemm_ref)."""
    M, K = a.shape
    N = b.shape[1]
    st = load().fo_gemm_ref(_ptr(a), _ptr(b), _ptr(c), M, K, N, _dt(a), _dt(c), tile,
                            _stream(stream))
    if raw:
        return st
    _raise_on(st, "fo_gemm_ref")
    return st


def swiglu(y, h, stream=None, raw: bool = False):
    """h = silu(y[:, :inter]) * y[:, inter:] (fo_swiglu); y [rows, 2*inter] bf16, h [rows, inter]
    bf16."""
    rows, inter = h.shape
    st = load().fo_swiglu(_ptr(y), _ptr(h), rows, inter, _stream(stream))
    if raw:
        return st
    _raise_on(st, "fo_swiglu")
    return st


def transfer_ref(kind: str, src, dst, P: int, rank: int, slice_bytes: int, stream=None,
                 o: Opts | None = None, raw: bool = False):
    """The emulated transfers of one call alone (fo_transfer_ref)."""
    arr = _ptr_array(src)
    st = load().fo_transfer_ref(0 if kind == "ag" else 1, ctypes.cast(arr, ctypes.c_void_p),
                                _ptr(dst), P, rank, slice_bytes, _stream(stream),
                                ctypes.byref(o) if o is not None else None)
    if raw:
        return st
    _raise_on(st, "fo_transfer_ref")
    return st


def check(stream=None) -> int:
    """fo_check: synchronize, wait for the DMA transfers, report wait timeouts and failed copies
    (raises FoError)."""
    st = load().fo_check(_stream(stream))
    _raise_on(st, "fo_check")
    return st


def slice_order(kind: str, P: int, rank: int, order: int = ORDER_FLASH) -> list:
    out = (ctypes.c_int32 * P)()
    st = load().fo_slice_order(0 if kind == "ag" else 1, order, P, rank, out)
    _raise_on(st, "fo_slice_order")
    return list(out)


def tile_info(P: int, m: int, K: int, N: int, in_dt: int = BF16, tile: int = TILE_AUTO,
              out_dt: int = BF16):
    """Tile rows, tile columns and workgroups of one call (fo_tile_info); out_dt F32 for RS."""
    bm, bn, wg = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    st = load().fo_tile_info(P, m, K, N, in_dt, out_dt, tile, ctypes.byref(bm), ctypes.byref(bn),
                             ctypes.byref(wg))
    _raise_on(st, "fo_tile_info")
    return bm.value, bn.value, wg.value


def attn_schedule(P: int, m: int, hq: int, n_cu: int):
    """Work lists of a causal attention launch (fo_attn_schedule): a list of (workgroup, slice,
    query tile, head, w) entries in launch order, and the number of workgroups."""
    lib = load()
    cnt, wgs = ctypes.c_int64(), ctypes.c_int32()
    _raise_on(lib.fo_attn_schedule(P, m, hq, n_cu, None, 0, ctypes.byref(cnt), ctypes.byref(wgs)),
              "fo_attn_schedule")
    buf = (ctypes.c_int32 * max(1, 5 * cnt.value))()
    _raise_on(lib.fo_attn_schedule(P, m, hq, n_cu, buf, cnt.value, ctypes.byref(cnt),
                                   ctypes.byref(wgs)), "fo_attn_schedule")
    return [tuple(buf[5 * i:5 * i + 5]) for i in range(cnt.value)], wgs.value


def tile_order(kind: str, P: int, m: int, K: int, N: int, in_dt: int = BF16,
               o: Opts | None = None, out_dt: int = BF16):
    """Dispatch order of one call: a list of (position, row group, tile row, tile column) per
    workgroup (fo_tile_order)."""
    lib = load()
    cnt = ctypes.c_int64()
    k = 0 if kind == "ag" else 1
    ob = ctypes.byref(o) if o is not None else None
    _raise_on(lib.fo_tile_order(k, P, m, K, N, in_dt, out_dt, ob, None, 0, ctypes.byref(cnt)),
              "fo_tile_order")
    buf = (ctypes.c_int32 * (4 * cnt.value))()
    _raise_on(lib.fo_tile_order(k, P, m, K, N, in_dt, out_dt, ob, buf, cnt.value,
                                ctypes.byref(cnt)), "fo_tile_order")
    return [tuple(buf[4 * i:4 * i + 4]) for i in range(cnt.value)]


def version() -> int:
    return int(load().fo_version())


def runtimes_mapped(name: str = "libamdhip64") -> set:
    """Paths of the runtime library `name` (libamdhip64, libhsa-runtime64) mapped into this
    process (one of each expected)."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if name in line:
                paths.add(os.path.realpath(line.split()[-1]))
    return paths


def attn(qkv_local, qkv_peer, qkv_recv, out, P: int, rank: int, hq: int, hkv: int,
         causal: bool = True, compute_stream=None, o: Opts | None = None, raw: bool = False,
         out_peer=None):
    """Query-split attention between the two Flash All-to-Alls (fo_attn). qkv_local
    [m, (hq+2hkv)*128] bf16, qkv_peer list of P tensors (or None), qkv_recv [P*m, same], out
    [P*m, hq*128] bf16, out_peer list of P [m, hq*128] bf16 tensors receiving each slice's rows
    (entry [rank] unused; None: no return exchange)."""
    m, row = qkv_local.shape
    d = row // (hq + 2 * hkv)
    peers = None if qkv_peer is None else _ptr_array(qkv_peer)
    outs = None if out_peer is None else _ptr_array(out_peer)
    st = load().fo_attn(_ptr(qkv_local), ctypes.cast(peers, ctypes.c_void_p) if peers else None,
                        _ptr(qkv_recv), _ptr(out),
                        ctypes.cast(outs, ctypes.c_void_p) if outs else None, P, rank, m, hq, hkv,
                        d, int(causal), _stream(compute_stream),
                        ctypes.byref(o) if o is not None else None)
    if raw:
        return st
    _raise_on(st, "fo_attn")
    return st


def attn_ref(qkv, out, hq: int, hkv: int, causal: bool = True, stream=None, raw: bool = False):
    """The same attention on one resident sequence (fo_attn_ref): qkv [S, (hq+2hkv)*128] bf16,
    out [S, hq*128] bf16."""
    S, row = qkv.shape
    d = row // (hq + 2 * hkv)
    st = load().fo_attn_ref(_ptr(qkv), _ptr(out), S, hq, hkv, d, int(causal), _stream(stream))
    if raw:
        return st
    _raise_on(st, "fo_attn_ref")
    return st
