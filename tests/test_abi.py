"""CPU tests of the C ABI boundary: the library loads without a GPU, exports every entry point
its header declares, implements the slice schedule of the FlashOverlap page, and rejects bad
arguments before touching the device."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import oracle
from comm_overlapped_sliced_amd import flashovl as fo

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashovl.h")


@pytest.fixture(scope="module")
def lib():
    return fo.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fo_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"{n} declared in flashovl.h but not exported"
    assert set(names) == set(fo.EXPORTS)


def test_version_and_status_strings(lib):
    assert fo.version() == 1
    for s, name in enumerate(["FO_OK", "FO_ERR_INVALID_ARG", "FO_ERR_UNSUPPORTED", "FO_ERR_HIP",
                              "FO_ERR_TIMEOUT"]):
        assert lib.fo_status_str(s).decode() == name
    assert lib.fo_status_str(99).decode() == "FO_ERR_UNKNOWN"


def test_opts_defaults():
    o = fo.opts()
    assert (o.order, o.arrival, o.tile, o.links) == (0, 0, 0, 0)
    assert o.spin_timeout_us == 2_000_000
    assert list(o.kernel_events) == [None, None]
    assert o.row_groups == 0 and o.epilogue == fo.EPI_NONE and o.k_chunks == 0
    assert ctypes.sizeof(fo.Opts) == 56
    # the C layout: after the events, the epilogue, k_chunks, engines_per_link and a reserved word
    assert fo.Opts.kernel_events.offset == 24 and fo.Opts.epilogue.offset == 40
    assert fo.Opts.k_chunks.offset == 44 and fo.Opts.engines_per_link.offset == 48
    assert fo.Opts.reserved.offset == 52 and o.engines_per_link == 0 and o.reserved == 0
    assert fo.opts(k_chunks=4).k_chunks == 4


@pytest.mark.parametrize("P", list(range(1, 33)))
def test_slice_orders_follow_the_page(P):
    for r in range(P):
        ag = fo.slice_order("ag", P, r)
        rs = fo.slice_order("rs", P, r)
        assert ag[0] == r and sorted(ag) == list(range(P))     # local slice first
        assert rs[-1] == r and sorted(rs) == list(range(P))    # own chunk last
        assert ag == oracle.ag_order(P, r)
        assert rs == oracle.rs_order(P, r)
        assert fo.slice_order("ag", P, r, fo.ORDER_NATURAL) == list(range(P))
    for i in range(P - 1):  # every RS step is a derangement over the ranks
        tgt = [fo.slice_order("rs", P, r)[i] for r in range(P)]
        assert sorted(tgt) == list(range(P)) and all(t != r for r, t in enumerate(tgt))


def test_slice_order_rejects(lib):
    out = (ctypes.c_int32 * 4)()
    assert lib.fo_slice_order(2, 0, 4, 0, out) == fo.FO_ERR_INVALID_ARG
    assert lib.fo_slice_order(0, 0, 0, 0, out) == fo.FO_ERR_INVALID_ARG
    assert lib.fo_slice_order(0, 0, 4, 4, out) == fo.FO_ERR_INVALID_ARG
    assert lib.fo_slice_order(0, 7, 4, 0, out) == fo.FO_ERR_INVALID_ARG
    assert lib.fo_slice_order(0, 0, 33, 0, out) == fo.FO_ERR_INVALID_ARG


def test_tile_choice_for_the_workloads():
    # Tiles never cross a slice; 256x256 unless a rule below applies.
    assert fo.tile_info(8, 512, 8192, 7168)[:2] == (256, 256)    # 70B gate+up
    # 70B down in Flash-RS (fp32 out, K = 3584): transfer-bound, finer tiles release sooner
    assert fo.tile_info(8, 512, 3584, 8192, out_dt=fo.F32)[:2] == (128, 256)
    assert fo.tile_info(8, 512, 3584, 8192)[:2] == (256, 256)    # the same with bf16 out
    assert fo.tile_info(1, 4096, 3584, 8192, out_dt=fo.F32)[:2] == (256, 256)  # monolithic
    # 405B
    assert fo.tile_info(8, 1024, 16384, 13312)[:2] == (256, 256)
    assert fo.tile_info(8, 1024, 6656, 16384, out_dt=fo.F32)[:2] == (256, 256)
    # 70B gate+up sweep, M = 2048 .. 16384
    for m in (256, 512, 1024, 2048):
        assert fo.tile_info(8, m, 8192, 7168)[:2] == (256, 256)
    bm, bn, wg = fo.tile_info(8, 128, 8192, 7168)       # M = 1024: slices of 128 rows
    assert (bm, bn) == (128, 256) and wg == 8 * 28
    assert fo.tile_info(8, 512, 8192, 200)[:2] == (256, 128)
    assert fo.tile_info(4, 64, 256, 512, fo.F32)[:2] == (64, 64)
    assert fo.tile_info(8, 512, 8192, 7168, fo.BF16, fo.TILE_128x128) == (128, 128, 8 * 4 * 56)


# --- argument checks: all rejected before any HIP call (no GPU in this container) ---------

A = 0x10000000   # fake, 16-byte aligned addresses that are never dereferenced
B = 0x20000000
C = 0x30000000
D = 0x40000000


def _ag(lib, **kw):
    args = dict(x_local=A, x_peer=None, x_recv=B, w=C, y=D, P=4, rank=0, m=64, K=256, N=512,
                in_dt=fo.BF16, out_dt=fo.BF16, cs=None, opts=None)
    args.update(kw)
    peers = args["x_peer"]
    if peers is not None:
        arr = (ctypes.c_void_p * len(peers))(*peers)
        peers = ctypes.cast(arr, ctypes.c_void_p)
    return lib.fo_ag_gemm(args["x_local"], peers, args["x_recv"], args["w"], args["y"], args["P"],
                          args["rank"], args["m"], args["K"], args["N"], args["in_dt"],
                          args["out_dt"], args["cs"], args["opts"])


@pytest.mark.parametrize("kw", [
    dict(P=0), dict(P=33), dict(rank=4), dict(rank=-1), dict(m=-1), dict(K=-8),
    dict(K=260), dict(N=500), dict(in_dt=5), dict(out_dt=2), dict(x_local=None), dict(w=None),
    dict(K=(1 << 21) + 8), dict(N=(1 << 20) + 8),  # past the kernel's 31-bit tile offsets
    dict(y=None), dict(x_recv=None), dict(x_local=A + 2), dict(w=C + 8), dict(y=D + 1),
    dict(y=A),                                   # output overlaps the local slice
    dict(y=B + 4096),                            # output overlaps the receive buffer
    dict(x_peer=[0x50000000, None, 0x60000000, 0x70000000], rank=0),  # a peer missing
    dict(x_peer=[0x50000000, B, 0x60000000, 0x70000000], rank=0),     # peer inside x_recv
])
def test_ag_rejects(lib, kw):
    assert _ag(lib, **kw) == fo.FO_ERR_INVALID_ARG
    assert lib.fo_last_error().decode() != ""


def test_bad_engines_per_link_and_reserved_rejected(lib):
    for kw in (dict(engines_per_link=4), dict(engines_per_link=-1), dict(reserved=1)):
        o = fo.opts()
        for k, v in kw.items():
            setattr(o, k, v)
        assert _rs(lib, opts=ctypes.byref(o)) == fo.FO_ERR_INVALID_ARG, kw
        assert _attn(lib, opts=ctypes.byref(o)) == fo.FO_ERR_INVALID_ARG, kw


def test_ag_rejects_bad_opts(lib):
    for field, val in [("order", 9), ("arrival", 7), ("tile", 11), ("links", 33), ("links", -1),
                       ("row_groups", 9), ("row_groups", -1), ("epilogue", 2),
                       ("epilogue", -1), ("k_chunks", 9), ("k_chunks", -1)]:
        o = fo.opts()
        setattr(o, field, val)
        assert _ag(lib, opts=ctypes.byref(o)) == fo.FO_ERR_INVALID_ARG
    o = fo.opts(arrival=fo.ARR_LOCKSTEP)
    assert _ag(lib, opts=ctypes.byref(o)) == fo.FO_ERR_INVALID_ARG


def test_ag_k_chunks_unsupported_shapes(lib):
    # K-chunk-major slices: bf16 only, K a multiple of 256 per chunk, slices of at most 2^30 bytes
    o = ctypes.byref(fo.opts(k_chunks=2))
    assert _ag(lib, opts=o, K=256) == fo.FO_ERR_UNSUPPORTED          # 128 columns per chunk
    assert _ag(lib, opts=o, K=768) == fo.FO_ERR_UNSUPPORTED          # 384 columns per chunk
    assert _ag(lib, opts=o, K=512, in_dt=fo.F32, out_dt=fo.F32) == fo.FO_ERR_UNSUPPORTED
    assert _ag(lib, opts=o, m=65536, K=16384) == fo.FO_ERR_UNSUPPORTED  # 2^31-byte slices
    assert "k_chunks" in lib.fo_last_error().decode()


def test_k_chunks_only_for_ag(lib):
    o = ctypes.byref(fo.opts(k_chunks=2))
    assert _rs(lib, opts=o, K=512) == fo.FO_ERR_INVALID_ARG
    assert _attn(lib, opts=o) == fo.FO_ERR_INVALID_ARG
    # 0 and 1 both mean row-major, accepted everywhere
    for c in (0, 1):
        o = ctypes.byref(fo.opts(k_chunks=c))
        assert _rs(lib, opts=o, m=0) == fo.FO_OK
        assert _attn(lib, opts=o, m=0) == fo.FO_OK


def test_ag_swiglu_epilogue_rejects(lib):
    # the fused SwiGLU write-back needs bf16 in and out and N a multiple of 16
    o = ctypes.byref(fo.opts(epilogue=fo.EPI_SWIGLU))
    assert _ag(lib, opts=o, out_dt=fo.F32) == fo.FO_ERR_INVALID_ARG
    assert _ag(lib, opts=o, in_dt=fo.F32, out_dt=fo.F32) == fo.FO_ERR_INVALID_ARG
    assert _ag(lib, opts=o, N=520) == fo.FO_ERR_INVALID_ARG
    assert "SwiGLU" in lib.fo_last_error().decode()
    # y is [P*m, N/2] bf16: one that reaches into x_recv is rejected; m = 0 is a no-op
    half = 4 * 64 * 256 * 2
    assert _ag(lib, opts=o, y=B - half + 16) == fo.FO_ERR_INVALID_ARG
    assert _ag(lib, opts=o, m=0) == fo.FO_OK
    assert _rs(lib, opts=o) == fo.FO_ERR_INVALID_ARG
    src = (ctypes.c_void_p * 4)(0x50000000, 0x60000000, 0x70000000, 0x78000000)
    assert lib.fo_transfer_ref(0, ctypes.cast(src, ctypes.c_void_p), B, 4, 0, 4096, None,
                               o) == fo.FO_ERR_INVALID_ARG


def test_ag_empty_is_a_no_op(lib):
    # m = 0 or N = 0: valid, nothing to compute, nothing enqueued
    assert _ag(lib, m=0) == fo.FO_OK
    assert _ag(lib, N=0) == fo.FO_OK


def _rs(lib, **kw):
    args = dict(x=A, w=B, send=C, out=D, peers=None, recv=0x50000000, P=4, rank=1, m=64, K=256,
                N=512, in_dt=fo.BF16, opts=None)
    args.update(kw)
    peers = args["peers"]
    if peers is not None:
        arr = (ctypes.c_void_p * len(peers))(*peers)
        peers = ctypes.cast(arr, ctypes.c_void_p)
    return lib.fo_gemm_rs(args["x"], args["w"], args["send"], args["out"], peers, args["recv"],
                          args["P"], args["rank"], args["m"], args["K"], args["N"], args["in_dt"],
                          None, args["opts"])


@pytest.mark.parametrize("kw", [
    dict(P=0), dict(rank=4), dict(N=12), dict(K=7), dict(x=None), dict(out=None),
    dict(send=None), dict(recv=None), dict(out=A), dict(send=B), dict(out=0x50000000),
    dict(send=D - 4), dict(x=A + 4), dict(out=D + 2),
    dict(peers=[0x60000000, 0x70000000, None, 0x78000000]),
    dict(peers=[0x60000000, 0x70000000, 0x50000000, 0x78000000]),  # peer inside recv_buf
])
def test_rs_rejects(lib, kw):
    assert _rs(lib, **kw) == fo.FO_ERR_INVALID_ARG


def test_rs_bad_order_rejected(lib):
    o = fo.opts(order=fo.ORDER_NATURAL)
    o.order = 5
    assert _rs(lib, opts=ctypes.byref(o)) == fo.FO_ERR_INVALID_ARG


def test_transfer_ref_rejects(lib):
    src = (ctypes.c_void_p * 4)(0x50000000, 0x60000000, 0x70000000, 0x78000000)
    ps = ctypes.cast(src, ctypes.c_void_p)
    assert lib.fo_transfer_ref(2, ps, B, 4, 0, 4096, None, None) == fo.FO_ERR_INVALID_ARG
    assert lib.fo_transfer_ref(0, ps, B, 4, 4, 4096, None, None) == fo.FO_ERR_INVALID_ARG
    assert lib.fo_transfer_ref(0, ps, B, 4, 0, 4098, None, None) == fo.FO_ERR_INVALID_ARG
    assert lib.fo_transfer_ref(0, None, B, 4, 0, 4096, None, None) == fo.FO_ERR_INVALID_ARG
    assert lib.fo_transfer_ref(0, ps, 0x60000000 - 8192, 4, 0, 4096, None, None) == fo.FO_ERR_INVALID_ARG
    assert lib.fo_transfer_ref(0, ps, B, 4, 0, 0, None, None) == fo.FO_OK


def test_ref_rejects(lib):
    assert lib.fo_gemm_ref(A, B, C, 64, 256, 500, fo.BF16, fo.BF16, 0, None) == fo.FO_ERR_INVALID_ARG
    assert lib.fo_gemm_ref(A, B, A, 64, 256, 512, fo.BF16, fo.BF16, 0, None) == fo.FO_ERR_INVALID_ARG
    assert lib.fo_gemm_ref(A, B, C, 64, 256, 512, fo.BF16, fo.BF16, 9, None) == fo.FO_ERR_INVALID_ARG
    assert lib.fo_gemm_ref(A, B, C, 64, 256, (1 << 20) + 8, fo.BF16, fo.BF16, 0, None) == fo.FO_ERR_INVALID_ARG
    assert lib.fo_gemm_ref(None, B, C, 64, 256, 512, fo.BF16, fo.BF16, 0, None) == fo.FO_ERR_INVALID_ARG
    assert lib.fo_gemm_ref(A, B, C, 0, 256, 512, fo.BF16, fo.BF16, 0, None) == fo.FO_OK


def test_swiglu_rejects(lib):
    assert lib.fo_swiglu(A, C, 64, 100, None) == fo.FO_ERR_INVALID_ARG   # inter % 8
    assert lib.fo_swiglu(A + 2, C, 64, 128, None) == fo.FO_ERR_INVALID_ARG  # misaligned
    assert lib.fo_swiglu(None, C, 64, 128, None) == fo.FO_ERR_INVALID_ARG
    assert lib.fo_swiglu(A, A + 4096, 64, 128, None) == fo.FO_ERR_INVALID_ARG  # h inside y
    assert lib.fo_swiglu(A, C, -1, 128, None) == fo.FO_ERR_INVALID_ARG
    assert lib.fo_swiglu(A, C, 0, 128, None) == fo.FO_OK  # nothing to do


def _attn(lib, **kw):
    args = dict(local=A, peers=None, recv=B, out=C, out_peer=None, P=4, rank=0, m=64, hq=8,
                hkv=2, d=128, causal=1, opts=None)
    args.update(kw)

    def arr(ptrs):
        if ptrs is None:
            return None
        a = (ctypes.c_void_p * len(ptrs))(*ptrs)
        return ctypes.cast(a, ctypes.c_void_p)

    return lib.fo_attn(args["local"], arr(args["peers"]), args["recv"], args["out"],
                       arr(args["out_peer"]), args["P"], args["rank"], args["m"], args["hq"],
                       args["hkv"], args["d"], args["causal"], None, args["opts"])


@pytest.mark.parametrize("kw", [dict(hq=6, hkv=4), dict(hq=0), dict(hkv=0), dict(causal=2),
                                dict(m=-1), dict(P=0), dict(rank=4), dict(local=0),
                                dict(out=0), dict(recv=0), dict(out=A + 8), dict(local=A + 4),
                                dict(out=B + 64),  # out overlaps qkv_recv
                                dict(m=1 << 22)],
                         ids=lambda k: ",".join(f"{a}={b}" for a, b in k.items()))
def test_attn_rejects(lib, kw):
    assert _attn(lib, **kw) == fo.FO_ERR_INVALID_ARG
    assert lib.fo_last_error().decode() != ""


def test_attn_head_dim_is_unsupported(lib):
    assert _attn(lib, d=64) == fo.FO_ERR_UNSUPPORTED
    assert lib.fo_attn_ref(A, C, 64, 8, 2, 96, 1, None) == fo.FO_ERR_UNSUPPORTED


def test_attn_rejects_bad_opts(lib):
    for kw in (dict(arrival=fo.ARR_LOCKSTEP), dict(tile=fo.TILE_256x256), dict(row_groups=9),
               dict(epilogue=fo.EPI_SWIGLU), dict(order=7)):
        o = fo.opts()
        for k, v in kw.items():
            setattr(o, k, v)
        assert _attn(lib, opts=ctypes.byref(o)) == fo.FO_ERR_INVALID_ARG, kw
    peers = [0x50000000, 0, 0x60000000, 0x70000000]   # a NULL peer with arrivals on
    assert _attn(lib, peers=peers) == fo.FO_ERR_INVALID_ARG


def test_attn_return_exchange_rejects(lib):
    """out_peer (the return All-to-All): every entry but the rank's present, 16-byte aligned, and
    clear of out, of the inputs and of the other entries; 2P slots of signals needed."""
    E, F, G = 0x60000000, 0x68000000, 0x70000000   # out slices are 64 x 8 x 256 B = 128 KiB
    ok = [0, E, F, G]
    for bad in ([0, 0, F, G], [0, E + 8, F, G], [0, C, F, G], [0, E, E + 4096, G],
                [0, E, F, A]):
        assert _attn(lib, out_peer=bad) == fo.FO_ERR_INVALID_ARG, bad
    assert _attn(lib, out_peer=ok, m=0) == fo.FO_OK
    big = [0] + [0x60000000 + i * (1 << 20) for i in range(16)]
    assert _attn(lib, out_peer=big, P=17, m=64) == fo.FO_ERR_UNSUPPORTED


def test_attn_empty_is_a_no_op(lib):
    assert _attn(lib, m=0) == fo.FO_OK
    assert lib.fo_attn_ref(A, C, 0, 8, 2, 128, 1, None) == fo.FO_OK
    assert lib.fo_attn_ref(A, A + 16, 4, 8, 2, 128, 1, None) == fo.FO_ERR_INVALID_ARG


def test_rs_noalloc_rejects(lib):
    """fo_gemm_rs_noalloc checks its arguments like fo_gemm_rs, before touching the device, and
    takes resident partials only."""
    def call(**kw):
        a = dict(x=A, w=B, send=C, out=D, recv=0x50000000, P=4, rank=1, m=64, K=256, N=512,
                 in_dt=fo.BF16, opts=None)
        a.update(kw)
        return lib.fo_gemm_rs_noalloc(a["x"], a["w"], a["send"], a["out"], a["recv"], a["P"],
                                      a["rank"], a["m"], a["K"], a["N"], a["in_dt"], None,
                                      a["opts"])
    for kw in (dict(P=0), dict(P=33), dict(rank=4), dict(N=12), dict(x=None), dict(recv=None),
               dict(out=A), dict(send=D - 4), dict(x=A + 4)):
        assert call(**kw) == fo.FO_ERR_INVALID_ARG, kw
    for arrival in (fo.ARR_EAGER, fo.ARR_LOCKSTEP):
        o = fo.opts(arrival=arrival)
        assert call(opts=ctypes.byref(o)) == fo.FO_ERR_INVALID_ARG
    o = fo.opts(epilogue=fo.EPI_SWIGLU)
    assert call(opts=ctypes.byref(o)) == fo.FO_ERR_INVALID_ARG
    assert call(m=0) == fo.FO_OK and call(N=0) == fo.FO_OK  # nothing to do, nothing touched
