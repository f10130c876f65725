"""Benchmark of the Flash-Overlap hot path on one MI355X.

One step is one pass of the whole path for one tensor-parallel rank (rank 0 of TP8) of the
Llama-3.1-70B MLP: the gate+up projection as Flash-AG (fo_ag_gemm, M=4096 tokens in 8 slices,
K=8192, N=7168, bf16) and the down projection as Flash-RS (fo_gemm_rs, M=4096, K=3584, N=8192,
seven incoming fp32 partials), each with its emulated peer arrivals. Inputs are synthetic and
seeded, resident in HBM before timing starts.

Prints one JSON line: throughput (TFLOP/s of the step), the roofline of the dominant kernel
(measured with HIP events around each GEMM kernel launch on its own stream), the
exposed-transfer decomposition, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch loaded (the library records them itself,
    which torch.cuda.Event would not see)."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")  # the copy already in the process
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        e = self.ct.c_void_p()
        if self.hip.hipEventCreate(self.ct.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def record(self, e: int, stream: int) -> None:
        if self.hip.hipEventRecord(e, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--links", type=int, default=0,
                    help="emulated links per call (0: one DMA engine per peer; 1: one link)")
    ap.add_argument("--row-groups", type=int, default=0,
                    help="row groups per slice (0: one per tile row; 1: whole slices)")
    ap.add_argument("--ag-k-chunks", type=int, default=0,
                    help="Flash-AG slices stored and sent in this many K blocks in the timed step "
                         "(opts.k_chunks; 0: row-major slices, the activation's own layout); the "
                         "exposure section measures 4 K blocks beside the row-major call either "
                         "way")
    ap.add_argument("--engines-per-link", type=int, default=0,
                    help="DMA engines per emulated link (opts.engines_per_link; 0: the library's "
                         "default)")
    ap.add_argument("--no-sweeps", action="store_true",
                    help="skip the other workloads (1K-16K, 405B, MLP block and attention sweeps)")
    ap.add_argument("--exposure-reps", type=int, default=10)
    ap.add_argument("--no-exposure", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample (0 disables)")
    ap.add_argument("--settle-seconds", type=float, default=1.5,
                    help="right before the warm-up and timed steps, run the step back to back "
                         "this long, so that the timed steps find the clocks and power at their "
                         "steady state (the shader clock is sampled meanwhile; 0 disables)")
    ap.add_argument("--clock-seconds", type=float, default=1.5,
                    help="sample the SMU's shader clock, and after the timed region run the "
                         "monolithic gate+up GEMM alone this long (0 disables both)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="also run one plain device copy of BYTES bytes after the warmup: the "
                         "reference that scales the HBM byte counters of a profiled run")
    return ap.parse_args()


def exposure_entry(t_ref, t0, t_pure, t_slice, t_xfer):
    """One call's exposure record (times in ms in, us out). t_pure is the fastest pure GEMM the
    library has for the product (min of fo_gemm_ref and the sliced call with every slice
    resident); exposed_frac = (T_slice - T_pure) / T_xfer, and against fo_gemm_ref alone."""
    return {"t_ref_us": t_ref * 1e3, "t_slice0_us": t0 * 1e3, "t_pure_us": t_pure * 1e3,
            "t_slice_us": t_slice * 1e3, "t_xfer_us": t_xfer * 1e3,
            "exposed_frac": (t_slice - t_pure) / t_xfer,
            "exposed_frac_vs_ref": (t_slice - t_ref) / t_xfer}


def rs_floor(t_slice0, t_pure, t_xfer, tiles, n_cu):
    """A floor for Flash-RS in lockstep under this emulation (a model, times in ms in, us out):
    no partial can leave before the first round of tiles has stored its row groups (about one
    round, T_slice0 over the rounds of tiles), and the links then need T_xfer for the partials
    (the transfers alone, engines in parallel). floor = max(T_pure, t_round + T_xfer); the
    exposed fraction at the floor = (floor - T_pure) / T_xfer."""
    rounds = max(1, -(-tiles // n_cu))
    t_round = t_slice0 / rounds
    floor = max(t_pure, t_round + t_xfer)
    return {"t_first_release_model_us": t_round * 1e3, "rounds_of_tiles": rounds,
            "floor_us": floor * 1e3, "exposed_floor": (floor - t_pure) / t_xfer}


def attention_case(fo, dev, stream, timed, reps, c, ranks, log=None):
    """Query-split attention between the two All-to-Alls of Ulysses parallelism on one share: the
    resident attention (T_ref), the call with every slice resident and nothing sent (T_slice0),
    the inbound exchange alone overlapped (Flash, in only), both exchanges overlapped (Flash, the
    own slice dispatched last), both in the data-slicing index order, and the transfers alone:
    inbound (T_xfer_in) and the return of the output rows (T_xfer_out). Vanilla = T_xfer_in +
    T_ref + T_xfer_out, nothing overlapped."""
    import numpy as np
    import torch
    qkv_np = c.qkv()
    qkv = torch.from_numpy(qkv_np.view(np.int16)).to(dev).view(torch.bfloat16)
    del qkv_np
    slices = [qkv[s * c.m:(s + 1) * c.m].contiguous() for s in range(c.P)]
    recv = torch.empty_like(qkv)
    out = torch.empty((c.S, c.hq * c.head_dim), dtype=torch.bfloat16, device=dev)
    back_buf = torch.empty_like(out)  # the peers' receive buffers of the return exchange
    back = [back_buf[s * c.m:(s + 1) * c.m] for s in range(c.P)]
    t_ref = timed(lambda: fo.attn_ref(qkv, out, c.hq, c.hkv, c.causal, stream=stream), reps)
    res = {"workload": c.name, "S": c.S, "P": c.P, "hq": c.hq, "hkv": c.hkv,
           "head_dim": c.head_dim, "causal": c.causal, "gflop": c.flops / 1e9,
           "t_ref_us": t_ref * 1e3, "tflops_ref": c.flops / t_ref / 1e9}
    slice_b = c.m * c.row * 2
    oslice_b = c.m * c.hq * c.head_dim * 2
    out_slices = [out[s * c.m:(s + 1) * c.m] for s in range(c.P)]
    for rb in ranks:
        for s in range(c.P):
            recv[s * c.m:(s + 1) * c.m] = slices[s]
        t0 = timed(lambda: fo.attn(slices[rb], None, recv, out, c.P, rb, c.hq, c.hkv, c.causal,
                                   compute_stream=stream, o=fo.opts(arrival=fo.ARR_NONE)), reps)
        t_in = timed(lambda: fo.attn(slices[rb], slices, recv, out, c.P, rb, c.hq, c.hkv,
                                     c.causal, compute_stream=stream), reps)
        t1 = timed(lambda: fo.attn(slices[rb], slices, recv, out, c.P, rb, c.hq, c.hkv, c.causal,
                                   compute_stream=stream, out_peer=back), reps)
        tn = timed(lambda: fo.attn(slices[rb], slices, recv, out, c.P, rb, c.hq, c.hkv, c.causal,
                                   compute_stream=stream, o=fo.opts(order=fo.ORDER_NATURAL),
                                   out_peer=back), reps)
        tx_in = timed(lambda: fo.transfer_ref("ag", slices, recv, c.P, rb, slice_b, stream,
                                              fo.opts(row_groups=1)), reps)
        tx_out = timed(lambda: fo.transfer_ref("ag", out_slices, back_buf, c.P, rb, oslice_b,
                                               stream, fo.opts(row_groups=1)), reps)
        tx = tx_in + tx_out
        van = tx_in + t_ref + tx_out
        t_pure = min(t_ref, t0)
        res[f"rank{rb}"] = {"t_slice0_us": t0 * 1e3, "t_flash_inbound_only_us": t_in * 1e3,
                            "t_slice_us": t1 * 1e3, "data_slicing_us": tn * 1e3,
                            "t_xfer_in_us": tx_in * 1e3, "t_xfer_out_us": tx_out * 1e3,
                            "vanilla_us": van * 1e3, "t_pure_us": t_pure * 1e3,
                            "exposed_frac": (t1 - t_pure) / tx,
                            "exposed_frac_data_slicing": (tn - t_pure) / tx,
                            "latency_reduction_flash": (van - t1) / van,
                            "latency_reduction_data_slicing": (van - tn) / van}
        (log or print)(f"attention S={c.S} rank {rb}: ref {t_ref*1e3:.0f} us ({res['tflops_ref']:.0f} TFLOP/s), "
            f"slice0 {t0*1e3:.0f}, flash in-only {t_in*1e3:.0f}, flash both {t1*1e3:.0f}, data "
            f"slicing {tn*1e3:.0f}, xfer in {tx_in*1e3:.0f} out {tx_out*1e3:.0f}, vanilla "
            f"{van*1e3:.0f} -> exposed {(t1 - t_pure) / tx:.2f} (data slicing "
            f"{(tn - t_pure) / tx:.2f}), {(van - t1) / van:.3f} less than vanilla "
            f"(data slicing {(van - tn) / van:.3f})")
    del qkv, slices, recv, out, back_buf, back
    torch.cuda.empty_cache()
    return res


def attention_section(fo, dev, stream, timed, reps, log, sweep=True):
    """The Llama-3.1-70B Ulysses share at 8K tokens (ranks 0 and P-1), and the same share at 2K to
    16K tokens (rank 0): the page reports a latency gain that grows with the sequence length."""
    from comm_overlapped_sliced_amd import configs
    c = configs.L70B_ATTN
    res = attention_case(fo, dev, stream, timed, reps, c, (0, c.P - 1), log)
    if sweep:
        res["sequence_sweep"] = [attention_case(fo, dev, stream, timed, reps, cs, (0,), log)
                                 for cs in configs.SWEEP_ATTN]
    return res


def mlp_sweep_section(fo, dev, stream, timed, reps, log, kc):
    """The MLP block of the page's latency experiment (gate+up Flash-AG -> SwiGLU -> down Flash-RS,
    one TP8 rank's share of the Llama-3.1-70B MLP, rank 0) at 1K to 16K tokens: vanilla (each
    projection's transfers, then its GEMM, nothing overlapped, plus the activation kernel), data
    slicing (index order, whole slices) and Flash (row groups; gate+up slices row-major, or in kc
    K blocks when the timed step uses them),
    with the activation as its own kernel and fused into the gate+up write-back. The pure GEMMs
    of vanilla are the fastest the library has for each product (fo_gemm_ref or the sliced call
    with everything resident)."""
    import numpy as np
    import torch
    from comm_overlapped_sliced_amd import configs

    def dev_of(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    def k_blocks(t, c):
        m_, k_ = t.shape
        return t.reshape(m_, c, k_ // c).permute(1, 0, 2).contiguous().reshape(m_, k_)

    w_gu = dev_of(configs.SWEEP_AG[0].w())
    w_dn = dev_of(configs.L70B_RS.w())
    res = []
    for agc in configs.SWEEP_AG:
        M, P = agc.M, agc.P
        m = M // P
        rsc = configs.scaled(configs.L70B_RS, M=M)
        x = dev_of(agc.x())
        rows = [x[s * m:(s + 1) * m].contiguous() for s in range(P)]
        c = kc if kc > 1 and agc.K % (256 * kc) == 0 else 0
        chunked = [k_blocks(t, c) for t in rows] if c else rows
        recv = torch.empty_like(x)
        y = torch.empty((M, agc.N), dtype=torch.bfloat16, device=dev)
        h = torch.empty((M, rsc.K), dtype=torch.bfloat16, device=dev)
        peers = [dev_of(rsc.partial(q)) for q in range(P)]
        send = torch.empty((M, rsc.N), dtype=torch.float32, device=dev)
        out = torch.empty((m, rsc.N), dtype=torch.float32, device=dev)
        rrecv = torch.empty((M, rsc.N), dtype=torch.float32, device=dev)
        yref = torch.empty((M, rsc.N), dtype=torch.float32, device=dev)
        for s_ in range(P):
            recv[s_ * m:(s_ + 1) * m] = chunked[s_]
            rrecv[s_ * m:(s_ + 1) * m] = peers[s_]
        o_none = fo.opts(arrival=fo.ARR_NONE, k_chunks=c)
        t_ag = min(timed(lambda: fo.gemm_ref(x, w_gu, y, stream=stream), reps),
                   timed(lambda: fo.ag_gemm(chunked[0], None, recv, w_gu, y, P, 0,
                                            compute_stream=stream, o=o_none), reps))
        t_rs = min(timed(lambda: fo.gemm_ref(h, w_dn, yref, stream=stream), reps),
                   timed(lambda: fo.gemm_rs(h, w_dn, send, out, None, rrecv, P, 0,
                                            compute_stream=stream,
                                            o=fo.opts(arrival=fo.ARR_NONE)), reps))
        t_act = timed(lambda: fo.swiglu(y, h, stream), reps)
        tx_a = timed(lambda: fo.transfer_ref("ag", rows, recv, P, 0, m * agc.K * 2, stream,
                                             fo.opts(row_groups=1)), reps)
        tx_r = timed(lambda: fo.transfer_ref("rs", peers, rrecv, P, 0, m * rsc.N * 4, stream,
                                             fo.opts(row_groups=1)), reps)
        van = t_ag + tx_a + t_act + t_rs + tx_r

        def block(natural, fused=False, fine=False):
            # data slicing in whole row-major slices (the page's unit), or (fine) in the units
            # Flash uses, so that only the order differs
            if natural and not fine:
                o_ag = fo.opts(order=fo.ORDER_NATURAL, row_groups=1)
                o_rs = fo.opts(order=fo.ORDER_NATURAL, row_groups=1)
            else:
                o_ag = fo.opts(order=fo.ORDER_NATURAL if natural else fo.ORDER_FLASH, k_chunks=c)
                o_rs = fo.opts(order=fo.ORDER_NATURAL if natural else fo.ORDER_FLASH)
            sl = rows if (natural and not fine) else chunked
            if fused:
                o_ag.epilogue = fo.EPI_SWIGLU
                fo.ag_gemm(sl[0], sl, recv, w_gu, h, P, 0, compute_stream=stream, o=o_ag)
            else:
                fo.ag_gemm(sl[0], sl, recv, w_gu, y, P, 0, compute_stream=stream, o=o_ag)
                fo.swiglu(y, h, stream)
            fo.gemm_rs(h, w_dn, send, out, peers, rrecv, P, 0, compute_stream=stream, o=o_rs)

        t_ds = timed(lambda: block(True), reps)
        t_dsf = timed(lambda: block(True, fine=True), reps)
        t_fl = timed(lambda: block(False), reps)
        t_ff = timed(lambda: block(False, True), reps)
        ent = {"M": M, "vanilla_us": van * 1e3, "data_slicing_us": t_ds * 1e3,
               "data_slicing_fine_units_us": t_dsf * 1e3,
               "flash_us": t_fl * 1e3, "flash_fused_us": t_ff * 1e3,
               "t_xfer_us": (tx_a + tx_r) * 1e3, "t_pure_gemms_us": (t_ag + t_rs) * 1e3,
               "latency_reduction_data_slicing": (van - t_ds) / van,
               "latency_reduction_flash": (van - t_fl) / van,
               "latency_reduction_flash_fused": (van - t_ff) / van,
               "removed_data_slicing": (van - t_ds) / (tx_a + tx_r),
               "removed_flash": (van - t_fl) / (tx_a + tx_r)}
        res.append(ent)
        log(f"MLP block M={M} rank 0: vanilla {van*1e3:.0f} us, data slicing {t_ds*1e3:.0f} "
            f"({ent['latency_reduction_data_slicing']:.3f} less; in Flash's units {t_dsf*1e3:.0f}), "
            f"flash {t_fl*1e3:.0f} "
            f"({ent['latency_reduction_flash']:.3f} less), fused {t_ff*1e3:.0f} "
            f"({ent['latency_reduction_flash_fused']:.3f} less); transfer removed: data slicing "
            f"{ent['removed_data_slicing']:.2f}, flash {ent['removed_flash']:.2f}")
        del x, rows, chunked, recv, y, h, peers, send, out, rrecv, yref
        torch.cuda.empty_cache()
    return res


def sweep_section(fo, dev, stream, timed, reps, log, kc):
    """The other workloads of the measurement, each in the three forms of the metric: the 70B
    gate+up AG-GEMM at 1K to 16K tokens and the 405B AG and RS shares at 8K tokens, rank 0, one
    link per peer, row groups (AG slices row-major, or in kc K blocks when the timed step uses
    them and K allows). Per call: T_ref
    (monolithic GEMM), T_slice0 (slices resident), T_slice (arrivals), T_xfer (the same copies
    alone); TFLOP/s and the share of the bf16 peak from T_slice; exposed = (T_slice - T_ref) /
    T_xfer."""
    import numpy as np
    import torch
    from comm_overlapped_sliced_amd import configs

    def dev_of(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    def k_blocks(t, c):
        m_, k_ = t.shape
        return t.reshape(m_, c, k_ // c).permute(1, 0, 2).contiguous().reshape(m_, k_)

    def groups_of(kind, case, chunks):
        order = fo.tile_order(kind, case.P, case.m, case.K, case.N, o=fo.opts(k_chunks=chunks),
                              out_dt=fo.F32 if kind == "rs" else fo.BF16)
        return max(g for _, g, _, _ in order) + 1

    res = []
    for case in configs.SWEEP_AG + (configs.L405B_AG, configs.L405B_RS):
        P, m = case.P, case.m
        x = dev_of(case.x())
        w = dev_of(case.w())
        if case.call == "ag":
            c = kc if kc > 1 and case.K % (256 * kc) == 0 else 0
            rows = [x[s_ * m:(s_ + 1) * m].contiguous() for s_ in range(P)]
            sl = [k_blocks(t, c) for t in rows] if c else rows
            recv = torch.empty_like(x)
            y = torch.empty((case.M, case.N), dtype=torch.bfloat16, device=dev)
            for s_ in range(P):
                recv[s_ * m:(s_ + 1) * m] = sl[s_]
            t_ref = timed(lambda: fo.gemm_ref(x, w, y, stream=stream), reps)
            t0 = timed(lambda: fo.ag_gemm(sl[0], None, recv, w, y, P, 0, compute_stream=stream,
                                          o=fo.opts(arrival=fo.ARR_NONE, k_chunks=c)), reps)
            t1 = timed(lambda: fo.ag_gemm(sl[0], sl, recv, w, y, P, 0, compute_stream=stream,
                                          o=fo.opts(k_chunks=c)), reps)
            pieces = groups_of("ag", case, c) * max(1, c)
            tx = timed(lambda: fo.transfer_ref("ag", sl, recv, P, 0, m * case.K * 2, stream,
                                               fo.opts(row_groups=min(8, pieces))), reps)
            del rows, sl, recv, y
        else:
            c = 0
            peers = [dev_of(case.partial(q)) for q in range(P)]
            send = torch.empty((case.M, case.N), dtype=torch.float32, device=dev)
            out = torch.empty((m, case.N), dtype=torch.float32, device=dev)
            recv = torch.empty((case.M, case.N), dtype=torch.float32, device=dev)
            t_ref = timed(lambda: fo.gemm_ref(x, w, send, stream=stream), reps)
            t0 = timed(lambda: fo.gemm_rs(x, w, send, out, None, recv, P, 0,
                                          compute_stream=stream,
                                          o=fo.opts(arrival=fo.ARR_NONE)), reps)
            t1 = timed(lambda: fo.gemm_rs(x, w, send, out, peers, recv, P, 0,
                                          compute_stream=stream), reps)
            tx = timed(lambda: fo.transfer_ref("rs", peers, recv, P, 0, m * case.N * 4, stream,
                                               fo.opts(row_groups=groups_of("rs", case, 0))),
                       reps)
            del peers, send, out, recv
        del x, w
        torch.cuda.empty_cache()
        tf = case.flops / t1 / 1e9
        ent = {"workload": case.name, "call": case.call, "M": case.M, "K": case.K, "N": case.N,
               "k_blocks": c, "tflops": tf, "pct_bf16_peak": 100.0 * tf / PEAK_BF16_TFLOPS}
        ent.update(exposure_entry(t_ref, t0, min(t_ref, t0), t1, tx))
        if case.call == "rs":
            n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
            ent["floor_model"] = rs_floor(t0, min(t_ref, t0), tx, fo.tile_info(
                P, m, case.K, case.N, out_dt=fo.F32)[2], n_cu)
        res.append(ent)
        log(f"sweep {case.call} M={case.M} K={case.K} N={case.N}: ref {t_ref*1e3:.0f} us, slice0 "
            f"{t0*1e3:.0f}, slice {t1*1e3:.0f}, xfer {tx*1e3:.0f} -> {tf:.0f} TFLOP/s "
            f"({ent['pct_bf16_peak']:.1f}% of peak), exposed {ent['exposed_frac']:.2f} "
            f"({ent['exposed_frac_vs_ref']:.2f} against fo_gemm_ref)")
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU (one rank's share of the tensor-parallel layer); "
              "--gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from comm_overlapped_sliced_amd import clocks, configs, flashovl as fo

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fo.load()
    fo.set_default_engines_per_link(args.engines_per_link)
    stream = torch.cuda.current_stream()
    # the shader clock sampler (a child process reading the SMU's metrics; off with
    # --clock-seconds 0, as in the profiler's runs)
    sampler = clocks.Sampler()
    if args.clock_seconds > 0:
        sampler.start()

    ag_case, rs_case = configs.L70B_AG, configs.L70B_RS
    P, r = ag_case.P, args.rank

    def dev_of(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    t0 = time.time()
    xa = ag_case.x()
    ag_slices = [dev_of(np.ascontiguousarray(xa[s * ag_case.m:(s + 1) * ag_case.m]))
                 for s in range(P)]
    ag_full = dev_of(xa)
    del xa
    # The timed step's Flash-AG slices: row-major (the activation's layout), or with
    # --ag-k-chunks c > 1 in the K-block layout of opts.k_chunks (block j = columns j*K/c .. of
    # every row), which a sender would have to produce. The exposure section measures the K-block
    # form (kb blocks) beside the row-major one either way.
    kc = args.ag_k_chunks
    kb = kc if kc > 1 else 4

    def k_blocks(t, c):
        m_, k_ = t.shape
        return t.reshape(m_, c, k_ // c).permute(1, 0, 2).contiguous().reshape(m_, k_)

    ag_chunked = [k_blocks(t, kb) for t in ag_slices]
    ag_w = dev_of(ag_case.w())
    ag_recv = torch.empty((ag_case.M, ag_case.K), dtype=torch.bfloat16, device=dev)
    ag_y = torch.empty((ag_case.M, ag_case.N), dtype=torch.bfloat16, device=dev)
    rs_x = dev_of(rs_case.x())
    rs_w = dev_of(rs_case.w())
    rs_peer = [dev_of(rs_case.partial(q)) for q in range(P)]
    rs_send = torch.empty((rs_case.M, rs_case.N), dtype=torch.float32, device=dev)
    rs_out = torch.empty((rs_case.m, rs_case.N), dtype=torch.float32, device=dev)
    rs_recv = torch.empty((rs_case.M, rs_case.N), dtype=torch.float32, device=dev)
    ref_y_ag = torch.empty_like(ag_y)
    ref_y_rs = torch.empty((rs_case.M, rs_case.N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s")
    # Python's collector: a full collection of this process's heap takes ~50 ms on the host,
    # long enough to starve the GPU for dozens of steps; the objects made so far are frozen
    # out of later collections, and the collector is off from the back-to-back window to the end
    # of the timed steps
    gc.collect()
    gc.freeze()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def ag_call(evs=None, arrival=fo.ARR_DEFAULT, links=args.links, groups=args.row_groups,
                order=fo.ORDER_FLASH, rank=r, epilogue=fo.EPI_NONE, y=None, chunks=kc):
        o = fo.opts(order=order, links=links, row_groups=groups, arrival=arrival,
                    kernel_events=evs, epilogue=epilogue, k_chunks=chunks)
        sl = ag_chunked if chunks > 1 else ag_slices
        peers = None if arrival == fo.ARR_NONE else sl
        fo.ag_gemm(sl[rank], peers, ag_recv, ag_w, ag_y if y is None else y, P, rank,
                   compute_stream=stream, o=o)

    def rs_call(evs=None, arrival=fo.ARR_DEFAULT, links=args.links, groups=args.row_groups,
                order=fo.ORDER_FLASH, rank=r, x=None):
        o = fo.opts(order=order, links=links, row_groups=groups, arrival=arrival,
                    kernel_events=evs)
        peers = None if arrival == fo.ARR_NONE else rs_peer
        fo.gemm_rs(rs_x if x is None else x, rs_w, rs_send, rs_out, peers, rs_recv, P, rank,
                   compute_stream=stream, o=o)

    def step(evs=None):
        ag_call(evs[0] if evs else None)
        rs_call(evs[1] if evs else None)

    def timed(fn, reps):
        """Steady-state duration (ms) of one fn() on the compute stream: `reps` calls enqueued
        back to back, as a training step enqueues them, so that the host's set-up of a call
        (signals, the enqueueing of its copies) runs ahead of the GPU instead of delaying the
        first copy; median over three such batches. Calls for at least 20 ms first: after a
        stretch with little to compute (transfers alone, the host) the first few milliseconds of
        GEMM calls run up to ~50 us per call slower while the clocks come back up."""
        t_end = time.perf_counter() + 0.02
        n = 0
        while n < 3 or time.perf_counter() < t_end:
            fn()
            n += 1
            if n % 4 == 0:
                torch.cuda.synchronize()
        out = []
        for _ in range(3):
            a, b = ev(), ev()
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
            b.synchronize()
            out.append(a.elapsed_time(b) / reps)
        return statistics.median(out)

    # one step first: the first call on a device sets up its engines and signals
    step()
    fo.check(stream)
    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        # a 512 MiB fill between the writes of src and the copy leaves no src line in the
        # 256 MB last-level cache
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        flush.fill_(3)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {n} bytes read and written by one copy kernel")
        del src, dst, flush

    # ---- exposed-transfer decomposition (before the timed region) ------------------------
    exposure = None
    if not args.no_exposure:
        exposure = {}
        reps = args.exposure_reps
        # one DMA engine per peer (the xGMI mesh) with row-group arrivals (the default), the same
        # with whole slices (the page's granularity), and every transfer over one link (the
        # ring of the page's Flash-AG, where all slices come from one neighbour)
        # (name, links, row groups, Flash-AG K blocks). The K-block variant changes Flash-AG
        # only, so its RS entry repeats the row-major one.
        variants = [("mesh_rowgroups", 0, 0, 0), ("mesh_rowgroups_kblocks", 0, 0, kb),
                    ("mesh_slices", 0, 1, 0), ("onelink_slices", 1, 1, 0)]

        def groups_of(kind, case, req, chunks=0):
            order = fo.tile_order(kind, P, case.m, case.K, case.N,
                                  o=fo.opts(row_groups=req, k_chunks=chunks),
                                  out_dt=fo.F32 if kind == "rs" else fo.BF16)
            return max(g for _, g, _, _ in order) + 1

        n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
        rs_tiles = fo.tile_info(P, rs_case.m, rs_case.K, rs_case.N, out_dt=fo.F32)[2]
        t_ref_ag = timed(lambda: fo.gemm_ref(ag_full, ag_w, ref_y_ag, stream=stream), reps)
        t_ref_rs = timed(lambda: fo.gemm_ref(rs_x, rs_w, ref_y_rs, stream=stream), reps)
        t0_rs = timed(lambda: rs_call(arrival=fo.ARR_NONE), reps)
        t0_ag = {chunks: timed(lambda: ag_call(arrival=fo.ARR_NONE, chunks=chunks), reps)
                 for chunks in sorted({v[3] for v in variants})}
        # the pure-GEMM latency of the exposed fraction: the fastest way the library has to
        # compute the same product with nothing in flight (the monolithic GEMM, or the sliced
        # call with every slice already resident when its tile placement suits the L2 better)
        t_pure_ag = min([t_ref_ag] + list(t0_ag.values()))
        t_pure_rs = min(t_ref_rs, t0_rs)
        for name, links, req, chunks in variants:
            # the same copies alone: each row group of each slice in `chunks` equal K blocks
            to_ag = fo.opts(links=links,
                            row_groups=groups_of("ag", ag_case, req, chunks) * max(1, chunks))
            to_rs = fo.opts(links=links, row_groups=groups_of("rs", rs_case, req))
            tx_ag = timed(lambda: fo.transfer_ref("ag", ag_slices, ag_recv, P, r,
                                                  ag_case.m * ag_case.K * 2, stream, to_ag), reps)
            ts_ag = timed(lambda: ag_call(links=links, groups=req, chunks=chunks), reps)
            if chunks > 1 and "mesh_rowgroups" in exposure:
                tx_rs, ts_rs = tx_rs_prev, ts_rs_prev
            else:
                tx_rs = timed(lambda: fo.transfer_ref("rs", rs_peer, rs_recv, P, r,
                                                      rs_case.m * rs_case.N * 4, stream, to_rs),
                              reps)
                ts_rs = timed(lambda: rs_call(links=links, groups=req), reps)
            tx_rs_prev, ts_rs_prev = tx_rs, ts_rs
            exposure[name] = {
                "ag": exposure_entry(t_ref_ag, t0_ag[chunks], t_pure_ag, ts_ag, tx_ag),
                "rs": exposure_entry(t_ref_rs, t0_rs, t_pure_rs, ts_rs, tx_rs),
            }
            exposure[name]["rs"]["floor_model"] = rs_floor(
                t0_rs, t_pure_rs, tx_rs, rs_tiles, n_cu)
            log(f"exposure {name}: AG ref {t_ref_ag*1e3:.0f} us slice0 {t0_ag[chunks]*1e3:.0f} "
                f"pure {t_pure_ag*1e3:.0f} slice {ts_ag*1e3:.0f} xfer {tx_ag*1e3:.0f} -> "
                f"{exposure[name]['ag']['exposed_frac']:.3f}; RS ref {t_ref_rs*1e3:.0f} slice0 "
                f"{t0_rs*1e3:.0f} slice {ts_rs*1e3:.0f} xfer {tx_rs*1e3:.0f} -> "
                f"{exposure[name]['rs']['exposed_frac']:.3f} (floor model "
                f"{exposure[name]['rs']['floor_model']['exposed_floor']:.3f})")
        # the page's comparison (FlashOverlap page, section 1 and section 4): vanilla (all
        # transfers, then the GEMM, nothing overlapped), data slicing (slices in index order) and
        # Flash (the page's order), each pair at the same granularity and over the same links, so
        # that the difference is the order alone: whole row-major slices (the page's unit), and
        # the fine units of the step (row groups; Flash-AG slices in K blocks); one DMA engine
        # per peer (the mesh) and every transfer over one link (a ring from one neighbour, where
        # the page's tail argument applies); at rank 0 and at rank P-1, the rank data slicing
        # serves worst (its own RS chunk and its local AG slice come last in index order).
        # "removed" = the share of the transfer time that does not show in the latency.
        base = {}
        units = {"whole_slices": (1, 0), "fine": (args.row_groups, kc)}
        for kind, t_pure, call, case in (("ag", t_pure_ag, ag_call, ag_case),
                                          ("rs", t_pure_rs, rs_call, rs_case)):
            ent = {"t_pure_us": t_pure * 1e3}
            for rb in (0, P - 1):
                for lname, links in (("mesh", 0), ("onelink", 1)):
                    for uname, (req, chunks) in units.items():
                        c = chunks if kind == "ag" else 0
                        pieces = groups_of(kind, case, req, c) * max(1, c)
                        tx = timed(lambda: fo.transfer_ref(
                            kind, ag_slices if kind == "ag" else rs_peer,
                            ag_recv if kind == "ag" else rs_recv, P, rb,
                            case.m * (case.K * 2 if kind == "ag" else case.N * 4), stream,
                            fo.opts(links=links, row_groups=min(8, pieces))), reps)
                        kw = dict(rank=rb, links=links, groups=req)
                        if kind == "ag":
                            kw["chunks"] = c
                        t_ds = timed(lambda: call(order=fo.ORDER_NATURAL, **kw), reps)
                        t_fl = timed(lambda: call(**kw), reps)
                        van = t_pure + tx
                        ent[f"rank{rb}_{lname}_{uname}"] = {
                            "t_xfer_us": tx * 1e3, "vanilla_us": van * 1e3,
                            "data_slicing_us": t_ds * 1e3, "flash_us": t_fl * 1e3,
                            "removed_data_slicing": (van - t_ds) / tx,
                            "removed_flash": (van - t_fl) / tx}
                        log(f"baselines {kind} rank {rb} {lname} {uname}: vanilla {van*1e3:.0f} "
                            f"us, data slicing {t_ds*1e3:.0f} us ({(van - t_ds) / tx:.2f} "
                            f"removed), flash {t_fl*1e3:.0f} us ({(van - t_fl) / tx:.2f} removed)")
            base[kind] = ent
        exposure["baselines"] = base
        tw = fo.opts(row_groups=1)

        # the MLP block of the page's latency experiment: AG (gate+up) -> SwiGLU -> RS (down),
        # the RS reading the activation H that SwiGLU makes of the AG output. Vanilla = each
        # projection's transfers, then its GEMM, nothing overlapped.
        mlp_h = torch.empty((rs_case.M, rs_case.K), dtype=torch.bfloat16, device=dev)
        t_act = timed(lambda: fo.swiglu(ag_y, mlp_h, stream), reps)

        def block(rank, natural, fused=False):
            g = 1 if natural else args.row_groups
            o = fo.ORDER_NATURAL if natural else fo.ORDER_FLASH
            c = 0 if natural else kc  # data slicing keeps row-major slices
            if fused:  # the activation in the gate+up projection's write-back
                ag_call(order=o, groups=g, rank=rank, epilogue=fo.EPI_SWIGLU, y=mlp_h, chunks=c)
            else:
                ag_call(order=o, groups=g, rank=rank, chunks=c)
                fo.swiglu(ag_y, mlp_h, stream)
            rs_call(order=o, groups=g, rank=rank, x=mlp_h)

        t_ag_fused = timed(lambda: ag_call(epilogue=fo.EPI_SWIGLU, y=mlp_h), reps)
        t_ag = timed(lambda: ag_call(), reps)
        mlp = {"swiglu_us": t_act * 1e3,
               "swiglu_gbps": (ag_case.M * ag_case.N * 2 + rs_case.M * rs_case.K * 2) / t_act / 1e6,
               "ag_us": t_ag * 1e3, "ag_swiglu_fused_us": t_ag_fused * 1e3}
        for rb in (0, P - 1):
            tx_a = timed(lambda: fo.transfer_ref("ag", ag_slices, ag_recv, P, rb,
                                                 ag_case.m * ag_case.K * 2, stream, tw), reps)
            tx_r = timed(lambda: fo.transfer_ref("rs", rs_peer, rs_recv, P, rb,
                                                 rs_case.m * rs_case.N * 4, stream, tw), reps)
            van = t_pure_ag + tx_a + t_act + t_pure_rs + tx_r
            t_fl = timed(lambda: block(rb, False), reps)
            t_ff = timed(lambda: block(rb, False, True), reps)
            t_ds = timed(lambda: block(rb, True), reps)
            mlp[f"rank{rb}"] = {"vanilla_us": van * 1e3, "data_slicing_us": t_ds * 1e3,
                                "flash_us": t_fl * 1e3, "flash_fused_us": t_ff * 1e3,
                                "latency_reduction_data_slicing": (van - t_ds) / van,
                                "latency_reduction_flash": (van - t_fl) / van,
                                "latency_reduction_flash_fused": (van - t_ff) / van}
            log(f"MLP block rank {rb}: vanilla {van*1e3:.0f} us, data slicing {t_ds*1e3:.0f} us "
                f"({(van - t_ds) / van:.3f} less), flash {t_fl*1e3:.0f} us ({(van - t_fl) / van:.3f} "
                f"less), flash with the fused activation {t_ff*1e3:.0f} us ({(van - t_ff) / van:.3f} less)")
        log(f"SwiGLU {t_act*1e3:.1f} us, {mlp['swiglu_gbps']:.0f} GB/s; AG {t_ag*1e3:.0f} us, "
            f"AG with the SwiGLU epilogue {t_ag_fused*1e3:.0f} us")
        exposure["mlp_block"] = mlp
        fo.check(stream)
        exposure["attention"] = attention_section(fo, dev, stream, timed, reps, log,
                                                  sweep=not args.no_sweeps)
        fo.check(stream)
        step()
        fo.check(stream)

    # ---- sustained window, then the timed region ------------------------------------------
    # The same step back to back for about args.settle_seconds (the sampler reads the clock the
    # chip sustains under it), then the W warm-up steps and the K timed steps without a break.
    # After idling or a change of load (the sections above) the power controller overshoots and
    # settles over ~40 steps (~35 ms: steps of 843, 1027, then 815 us), so timed steps started
    # right after the attention sweep measured that transient instead of the steady state a
    # training loop runs in.
    he = HipEvents()
    kevs = [((he.create(), he.create()), (he.create(), he.create())) for _ in range(args.steps)]
    gc.collect()
    gc.disable()
    sustained = None
    if args.settle_seconds > 0:
        t_one = time.perf_counter()
        step()
        torch.cuda.synchronize()
        t_one = time.perf_counter() - t_one
        n_sus = max(1, int(args.settle_seconds / max(1e-4, t_one)))
        torch.cuda.synchronize()
        s0 = time.monotonic_ns()
        for i in range(n_sus):
            step()
            if i % 64 == 63:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        s1 = time.monotonic_ns()
        sustained = (s0, s1, n_sus)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    g0, g1 = ev(), ev()
    h0 = time.perf_counter()
    c0 = time.monotonic_ns()
    g0.record(stream)
    for i in range(args.steps):
        step(kevs[i])
    g1.record(stream)
    torch.cuda.synchronize()
    c1 = time.monotonic_ns()
    host_s = time.perf_counter() - h0
    gc.enable()
    fo.check(stream)
    clock_timed = sampler.window(c0, c1)
    clock_sustained = None
    if sustained is not None:
        s0, s1, n_sus = sustained
        clock_sustained = sampler.window(s0, s1)
        clock_sustained["steps"] = n_sus
        clock_sustained["us_per_step"] = round((s1 - s0) / 1e3 / n_sus, 1)
        clock_sustained["when"] = "right before the warm-up and timed steps"
    if args.clock_seconds > 0:
        # the monolithic gate+up GEMM alone, back to back, for the same time: the clock the chip
        # holds under a pure MFMA load, and the fraction of the peak at that clock
        n_g = max(1, int(args.clock_seconds / 0.4e-3))
        torch.cuda.synchronize()
        g0_ns = time.monotonic_ns()
        ge0, ge1 = ev(), ev()
        ge0.record(stream)
        for i in range(n_g):
            fo.gemm_ref(ag_full, ag_w, ref_y_ag, stream=stream)
            if i % 256 == 255:
                torch.cuda.synchronize()
        ge1.record(stream)
        torch.cuda.synchronize()
        g1_ns = time.monotonic_ns()
        clock_gemm = sampler.window(g0_ns, g1_ns)
        t_g = ge0.elapsed_time(ge1) / n_g
        clock_gemm.update({"call": "fo_gemm_ref, 70B gate+up (M=4096, K=8192, N=7168)",
                           "calls": n_g, "us_per_call": round(t_g * 1e3, 1),
                           "tflops": round(ag_case.flops / (t_g * 1e-3) / 1e12, 1)})
        if clock_gemm.get("sclk_mhz"):
            clock_gemm["frac_at_sclk"] = round(clock_gemm["tflops"] /
                                               clocks.peak_at(clock_gemm["sclk_mhz"]), 4)
        if clock_sustained is not None:
            clock_sustained["gemm_only"] = clock_gemm
    sampler.stop()
    log(f"shader clock: timed region {clock_timed}; sustained {clock_sustained}")
    total_ms = g0.elapsed_time(g1)
    ms_per_step = total_ms / args.steps
    flops = ag_case.flops + rs_case.flops
    value = flops / (ms_per_step * 1e-3) / 1e12

    k_ag = [he.elapsed_ms(a, b) for (a, b), _ in kevs]
    k_rs = [he.elapsed_ms(a, b) for _, (a, b) in kevs]
    mean_ag, mean_rs = statistics.mean(k_ag), statistics.mean(k_rs)
    if mean_ag * ag_case.flops >= 0 and mean_ag >= mean_rs:
        dom, dom_ms, dom_flops = "ag", mean_ag, ag_case.flops
    else:
        dom, dom_ms, dom_flops = "rs", mean_rs, rs_case.flops
    bm, bn, wg = fo.tile_info(P, ag_case.m if dom == "ag" else rs_case.m,
                              ag_case.K if dom == "ag" else rs_case.K,
                              ag_case.N if dom == "ag" else rs_case.N,
                              out_dt=fo.BF16 if dom == "ag" else fo.F32)
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    roofline = {
        "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": traffic_for(dom),
        "kernel": f"gemm_bf16_kernel<{bm},{bn}> ({'fo_ag_gemm' if dom == 'ag' else 'fo_gemm_rs'})",
        "kernel_us": round(dom_ms * 1e3, 1), "tiles": wg,
        "ag_kernel_us": round(mean_ag * 1e3, 1), "rs_kernel_us": round(mean_rs * 1e3, 1),
        # both launches of the step against the same peak; each launch's time includes its
        # in-kernel waits for the emulated transfers (the RS one waits for 117 MB of partials)
        "per_kernel": {
            kind: {"kernel_us": round(t * 1e3, 1),
                   "achieved": round(f / (t * 1e-3) / 1e12, 1),
                   "frac": round(f / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                   "traffic": traffic_for(kind)}
            for kind, t, f in (("ag", mean_ag, ag_case.flops), ("rs", mean_rs, rs_case.flops))},
    }
    # the peak at the clock the chip ran at: the timed region's samples, else the sustained run's
    sclk = clock_timed.get("sclk_mhz") or (clock_sustained or {}).get("sclk_mhz")
    if sclk:
        pk = clocks.peak_at(sclk)
        roofline["sclk_mhz"] = sclk
        roofline["sclk_source"] = ("SMU gfx clocks sampled in the timed region"
                                   if clock_timed.get("sclk_mhz") else
                                   "SMU gfx clocks sampled while the step ran back to back")
        roofline["peak_at_sclk"] = round(pk, 1)
        roofline["frac_at_sclk"] = round(achieved / pk, 4)
    log(f"timed: {args.steps} steps {total_ms:.2f} ms (host {host_s*1e3:.2f} ms), "
        f"{ms_per_step*1e3:.1f} us/step, {value:.1f} TFLOP/s; AG kernel {mean_ag*1e3:.1f} us, "
        f"RS kernel {mean_rs*1e3:.1f} us")

    # the other workloads after the timed region (their large GEMMs heat the chip)
    if exposure is not None and not args.no_sweeps:
        exposure["sweep"] = sweep_section(fo, dev, stream, timed, args.exposure_reps, log, kc)
        fo.check(stream)
        exposure["mlp_block"]["sequence_sweep"] = mlp_sweep_section(
            fo, dev, stream, timed, args.exposure_reps, log, kc)
        fo.check(stream)

    cpu = cpu_baseline(ag_case, rs_case, args.cpu_seconds) if args.cpu_seconds > 0 else None

    line = {
        "metric": "sliced AG/RS-GEMM TFLOP/s, % bf16 MFMA peak, exposed-transfer % (1 GPU)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Llama-3.1-70B MLP, one TP8 rank share (rank %d): Flash-AG "
                   "gate+up M=4096 K=8192 N=7168 + Flash-RS down M=4096 K=3584 N=8192, "
                   "P=8 slices" % r,
                   "transfers": "SDMA engines, %s, engines per link: %s" % (
                       "one link per peer" if args.links == 0 else "%d link(s)" % args.links,
                       args.engines_per_link or "library default (an engine pair, each "
                                                "transfer split across it)"),
                   "row_groups": "one per tile row" if args.row_groups == 0 else args.row_groups,
                   "ag_k_blocks": kc if kc > 1 else "row-major slices",
                   "ag_arrival": "eager", "rs_arrival": "lockstep",
                   "engines_per_link": args.engines_per_link or "library default"},
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "exposed_transfer": exposure,
        "roofline": roofline,
        "clock": {"timed_region": clock_timed, "sustained": clock_sustained,
                  "nominal_mhz": 2400, "peak_bf16_at_nominal": PEAK_BF16_TFLOPS},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def traffic_for(dom: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on the kernel
    source as it is now (else null)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    src = os.path.join(ROOT, "comm_overlapped_sliced_amd", "csrc", "fo_gemm.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    ent = data.get(dom)
    if not ent or ent.get("kernel_source_sha256") != sha:
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(ag_case, rs_case, target_s: float):
    """The oracle (plain fp64 C, OpenMP) on a bounded sample of the step's two products: rows of
    the Flash-AG product (X times the full W), then rows of the Flash-RS product, in batches of
    doubling size (32 rows per thread first) until about target_s seconds have been spent. Every
    batch is a full oracle call on rows not computed before; the rate is all flops over all time."""
    import oracle

    orc = oracle.default()
    threads = orc.num_threads()
    parts, fl, secs = [], 0.0, 0.0
    for case in (ag_case, rs_case):
        if secs >= target_s:
            break
        x = case.x()
        w = case.w()
        done, batch = 0, 32 * threads
        while done < case.M and secs < target_s:
            n = min(batch, case.M - done)
            t0 = time.perf_counter()
            orc.gemm(x[done:done + n], w)
            secs += time.perf_counter() - t0
            fl += 2.0 * n * case.K * case.N
            done += n
            batch *= 2
        parts.append(f"first {done} of {case.M} rows of the {case.call.upper()} product "
                     f"(K={case.K}, N={case.N})")
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(fl / secs / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "sample": "; ".join(parts) + f"; fp64, {secs:.1f} s",
            "host": {"nproc": os.cpu_count(), "cpu_model": model}}


if __name__ == "__main__":
    main()
