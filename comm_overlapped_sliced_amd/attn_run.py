"""The resident query-split attention on one Ulysses rank share, for the profiler: seeded inputs
of the Llama-3.1-70B share (8 query heads, 1 key/value head of dimension 128, causal),
fo_attn_ref back to back for `--warmup-ms` (the clocks settle after a change of load), then
`--calls` calls timed with HIP events.

    python -m comm_overlapped_sliced_amd.attn_run --seq 8192 --calls 50
"""
from __future__ import annotations

import argparse
import sys
import time


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(prog="python -m comm_overlapped_sliced_amd.attn_run")
    ap.add_argument("--seq", type=int, default=8192)
    ap.add_argument("--calls", type=int, default=50)
    ap.add_argument("--warmup-ms", type=float, default=50.0)
    a = ap.parse_args(argv)

    import numpy as np
    import torch

    from comm_overlapped_sliced_amd import configs, flashovl as fo

    c = next((x for x in configs.SWEEP_ATTN if x.S == a.seq), None)
    if c is None:
        print(f"no attention workload at {a.seq} tokens", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fo.load()
    stream = torch.cuda.current_stream()
    qkv = torch.from_numpy(c.qkv().view(np.int16)).to(dev).view(torch.bfloat16)
    out = torch.empty((c.S, c.hq * c.head_dim), dtype=torch.bfloat16, device=dev)
    # the first call sets the library up on the device (copy engines included): not warm-up
    fo.attn_ref(qkv, out, c.hq, c.hkv, c.causal, stream=stream)
    torch.cuda.synchronize()
    t_end = time.perf_counter() + a.warmup_ms * 1e-3
    n = 0
    while n < 3 or time.perf_counter() < t_end:
        fo.attn_ref(qkv, out, c.hq, c.hkv, c.causal, stream=stream)
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(a.calls):
        fo.attn_ref(qkv, out, c.hq, c.hkv, c.causal, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    fo.check(stream)
    us = e0.elapsed_time(e1) / a.calls * 1e3
    print(f"attn timed: S={c.S}, {a.calls} calls, {us:.1f} us per call, "
          f"{c.flops / (us * 1e-6) / 1e12:.1f} TFLOP/s", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
