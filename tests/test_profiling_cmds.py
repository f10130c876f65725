"""The rocprofv3 harness builds commands that the profiler can run: the program after `--` is
python itself (no launcher in between) on bench.py or the attention module (attn_run), counter
passes trace kernels only (no copy, HIP, HSA, marker or system traces beside --pmc) and ask for
at most 8 SQ and 4 TCC counters, and every pass writes under its own directory."""
from __future__ import annotations

import pytest

from comm_overlapped_sliced_amd import profiling

TRACE_DOMAINS = {"--memory-copy-trace", "--hip-trace", "--hsa-trace", "--marker-trace",
                 "--sys-trace", "-s", "--runtime-trace", "-r", "--scratch-memory-trace"}
TCC_COST = {"FETCH_SIZE": 3, "WRITE_SIZE": 2}


@pytest.mark.parametrize("name", [p[0] for p in profiling.PASSES])
def test_pass_command(name):
    argv = profiling.command(name, "out", python="python3")
    assert argv[0] == "rocprofv3"
    sep = argv.index("--")
    assert argv[sep + 1] == "python3"
    assert argv[sep + 2] == "bench.py" or argv[sep + 2:sep + 4] == [
        "-m", "comm_overlapped_sliced_amd.attn_run"]
    opts = argv[1:sep]
    assert opts[opts.index("-d") + 1] == f"out/{name}"
    if "--pmc" in opts:
        assert not TRACE_DOMAINS & set(opts)
        i = opts.index("--pmc") + 1
        counters = []
        while i < len(opts) and not opts[i].startswith("-"):
            counters.append(opts[i])
            i += 1
        assert counters
        assert sum(1 for c in counters if c.startswith("SQ_")) <= 8
        assert sum(TCC_COST.get(c, 0) for c in counters) <= 4


def test_pass_names_unique():
    names = [p[0] for p in profiling.PASSES]
    assert len(names) == len(set(names))
    with pytest.raises(KeyError):
        profiling.command("nope", "out")
