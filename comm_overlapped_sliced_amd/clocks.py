"""Shader clock and power of the GPU while a measurement runs, from the SMU's metrics table.

The MFMA peak of an MI355X (256 CUs x 4096 bf16 flop per clock) is quoted at the 2.4 GHz top
clock; under a sustained MFMA load the chip holds its power limit by lowering the clock, so a
roofline fraction against the nominal peak mixes kernel quality with the clock the chip could
sustain. This module samples, from a child process (no HIP in it), the per-XCD gfx clock, the
socket power and the accumulated residency in package-power (PPT) throttling that the SMU
publishes, so that a benchmark can report the clock its timed region ran at and the fraction of
the peak at that clock beside the nominal one.

Usage from a benchmark: ``s = Sampler(); s.start(); ...; w = s.window(t0_ns, t1_ns); s.stop()``
with ``time.monotonic_ns()`` bounds (the child stamps its samples with the same clock).

As a script (the child): prints one JSON line per sample until its stdin closes.
"""
from __future__ import annotations

import json
import os
import statistics
import subprocess
import sys
import threading
import time

MFMA_BF16_FLOP_PER_CLK_CU = 4096


def _child(period_s: float) -> int:
    try:
        import amdsmi
    except Exception as e:  # noqa: BLE001 - reported to the parent as a sample error
        print(json.dumps({"error": f"amdsmi not importable: {e}"}), flush=True)
        return 0
    try:
        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        want = os.environ.get("FO_CLOCKS_BDF", "").lower()
        h = handles[0]
        for cand in handles:
            try:
                if want and amdsmi.amdsmi_get_gpu_device_bdf(cand).lower().endswith(want):
                    h = cand
            except Exception:  # noqa: BLE001
                pass
        print(json.dumps({"gpus": len(handles),
                          "bdf": amdsmi.amdsmi_get_gpu_device_bdf(h)}), flush=True)
    except Exception as e:  # noqa: BLE001
        print(json.dumps({"error": f"amdsmi init: {e}"}), flush=True)
        return 0
    stop = threading.Event()
    threading.Thread(target=lambda: (sys.stdin.read(), stop.set()), daemon=True).start()
    while not stop.is_set():
        t = time.monotonic_ns()
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
            clks = [c for c in m.get("current_gfxclks", []) if isinstance(c, int) and c > 0]
            rec = {"t": t, "gfxclks": clks,
                   "power_w": m.get("current_socket_power"),
                   "ppt_acc": m.get("ppt_residency_acc"),
                   "acc": m.get("accumulation_counter"),
                   "energy": m.get("energy_accumulator")}
        except Exception as e:  # noqa: BLE001
            rec = {"t": t, "error": str(e)}
        print(json.dumps(rec), flush=True)
        stop.wait(period_s)
    amdsmi.amdsmi_shut_down()
    return 0


class Sampler:
    """A child process sampling the SMU metrics every `period_s`; see the module docstring."""

    def __init__(self, period_s: float = 0.002, bdf: str = ""):
        self.period_s = period_s
        self.bdf = bdf
        self.samples: list = []
        self.info: dict = {}
        self._proc = None
        self._reader = None

    def start(self) -> None:
        env = dict(os.environ, FO_CLOCKS_BDF=self.bdf)
        self._proc = subprocess.Popen(
            [sys.executable, "-u", "-m", "comm_overlapped_sliced_amd.clocks", str(self.period_s)],
            stdin=subprocess.PIPE, stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True,
            cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))), env=env)
        self._reader = threading.Thread(target=self._read, daemon=True)
        self._reader.start()
        deadline = time.monotonic() + 20.0
        while not self.info and not self.samples and time.monotonic() < deadline:
            time.sleep(0.01)

    def _read(self) -> None:
        for line in self._proc.stdout:
            try:
                rec = json.loads(line)
            except ValueError:
                continue
            if "t" in rec:
                self.samples.append(rec)
            else:
                self.info.update(rec)

    def stop(self) -> None:
        if self._proc is None:
            return
        try:
            self._proc.stdin.close()
            self._proc.wait(timeout=10)
        except Exception:  # noqa: BLE001
            self._proc.kill()
        self._reader.join(timeout=5)
        self._proc = None

    def window(self, t0_ns: int, t1_ns: int) -> dict:
        """Clock and power over the samples taken in [t0_ns, t1_ns]: the mean over samples of
        the mean gfx clock over the XCDs (MHz), its range, the mean socket power, and the share
        of the window the SMU accumulated as package-power throttling (from the residency
        counters of the first and last sample, when it publishes them)."""
        s = [x for x in self.samples if t0_ns <= x["t"] <= t1_ns and x.get("gfxclks")]
        out = {"samples": len(s), "window_ms": round((t1_ns - t0_ns) / 1e6, 2)}
        if self.info.get("error"):
            out["error"] = self.info["error"]
        if not s:
            return out
        per = [statistics.mean(x["gfxclks"]) for x in s]
        out["sclk_mhz"] = round(statistics.mean(per), 1)
        out["sclk_mhz_min"] = round(min(min(x["gfxclks"]) for x in s), 1)
        out["sclk_mhz_max"] = round(max(max(x["gfxclks"]) for x in s), 1)
        pw = [x["power_w"] for x in s if isinstance(x.get("power_w"), (int, float))]
        if pw:
            out["socket_power_w"] = round(statistics.mean(pw), 1)
        a, b = s[0], s[-1]
        if all(isinstance(v.get(k), int) for v in (a, b) for k in ("ppt_acc", "acc")) and \
                b["acc"] > a["acc"]:
            out["ppt_throttle_share"] = round((b["ppt_acc"] - a["ppt_acc"]) / (b["acc"] - a["acc"]), 3)
        return out


def peak_at(sclk_mhz: float, n_cu: int = 256) -> float:
    """Dense bf16 MFMA peak (TFLOP/s) of n_cu CUs at the given shader clock."""
    return n_cu * MFMA_BF16_FLOP_PER_CLK_CU * sclk_mhz * 1e6 / 1e12


if __name__ == "__main__":
    sys.exit(_child(float(sys.argv[1]) if len(sys.argv) > 1 else 0.002))
