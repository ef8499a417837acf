"""The benchmark's host side without a GPU: it refuses more than one GPU with
a message, its workload table names real workloads, and every committed
counter summary it reads was taken on the kernel sources as they stand (a
summary taken on other sources would make it report no traffic)."""
from __future__ import annotations

import re
import subprocess
import sys
from pathlib import Path

import bench
from sparse_attention_lightning_amd import workloads as W

ROOT = Path(__file__).resolve().parents[1]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_other_workloads_are_real_configs():
    names = set()
    for cfg, kf in bench.OTHER_WORKLOADS:
        assert 0 <= cfg < len(W.CONFIG_NAMES) and cfg != 3
        assert kf in (None, "fp8")
        names.add((W.CONFIG_NAMES[cfg], kf))
    assert len(names) == len(bench.OTHER_WORKLOADS)


def test_counter_summaries_match_the_sources():
    summaries = sorted((ROOT / "profiles").glob("*_traffic.md"))
    assert summaries, "no counter summaries committed"
    for f in summaries:
        kernel = next(k for k in bench.KERNEL_SOURCES if f.name.startswith(k + "_"))
        text = f.read_text()
        m = re.search(r"source digest:\s*([0-9a-f]+)", text)
        assert m, f"{f.name} names no source digest"
        assert m.group(1) == bench.source_digest(kernel), f"{f.name} was taken on other sources of {kernel}"
        assert re.search(r"hbm bytes per launch:\s*[0-9.eE+]+", text), f"{f.name} gives no byte count"
