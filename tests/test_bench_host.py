"""bench.py's host-side bookkeeping, without a GPU: the source hash behind
the counted-traffic table covers every local header a kernel includes, a
record taken on other sources reports no traffic, and a multi-GPU request
is refused with a message."""
import os
import re
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_top_sparse_amd", "csrc")


def test_kernel_sources_follow_includes():
    for symbol, src in bench.KERNEL_SOURCES.items():
        files = bench.kernel_sources(symbol)
        assert files[0] == src
        # every local header named by any listed file is itself listed
        for f in files:
            text = open(os.path.join(CSRC, f)).read()
            for h in re.findall(r'^#include "([^"]+)"', text, flags=re.M):
                if os.path.exists(os.path.join(CSRC, h)):
                    assert h in files, (symbol, f, h)
    # the scan compiles step 4's prefix from the bucket header
    assert "mita_bucket.hpp" in bench.kernel_sources("k_scan")


def test_counted_traffic_turns_null_on_other_sources(monkeypatch):
    recs = bench.COUNTED_TRAFFIC["len_1m"]
    monkeypatch.setitem(recs, "k_attend", {"sha": "000000000000", "bytes": 1})
    assert bench.counted_traffic("len_1m", "k_attend") is None
    monkeypatch.setitem(recs, "k_attend", {"sha": bench.kernel_sha("k_attend"), "bytes": 7})
    assert bench.counted_traffic("len_1m", "k_attend") == 7


def test_multi_gpu_request_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
