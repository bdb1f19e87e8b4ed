"""Host-side logic of bench.py: the committed counter figures it reports as
`roofline.traffic`, and the contract of its command line (no GPU needed)."""
import json
import os
import subprocess
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, REPO)
import bench  # noqa: E402


def _entries():
    with open(os.path.join(REPO, "profiles", "pmc_traffic.json")) as fh:
        return json.load(fh)


def test_traffic_entries_well_formed():
    """Every committed counter figure names the kernel sources it was taken
    on (the bench reports null once those change) and adds up."""
    data = _entries()
    assert data, "no counter figures committed"
    for key, ent in data.items():
        assert len(ent["src_sha256"]) == 64, key
        assert ent["bytes_per_launch"] == pytest.approx(ent["fetch_bytes"] + ent["write_bytes"])
        assert ent["fetch_factor"] > 0 and ent["write_factor"] > 0


def test_traffic_lookup_rules():
    data = _entries()
    key = "gemm_tiled_kernel<gated>@mixtral"
    h = data[key]["src_sha256"]   # the sources the figure was taken on
    assert bench.pmc_traffic(key, h, 1) == data[key]["bytes_per_launch"]
    # a forced plan runs other kernels than the counters saw
    assert bench.pmc_traffic(key, h, 1, 0, 4) is None
    # changed sources void the figure
    assert bench.pmc_traffic(key, "0" * 64, 1) is None
    # unknown workload
    assert bench.pmc_traffic("gemm_tiled_kernel<gated>@tiny", h, 1) is None
    # figures of one routing seed answer for that seed only
    seeded = [k for k, e in data.items() if e.get("seed") is not None]
    for k in seeded:
        s, hk = data[k]["seed"], data[k]["src_sha256"]
        assert bench.pmc_traffic(k, hk, 1, s) == data[k]["bytes_per_launch"]
        assert bench.pmc_traffic(k, hk, 1, s + 1) is None


def test_several_gpus_is_refused():
    r = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=REPO, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)


def test_source_hash_ignores_comments_only():
    a = "int f(int x) {\n  return x + 1;  // one more\n}\n/* block\n comment */\n"
    b = "int f(int x) {\n    return x + 1;\n}\n"
    c = "int f(int x) {\n  return x + 2;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
