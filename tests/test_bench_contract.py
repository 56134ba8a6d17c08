"""Host-side checks of bench.py's command-line contract and its traffic table.

These run without a GPU: bench.py measures one GPU only and must refuse more
before it touches the device; the committed HBM-traffic table must be well
formed, and where its entry for the dominant kernel is current (taken on the
present sources; otherwise bench.py reports null) it must match the kernel's
algorithmic bytes.
"""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_table_has_counters_and_calibration():
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
        table = json.load(f)
    entries = {k: v for k, v in table.items() if not k.startswith("_")}
    assert "quantize_pc_kernel:quantize_k" in entries
    for key, e in entries.items():
        assert e["fetch_kib"] > 0 and e["write_kib"] > 0, key
        assert 1.5 < e["fetch_scale"] < 2.5 and 0.5 < e["write_scale"] < 1.5, key
        assert len(e["source_sha"]) == 16 and e["dispatches"] >= 1, key


def test_traffic_of_the_dominant_kernel_matches_its_algorithmic_bytes():
    # the decode step's dominant call: the counters were taken on these sources
    t = bench._traffic("quantize_pc_kernel:quantize_k", ["quantize.hip", "tq_device.h"])
    if t is None:
        pytest.skip("kernel sources changed since the counters were taken (bench reports null)")
    # within a few percent of the algorithmic bytes per launch (262144 keys:
    # 256 B read, 48 B of codes and signs and 4 B of norms written)
    assert abs(t / (262144 * (256 + 48 + 4)) - 1.0) < 0.05


def _counter_csv(path, counter, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for did, name, v in rows:
            f.write('%d,"%s",%s,%r\n' % (did, name, counter, v))


def test_write_traffic_scales_by_the_first_copy(tmp_path):
    """--write-traffic: the first copy kernel is the 512 MiB calibration, each
    entry is the mean over its instance's dispatches, rows of one dispatch add."""
    inst = bench.TRAFFIC_INSTANCES["quantize_pc_kernel:quantize_k"][0]
    other = "void ns::logit_kernel<128, 3, true, 1, false>(Args)"
    fetch = [(1, "void at::native::direct_copy_kernel(...)", 262144.0),
             (2, "void at::native::direct_copy_kernel(...)", 999999.0),     # a later, larger copy
             (3, "void ns::%s(Args)" % inst, 30000.0), (4, "void ns::%s(Args)" % inst, 34000.0),
             (5, other, 1000.0), (5, other, 500.0)]
    write = [(1, "void at::native::direct_copy_kernel(...)", 524288.0),
             (3, "void ns::%s(Args)" % inst, 13000.0), (4, "void ns::%s(Args)" % inst, 13000.0),
             (5, other, 100.0)]
    _counter_csv(str(tmp_path / "f" / "host" / "p_counter_collection.csv"), "FETCH_SIZE", fetch)
    _counter_csv(str(tmp_path / "w" / "host" / "p_counter_collection.csv"), "WRITE_SIZE", write)
    out = tmp_path / "t.json"
    bench.write_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(out))
    table = json.loads(out.read_text())
    e = table["quantize_pc_kernel:quantize_k"]
    assert e["fetch_scale"] == 2.0 and e["write_scale"] == 1.0
    assert e["fetch_kib"] == 32000.0 and e["write_kib"] == 13000.0 and e["dispatches"] == 2
    lc = table["logit_kernel:long_context"]
    assert lc["fetch_kib"] == 1500.0 and lc["write_kib"] == 100.0 and lc["dispatches"] == 1
    assert "dequant_kernel:dequantize_v" not in table
