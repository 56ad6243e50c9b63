"""Host logic of bench.py that needs no GPU: the refusal of several GPUs, the kernel-source
hash that keys the committed HBM-traffic counters (comment edits keep it, code edits change it),
and the attended-pair count that the query-block roofline's flops come from."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_code_only_drops_comments_and_spacing_but_keeps_code():
    b = load_bench()
    base = 'int a = 1;  // note\n/* block\n comment */ const char* s = "x // y";\n'
    assert b._code_only(base) == 'int a = 1; const char* s = "x // y";'
    assert b._code_only(base.replace("note", "other note")) == b._code_only(base)
    assert b._code_only(base.replace("a = 1", "a = 2")) != b._code_only(base)


def test_traffic_record_lookup():
    b = load_bench()
    with open(b.TRAFFIC_FILE) as f:
        rec = json.load(f)
    assert {r["workload"] for r in rec["records"]} >= {"config2"}
    for r in rec["records"]:
        assert r["hbm_bytes_per_launch"] == r["fetch_bytes_per_launch"] + r["write_bytes_per_launch"]
        assert 1.0 <= r["fetch_bytes_per_launch"] / r["algorithmic_bytes_per_launch"] < 1.05
    # reported only while the kernel code is the profiled one
    expect = rec["records"][0]["hbm_bytes_per_launch"]
    got = b.measured_traffic(rec["records"][0]["workload"], rec["records"][0]["schedule"])
    assert got == (expect if rec["kernel_source_hash"] == b.kernel_source_hash() else None)
    assert b.measured_traffic("no such workload", "balanced") is None


def test_several_gpus_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_attended_pairs_matches_a_brute_force_count():
    """(query token, key) pairs per query head: token i of q_len sits at L - q_len + i and
    attends keys max(0, p + 1 - W) .. p; counted here key by key."""
    b = load_bench()
    from workloads import make_workload

    for window in (0, 5, 40):
        wl = make_workload(name="pairs", seq_lens=[0, 1, 3, 7, 30, 100], num_q_heads=4,
                           num_kv_heads=2, head_dim=64, block_size=16, seed=[1, window],
                           window=window, q_len=7)
        want = 0
        for L in wl.seq_lens:
            for i in range(wl.q_len):
                p = int(L) - wl.q_len + i
                for t in range(0, max(p + 1, 0)):
                    if window == 0 or t > p - window:
                        want += 1
        assert b.attended_pairs(wl) == want
        assert isinstance(b.attended_pairs(wl), int) and want > 0
