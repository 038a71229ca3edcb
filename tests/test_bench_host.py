"""Host logic of the benchmark that needs no GPU: the key that ties the
recorded HBM byte counters to the kernel code they were taken on, and the
algorithmic byte counts."""
import json
import os

import bench


def test_code_key_ignores_comments_and_layout():
    a = "int f(int x) {\n    return x + 1;  // one more\n}\n/* block\n comment */\n"
    b = "int f(int x) { return x + 1; }\n"
    c = "int f(int x) {\n    return x + 2;  // one more\n}\n"
    assert bench.code_only(a) == bench.code_only(b)
    assert bench.code_only(a) != bench.code_only(c)


def test_source_key_changes_with_the_code_only():
    orig = {}

    def read(name):
        path = os.path.join(bench.ROOT, "linear_recurrence_sequence_diag_amd", "csrc", name)
        if name not in orig:
            with open(path) as f:
                orig[name] = f.read()
        return orig[name]

    base = bench.kernel_sources_sha256("real", read)
    assert base == bench.kernel_sources_sha256("real")
    commented = bench.kernel_sources_sha256(
        "real", lambda n: read(n) + ("\n// a note\n" if n == "fused.hip" else ""))
    assert commented == base
    changed = bench.kernel_sources_sha256(
        "real", lambda n: read(n) + ("\nstatic int extra;\n" if n == "fused.hip" else ""))
    assert changed != base


def test_traffic_record_is_well_formed():
    path = os.path.join(bench.ROOT, "profiles", "hbm_traffic.json")
    with open(path) as f:
        rec = json.load(f)
    assert rec["copy_factor"]["FETCH_SIZE"] > 0 and rec["copy_factor"]["WRITE_SIZE"] > 0
    for name, w in rec["workloads"].items():
        assert len(w["source_sha256"]) == 64, name
        for d in ("forward", "backward"):
            assert w[d]["fetch_kib"] > 0 and w[d]["write_kib"] > 0, (name, d)


def test_algorithmic_bytes():
    # forward 3 s N + 4 B D, backward 5 s N (the fp32 state `last` in the forward)
    B, T, D = 2, 3, 5
    N = B * T * D
    fwd, bwd = bench.algorithmic_bytes(B, T, D, 2)
    assert fwd == 3 * 2 * N + 4 * B * D
    assert bwd == 5 * 2 * N
