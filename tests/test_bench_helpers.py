"""Host-side helpers of bench.py: the kernel-source digest that ties a
committed counter summary (profiles/traffic_*.txt) to the code it was taken
on.  Comments and blank space do not count as a change of the kernel; any
change of code does."""

import os

import bench


def test_code_only_ignores_prose_not_code():
    src = "int f(int x) {\n  // doubled\n  return 2 * x; /* twice */\n}\n"
    assert bench._code_only(src) == bench._code_only("/* header */\nint f(int x) {\n\n  return   2 * x;\n}\n")
    assert bench._code_only(src) != bench._code_only(src.replace("2 * x", "3 * x"))
    # block comments spanning lines are removed whole
    assert bench._code_only("a;/* x\ny */b;") == "a; b;"


def test_committed_traffic_summaries_name_known_kernels():
    prof = os.path.join(bench.ROOT, "profiles")
    names = [n for n in os.listdir(prof) if n.startswith("traffic_") and n.endswith(".txt")]
    assert names
    for n in names:
        kern = max((k for k in bench.KERNEL_SOURCE if n.startswith(f"traffic_{k}_")), key=len)
        workload = n[len(f"traffic_{kern}_"):-len(".txt")]
        fields = dict(l.split(":", 1) for l in open(os.path.join(prof, n)) if ":" in l and not l.startswith("#"))
        assert int(fields["traffic_bytes"]) > 0
        # the lookup bench.py makes returns the bytes while the code matches
        if fields["source_sha256"].strip() == bench.source_digest(kern):
            assert bench.measured_traffic(kern, workload) == int(fields["traffic_bytes"])
        else:
            assert bench.measured_traffic(kern, workload) is None
