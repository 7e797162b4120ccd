"""The counter summary bench.py builds from two rocprofv3 --pmc CSVs: each
counter is scaled by its own reading for the 1 GiB copy, the switch dispatches
are averaged, and the SGMM dispatches are split into passes at each
segmentation (one or two launches) or, where a pass has none (up to 64
rows), at its shrink launch; prefill passes first, then the mixed-decode
steps. Synthetic CSVs in
the profile run's dispatch order; no GPU."""
import csv
import json

import bench

SWITCH = "void dlm::switch_bf16_kernel<1, 256>(dlm::SwitchArgs)"
SG = ("segment", "shrink", "vsum", "expand")
_SHRINK = "void dlm::(anonymous namespace)::sgmm_shrink_bf16<1, true>(dlm::SgmmArgs)"
_VSUM = "dlm::(anonymous namespace)::sgmm_vsum_kernel(dlm::SgmmArgs)"
_EXPAND = "void dlm::(anonymous namespace)::sgmm_expand_bf16<1, true>(dlm::SgmmArgs)"
_COUNT = "dlm::(anonymous namespace)::sgmm_seg_count(int const*, float const*, long, int, char*, dlm::SgLayout)"
_PLACE = ("dlm::(anonymous namespace)::sgmm_seg_place(int const*, float const*, long, int, char*, "
          "dlm::SgLayout, int*)")
# (kernel name, share of the kind's counter value) per dispatch: the prefill
# (4096 rows) segments with a count and a placing launch, mixed decode (64 rows)
# has no segmentation launch (its shrink and expand order the rows)
KERNELS = [{"segment": [(_COUNT, 0.25), (_PLACE, 0.75)], "shrink": [(_SHRINK, 1.0)], "vsum": [(_VSUM, 1.0)],
            "expand": [(_EXPAND, 1.0)]},
           {"segment": [], "shrink": [(_SHRINK, 1.0)], "vsum": [(_VSUM, 1.0)],
            "expand": [(_EXPAND, 1.0)]}]


def _csv(path, counter, per_kernel, copy_kib):
    d = 0
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for v in (100.0, 300.0):
            d += 1
            w.writerow([d, SWITCH, counter, v])
        for wl in range(2):
            for _ in range(bench.SGMM_PROFILE_PASSES):
                for k in SG:
                    for name, share in KERNELS[wl][k]:
                        d += 1
                        w.writerow([d, name, counter, per_kernel[wl][k] * share])
        d += 1
        w.writerow([d, "__amd_rocclr_copyBuffer", counter, copy_kib])


def test_traffic_summary_from_counter_csvs(tmp_path):
    pk = [dict(segment=1.0, shrink=1000.0, vsum=10.0, expand=2000.0),
          dict(segment=2.0, shrink=3000.0, vsum=20.0, expand=4000.0)]
    F, W, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.json"
    _csv(F, "FETCH_SIZE", pk, 2 ** 19)    # the copy's reads counted at half
    _csv(W, "WRITE_SIZE", pk, 2 ** 20)
    bench.traffic_from(str(F), str(W), lambda m: None, out_path=str(out))
    t = json.loads(out.read_text())
    sw = t["switch_bf16_7b"]
    assert sw["fetch"]["launches"] == 2 and sw["fetch"]["scale"] == 2.0 and sw["write"]["scale"] == 1.0
    assert sw["bytes_per_launch"] == 200.0 * 1024 * 2 + 200.0 * 1024
    pre, mix = t["sgmm_sgmm-prefill"], t["sgmm_mixed-decode"]
    assert pre["kernels"]["shrink"] == {"read": 1000.0 * 1024 * 2, "write": 1000.0 * 1024}
    # both segmentation launches of a prefill pass count as its segment
    assert pre["kernels"]["segment"] == {"read": 1.0 * 1024 * 2, "write": 1.0 * 1024}
    assert mix["kernels"]["segment"] == {"read": 0.0, "write": 0.0}
    assert mix["kernels"]["shrink"] == {"read": 3000.0 * 1024 * 2, "write": 3000.0 * 1024}
    assert mix["kernels"]["expand"] == {"read": 4000.0 * 1024 * 2, "write": 4000.0 * 1024}
    assert pre["read_per_step"] == sum(pk[0].values()) * 1024 * 2
    assert mix["write_per_step"] == (sum(pk[1].values()) - pk[1]["segment"]) * 1024
    assert pre["algo_bytes_per_step"] == 1007812608   # 4096 tokens x 7 projections, Zipf pairs
    assert pre["source_hash"] == bench._src_hash(bench.SGMM_SOURCES)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 (or a multi-rank launch) exits
    with a message before touching a device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for args, env in ((["--gpus", "2"], {}), (["--gpus", "1"], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *args], capture_output=True,
                           text=True, timeout=120, env={**os.environ, **env})
        assert r.returncode == 2, (args, env, r.returncode)
        assert "one GPU" in r.stderr and not r.stdout.strip()
