"""bench.py reports measured HBM traffic only while the counter summary in
profiles/ matches the library it was taken from: every source and every
unit's compiler flags.  A changed source or flag must give None (host-only
check on a copy of the tree: no GPU, no library call)."""
import hashlib
import json
import os
import shutil

import bench
from bitwise_reproducible_lsq_amd import build as brl_build


def _summary(root, kernels):
    srcs = ["bitwise_reproducible_lsq_amd/csrc/replay.hip", "include/brlsq.h"]
    flags = {u: [f for f in brl_build.FLAGS + brl_build.EXTRA.get(u, []) if not f.startswith("-I")]
             for u in brl_build.SOURCES}
    return {"sources_sha256": {s: hashlib.sha256(open(os.path.join(root, s), "rb").read()).hexdigest()
                               for s in srcs},
            "flags_sha256": hashlib.sha256(json.dumps(flags, sort_keys=True).encode()).hexdigest(),
            "kernels": {k: {"bytes": b} for k, b in kernels.items()}}


def test_traffic_follows_sources_and_flags(tmp_path, monkeypatch):
    root = str(tmp_path)
    for d in (os.path.join("bitwise_reproducible_lsq_amd", "csrc"), "include"):
        shutil.copytree(os.path.join(bench.ROOT, d), os.path.join(root, d))
    os.makedirs(os.path.join(root, "profiles"))
    kernels = {"k [a]": 1000.0, "k [b]": 2500.0}
    with open(os.path.join(root, "profiles", "hbm_traffic_bench_step.json"), "w") as f:
        json.dump(_summary(root, kernels), f)
    monkeypatch.setattr(bench, "ROOT", root)
    assert bench.measured_traffic(["k [a]"]) == 1000
    assert bench.measured_traffic(["k [a]", "k [b]"], weights=[1, 4]) == 2200   # (1000 + 4 * 2500) / 5
    assert bench.measured_traffic(["k [c]"]) is None
    # another compiler flag: stale
    monkeypatch.setattr(brl_build, "FLAGS", brl_build.FLAGS + ["-DSOMETHING"])
    assert bench.measured_traffic(["k [a]"]) is None
    monkeypatch.undo()
    monkeypatch.setattr(bench, "ROOT", root)
    assert bench.measured_traffic(["k [a]"]) == 1000
    # a changed source: stale
    with open(os.path.join(root, "bitwise_reproducible_lsq_amd", "csrc", "replay.hip"), "a") as f:
        f.write("\n// changed\n")
    assert bench.measured_traffic(["k [a]"]) is None
