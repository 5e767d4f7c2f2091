"""Address and undefined-behaviour sanitizer run of the host-side planner
(csrc/plan.cpp) and owner-assignment solver (csrc/assign.cpp).

tests/native/host_check.cpp drives both sources; this test compiles it with
g++ -fsanitize=address,undefined (no recovery: any report ends the process
with an error) and checks that what it prints equals what the library returns
for the same inputs: plan texts of every workload and of ragged mixed sets
under forced forms, tile plans, lane counts and a small workspace cap (which
splits sets into chunks), owner assignments, and a tune-cache round trip
with a damaged file."""
import os
import random
import shutil
import subprocess

import pytest

import workloads as WL
import matrix_orthogonalizing_optimizer_muon_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "matrix_orthogonalizing_optimizer_muon_amd", "csrc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=24")


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("san") / "host_check")
    cmd = [gxx, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", f"-I{CSRC}", os.path.join(ROOT, "tests", "native", "host_check.cpp"),
           os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "assign.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe, args, stdin):
    r = subprocess.run([exe, *map(str, args)], input=stdin, capture_output=True, text=True, env=ENV,
                       timeout=300)
    assert r.returncode == 0, f"{args}: rc {r.returncode}\n{r.stderr[-4000:]}"
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    return r.stdout


DT = {WL.F32: 0, WL.BF16: 1}
PREC = {"auto": 0, "fp32": 1, "bf16": 2}
FORM = {"auto": 0, "direct": 1, "gram": 2}


def _cases():
    out = []
    for cfg in (1, 2, 3, 4, 5):
        wl = WL.workload(cfg)
        out.append((f"workload{cfg}", list(wl.shapes), [wl.dtype] * wl.n_matrices, {}))
    rng = random.Random(3)
    shapes = [(rng.randint(1, 1500), rng.randint(1, 1500)) for _ in range(24)] + [(1, 1), (1, 5000), (4097, 3)]
    dts = [rng.choice([WL.F32, WL.BF16]) for _ in shapes]
    out.append(("ragged", shapes, dts, {}))
    for t in range(10):
        out.append((f"ragged_tile{t}", shapes, dts, {"tile": t}))
    out.append(("ragged_gram", shapes, dts, {"form": "gram"}))
    out.append(("ragged_direct_bf16", shapes, dts, {"form": "direct", "precision": "bf16"}))
    out.append(("ragged_fp32", shapes, dts, {"precision": "fp32"}))
    out.append(("ragged_lanes3_cap", shapes, dts, {"lanes": 3, "workspace_cap": 64 << 20}))
    wl = WL.workload(2)
    out.append(("blocks_lanes4_cap", list(wl.shapes), [wl.dtype] * 16, {"lanes": 4, "workspace_cap": 100 << 20}))
    return out


@pytest.mark.parametrize("name,shapes,dts,kw", _cases(), ids=[c[0] for c in _cases()])
def test_planner_under_sanitizers_matches_library(harness, name, shapes, dts, kw):
    stdin = "".join(f"{r} {c} {DT[d]}\n" for (r, c), d in zip(shapes, dts))
    args = ["plan", kw.get("tile", -1), FORM[kw.get("form", "auto")], kw.get("lanes", 1),
            kw.get("workspace_cap", 0), PREC[kw.get("precision", "auto")]]
    got = _run(harness, args, stdin)
    plan = M.MuonPlan(shapes, dts, host_only=True, tune="off", tile=kw.get("tile"),
                      form=kw.get("form", "auto"), lanes=kw.get("lanes"),
                      precision=kw.get("precision", "auto"), workspace_cap=kw.get("workspace_cap", 0))
    want = plan.serialize()
    want = want.decode() if isinstance(want, bytes) else want
    assert got == want
    plan.close()


def test_assignment_under_sanitizers_matches_library(harness):
    rng = random.Random(17)
    for trial in range(40):
        n = rng.randint(0, 60)
        k = rng.randint(1, 9)
        costs = [round(rng.uniform(0.5, 100.0), 3) for _ in range(n)]
        limit = rng.choice([1, 100, 2000000])
        out = _run(harness, ["assign", k, limit], "".join(f"{c!r}\n" for c in costs)).split("\n")
        span, optimal = out[0].split()
        owner = [int(x) for x in out[1:] if x]
        want = M.assign_owners(costs, k, node_limit=limit)
        assert (owner, float(span), optimal == "1") == want


def test_tune_cache_round_trip_under_sanitizers(harness, tmp_path):
    out = _run(harness, ["cache", tmp_path / "tune.txt"], "")
    assert out.splitlines() == ["shapes 2 sets 1 other 0", "m=256 n=512 path=0 form=2 tile=0",
                                "m=1024 n=4096 path=1 form=1 tile=6", "set key tile=2 lanes=3",
                                "damaged shapes 2 sets 1"]
