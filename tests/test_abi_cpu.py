"""The C-ABI library on the CPU: it loads, exports every function include/muon.h
declares, and its host-only planner is deterministic and validates input.
No compute call is made (no GPU here)."""
import ctypes
import os
import re

import pytest

import matrix_orthogonalizing_optimizer_muon_amd as M
from matrix_orthogonalizing_optimizer_muon_amd import _lib as L
import workloads as WL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "muon.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_function_is_exported_and_bound():
    lib = L.lib()
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
        assert n in L.PROTOTYPES, f"{n} has no ctypes prototype"
    assert set(L.PROTOTYPES) == set(names)
    assert lib.muon_abi_version() == 13


def test_struct_sizes_match_header_layout():
    assert ctypes.sizeof(L.MatrixDesc) == 24
    assert ctypes.sizeof(L.PlanOpts) == 56
    opts = L.PlanOpts()
    assert L.lib().muon_plan_opts_default(ctypes.byref(opts)) == 0
    assert opts.struct_size == ctypes.sizeof(L.PlanOpts)
    assert opts.nesterov == 1 and abs(opts.eps - 1e-7) < 1e-12 and abs(opts.rms_scale - 0.2) < 1e-7
    assert opts.tile == -1 and opts.form == 0 and opts.precision == 0 and opts.lanes == 0
    assert ctypes.sizeof(L.PlanInfo) == 64


def _host(shapes, dtype="bf16", **kw):
    return M.MuonPlan(shapes, dtype, host_only=True, **kw)


def test_grouping_of_c2_and_plan_determinism():
    wl = WL.workload(2)
    a = _host(wl.shapes)
    b = _host(wl.shapes)
    assert a.serialize() == b.serialize()
    info = a.info()
    assert info["n_matrices"] == 16 and info["n_chunks"] == 1
    # canonical keys: 1024x1024, 1024x3072, 1024x4096 (up is the transposed down shape)
    assert info["n_groups"] == 3
    assert a.matrix_choice(2)["group"] == a.matrix_choice(3)["group"]
    assert a.matrix_choice(0)["group"] != a.matrix_choice(1)["group"]
    # symmetric-aware flops at T = 5: T (m^2 n + m^2(m+1)... ) summed per matrix
    want = 0.0
    for r, c in wl.shapes:
        m, n = min(r, c), max(r, c)
        want += 5 * (n * m * (m + 1) + m * m * (m + 1) + 2.0 * m * m * n)
    assert info["ns_flops_min"] == pytest.approx(want, rel=1e-12)
    assert info["ns_flops_issued"] >= info["ns_flops_min"]


def test_plan_is_invariant_to_repeat_and_records_order():
    shapes = [(300, 100), (100, 300), (64, 64), (300, 100)]
    p1 = _host(shapes)
    for _ in range(20):
        assert _host(shapes).serialize() == p1.serialize()
    # equal shapes share a group; the transposed shape shares its canonical key
    g = [p1.matrix_choice(i)["group"] for i in range(4)]
    assert g[0] == g[1] == g[3] and g[2] != g[0]


def test_workspace_cap_makes_chunks_and_rejects_oversize():
    shapes = [(1024, 4096)] * 6
    one = _host(shapes)
    ws1 = one.info()["workspace_bytes"] // 6
    p = _host(shapes, workspace_cap=2 * ws1)
    info = p.info()
    assert info["n_chunks"] == 3
    assert info["workspace_bytes"] == 2 * ws1
    assert [p.matrix_choice(i)["chunk"] for i in range(6)] == [0, 0, 1, 1, 2, 2]
    with pytest.raises(M.MuonError) as e:
        _host(shapes, workspace_cap=ws1 - 1)
    assert e.value.code == L.MUON_ENOMEM


def test_invalid_arguments():
    lib = L.lib()
    out = ctypes.c_void_p()
    assert lib.muon_plan_create(None, 1, None, ctypes.byref(out)) == L.MUON_EINVAL
    descs = (L.MatrixDesc * 1)()
    descs[0].rows, descs[0].cols, descs[0].dtype = 0, 8, 1
    assert lib.muon_plan_create(descs, 1, None, ctypes.byref(out)) in (L.MUON_EUNSUPPORTED, L.MUON_EINVAL)
    descs[0].rows, descs[0].dtype = 8, 7
    assert lib.muon_plan_create(descs, 1, None, ctypes.byref(out)) == L.MUON_EUNSUPPORTED
    assert lib.muon_plan_create(descs, 0, None, ctypes.byref(out)) == L.MUON_EINVAL
    descs[0].dtype, descs[0].reserved = 1, 3
    assert lib.muon_plan_create(descs, 1, None, ctypes.byref(out)) == L.MUON_EINVAL
    assert lib.muon_last_error()
    with pytest.raises(M.MuonError):
        _host([(8, 8)], eps=-1.0)
    assert lib.muon_plan_destroy(None) == L.MUON_OK


def test_step_refuses_host_only_plan():
    p = _host([(16, 32)])
    lib = L.lib()
    arr = (ctypes.c_void_p * 1)(1)
    rc = lib.muon_step(p._h, arr, arr, arr, 0.02, 0.95, 0.01, 5, None, None)
    assert rc == L.MUON_ESTATE


def test_forced_forms_and_cost_model():
    p = _host([(512, 16384), (1024, 1024)], form="gram")
    assert p.matrix_choice(0)["form"] == "gram" and p.matrix_choice(1)["form"] == "gram"
    q = _host([(512, 16384), (1024, 1024)], form="direct")
    assert q.info()["n_gram"] == 0
    # the cost model never picks Gram for a square matrix
    r = _host([(2048, 2048)])
    assert r.matrix_choice(0)["form"] == "direct"


def _set_key(entries, forced_lanes=0):
    """Key of a matrix set in the tune cache: FNV-1a (64-bit) of
    "m,n,path,count,form,tile;" per canonical shape key, keys in (path, m, n)
    order, then "lanes=<forced lane count>"."""
    text = "".join(f"{m},{n},{p},{c},{f},{t};" for (p, m, n, c, f, t) in sorted(entries))
    text += f"lanes={forced_lanes}"
    h = 1469598103934665603
    for b in text.encode():
        h = ((h ^ b) * 1099511628211) % (1 << 64)
    return f"{h:016x}"


def test_tune_cache_set_line_gives_every_direct_shape_one_tile_plan(tmp_path):
    shapes = [(3072, 1024), (1024, 3072), (1024, 1024), (1024, 1024), (4096, 1024)]
    shape_lines = ("muon-tune-v4 host m=1024 n=1024 path=1 form=1 tile=0 us=1\n"
                   "muon-tune-v4 host m=1024 n=3072 path=1 form=1 tile=0 us=1\n"
                   "muon-tune-v4 host m=1024 n=4096 path=1 form=1 tile=1 us=1\n")
    key = _set_key([(1, 1024, 1024, 2, 1, 0), (1, 1024, 3072, 2, 1, 0), (1, 1024, 4096, 1, 1, 1)])
    other = _set_key([(1, 1024, 1024, 2, 1, 0)])
    path = tmp_path / "tune.txt"
    path.write_text(shape_lines)
    per_shape = _host(shapes, cache_path=str(path))
    assert [per_shape.matrix_choice(i)["tile"] for i in range(5)] == [0, 0, 0, 0, 1]
    path.write_text(shape_lines + f"muon-tune-v4 host set={key} tile=2 us=5\n")
    p = _host(shapes, cache_path=str(path))
    assert [p.matrix_choice(i)["tile"] for i in range(5)] == [2] * 5
    assert p.info()["n_lanes"] == 1
    path.write_text(shape_lines + f"muon-tune-v4 host set={key} tile=-1 lanes=2 us=5\n")
    q = _host(shapes, cache_path=str(path))
    assert [q.matrix_choice(i)["tile"] for i in range(5)] == [0, 0, 0, 0, 1]
    assert q.info()["n_lanes"] == 2 and {q.matrix_choice(i)["lane"] for i in range(5)} == {0, 1}
    # -1 keeps the per-shape choices; other sets, bad keys, tiles and lane counts are ignored
    for line in (f"set={key} tile=-1 us=5", f"set={other} tile=2 us=5", f"set={key[:-1]} tile=2 us=5",
                 f"set={key.upper()} tile=2 us=5", f"set={key} tile=10 us=5", f"set={key} us=5",
                 f"set={key} tile=2 lanes=5 us=5", f"set={key} tile=2 lanes=0 us=5"):
        path.write_text(shape_lines + f"muon-tune-v4 host {line}\n")
        q = _host(shapes, cache_path=str(path))
        assert q.serialize() == per_shape.serialize(), line
    # a forced tile plan takes only the lane count of its own set line
    path.write_text(shape_lines + f"muon-tune-v4 host set={key} tile=2 lanes=2 us=5\n")
    f = _host(shapes, cache_path=str(path), tile=1)
    assert [f.matrix_choice(i)["tile"] for i in range(5)] == [1] * 5 and f.info()["n_lanes"] == 1
    fkey = _set_key([(1, 1024, 1024, 2, 1, 1), (1, 1024, 3072, 2, 1, 1), (1, 1024, 4096, 1, 1, 1)])
    path.write_text(shape_lines + f"muon-tune-v4 host set={fkey} tile=2 lanes=4 us=5\n")
    f = _host(shapes, cache_path=str(path), tile=1)
    assert [f.matrix_choice(i)["tile"] for i in range(5)] == [1] * 5 and f.info()["n_lanes"] == 4
    # forced lanes: the set line (keyed with the forced count) gives only the tile plan
    lkey = _set_key([(1, 1024, 1024, 2, 1, 0), (1, 1024, 3072, 2, 1, 0), (1, 1024, 4096, 1, 1, 1)], 2)
    path.write_text(shape_lines + f"muon-tune-v4 host set={lkey} tile=2 lanes=4 us=5\n")
    g = _host(shapes, cache_path=str(path), lanes=2)
    assert [g.matrix_choice(i)["tile"] for i in range(5)] == [2] * 5 and g.info()["n_lanes"] == 2


def test_lanes_cut_each_chunk_into_runs_of_equal_work():
    wl = WL.workload(2)
    for lanes in (1, 2, 3, 4):
        p = _host(wl.shapes, lanes=lanes)
        assert p.info()["n_lanes"] == lanes
        ch = [p.matrix_choice(i) for i in range(len(wl.shapes))]
        # lanes follow the group order: sorting by (group, index) gives non-decreasing lanes
        order = sorted(range(len(ch)), key=lambda i: (ch[i]["group"], i))
        got = [ch[i]["lane"] for i in order]
        assert got == sorted(got) and set(got) == set(range(lanes))
        work = [0.0] * lanes
        for i, (r, c) in enumerate(wl.shapes):
            m, n = min(r, c), max(r, c)
            work[ch[i]["lane"]] += n * m * (m + 1) + m * m * (m + 1) + 2.0 * m * m * n
        # no lane exceeds its share by more than one matrix's work
        biggest = max(2.0 * min(s) ** 2 * max(s) * 2 for s in wl.shapes)
        assert max(work) <= sum(work) / lanes + biggest
        # the plan text names every lane
        assert f"lanes={lanes}".encode() in p.serialize()
    with pytest.raises(M.MuonError):
        _host(wl.shapes, lanes=5)


def test_tune_cache_is_read_and_bad_lines_ignored(tmp_path):
    path = tmp_path / "tune.txt"
    path.write_text(
        "garbage line\n"
        "muon-tune-v4 host m=512 n=16384 path=1 form=2 tile=1 us=400\n"
        "muon-tune-v4 host m=1024 n=1024 path=1 form=9 tile=0 us=1\n"
        "muon-tune-v4 host m=2048 n=2048 path=1 form=1 tile=10 us=1\n"
        "muon-tune-v1 host m=256 n=256 path=1 form=2 tile=0 us_direct=1 us_gram=1\n"
        "muon-tune-v4 otherdev m=64 n=64 path=1 form=2 tile=0 us=1\n")
    shapes = [(512, 16384), (1024, 1024), (64, 64), (2048, 2048), (256, 256)]
    p = _host(shapes, cache_path=str(path))
    model = _host(shapes, tune="off")
    c0 = p.matrix_choice(0)
    assert (c0["form"], c0["tile"]) == ("gram", 1)   # from the cache
    for i in range(1, 5):                            # malformed, other device, old format -> model
        got, want = p.matrix_choice(i), model.matrix_choice(i)
        assert (got["form"], got["tile"]) == (want["form"], want["tile"])
    p2 = _host(shapes, cache_path=str(path))
    assert p2.serialize() == p.serialize()
    # tune off ignores the cache
    p3 = _host([(512, 16384)], cache_path=str(path), tune="off")
    assert p3.serialize() == _host([(512, 16384)], tune="off").serialize()
    # a forced form or tile never takes a cached choice that violates it
    p4 = _host([(512, 16384)], cache_path=str(path), form="direct")
    assert p4.matrix_choice(0)["form"] == "direct"


def test_orthogonalize_marshalling_and_host_only_refusal():
    p = _host([(16, 32), (32, 16)])
    lib = L.lib()
    ins = (ctypes.c_void_p * 2)(16, 32)
    outs = (ctypes.c_void_p * 2)(64, 128)
    sched = (ctypes.c_float * 3)(1.5, -0.5, 0.0)
    assert lib.muon_orthogonalize(p._h, ins, outs, 1, sched, None) == L.MUON_ESTATE
    assert lib.muon_orthogonalize(None, ins, outs, 1, sched, None) == L.MUON_EINVAL
    assert lib.muon_orthogonalize(p._h, ins, outs, 65, None, None) == L.MUON_EINVAL


def test_adamw_entry_points_refuse_bad_arguments_without_a_device():
    lib = L.lib()
    out = ctypes.c_void_p()
    ne = (ctypes.c_int64 * 2)(10, 20)
    dt = (ctypes.c_int32 * 2)(L.MUON_F32, L.MUON_BF16)
    assert lib.muon_adamw_plan_create(None, dt, 2, ctypes.byref(out)) == L.MUON_EINVAL
    assert lib.muon_adamw_plan_create(ne, dt, 0, ctypes.byref(out)) == L.MUON_EINVAL
    bad = (ctypes.c_int32 * 2)(L.MUON_F32, 9)
    assert lib.muon_adamw_plan_create(ne, bad, 2, ctypes.byref(out)) == L.MUON_EUNSUPPORTED
    arr = (ctypes.c_void_p * 1)(16)
    assert lib.muon_adamw_step(None, arr, arr, arr, arr, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, None) == L.MUON_EINVAL
    assert lib.muon_adamw_plan_destroy(None) == L.MUON_OK


def test_probes_refuse_bad_arguments_without_a_device():
    lib = L.lib()
    tf, fl, gbs = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    assert lib.muon_probe_mfma_bf16(0, ctypes.byref(tf), ctypes.byref(fl)) == L.MUON_EINVAL
    assert lib.muon_probe_mfma_bf16((1 << 24) + 1, ctypes.byref(tf), None) == L.MUON_EINVAL
    assert lib.muon_probe_mfma_bf16(10, None, None) == L.MUON_EINVAL
    a, b = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 24)   # never dereferenced
    assert lib.muon_probe_hbm_copy(None, b, 1024, 1, ctypes.byref(gbs)) == L.MUON_EINVAL
    assert lib.muon_probe_hbm_copy(a, b, 1000, 1, ctypes.byref(gbs)) == L.MUON_EINVAL      # not 16 | bytes
    assert lib.muon_probe_hbm_copy(a, b, 0, 1, ctypes.byref(gbs)) == L.MUON_EINVAL
    assert lib.muon_probe_hbm_copy(ctypes.c_void_p((1 << 20) + 8), b, 1024, 1, ctypes.byref(gbs)) == L.MUON_EINVAL
    assert lib.muon_probe_hbm_copy(a, ctypes.c_void_p((1 << 20) + 512), 1024, 1, ctypes.byref(gbs)) == L.MUON_EINVAL
    assert lib.muon_probe_hbm_copy(a, b, 1024, 0, ctypes.byref(gbs)) == L.MUON_EINVAL
    assert lib.muon_probe_hbm_copy(a, b, 1024, 1, None) == L.MUON_EINVAL


def test_graph_toggle_refuses_null_and_host_only_plans():
    lib = L.lib()
    assert lib.muon_plan_set_graph(None, 1) == L.MUON_EINVAL
    p = _host([(64, 128)])
    with pytest.raises(M.MuonError):
        p.set_graph(True)


_PLAN_DIGESTS = r"""
import hashlib, sys
import matrix_orthogonalizing_optimizer_muon_amd as M
import workloads as WL
cache = sys.argv[1]
for cfg in (1, 2, 3, 4, 5):
    wl = WL.workload(cfg)
    p = M.MuonPlan(wl.shapes, wl.dtype, host_only=True, cache_path=cache)
    print(cfg, hashlib.sha256(p.serialize()).hexdigest(), flush=True)
"""


def test_plans_are_byte_identical_across_runs_and_processes(tmp_path):
    """The plan is a function of (shapes, options, cache): 100 creations in this
    process and two fresh processes reading the same cache file give the same
    bytes for every workload's matrix set."""
    import hashlib
    import subprocess
    import sys
    cache = tmp_path / "tune.txt"
    cache.write_text("muon-tune-v4 host m=1024 n=4096 path=1 form=1 tile=6 us=1\n"
                     "muon-tune-v4 host m=512 n=16384 path=1 form=2 tile=8 us=1\n")
    here = {}
    for cfg in (1, 2, 3, 4, 5):
        wl = WL.workload(cfg)
        here[cfg] = hashlib.sha256(
            M.MuonPlan(wl.shapes, wl.dtype, host_only=True, cache_path=str(cache)).serialize()).hexdigest()
    wl2 = WL.workload(2)
    for _ in range(100):
        p = M.MuonPlan(wl2.shapes, wl2.dtype, host_only=True, cache_path=str(cache))
        assert hashlib.sha256(p.serialize()).hexdigest() == here[2]
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, PYTHONPATH=root + os.pathsep + os.environ.get("PYTHONPATH", ""))
    for _ in range(2):
        out = subprocess.run([sys.executable, "-c", _PLAN_DIGESTS, str(cache)], capture_output=True,
                             text=True, env=env, cwd=root, timeout=300)
        assert out.returncode == 0, out.stderr
        got = {int(a): b for a, b in (line.split() for line in out.stdout.split("\n") if line.strip())}
        assert got == here
    # the cached choices were taken
    p = M.MuonPlan(wl2.shapes, wl2.dtype, host_only=True, cache_path=str(cache))
    assert {p.matrix_choice(i)["tile"] for i in range(len(wl2.shapes))
            if max(wl2.shapes[i]) == 4096 and min(wl2.shapes[i]) == 1024} == {6}
