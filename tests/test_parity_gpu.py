"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerance (relative Frobenius error of the fp32 pre-rounding update U):
1e-4 on the fp32 path, 2e-2 on the bf16-MFMA path."""
import numpy as np
import pytest

import workloads as WL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import matrix_orthogonalizing_optimizer_muon_amd as mod
    return mod


def _plan(M, shapes, dtype, **kw):
    kw.setdefault("tune", "off")
    return M.MuonPlan(shapes, dtype, **kw)


def test_single_fp32_256x512_matrix(M):
    from gpu_util import run_and_compare
    wl = WL.workload(1)
    Ws = [WL.draw(wl, 0, 0, WL.KIND_W)]
    Gs = [WL.draw(wl, 0, 0, WL.KIND_G)]
    Bs = [WL.Stored(np.zeros((256, 512)), np.zeros((256, 512), np.float32), WL.F32)]
    plan = _plan(M, wl.shapes, "f32")
    errs = run_and_compare(plan, Ws, Gs, Bs, WL.F32)
    print("c1", errs)


@pytest.mark.parametrize("coeffs,T", [((1.0, 0.0, 0.0), 1), ((0.0, 1.0, 0.0), 1),
                                      ((0.0, 0.0, 1.0), 1), ((3.4445, -4.7750, 2.0315), 2),
                                      ((1.5, -0.5, 0.0), 7)])
@pytest.mark.parametrize("dtype", [WL.F32, WL.BF16])
def test_single_stage_isolation(M, coeffs, T, dtype):
    """(1,0,0): X_T = X0 (elementwise + transpose paths); (0,1,0): A X; (0,0,1): A^2 X."""
    from gpu_util import make_state, run_and_compare
    shapes = [(200, 136), (136, 200)]
    Ws, Gs, Bs = make_state(shapes, dtype, seed=11)
    plan = _plan(M, shapes, dtype)
    run_and_compare(plan, Ws, Gs, Bs, dtype, ns_steps=T, coeffs=coeffs)


@pytest.mark.parametrize("dtype", [WL.F32, WL.BF16])
def test_ragged_mixed_shapes_one_plan(M, dtype):
    from gpu_util import make_state, run_and_compare
    shapes = [(100, 300), (300, 100), (129, 257), (1, 64), (64, 1), (513, 77), (7, 7),
              (256, 256), (300, 100)]
    Ws, Gs, Bs = make_state(shapes, dtype, seed=3, buf_scale=0.01)
    plan = _plan(M, shapes, dtype)
    run_and_compare(plan, Ws, Gs, Bs, dtype)


@pytest.mark.parametrize("form", ["direct", "gram"])
@pytest.mark.parametrize("dtype", [WL.F32, WL.BF16])
def test_plain_momentum_option(M, dtype, form):
    """nesterov=False orthogonalizes the momentum buffer itself (nonzero
    incoming buffers), with NS and with ns_steps = 0 (X_T = X0)."""
    from gpu_util import make_state, run_and_compare
    shapes = [(100, 300), (300, 100), (129, 257), (513, 77), (256, 640)]
    Ws, Gs, Bs = make_state(shapes, dtype, seed=21, buf_scale=0.01)
    plan = _plan(M, shapes, dtype, nesterov=False, form=form)
    run_and_compare(plan, Ws, Gs, Bs, dtype, nesterov=False)
    Ws2, Gs2, _ = make_state(shapes, dtype, seed=22)
    run_and_compare(plan, Ws2, Gs2, Bs, dtype, nesterov=False, ns_steps=0)


@pytest.mark.parametrize("dtype", [WL.F32, WL.BF16])
def test_gram_form_matches_oracle(M, dtype):
    from gpu_util import make_state, run_and_compare
    shapes = [(64, 1000), (1000, 64), (256, 2048), (130, 700)]
    Ws, Gs, Bs = make_state(shapes, dtype, seed=5)
    plan = _plan(M, shapes, dtype, form="gram")
    assert all(plan.matrix_choice(i)["form"] == "gram" for i in range(len(shapes)))
    run_and_compare(plan, Ws, Gs, Bs, dtype)
    for T in (1, 2, 0):
        run_and_compare(plan, Ws, Gs, Bs, dtype, ns_steps=T)


def test_ns_steps_zero_and_schedule(M):
    from gpu_util import make_state, run_and_compare
    shapes = [(96, 160), (160, 96)]
    Ws, Gs, Bs = make_state(shapes, WL.F32, seed=8)
    plan = _plan(M, shapes, "f32")
    run_and_compare(plan, Ws, Gs, Bs, WL.F32, ns_steps=0)
    sched = [(3.4445, -4.7750, 2.0315), (1.5, -0.5, 0.0), (2.0, -1.5, 0.5)]
    run_and_compare(plan, Ws, Gs, Bs, WL.F32, ns_steps=3, coeffs=sched)


@pytest.mark.parametrize("tune", ["off", "once"])
def test_transformer_block_set_three_steps_all_matrices(M, tune, tmp_path):
    """The transformer-block workload: 16 bf16 matrices, 3 steps, fresh
    gradients each step, momentum and weights carried over; with the cost
    model's plan and with the plan bench.py times (shapes and the whole set
    timed once into a fresh cache: tile plan and NS lanes)."""
    import torch
    from gpu_util import to_device, to_f64, rel
    from oracle import muon_oracle as O
    wl = WL.workload(2)
    plan = _plan(M, wl.shapes, "bf16", tune=tune, cache_path=str(tmp_path / "tune.txt"))
    print("transformer block set plan", tune, plan.info()["n_lanes"], "lanes,",
          sorted({(plan.matrix_choice(i)["form"], plan.matrix_choice(i)["tile"]) for i in range(wl.n_matrices)}))
    P = [to_device(WL.draw(wl, i, 0, WL.KIND_W)) for i in range(wl.n_matrices)]
    B = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in wl.shapes]
    cap = [torch.empty(s, dtype=torch.float32, device="cuda") for s in wl.shapes]
    worst = 0.0
    for step in range(wl.steps):
        Gst = [WL.draw(wl, i, step, WL.KIND_G) for i in range(wl.n_matrices)]
        G = [to_device(g) for g in Gst]
        W_before = [to_f64(p) for p in P]
        buf_before = [to_f64(b) for b in B]
        plan.set_update_capture(cap)
        plan.step(P, G, B)
        torch.cuda.synchronize()
        for i in range(wl.n_matrices):
            ref = O.muon_step_ref(W_before[i], Gst[i].value, buf_before[i], param_dtype="bf16")
            e = rel(cap[i].cpu().numpy().astype(np.float64), ref["U"])
            worst = max(worst, e)
            assert e <= 2e-2, f"step {step} matrix {i}: {e:.3e}"
            assert rel(to_f64(B[i]), ref["buf_new"]) <= 1e-6
            # weights: the GPU stores RNE(W + U_gpu); its delta carries the error of U plus
            # the bf16 rounding floor the oracle's own rounding of W + U shows
            Wn = to_f64(P[i])
            nU = np.linalg.norm(ref["U"])
            floor = np.linalg.norm(ref["W_new_stored"] - ref["W_new"]) / nU
            assert rel(Wn - W_before[i], ref["U"]) <= 2e-2 + 2.5 * floor
    plan.set_update_capture(None)
    print("transformer block set worst rel err", worst)


def test_bitwise_determinism(M):
    import torch
    from gpu_util import make_state, device_state
    shapes = [(384, 640), (640, 384), (128, 1024)]
    Ws, Gs, Bs = make_state(shapes, WL.BF16, seed=21, buf_scale=0.01)
    plan = _plan(M, shapes, "bf16")
    outs = []
    for _ in range(2):
        P, G, B = device_state(Ws, Gs, Bs)
        plan.step(P, G, B)
        torch.cuda.synchronize()
        outs.append([p.view(torch.int16).cpu().numpy().copy() for p in P] +
                    [b.cpu().numpy().copy() for b in B])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_zero_grad_lr_zero_and_nonfinite_flag(M):
    import torch
    from gpu_util import make_state, device_state, to_f64
    shapes = [(64, 96), (96, 64)]
    Ws, Gs, Bs = make_state(shapes, WL.F32, seed=2)
    plan = _plan(M, shapes, "f32")
    # zero gradient and zero momentum: pure decoupled decay
    P, G, B = device_state(Ws, Gs, Bs)
    for g in G:
        g.zero_()
    cap = [torch.empty(s, dtype=torch.float32, device="cuda") for s in shapes]
    plan.set_update_capture(cap)
    plan.step(P, G, B, lr=0.02, wd=0.01)
    torch.cuda.synchronize()
    for i in range(2):
        want = -0.02 * 0.01 * Ws[i].value
        assert np.max(np.abs(cap[i].cpu().numpy() - want)) <= 1e-9
    # lr = 0 leaves weights bit-identical and still moves the momentum
    P, G, B = device_state(Ws, Gs, Bs)
    before = [p.clone() for p in P]
    plan.step(P, G, B, lr=0.0)
    torch.cuda.synchronize()
    for a, b in zip(P, before):
        assert torch.equal(a, b)
    assert np.allclose(to_f64(B[0]), Gs[0].value, rtol=0, atol=0)
    plan.set_update_capture(None)
    assert plan.flags(clear=True) == 0
    # a NaN gradient raises the non-finite flag
    P, G, B = device_state(Ws, Gs, Bs)
    G[1][3, 5] = float("nan")
    plan.step(P, G, B)
    assert plan.flags(clear=True) & 1
    assert plan.flags() == 0


def test_plan_errors_and_host_checks(M):
    import torch
    with pytest.raises(M.MuonError):
        _plan(M, [(0, 5)], "bf16")
    plan = _plan(M, [(32, 64)], "bf16")
    good = [torch.zeros(32, 64, dtype=torch.bfloat16, device="cuda")]
    mom = [torch.zeros(32, 64, dtype=torch.float32, device="cuda")]
    with pytest.raises(ValueError):
        plan.step([torch.zeros(64, 32, dtype=torch.bfloat16, device="cuda")], good, mom)
    with pytest.raises(ValueError):
        plan.step(good, [torch.zeros(32, 64, dtype=torch.float32, device="cuda")], mom)
    with pytest.raises(M.MuonError):
        plan.step([good[0].clone()], good, mom, ns_steps=-1)


@pytest.mark.parametrize("tile", [0, 1, 2, 3, 4, 5, 6, 7, 8, 9])
def test_bf16_direct_every_tile_plan(M, tile):
    """Each NT tile plan (symmetric / m x n output tiles), ragged and tall shapes
    in one batched plan, T = 5, 1 and 2."""
    from gpu_util import make_state, run_and_compare
    shapes = [(300, 700), (700, 300), (129, 1000), (520, 520), (64, 2048), (300, 700)]
    Ws, Gs, Bs = make_state(shapes, WL.BF16, seed=40 + tile, buf_scale=0.01)
    plan = _plan(M, shapes, "bf16", tile=tile, form="direct")
    assert all(plan.matrix_choice(i)["tile"] == tile for i in range(len(shapes)))
    for T in (5, 1, 2):
        run_and_compare(plan, Ws, Gs, Bs, WL.BF16, ns_steps=T)


@pytest.mark.parametrize("tile", [0, 1, 2, 5, 6, 7, 8, 9])
def test_bf16_gram_every_tile_plan(M, tile):
    from gpu_util import make_state, run_and_compare
    shapes = [(200, 1500), (1500, 200), (256, 4096)]
    Ws, Gs, Bs = make_state(shapes, WL.BF16, seed=60 + tile)
    plan = _plan(M, shapes, "bf16", tile=tile, form="gram")
    assert all(plan.matrix_choice(i)["form"] == "gram" for i in range(len(shapes)))
    for T in (5, 1):
        run_and_compare(plan, Ws, Gs, Bs, WL.BF16, ns_steps=T)


def _mixed_lane_state():
    from gpu_util import make_state
    sb = [(300, 700), (700, 300), (129, 1000), (520, 520), (200, 1500), (64, 2048)]
    sf = [(256, 512), (96, 96)]
    Wb, Gb, Bb = make_state(sb, WL.BF16, seed=81, buf_scale=0.01)
    Wf, Gf, Bf = make_state(sf, WL.F32, seed=82, buf_scale=0.01)
    return sb + sf, ["bf16"] * len(sb) + ["f32"] * len(sf), Wb + Wf, Gb + Gf, Bb + Bf


@pytest.mark.parametrize("lanes,chunked,profiled", [(2, False, False), (3, False, False),
                                                     (4, False, False), (2, True, False),
                                                     (3, False, True)])
def test_lanes_give_bitwise_the_one_lane_result(M, lanes, chunked, profiled):
    """NS lanes change only which stream a launch goes to: three consecutive
    steps (bf16 direct and Gram, fp32 matrices, one or several workspace chunks)
    leave parameters and momenta bitwise equal to the one-lane plan's; so does
    profiling, which runs the lanes one after another with dispatch events."""
    import torch
    from gpu_util import device_state
    shapes, dts, Ws, Gs, Bs = _mixed_lane_state()
    cap = 0
    if chunked:
        cap = _plan(M, shapes, dts).info()["workspace_bytes"] // 2
    outs = []
    for L in (1, lanes):
        plan = _plan(M, shapes, dts, lanes=L, workspace_cap=cap)
        info = plan.info()
        assert info["n_lanes"] == L and (info["n_chunks"] >= 2) == chunked
        P, G, B = device_state(Ws, Gs, Bs)
        if profiled and L > 1:
            plan.set_profiling(True)
        for _ in range(3):
            plan.step(P, G, B)
        torch.cuda.synchronize()
        if profiled and L > 1:
            kt = plan.kernel_times(reset=False)
            iv = plan.launch_intervals()
            plan.set_profiling(False)
            # every launch recorded, with a dispatch interval of positive length;
            # serial lanes: no two intervals overlap
            assert sum(k["launches"] for k in kt) == len(iv) > 0
            assert all(0 <= x["start_ms"] < x["end_ms"] for x in iv)
            spans = sorted((x["start_ms"], x["end_ms"]) for x in iv)
            assert all(b[0] >= a[1] - 5e-3 for a, b in zip(spans, spans[1:]))
        assert plan.flags() == 0
        outs.append([p.view(torch.int16).cpu().numpy().copy() if p.dtype == torch.bfloat16
                     else p.cpu().numpy().copy() for p in P] + [b.cpu().numpy().copy() for b in B])
        plan.close()
    for i, (a, b) in enumerate(zip(*outs)):
        assert np.array_equal(a, b), i


def test_lanes_match_oracle(M):
    from gpu_util import run_and_compare
    shapes, dts, Ws, Gs, Bs = _mixed_lane_state()
    plan = _plan(M, shapes, dts, lanes=4)
    assert len({plan.matrix_choice(i)["lane"] for i in range(len(shapes))}) >= 3
    bf = [i for i, d in enumerate(dts) if d == "bf16"]
    f32 = [i for i, d in enumerate(dts) if d == "f32"]
    run_and_compare(plan, Ws, Gs, Bs, WL.BF16, check=bf)
    run_and_compare(plan, Ws, Gs, Bs, WL.F32, check=f32)


@pytest.mark.parametrize("shapes,edge", [
    ([(256, 512), (100, 300), (300, 100)], 64),   # few 128-tiles: 64 x 64 fp32 tiles
    ([(512, 512)] * 15 + [(512, 1000)], 128),     # 256 128-tiles of m x n: 128 x 128
])
def test_fp32_tile_edge_matches_oracle(M, shapes, edge):
    """The fp32 kernel's tile edge follows the set's size (64 when its m x n
    products have fewer 128-tiles than the GPU has CUs); both edges meet the
    fp32 bar, direct form over T = 5 and 2, Gram form over T = 5."""
    from gpu_util import make_state, run_and_compare
    Ws, Gs, Bs = make_state(shapes, WL.F32, seed=120 + edge, buf_scale=0.01)
    plan = _plan(M, shapes, "f32", form="direct")
    assert f"edge={edge} ".encode() in plan.serialize()
    check = [0, 1, 2, len(shapes) - 1]
    for T in (5, 2):
        run_and_compare(plan, Ws, Gs, Bs, WL.F32, ns_steps=T, check=check)
    gram = _plan(M, shapes, "f32", form="gram")
    assert f"edge={edge} ".encode() in gram.serialize()
    run_and_compare(gram, Ws, Gs, Bs, WL.F32, ns_steps=5, check=check)


@pytest.mark.parametrize("case", range(12))
def test_seeded_random_shapes_match_oracle(M, case):
    """Seeded random plans: 3-4 shapes with sides from 1 to 1500 (primes,
    single rows and columns, both orientations), a random bf16 tile plan,
    form and NS step count, or the fp32 path; every matrix against the oracle."""
    from gpu_util import make_state, run_and_compare
    rng = np.random.default_rng(1000 + case)
    sides = [1, 2, 7, 31, 64, 127, 128, 129, 257, 383, 512, 641, 1000, 1021, 1500]
    shapes = []
    for _ in range(int(rng.integers(3, 5))):
        a, b = int(rng.choice(sides)), int(rng.choice(sides))
        if min(a, b) == max(a, b) == 1:
            b = 64
        shapes.append((a, b))
    dtype = WL.F32 if case % 4 == 3 else WL.BF16
    T = int(rng.integers(1, 7))
    if dtype == WL.BF16:
        form = "gram" if case % 5 == 4 else "direct"
        tiles = [0, 1, 2, 5, 6, 7, 8, 9] if form == "gram" else list(range(10))
        tile = int(rng.choice(tiles))
        plan = _plan(M, shapes, "bf16", tile=tile, form=form)
    else:
        form, tile = ("gram" if case == 7 else "direct"), None
        plan = _plan(M, shapes, "f32", form=form)
    print(f"case {case}: {dtype} shapes {shapes} form {form} tile {tile} T {T}", flush=True)
    Ws, Gs, Bs = make_state(shapes, dtype, seed=2000 + case, buf_scale=0.01)
    run_and_compare(plan, Ws, Gs, Bs, dtype, ns_steps=T)
