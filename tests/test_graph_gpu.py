"""Graph replay of muon_step (muon_plan_set_graph): a step that repeats the
previous step's arguments is captured into a HIP graph and later ones replay
it.  Every step, eager, captured or replayed, leaves parameters and momenta
bitwise equal to the same steps run without graphs (the same kernels in the
same order on each stream), with one or several lanes and workspace chunks,
with fresh gradients written into the same buffers before each step, and with
the program's own eager work and synchronizations between the replays."""
import pytest

import workloads as WL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import matrix_orthogonalizing_optimizer_muon_amd as mod
    return mod


def _state():
    from gpu_util import make_state
    sb = [(300, 700), (700, 300), (129, 1000), (520, 520), (64, 2048)]
    sf = [(256, 512), (96, 96)]
    Wb, Gb, Bb = make_state(sb, WL.BF16, seed=91, buf_scale=0.01)
    Wf, Gf, Bf = make_state(sf, WL.F32, seed=92, buf_scale=0.01)
    return sb + sf, ["bf16"] * len(sb) + ["f32"] * len(sf), Wb + Wf, Gb + Gf, Bb + Bf


@pytest.mark.parametrize("lanes,chunked", [(1, False), (3, False), (2, True)])
def test_graph_replays_match_eager_steps_bitwise(M, lanes, chunked):
    import torch
    from gpu_util import device_state
    shapes, dts, Ws, Gs, Bs = _state()
    cap = 0
    if chunked:
        probe = M.MuonPlan(shapes, dts, tune="off")
        cap = probe.info()["workspace_bytes"] // 2
        probe.close()
    eager = M.MuonPlan(shapes, dts, tune="off", lanes=lanes, workspace_cap=cap)
    graph = M.MuonPlan(shapes, dts, tune="off", lanes=lanes, workspace_cap=cap)
    assert (graph.info()["n_chunks"] >= 2) == chunked and graph.info()["n_lanes"] == lanes
    graph.set_graph(True)
    Pe, Ge, Be = device_state(Ws, Gs, Bs)
    Pg, Gg, Bg = device_state(Ws, Gs, Bs)
    side = torch.cuda.Stream()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    other = torch.randn(1 << 20, device="cuda", generator=gen)
    # steps 0-3 share their arguments (eager, captured, replayed twice); step 4
    # changes lr (eager again), step 5 repeats it (captured), 6 and 7 replay
    for k in range(8):
        for ge, gg in zip(Ge, Gg):
            fresh = (torch.randn(ge.shape, device="cuda", generator=gen) * 0.02).to(ge.dtype)
            ge.copy_(fresh)
            gg.copy_(fresh)
        torch.cuda.synchronize()
        lr = 0.02 if k < 4 else 0.01
        eager.step(Pe, Ge, Be, lr=lr)
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            graph.step(Pg, Gg, Bg, lr=lr)
        torch.cuda.synchronize()
        other.mul_(0.5).add_(1.0)          # unrelated eager work between replays
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(Pe + Be, Pg + Bg)):
            assert torch.equal(a, b), f"step {k}, tensor {i}"
        print(f"graph lanes={lanes} chunked={chunked} step {k}: bitwise equal", flush=True)
    graph.set_graph(False)
    eager.close()
    graph.close()


def test_graph_mode_refuses_the_null_stream(M):
    import torch
    from gpu_util import device_state, make_state
    Ws, Gs, Bs = make_state([(64, 128)], WL.BF16, seed=93)
    P, G, B = device_state(Ws, Gs, Bs)
    plan = M.MuonPlan([(64, 128)], "bf16", tune="off")
    plan.set_graph(True)
    with pytest.raises(M.MuonError):
        plan.step(P, G, B, stream=0)
    plan.set_graph(False)
    plan.step(P, G, B, stream=0)           # eager again on the null stream
    torch.cuda.synchronize()
    plan.close()


@pytest.mark.parametrize("graph_mode", [False, True])
def test_step_inside_the_callers_graph_matches_eager_steps(M, graph_mode):
    """A caller that captures muon_step into a graph of its own (torch.cuda.graph,
    three NS lanes joined back into the capture stream) gets, on every replay,
    the same parameters and momenta as eager steps, bitwise; with the library's
    own graph mode on, the step inside a caller's capture is enqueued as usual."""
    import torch
    from gpu_util import device_state
    shapes, dts, Ws, Gs, Bs = _state()
    eager = M.MuonPlan(shapes, dts, tune="off", lanes=3)
    capt = M.MuonPlan(shapes, dts, tune="off", lanes=3)
    if graph_mode:
        capt.set_graph(True)
    Pe, Ge, Be = device_state(Ws, Gs, Bs)
    Pc, Gc, Bc = device_state(Ws, Gs, Bs)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    side = torch.cuda.Stream()
    # one eager step first: the pointer tables are uploaded outside the capture
    eager.step(Pe, Ge, Be)
    with torch.cuda.stream(side):
        capt.step(Pc, Gc, Bc)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capt.step(Pc, Gc, Bc)
    torch.cuda.synchronize()
    other = torch.randn(1 << 20, device="cuda", generator=gen)
    for k in range(4):
        for ge, gc in zip(Ge, Gc):
            fresh = (torch.randn(ge.shape, device="cuda", generator=gen) * 0.02).to(ge.dtype)
            ge.copy_(fresh)
            gc.copy_(fresh)
        torch.cuda.synchronize()
        eager.step(Pe, Ge, Be)
        g.replay()
        torch.cuda.synchronize()
        other.mul_(0.5).add_(1.0)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(Pe + Be, Pc + Bc)):
            assert torch.equal(a, b), f"replay {k}, tensor {i}"
        print(f"caller graph (library graph mode {graph_mode}) replay {k}: bitwise equal", flush=True)
    del g
    eager.close()
    capt.close()


def test_capture_with_pointers_not_yet_uploaded_is_refused(M):
    """A step, an orthogonalization or an AdamW step on a stream under capture
    whose pointers differ from the plan's previous call outside the capture is
    refused (ESTATE) with nothing enqueued: the pointer tables are uploaded
    outside graphs only.  The plans stay usable: the next eager calls match
    a fresh plan's bitwise."""
    import torch
    from gpu_util import device_state
    shapes, dts, Ws, Gs, Bs = _state()
    plan = M.MuonPlan(shapes, dts, tune="off", lanes=3)
    ref = M.MuonPlan(shapes, dts, tune="off", lanes=3)
    P, G, B = device_state(Ws, Gs, Bs)
    Pr, Gr, Br = device_state(Ws, Gs, Bs)
    outs = [torch.empty(s, device="cuda", dtype=torch.float32) for s in shapes]
    numels = [16384, 1000]
    aw = M.AdamWPlan(numels, ["f32", "bf16"])
    ap = [torch.randn(numels[0], device="cuda"), torch.randn(numels[1], device="cuda").to(torch.bfloat16)]
    ag = [torch.randn_like(t) for t in ap]
    am = [torch.zeros(k, device="cuda") for k in numels]
    av = [torch.zeros(k, device="cuda") for k in numels]
    torch.cuda.synchronize()
    calls = [
        ("muon_step", lambda: plan.step(P, G, B)),
        ("muon_orthogonalize", lambda: plan.orthogonalize(G, outs)),
        ("muon_adamw_step", lambda: aw.step(ap, ag, am, av, lr=1e-3)),
    ]
    for name, call in calls:
        g = torch.cuda.CUDAGraph()
        with pytest.raises(M.MuonError, match="stream capture"):
            with torch.cuda.graph(g):
                call()
        torch.cuda.synchronize()
        print(f"{name} under capture with new pointers: refused", flush=True)
        del g
    plan.step(P, G, B)
    ref.step(Pr, Gr, Br)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(P + B, Pr + Br)):
        assert torch.equal(a, b), f"tensor {i}"
    aw.step(ap, ag, am, av, lr=1e-3)
    torch.cuda.synchronize()
    assert all(torch.isfinite(t.float()).all() for t in ap + am + av)
    aw.close()
    plan.close()
    ref.close()
