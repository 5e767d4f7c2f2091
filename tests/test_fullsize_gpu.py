"""Parity at the full workload sizes, in the launch configuration bench.py times.

For each large workload one module-scoped fixture builds the plan over every
matrix the way bench.py does (form and tile plan timed once per shape, cached
in a fresh file), steps all of them at once with the fp32 update of a sample
of matrices captured, and keeps the sampled results on the host.  The sampled
matrices get the seeded host generator's values; the others get
device-generated values of the same laws (their values do not change which
kernels run).  Each test then grades a few sampled matrices against the fp64
oracle one by one (kept under about a minute of oracle time per test):

* relative Frobenius error of U <= 2e-2 and momentum <= 1e-6;
* the worst row and the worst column of U within 2.5 x 2e-2, each line's error
  norm taken over max(the line's own norm, the RMS norm of the lines), so a
  wrong row, column or strip fails even where the Frobenius error would not;
* the fraction of bf16 weights within one ulp of the oracle's rounded W_new
  is printed, not asserted (tiny weights make it ill-posed).

Samples (the plan for full-size parity): the Llama-7B set's layer 0 (all five
matrices) and two matrices from each of three seeded random layers; every
512x16384 matrix and four experts per shape of the MoE stack; the VLA set's
backbone layer 0 plus three seeded random backbone layers and every matrix of
the 12 action-expert layers."""
import time

import numpy as np
import pytest

import workloads as WL

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _random_layers(seed, lo, hi, k):
    rng = np.random.default_rng(seed)
    return sorted(int(x) for x in rng.choice(np.arange(lo, hi), size=k, replace=False))


# Llama-7B set: per layer QKV, O, gate, up, down
C4_LAYERS = _random_layers(7, 1, 32, 3)
C4_SAMPLE = {
    "layer0_qkv_o_gate": [0, 1, 2],
    "layer0_up_down": [3, 4],
    "random_layer_a": [5 * C4_LAYERS[0] + 0, 5 * C4_LAYERS[0] + 1],   # QKV, O
    "random_layer_b": [5 * C4_LAYERS[1] + 2, 5 * C4_LAYERS[1] + 4],   # gate, down
    "random_layer_c": [5 * C4_LAYERS[2] + 3, 5 * C4_LAYERS[2] + 1],   # up, O
}
# MoE stack: expert e of layer l is 3 (64 l + e) + {0 gate, 1 up, 2 down};
# the eight 512 x 16384 matrices close the list
_C5_EXPERTS = [(0, 0), (2, 17), (5, 40), (7, 63)]
C5_SAMPLE = {
    "experts": [3 * (64 * l + e) + k for l, e in _C5_EXPERTS for k in range(3)],
    "tall_skinny_gram": list(range(1536, 1544)),
}
# VLA set: backbone layer l is 4 l + {QKV, O, up, down}; expert layer j is 96 + 4 j + ...
C3_LAYERS = _random_layers(11, 1, 24, 3)
C3_SAMPLE = {
    "backbone_layer0": [0, 1, 2, 3],
    "backbone_random_layers": [4 * l + k for l in C3_LAYERS for k in range(4)],
    "action_expert_all_layers": list(range(96, 144)),
}


def _run(wl, sample, tmp_path):
    """One step over the whole workload; host results of the sampled matrices."""
    import torch
    import matrix_orthogonalizing_optimizer_muon_amd as M
    from gpu_util import to_device

    t0 = time.time()
    plan = M.MuonPlan(wl.shapes, wl.dtype, tune="once", cache_path=str(tmp_path / "tune.txt"))
    print(f"{wl.name}: plan {time.time() - t0:.1f}s, choices "
          f"{sorted({(min(s), max(s), plan.matrix_choice(i)['form'], plan.matrix_choice(i)['tile']) for i, s in enumerate(wl.shapes)})}",
          flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4321 + wl.cfg)
    P, G, B = [], [], []
    host = {}
    for i, (r, c) in enumerate(wl.shapes):
        if i in sample:
            Wst, Gst = WL.draw(wl, i, 0, WL.KIND_W), WL.draw(wl, i, 0, WL.KIND_G)
            host[i] = (Wst, Gst)
            P.append(to_device(Wst))
            G.append(to_device(Gst))
        else:
            P.append((torch.randn(r, c, device="cuda", generator=gen) * wl.w_scale).to(torch.bfloat16))
            G.append((torch.randn(r, c, device="cuda", generator=gen) * wl.grad_scale).to(torch.bfloat16))
        B.append(torch.zeros(r, c, device="cuda", dtype=torch.float32))
    cap = [torch.empty(s, dtype=torch.float32, device="cuda") if i in sample else None
           for i, s in enumerate(wl.shapes)]
    plan.set_update_capture(cap)
    plan.step(P, G, B)
    torch.cuda.synchronize()
    plan.set_update_capture(None)
    flags = plan.flags()
    out = {}
    for i in sample:
        out[i] = (cap[i].cpu().numpy(), P[i].contiguous().view(torch.int16).cpu().numpy(),
                  B[i].cpu().numpy())
    plan.close()
    del P, G, B, cap
    torch.cuda.empty_cache()
    print(f"{wl.name}: step done {time.time() - t0:.1f}s", flush=True)
    return {"wl": wl, "host": host, "gpu": out, "flags": flags}


def _check(run, idx):
    from gpu_util import rel, check_lines
    from oracle import muon_oracle as O

    assert run["flags"] == 0
    wl = run["wl"]
    for i in idx:
        Wst, Gst = run["host"][i]
        U, wbits, buf = run["gpu"][i]
        t0 = time.time()
        ref = O.muon_step_ref(Wst.value, Gst.value, np.zeros(Wst.value.shape), param_dtype="bf16")
        U = U.astype(np.float64)
        e = rel(U, ref["U"])
        eb = rel(buf.astype(np.float64), ref["buf_new"])
        row, col = check_lines(U, ref["U"], TOL, f"matrix {i} {wl.shapes[i]}")
        wn = WL.bf16_bits_to_f64(wbits.view(np.uint16))
        _m, ex = np.frexp(ref["W_new_stored"])
        ulp = np.ldexp(1.0, ex - 8)
        within = float(np.mean(np.abs(wn - ref["W_new_stored"]) <= ulp))
        print(f"  matrix {i} {wl.shapes[i]}: rel err U {e:.3e}, worst row {row:.3e}, worst column "
              f"{col:.3e}, momentum {eb:.1e}, bf16 W within 1 ulp {within:.4f} "
              f"(oracle {time.time() - t0:.1f}s)", flush=True)
        assert e <= TOL, f"matrix {i} {wl.shapes[i]}: {e:.3e}"
        assert eb <= 1e-6


def _all(sample):
    return sorted({i for v in sample.values() for i in v})


@pytest.fixture(scope="module")
def llama7b(tmp_path_factory):
    return _run(WL.workload(4), _all(C4_SAMPLE), tmp_path_factory.mktemp("c4"))


@pytest.fixture(scope="module")
def moe(tmp_path_factory):
    return _run(WL.workload(5), _all(C5_SAMPLE), tmp_path_factory.mktemp("c5"))


@pytest.fixture(scope="module")
def vla(tmp_path_factory):
    return _run(WL.workload(3), _all(C3_SAMPLE), tmp_path_factory.mktemp("c3"))


@pytest.mark.parametrize("part", list(C4_SAMPLE))
def test_llama7b_matrix_set_full_size(llama7b, part):
    _check(llama7b, C4_SAMPLE[part])


@pytest.mark.parametrize("part", list(C5_SAMPLE))
def test_moe_stack_full_size(moe, part):
    _check(moe, C5_SAMPLE[part])


@pytest.mark.parametrize("part", list(C3_SAMPLE))
def test_vla_mixed_shapes_full_size(vla, part):
    _check(vla, C3_SAMPLE[part])
