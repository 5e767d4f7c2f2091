"""MI355X (gfx950) Muon per-owner update step.

Python binding of libmuon_mi355x.so (C ABI in include/muon.h).  This module
only marshals arguments: it checks that the tensors it is handed match the
plan (shape, dtype, device, contiguity) so no kernel is launched on mismatched
memory, and passes raw device pointers to the library.  Every step of the
update runs in the library's HIP kernels; there is no fallback path.

    plan = MuonPlan([(3072, 1024), (1024, 1024)], "bf16")
    plan.step(params, grads, momenta, lr=0.02, beta=0.95, wd=0.01)
"""
import ctypes

from . import _lib as L
from ._lib import MuonError  # noqa: F401

__all__ = ["MuonPlan", "AdamWPlan", "MuonError", "library_path", "assign_owners",
           "probe_mfma_bf16", "probe_nt_bf16", "probe_nt_out_bf16", "probe_hbm_copy", "step_noalloc"]


def library_path():
    return L.LIB_PATH


def _dtype_code(d):
    if isinstance(d, int):
        return d
    s = str(d).replace("torch.", "")
    if s in ("f32", "float32", "fp32", "float"):
        return L.MUON_F32
    if s in ("bf16", "bfloat16"):
        return L.MUON_BF16
    raise ValueError(f"unsupported dtype {d!r}")


class MuonPlan:
    """A plan over a fixed list of matrix shapes (see muon_plan_create)."""

    def __init__(self, shapes, dtypes, *, nesterov=True, eps=1e-7, rms_scale=0.2,
                 precision="auto", form="auto", tile=None, tune="once", cache_path=None,
                 workspace_cap=0, host_only=False, lanes=None):
        lib = L.lib()
        shapes = [(int(r), int(c)) for r, c in shapes]
        if isinstance(dtypes, (list, tuple)):
            codes = [_dtype_code(d) for d in dtypes]
        else:
            codes = [_dtype_code(dtypes)] * len(shapes)
        if len(codes) != len(shapes):
            raise ValueError("one dtype per shape")
        self.shapes = shapes
        self.dtypes = codes
        n = len(shapes)
        descs = (L.MatrixDesc * max(n, 1))()
        for i, ((r, c), d) in enumerate(zip(shapes, codes)):
            descs[i].rows, descs[i].cols, descs[i].dtype, descs[i].reserved = r, c, d, 0
        opts = L.PlanOpts()
        L.check(lib.muon_plan_opts_default(ctypes.byref(opts)))
        opts.nesterov = 1 if nesterov else 0
        opts.eps = eps
        opts.rms_scale = rms_scale
        opts.precision = L.PRECISION[precision]
        opts.form = L.FORM[form]
        opts.tile = -1 if tile is None else int(tile)
        opts.tune = L.TUNE[tune]
        opts.host_only = 1 if host_only else 0
        opts.lanes = 0 if lanes is None else int(lanes)
        opts.workspace_cap_bytes = int(workspace_cap)
        self._cache = cache_path.encode() if cache_path else None
        opts.cache_path = self._cache
        handle = ctypes.c_void_p()
        L.check(lib.muon_plan_create(descs, n, ctypes.byref(opts), ctypes.byref(handle)))
        self._h = handle
        self._capture = None

    # ---------------------------------------------------------------- lifetime
    def close(self):
        if getattr(self, "_h", None):
            L.lib().muon_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # ------------------------------------------------------------------ checks
    def _check_tensors(self, name, ts, want_dtype_codes):
        import torch
        if len(ts) != len(self.shapes):
            raise ValueError(f"{name}: expected {len(self.shapes)} tensors, got {len(ts)}")
        dev = None
        for i, (t, shp, dc) in enumerate(zip(ts, self.shapes, want_dtype_codes)):
            if not isinstance(t, torch.Tensor):
                raise TypeError(f"{name}[{i}] is not a tensor")
            if not t.is_cuda:
                raise ValueError(f"{name}[{i}] is not on the GPU")
            if tuple(t.shape) != shp:
                raise ValueError(f"{name}[{i}] has shape {tuple(t.shape)}, plan says {shp}")
            want = torch.float32 if dc == L.MUON_F32 else torch.bfloat16
            if t.dtype != want:
                raise ValueError(f"{name}[{i}] has dtype {t.dtype}, plan says {want}")
            if not t.is_contiguous():
                raise ValueError(f"{name}[{i}] is not contiguous")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{name}[{i}] is on {t.device}, others on {dev}")
        return dev

    @staticmethod
    def _ptrs(ts):
        arr = (ctypes.c_void_p * max(len(ts), 1))()
        for i, t in enumerate(ts):
            arr[i] = t.data_ptr() if t is not None else None
        return arr

    @staticmethod
    def _stream(stream, device):
        import torch
        if stream is None:
            return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
        if isinstance(stream, torch.cuda.Stream):
            return ctypes.c_void_p(stream.cuda_stream)
        return ctypes.c_void_p(int(stream))

    # -------------------------------------------------------------------- step
    def step(self, params, grads, momenta, lr=0.02, beta=0.95, wd=0.01, ns_steps=5,
             coeffs=None, stream=None):
        """One Muon step (muon_step); coeffs is (a, b, c) or a list of ns_steps triples."""
        dev = self._check_tensors("params", params, self.dtypes)
        self._check_tensors("grads", grads, self.dtypes)
        self._check_tensors("momenta", momenta, [L.MUON_F32] * len(self.shapes))
        for i, (p, g, m) in enumerate(zip(params, grads, momenta)):
            if p.data_ptr() == g.data_ptr() or p.data_ptr() == m.data_ptr():
                raise ValueError(f"matrix {i}: params alias grads or momenta")
        P, G, M = self._ptrs(params), self._ptrs(grads), self._ptrs(momenta)
        s = self._stream(stream, dev)
        lib = L.lib()
        if coeffs is not None and len(coeffs) and isinstance(coeffs[0], (list, tuple)):
            if len(coeffs) != ns_steps:
                raise ValueError("schedule needs one (a, b, c) per NS step")
            flat = [float(x) for row in coeffs for x in row]
            arr = (ctypes.c_float * max(len(flat), 1))(*flat)
            L.check(lib.muon_step_schedule(self._h, P, G, M, lr, beta, wd, int(ns_steps), arr, s))
            return
        carr = None
        if coeffs is not None:
            if len(coeffs) != 3:
                raise ValueError("coeffs must be (a, b, c)")
            carr = (ctypes.c_float * 3)(*[float(x) for x in coeffs])
        L.check(lib.muon_step(self._h, P, G, M, lr, beta, wd, int(ns_steps), carr, s))

    def orthogonalize(self, inputs, outputs, ns_steps=5, coeffs=None, stream=None):
        """NS orthogonalization alone (muon_orthogonalize): outputs[i] (fp32, the
        input's shape) = NS_T(inputs[i] / (||inputs[i]||_F + eps)).  coeffs: None
        (quintic), (a, b, c) for every step, or a list of ns_steps triples."""
        dev = self._check_tensors("inputs", inputs, self.dtypes)
        self._check_tensors("outputs", outputs, [L.MUON_F32] * len(self.shapes))
        for i, (a, b) in enumerate(zip(inputs, outputs)):
            if a.data_ptr() == b.data_ptr():
                raise ValueError(f"matrix {i}: output aliases input")
        sched = None
        if coeffs is not None:
            rows = coeffs if len(coeffs) and isinstance(coeffs[0], (list, tuple)) else [coeffs] * ns_steps
            if len(rows) != ns_steps or any(len(r) != 3 for r in rows):
                raise ValueError("coeffs must be (a, b, c) or one (a, b, c) per NS step")
            flat = [float(x) for r in rows for x in r]
            sched = (ctypes.c_float * max(len(flat), 1))(*flat)
        L.check(L.lib().muon_orthogonalize(self._h, self._ptrs(inputs), self._ptrs(outputs),
                                           int(ns_steps), sched, self._stream(stream, dev)))

    def set_update_capture(self, dst):
        """dst: list of fp32 tensors (or None entries) shaped like the params, or None."""
        if dst is None:
            self._capture = None
            L.check(L.lib().muon_plan_set_update_capture(self._h, None))
            return
        import torch
        if len(dst) != len(self.shapes):
            raise ValueError("one capture tensor (or None) per matrix")
        for i, (t, shp) in enumerate(zip(dst, self.shapes)):
            if t is None:
                continue
            if not (t.is_cuda and t.dtype == torch.float32 and tuple(t.shape) == shp and t.is_contiguous()):
                raise ValueError(f"capture[{i}] must be a contiguous fp32 GPU tensor of shape {shp}")
        self._capture = list(dst)
        L.check(L.lib().muon_plan_set_update_capture(self._h, self._ptrs(self._capture)))

    # ------------------------------------------------------------ inspection
    def flags(self, clear=False):
        f = ctypes.c_uint32()
        L.check(L.lib().muon_plan_get_flags(self._h, ctypes.byref(f), 1 if clear else 0))
        return f.value

    def serialize(self):
        n = ctypes.c_size_t()
        lib = L.lib()
        L.check(lib.muon_plan_serialize(self._h, None, ctypes.byref(n)))
        buf = ctypes.create_string_buffer(n.value)
        L.check(lib.muon_plan_serialize(self._h, buf, ctypes.byref(n)))
        return buf.raw[: n.value]

    def info(self):
        i = L.PlanInfo()
        L.check(L.lib().muon_plan_info_get(self._h, ctypes.byref(i)))
        return {k: getattr(i, k) for k, _ in L.PlanInfo._fields_}

    def matrix_choice(self, i):
        f, t, g, c, ln = (ctypes.c_int32() for _ in range(5))
        L.check(L.lib().muon_plan_matrix_choice(self._h, int(i), ctypes.byref(f), ctypes.byref(t),
                                                ctypes.byref(g), ctypes.byref(c), ctypes.byref(ln)))
        return {"form": {1: "direct", 2: "gram"}[f.value], "tile": t.value, "group": g.value,
                "chunk": c.value, "lane": ln.value}

    def set_graph(self, enable=True):
        """Graph replay of repeated steps (muon_plan_set_graph); steps must then
        run on a stream other than the null stream."""
        L.check(L.lib().muon_plan_set_graph(self._h, 1 if enable else 0))

    def set_profiling(self, enable=True):
        L.check(L.lib().muon_plan_set_profiling(self._h, 1 if enable else 0))

    def matrix_cost(self, i):
        """Estimated step time of matrix i in microseconds (owner-assignment input)."""
        us = ctypes.c_double()
        L.check(L.lib().muon_plan_matrix_cost(self._h, int(i), ctypes.byref(us)))
        return us.value

    def launch_intervals(self, max_n=1 << 16):
        """Folded launches (call after kernel_times(reset=False)), in launch order."""
        arr = (L.LaunchInterval * max_n)()
        n = ctypes.c_int()
        L.check(L.lib().muon_plan_get_launch_intervals(self._h, arr, max_n, ctypes.byref(n)))
        return [{"name": arr[k].name.decode(), "kernel": arr[k].kernel.decode(),
                 "start_ms": arr[k].start_ms, "end_ms": arr[k].end_ms} for k in range(n.value)]

    def kernel_times(self, reset=True):
        arr = (L.KernelTime * 64)()
        n = ctypes.c_int()
        L.check(L.lib().muon_plan_get_kernel_times(self._h, arr, 64, ctypes.byref(n), 1 if reset else 0))
        return [{"name": arr[k].name.decode(), "kernel": arr[k].kernel.decode(),
                 "launches": arr[k].launches,
                 "total_ms": arr[k].total_ms, "flops": arr[k].flops, "bytes": arr[k].bytes}
                for k in range(n.value)]


def step_noalloc(param, grad, momentum, *, lr=0.02, beta=0.95, wd=0.01, ns_steps=5, coeffs=None,
                 nesterov=True, eps=1e-7, rms_scale=0.2, stream=None):
    """One Muon step of one matrix through muon_step_noalloc: no plan and no
    device allocation (the library's fixed per-device scratch array holds the
    workspace).  param / grad: 2-D contiguous fp32 or bf16 tensors of one
    dtype on the GPU; momentum: fp32 of the same shape."""
    import torch
    if param.dim() != 2 or grad.shape != param.shape or momentum.shape != param.shape:
        raise ValueError("param, grad and momentum must be 2-D tensors of one shape")
    if param.dtype not in (torch.float32, torch.bfloat16) or grad.dtype != param.dtype:
        raise ValueError("param and grad must share dtype float32 or bfloat16")
    if momentum.dtype != torch.float32:
        raise ValueError("momentum must be float32")
    for name, t in (("param", param), ("grad", grad), ("momentum", momentum)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
        if t.device != param.device:
            raise ValueError(f"{name} is on {t.device}, param on {param.device}")
    desc = L.MatrixDesc(int(param.shape[0]), int(param.shape[1]),
                        L.MUON_F32 if param.dtype == torch.float32 else L.MUON_BF16, 0)
    opts = L.PlanOpts()
    L.check(L.lib().muon_plan_opts_default(ctypes.byref(opts)))
    opts.nesterov = 1 if nesterov else 0
    opts.eps = eps
    opts.rms_scale = rms_scale
    co = None
    if coeffs is not None:
        co = (ctypes.c_float * 3)(*[float(x) for x in coeffs])
    L.check(L.lib().muon_step_noalloc(ctypes.byref(desc), ctypes.byref(opts),
                                      ctypes.c_void_p(param.data_ptr()), ctypes.c_void_p(grad.data_ptr()),
                                      ctypes.c_void_p(momentum.data_ptr()), float(lr), float(beta),
                                      float(wd), int(ns_steps), co,
                                      MuonPlan._stream(stream, param.device)))


def assign_owners(costs, n_owners, node_limit=0):
    """Makespan-minimizing assignment of items to owners (muon_assign_owners).

    Returns (owner list, makespan, proven optimal)."""
    n = len(costs)
    arr = (ctypes.c_double * max(n, 1))(*[float(c) for c in costs])
    out = (ctypes.c_int32 * max(n, 1))()
    span = ctypes.c_double()
    opt = ctypes.c_int32()
    L.check(L.lib().muon_assign_owners(arr, n, int(n_owners), int(node_limit), out,
                                       ctypes.byref(span), ctypes.byref(opt)))
    return [out[i] for i in range(n)], span.value, bool(opt.value)


def probe_mfma_bf16(iters=20000, random_operands=False):
    """Measured dense bf16 MFMA rate of the current device (muon_probe_mfma_bf16,
    or muon_probe_mfma_bf16_random with random register operands).

    Returns (TFLOP/s, flop count of the timed launch)."""
    tf = ctypes.c_double()
    fl = ctypes.c_double()
    fn = L.lib().muon_probe_mfma_bf16_random if random_operands else L.lib().muon_probe_mfma_bf16
    L.check(fn(int(iters), ctypes.byref(tf), ctypes.byref(fl)))
    return tf.value, fl.value


def probe_nt_bf16(P, Q, reps=5):
    """Measured rate of the NT contraction core alone (muon_probe_nt_bf16) on
    P Q^T: P (m x k) and Q (n x k) contiguous bf16 device tensors, m and n
    multiples of 256, k a multiple of 64.

    Returns (TFLOP/s, sum of all entries of P Q^T as the core accumulated it)."""
    import torch
    for t in (P, Q):
        if not (t.is_cuda and t.is_contiguous() and t.dtype == torch.bfloat16 and t.dim() == 2):
            raise ValueError("P and Q must be contiguous 2-D bf16 device tensors")
    if P.shape[1] != Q.shape[1]:
        raise ValueError("P and Q must have the same number of columns")
    tf = ctypes.c_double()
    cs = ctypes.c_double()
    L.check(L.lib().muon_probe_nt_bf16(ctypes.c_void_p(P.data_ptr()), ctypes.c_void_p(Q.data_ptr()),
                                       int(P.shape[0]), int(Q.shape[0]), int(P.shape[1]), int(reps),
                                       ctypes.byref(tf), ctypes.byref(cs)))
    return tf.value, cs.value


def probe_nt_out_bf16(P, Q, C, CT=None, mode=1, reps=5):
    """Measured rate of the NT contraction core with a bf16 output epilogue
    (muon_probe_nt_out_bf16): C (m x n) receives P Q^T rounded to bf16; modes
    2 and 3 also store its transpose into CT (n x m), mode 3 with nontemporal
    stores.  All contiguous bf16 device tensors; m and n multiples of 256, k a
    multiple of 64.  Returns TFLOP/s."""
    import torch
    m, k = P.shape
    n = Q.shape[0]
    want = [(P, (m, k)), (Q, (n, k)), (C, (m, n))] + ([(CT, (n, m))] if mode >= 2 else [])
    for t, shape in want:
        if not (t is not None and t.is_cuda and t.is_contiguous() and t.dtype == torch.bfloat16
                and tuple(t.shape) == shape):
            raise ValueError(f"P, Q, C and CT must be contiguous bf16 device tensors of shapes "
                             f"(m, k), (n, k), (m, n) and (n, m)")
    tf = ctypes.c_double()
    ct = ctypes.c_void_p(CT.data_ptr()) if CT is not None else ctypes.c_void_p(None)
    L.check(L.lib().muon_probe_nt_out_bf16(ctypes.c_void_p(P.data_ptr()), ctypes.c_void_p(Q.data_ptr()),
                                           ctypes.c_void_p(C.data_ptr()), ct, int(m), int(n), int(k),
                                           int(mode), int(reps), ctypes.byref(tf)))
    return tf.value


def probe_hbm_copy(dst, src, reps=10):
    """Measured copy rate (read plus written GB/s) between two equal-sized,
    contiguous device tensors (muon_probe_hbm_copy); dst receives src's bytes."""
    if not (dst.is_cuda and src.is_cuda and dst.is_contiguous() and src.is_contiguous()):
        raise ValueError("dst and src must be contiguous device tensors")
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb:
        raise ValueError("dst and src must hold the same number of bytes")
    gbs = ctypes.c_double()
    L.check(L.lib().muon_probe_hbm_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                                        nb, int(reps), ctypes.byref(gbs)))
    return gbs.value


class AdamWPlan:
    """Fused multi-tensor AdamW over a fixed list of tensors (muon_adamw_*): the
    non-matrix half of the Muon + AdamW hybrid."""

    def __init__(self, numels, dtypes):
        numels = [int(x) for x in numels]
        codes = [_dtype_code(d) for d in dtypes] if isinstance(dtypes, (list, tuple)) \
            else [_dtype_code(dtypes)] * len(numels)
        if len(codes) != len(numels):
            raise ValueError("one dtype per tensor")
        self.numels, self.dtypes = numels, codes
        n = len(numels)
        ne = (ctypes.c_int64 * max(n, 1))(*numels)
        dt = (ctypes.c_int32 * max(n, 1))(*codes)
        h = ctypes.c_void_p()
        L.check(L.lib().muon_adamw_plan_create(ne, dt, n, ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            L.lib().muon_adamw_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def step(self, params, grads, exp_avg, exp_avg_sq, *, lr, beta1=0.9, beta2=0.999, eps=1e-8,
             wd=0.01, step=1, stream=None):
        import torch
        n = len(self.numels)
        for name, ts, want in (("params", params, self.dtypes), ("grads", grads, self.dtypes),
                               ("exp_avg", exp_avg, [L.MUON_F32] * n),
                               ("exp_avg_sq", exp_avg_sq, [L.MUON_F32] * n)):
            if len(ts) != n:
                raise ValueError(f"{name}: {len(ts)} tensors, plan has {n}")
            for i, (t, d) in enumerate(zip(ts, want)):
                tdt = torch.float32 if d == L.MUON_F32 else torch.bfloat16
                if not t.is_cuda or t.dtype != tdt or t.numel() != self.numels[i] or not t.is_contiguous():
                    raise ValueError(f"{name}[{i}] must be a contiguous CUDA {tdt} of {self.numels[i]} elements")
        ptr = MuonPlan._ptrs
        dev = params[0].device if n else torch.device("cuda")
        L.check(L.lib().muon_adamw_step(self._h, ptr(params), ptr(grads), ptr(exp_avg), ptr(exp_avg_sq),
                                        float(lr), float(beta1), float(beta2), float(eps), float(wd),
                                        int(step), MuonPlan._stream(stream, dev)))
