"""ctypes declarations of include/muon.h and loading of libmuon_mi355x.so.

Loading fails loudly when the library is missing: there is no fallback path.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmuon_mi355x.so")

MUON_OK, MUON_EINVAL, MUON_EUNSUPPORTED, MUON_ENOMEM, MUON_EHIP, MUON_ESTATE = range(6)
MUON_F32, MUON_BF16 = 0, 1
PRECISION = {"auto": 0, "fp32": 1, "bf16": 2}
FORM = {"auto": 0, "direct": 1, "gram": 2}
TUNE = {"off": 0, "once": 1, "force": 2}
STATUS_NAMES = {0: "MUON_OK", 1: "MUON_EINVAL", 2: "MUON_EUNSUPPORTED", 3: "MUON_ENOMEM",
                4: "MUON_EHIP", 5: "MUON_ESTATE"}


class MatrixDesc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class PlanOpts(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("nesterov", ctypes.c_int32),
                ("eps", ctypes.c_float), ("rms_scale", ctypes.c_float),
                ("precision", ctypes.c_int32), ("form", ctypes.c_int32),
                ("tile", ctypes.c_int32),
                ("tune", ctypes.c_int32), ("host_only", ctypes.c_int32),
                ("lanes", ctypes.c_int32),
                ("workspace_cap_bytes", ctypes.c_uint64), ("cache_path", ctypes.c_char_p)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("n_matrices", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("n_chunks", ctypes.c_int32), ("n_gram", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64), ("ns_flops_min", ctypes.c_double),
                ("ns_flops_issued", ctypes.c_double), ("ew_bytes", ctypes.c_double),
                ("plan_hash", ctypes.c_uint64), ("n_lanes", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("kernel", ctypes.c_char * 32),
                ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double), ("flops", ctypes.c_double),
                ("bytes", ctypes.c_double)]


class LaunchInterval(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("kernel", ctypes.c_char * 32),
                ("start_ms", ctypes.c_double), ("end_ms", ctypes.c_double)]


_PP = ctypes.POINTER(ctypes.c_void_p)
_FP = ctypes.POINTER(ctypes.c_float)

# name -> (restype, argtypes); must list every function include/muon.h declares.
PROTOTYPES = {
    "muon_abi_version": (ctypes.c_int, []),
    "muon_last_error": (ctypes.c_char_p, []),
    "muon_plan_opts_default": (ctypes.c_int, [ctypes.POINTER(PlanOpts)]),
    "muon_plan_create": (ctypes.c_int, [ctypes.POINTER(MatrixDesc), ctypes.c_int,
                                        ctypes.POINTER(PlanOpts), ctypes.POINTER(ctypes.c_void_p)]),
    "muon_plan_destroy": (ctypes.c_int, [ctypes.c_void_p]),
    "muon_step": (ctypes.c_int, [ctypes.c_void_p, _PP, _PP, _PP, ctypes.c_float, ctypes.c_float,
                                 ctypes.c_float, ctypes.c_int, _FP, ctypes.c_void_p]),
    "muon_step_schedule": (ctypes.c_int, [ctypes.c_void_p, _PP, _PP, _PP, ctypes.c_float,
                                          ctypes.c_float, ctypes.c_float, ctypes.c_int, _FP,
                                          ctypes.c_void_p]),
    "muon_plan_set_update_capture": (ctypes.c_int, [ctypes.c_void_p, _PP]),
    "muon_plan_get_flags": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32),
                                           ctypes.c_int]),
    "muon_plan_serialize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.POINTER(ctypes.c_size_t)]),
    "muon_plan_info_get": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(PlanInfo)]),
    "muon_plan_matrix_choice": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int,
                                               ctypes.POINTER(ctypes.c_int32),
                                               ctypes.POINTER(ctypes.c_int32),
                                               ctypes.POINTER(ctypes.c_int32),
                                               ctypes.POINTER(ctypes.c_int32),
                                               ctypes.POINTER(ctypes.c_int32)]),
    "muon_plan_set_profiling": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int]),
    "muon_plan_set_graph": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int]),
    "muon_plan_get_kernel_times": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(KernelTime),
                                                  ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                                  ctypes.c_int]),
    "muon_plan_get_launch_intervals": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(LaunchInterval),
                                                      ctypes.c_int, ctypes.POINTER(ctypes.c_int)]),
    "muon_orthogonalize": (ctypes.c_int, [ctypes.c_void_p, _PP, _PP, ctypes.c_int,
                                          ctypes.POINTER(ctypes.c_float), ctypes.c_void_p]),
    "muon_adamw_plan_create": (ctypes.c_int, [ctypes.POINTER(ctypes.c_int64),
                                              ctypes.POINTER(ctypes.c_int32), ctypes.c_int,
                                              ctypes.POINTER(ctypes.c_void_p)]),
    "muon_adamw_step": (ctypes.c_int, [ctypes.c_void_p, _PP, _PP, _PP, _PP, ctypes.c_double,
                                       ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                       ctypes.c_double, ctypes.c_int64, ctypes.c_void_p]),
    "muon_adamw_plan_destroy": (ctypes.c_int, [ctypes.c_void_p]),
    "muon_probe_mfma_bf16": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                            ctypes.POINTER(ctypes.c_double)]),
    "muon_probe_mfma_bf16_random": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                                   ctypes.POINTER(ctypes.c_double)]),
    "muon_probe_nt_bf16": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_double)]),
    "muon_probe_nt_out_bf16": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]),
    "muon_probe_hbm_copy": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                           ctypes.c_int, ctypes.POINTER(ctypes.c_double)]),
    "muon_plan_matrix_cost": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int,
                                             ctypes.POINTER(ctypes.c_double)]),
    "muon_step_noalloc": (ctypes.c_int, [ctypes.POINTER(MatrixDesc), ctypes.POINTER(PlanOpts),
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_int,
                                         _FP, ctypes.c_void_p]),
    "muon_assign_owners": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int64, ctypes.POINTER(ctypes.c_int32),
                                          ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_int32)]),
}

_lib = None


class MuonError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m matrix_orthogonalizing_optimizer_muon_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(code):
    if code != MUON_OK:
        raise MuonError(code, lib().muon_last_error().decode(errors="replace"))
    return code
