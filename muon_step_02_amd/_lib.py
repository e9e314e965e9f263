"""ctypes binding of libmuon.so: structures mirror include/muon.h exactly."""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmuon.so")

MUON_F32 = 0
MUON_BF16 = 1
SCALE_MODES = {"moonlight": 0, "jordan": 1, "bernstein": 2, "none": 3}

STATUS = {
    0: "MUON_OK",
    1: "MUON_ERR_INVALID_ARG",
    2: "MUON_ERR_UNSUPPORTED_DEVICE",
    3: "MUON_ERR_WORKSPACE",
    4: "MUON_ERR_OVERLAP",
    5: "MUON_ERR_HIP",
    6: "MUON_ERR_UNALIGNED",
    7: "MUON_ERR_SCRATCH",
}

# every entry point include/muon.h declares
SYMBOLS = (
    "muon_init",
    "muon_destroy",
    "muon_workspace_size",
    "muon_step_batched",
    "adamw_step",
    "muon_status_str",
    "muon_test_gram_bf16",
    "muon_test_poly_bf16",
    "muon_test_update_bf16",
    "muon_profile_enable",
    "muon_profile_collect",
    "adamw_workspace_size",
    "adamw_step_clipped",
    "muon_test_split_matrices",
    "adamw_step_clipped_noalloc",
)

NUM_PHASES = 7
PHASES = ("momentum", "norm", "gram", "poly", "update", "apply", "adamw")


class MuonError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s: %s" % (what, STATUS.get(status, "status %d" % status)))


class MuonMatrix(ctypes.Structure):
    _fields_ = [
        ("param", ctypes.c_void_p),
        ("grad", ctypes.c_void_p),
        ("momentum", ctypes.c_void_p),
        ("update_out", ctypes.c_void_p),
        ("norm_out", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("ld_param", ctypes.c_int64),
        ("ld_grad", ctypes.c_int64),
        ("ld_mom", ctypes.c_int64),
        ("param_dtype", ctypes.c_int32),
        ("grad_dtype", ctypes.c_int32),
        ("qk_smax", ctypes.c_void_p),
        ("qk_block_rows", ctypes.c_int64),
    ]


class MuonHparams(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float),
        ("momentum", ctypes.c_float),
        ("weight_decay", ctypes.c_float),
        ("eps", ctypes.c_float),
        ("extra_scale", ctypes.c_float),
        ("nesterov", ctypes.c_int32),
        ("ns_steps", ctypes.c_int32),
        ("ns_dtype", ctypes.c_int32),
        ("scale_mode", ctypes.c_int32),
        ("coeffs", ctypes.POINTER(ctypes.c_float)),
        ("qk_tau", ctypes.c_float),
    ]


class AdamwTensor(ctypes.Structure):
    _fields_ = [
        ("param", ctypes.c_void_p),
        ("grad", ctypes.c_void_p),
        ("exp_avg", ctypes.c_void_p),
        ("exp_avg_sq", ctypes.c_void_p),
        ("numel", ctypes.c_int64),
        ("param_dtype", ctypes.c_int32),
        ("grad_dtype", ctypes.c_int32),
    ]


class PhaseTimes(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_float * 7), ("launches", ctypes.c_int32 * 7)]


class AdamwHparams(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float),
        ("beta1", ctypes.c_float),
        ("beta2", ctypes.c_float),
        ("eps", ctypes.c_float),
        ("weight_decay", ctypes.c_float),
        ("step", ctypes.c_int64),
    ]


_lib = None


def load():
    """Load libmuon.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libmuon.so not built: run `python -m muon_step_02_amd.build` "
                           "(expected at %s)" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.muon_init.argtypes = [i32, ctypes.POINTER(vp)]
    lib.muon_destroy.argtypes = [vp]
    lib.muon_workspace_size.argtypes = [vp, ctypes.POINTER(MuonMatrix), i32,
                                        ctypes.POINTER(MuonHparams), ctypes.POINTER(ctypes.c_size_t)]
    lib.muon_step_batched.argtypes = [vp, ctypes.POINTER(MuonMatrix), i32,
                                      ctypes.POINTER(MuonHparams), vp, ctypes.c_size_t, vp]
    lib.adamw_step.argtypes = [vp, ctypes.POINTER(AdamwTensor), i32, ctypes.POINTER(AdamwHparams), vp]
    lib.muon_status_str.argtypes = [i32]
    lib.muon_status_str.restype = ctypes.c_char_p
    lib.muon_test_gram_bf16.argtypes = [vp, vp, vp, i64, i64, i64, i64, f32, vp]
    lib.muon_test_poly_bf16.argtypes = [vp, vp, vp, i64, i64, f32, f32, f32, vp]
    lib.muon_test_update_bf16.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, f32, vp]
    lib.adamw_workspace_size.argtypes = [vp, ctypes.POINTER(AdamwTensor), i32,
                                         ctypes.POINTER(ctypes.c_size_t)]
    lib.adamw_step_clipped.argtypes = [vp, ctypes.POINTER(AdamwTensor), i32,
                                       ctypes.POINTER(AdamwHparams), f32, vp, vp, ctypes.c_size_t, vp]
    lib.muon_test_split_matrices.argtypes = [vp, ctypes.POINTER(MuonMatrix), i32,
                                             ctypes.POINTER(MuonHparams),
                                             ctypes.POINTER(ctypes.c_int32), i32,
                                             ctypes.POINTER(ctypes.c_int)]
    lib.adamw_step_clipped_noalloc.argtypes = [vp, ctypes.POINTER(AdamwTensor), i32,
                                               ctypes.POINTER(AdamwHparams), f32, vp, vp]
    lib.muon_profile_enable.argtypes = [vp, i32]
    lib.muon_profile_collect.argtypes = [vp, ctypes.POINTER(PhaseTimes)]
    for name in ("muon_init", "muon_destroy", "muon_workspace_size", "muon_step_batched",
                 "adamw_step", "muon_test_gram_bf16", "muon_test_poly_bf16",
                 "muon_test_update_bf16", "muon_profile_enable", "muon_profile_collect",
                 "adamw_workspace_size", "adamw_step_clipped", "muon_test_split_matrices",
                 "adamw_step_clipped_noalloc"):
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def exported_symbols():
    """Names of SYMBOLS that the loaded library actually exports."""
    lib = load()
    out = []
    for s in SYMBOLS:
        try:
            getattr(lib, s)
            out.append(s)
        except AttributeError:
            pass
    return out


def _check(status, what):
    if status != 0:
        raise MuonError(status, what)


def _stream_ptr(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    if hasattr(stream, "cuda_stream"):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(stream)


def _dt(t):
    import torch
    if t.dtype == torch.float32:
        return MUON_F32
    if t.dtype == torch.bfloat16:
        return MUON_BF16
    raise TypeError("only float32 and bfloat16 tensors are supported, got %s" % t.dtype)


def _ld(t):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2D row-major tensor (stride(1) == 1)")
    return t.stride(0)


def muon_matrix(param, grad, momentum, update_out=None, norm_out=None, qk_smax=None,
                qk_block_rows=0):
    """Descriptor of one Muon matrix from 2D tensors (row blocks are fine).
    ``qk_smax``: optional float32 device tensor of per-head max logits for
    QK-Clip, one per ``qk_block_rows`` rows."""
    import torch
    if momentum.dtype != torch.float32:
        raise TypeError("momentum must be float32")
    if grad.shape != param.shape or momentum.shape != param.shape:
        raise ValueError("param, grad and momentum shapes differ")
    rows, cols = param.shape
    if update_out is not None:
        if update_out.dtype != torch.float32 or not update_out.is_contiguous() or \
                tuple(update_out.shape) != (rows, cols):
            raise ValueError("update_out must be a contiguous float32 (rows, cols) tensor")
    if norm_out is not None and norm_out.dtype != torch.float32:
        raise ValueError("norm_out must be float32")
    if qk_smax is not None:
        if qk_smax.dtype != torch.float32 or not qk_smax.is_contiguous():
            raise ValueError("qk_smax must be a contiguous float32 tensor")
        if qk_block_rows < 1 or qk_smax.numel() * qk_block_rows < rows:
            raise ValueError("qk_smax needs one value per qk_block_rows rows")
    return MuonMatrix(
        param=param.data_ptr(), grad=grad.data_ptr(), momentum=momentum.data_ptr(),
        update_out=update_out.data_ptr() if update_out is not None else None,
        norm_out=norm_out.data_ptr() if norm_out is not None else None,
        rows=rows, cols=cols, ld_param=_ld(param), ld_grad=_ld(grad), ld_mom=_ld(momentum),
        param_dtype=_dt(param), grad_dtype=_dt(grad),
        qk_smax=qk_smax.data_ptr() if qk_smax is not None else None,
        qk_block_rows=qk_block_rows if qk_smax is not None else 0)


def muon_hparams(lr, momentum=0.95, weight_decay=0.1, eps=1e-7, extra_scale=1.0, nesterov=True,
                 ns_steps=5, ns_dtype="bf16", scale_mode="moonlight", coeffs=None, qk_tau=100.0):
    """Hyperparameters; ``coeffs`` is None or a flat list of 3*ns_steps floats."""
    hp = MuonHparams(lr=lr, momentum=momentum, weight_decay=weight_decay, eps=eps,
                     extra_scale=extra_scale, nesterov=1 if nesterov else 0, ns_steps=ns_steps,
                     ns_dtype=MUON_BF16 if ns_dtype == "bf16" else MUON_F32,
                     scale_mode=SCALE_MODES[scale_mode], qk_tau=qk_tau)
    if coeffs is not None:
        arr = (ctypes.c_float * len(coeffs))(*[float(c) for c in coeffs])
        hp._coeff_keepalive = arr
        hp.coeffs = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
    return hp


def adamw_tensor(param, grad, exp_avg, exp_avg_sq):
    import torch
    for t in (param, grad, exp_avg, exp_avg_sq):
        if not t.is_contiguous():
            raise ValueError("AdamW tensors must be contiguous")
    if exp_avg.dtype != torch.float32 or exp_avg_sq.dtype != torch.float32:
        raise TypeError("AdamW state must be float32")
    n = param.numel()
    if grad.numel() != n or exp_avg.numel() != n or exp_avg_sq.numel() != n:
        raise ValueError("AdamW tensor sizes differ")
    return AdamwTensor(param=param.data_ptr(), grad=grad.data_ptr(), exp_avg=exp_avg.data_ptr(),
                       exp_avg_sq=exp_avg_sq.data_ptr(), numel=n, param_dtype=_dt(param),
                       grad_dtype=_dt(grad))


def adamw_hparams(lr, step, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1):
    return AdamwHparams(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay,
                        step=step)


def muon_init(device=0):
    lib = load()
    h = ctypes.c_void_p()
    _check(lib.muon_init(int(device), ctypes.byref(h)), "muon_init")
    return h


def muon_destroy(h):
    _check(load().muon_destroy(h), "muon_destroy")


def _array(mats):
    arr = (MuonMatrix * len(mats))(*mats)
    return arr


def muon_workspace_size(h, mats, hp):
    sz = ctypes.c_size_t()
    arr = _array(mats)
    _check(load().muon_workspace_size(h, arr, len(mats), ctypes.byref(hp), ctypes.byref(sz)),
           "muon_workspace_size")
    return sz.value


def muon_step_batched(h, mats, hp, workspace, stream=None):
    """``workspace``: a uint8 CUDA tensor of at least muon_workspace_size bytes."""
    arr = _array(mats)
    _check(load().muon_step_batched(h, arr, len(mats), ctypes.byref(hp),
                                    ctypes.c_void_p(workspace.data_ptr()),
                                    workspace.numel() * workspace.element_size(),
                                    _stream_ptr(stream)),
           "muon_step_batched")


def adamw_step(h, tensors, hp, stream=None):
    arr = (AdamwTensor * len(tensors))(*tensors)
    _check(load().adamw_step(h, arr, len(tensors), ctypes.byref(hp), _stream_ptr(stream)),
           "adamw_step")


def adamw_workspace_size(h, tensors):
    arr = (AdamwTensor * len(tensors))(*tensors)
    sz = ctypes.c_size_t()
    _check(load().adamw_workspace_size(h, arr, len(tensors), ctypes.byref(sz)), "adamw_workspace_size")
    return sz.value


def adamw_step_clipped(h, tensors, hp, max_norm, workspace, norm_out=None, stream=None):
    """AdamW with the gradients clipped together to global norm ``max_norm``.
    ``workspace``: uint8 CUDA tensor of at least adamw_workspace_size bytes;
    ``norm_out``: optional float32 CUDA tensor receiving the norm."""
    arr = (AdamwTensor * len(tensors))(*tensors)
    _check(load().adamw_step_clipped(h, arr, len(tensors), ctypes.byref(hp), float(max_norm),
                                     ctypes.c_void_p(norm_out.data_ptr() if norm_out is not None else 0),
                                     ctypes.c_void_p(workspace.data_ptr()),
                                     workspace.numel() * workspace.element_size(),
                                     _stream_ptr(stream)),
           "adamw_step_clipped")


def adamw_step_clipped_noalloc(h, tensors, hp, max_norm, norm_out=None, stream=None):
    """adamw_step_clipped without a workspace: the library's fixed per-device
    scratch holds the partial sums (at most 2^18 chunks of 4096 elements)."""
    arr = (AdamwTensor * len(tensors))(*tensors)
    _check(load().adamw_step_clipped_noalloc(
        h, arr, len(tensors), ctypes.byref(hp), float(max_norm),
        ctypes.c_void_p(norm_out.data_ptr() if norm_out is not None else 0), _stream_ptr(stream)),
        "adamw_step_clipped_noalloc")


def muon_test_gram_bf16(h, X, A, m, n, ldx, lda, s2=1.0, stream=None):
    _check(load().muon_test_gram_bf16(h, X.data_ptr(), A.data_ptr(), m, n, ldx, lda, s2,
                                      _stream_ptr(stream)), "muon_test_gram_bf16")


def muon_test_poly_bf16(h, A, B, m, lda, a, b, c, stream=None):
    """B = a I + b A + c A A (bf16, m x m, leading dimension lda)."""
    _check(load().muon_test_poly_bf16(h, A.data_ptr(), B.data_ptr(), m, lda, a, b, c,
                                      _stream_ptr(stream)), "muon_test_poly_bf16")


def muon_test_update_bf16(h, X, B, Xo, m, n, ldx, ldb, s=1.0, stream=None):
    """Xo = s B X (bf16; X, Xo m x n with leading dimension ldx, B m x m)."""
    _check(load().muon_test_update_bf16(h, X.data_ptr(), B.data_ptr(), Xo.data_ptr(), m, n, ldx,
                                        ldb, s, _stream_ptr(stream)), "muon_test_update_bf16")


def muon_test_split_matrices(h, mats, hp):
    """Indices of the matrices whose tiles sit where the grouped GEMM
    launches' per-XCD tile ranges start or end, or that hold quarter tiles."""
    arr = _array(mats)
    cnt = ctypes.c_int()
    _check(load().muon_test_split_matrices(h, arr, len(mats), ctypes.byref(hp), None, 0,
                                           ctypes.byref(cnt)), "muon_test_split_matrices")
    out = (ctypes.c_int32 * max(cnt.value, 1))()
    _check(load().muon_test_split_matrices(h, arr, len(mats), ctypes.byref(hp), out, cnt.value,
                                           ctypes.byref(cnt)), "muon_test_split_matrices")
    return list(out[:cnt.value])


def muon_profile_enable(h, enable=True):
    _check(load().muon_profile_enable(h, 1 if enable else 0), "muon_profile_enable")


def muon_profile_collect(h):
    """{phase: (total_ms, launches)} since the previous collect."""
    pt = PhaseTimes()
    _check(load().muon_profile_collect(h, ctypes.byref(pt)), "muon_profile_collect")
    return {PHASES[i]: (pt.ms[i], pt.launches[i]) for i in range(NUM_PHASES)}
