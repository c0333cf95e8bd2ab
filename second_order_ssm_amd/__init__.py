"""Python binding of libtwomamba.so, the MI355X 2Mamba / 2Mamba-E operator.

Argument marshalling only: tensors are passed to the C ABI as raw device
pointers together with torch's current HIP stream; every step of the
computation runs in the library's HIP kernels.  PyTorch provides device memory
and streams, nothing else.  If the library is not built, every entry point
raises -- there is no fallback.

    out, state, norm = fwd(q, k, v, z, variant="sq", want_state=True)
    out = step(q, k, v, z, state, norm)          # state/norm updated in place
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["load", "abi_version", "status_str", "workspace_size", "fwd", "fwd_noalloc", "step", "library_path",
           "exp_cache", "exp_cache_fill", "exp_step_workspace_size", "exp_step", "bwd_workspace_size", "bwd", "conv2", "step_conv",
           "TwoMambaError", "SQ", "EXP", "LIN", "FLAG_NO_NORM", "FLAG_REFERENCE_KERNELS", "FLAG_FIRST_ORDER",
           "num_pairs", "twomamba", "ceiling_copy", "ceiling_mfma", "fwd_conv", "conv_workspace_size"]

_PKG = os.path.dirname(os.path.abspath(__file__))
# TWOMAMBA_LIBRARY names another build of the same library (e.g. the host-sanitized one)
library_path = os.environ.get("TWOMAMBA_LIBRARY") or os.path.join(_PKG, "libtwomamba.so")

SQ, EXP, LIN = 0, 1, 2
F32, BF16 = 0, 1
FLAG_NO_NORM = 1
FLAG_REFERENCE_KERNELS = 2
FLAG_FIRST_ORDER = 4
FLAG_ATTENTION_FORM = 8
FLAG_CHUNKED_FORM = 16
_DT = {torch.float32: F32, torch.bfloat16: BF16}
_VARIANT = {"sq": SQ, "exp": EXP, "lin": LIN}


class TwoMambaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({status_str(status)})")
        self.status = status


class FwdDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("T", ctypes.c_int),
                ("dk", ctypes.c_int), ("dv", ctypes.c_int), ("chunk", ctypes.c_int),
                ("scale", ctypes.c_float), ("variant", ctypes.c_int), ("dtype", ctypes.c_int),
                ("flags", ctypes.c_uint)]


class ExpCacheDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("dk", ctypes.c_int), ("dv", ctypes.c_int),
                ("max_len", ctypes.c_int), ("pos", ctypes.c_int), ("scale", ctypes.c_float),
                ("dtype", ctypes.c_int), ("flags", ctypes.c_uint)]


class ConvDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("T", ctypes.c_int), ("d", ctypes.c_int),
                ("dtype", ctypes.c_int), ("flags", ctypes.c_uint)]


class StepDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("dk", ctypes.c_int), ("dv", ctypes.c_int),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int), ("flags", ctypes.c_uint)]


_lib = None


def load(path: str | None = None):
    """Load (once) and return the ctypes handle of libtwomamba.so."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path
    if not os.path.exists(p):
        raise RuntimeError(f"libtwomamba.so not built ({p}); run `python -m second_order_ssm_amd.build`")
    lib = ctypes.CDLL(p)
    vp = ctypes.c_void_p
    lib.twomamba_abi_version.restype = ctypes.c_int
    lib.twomamba_status_str.restype = ctypes.c_char_p
    lib.twomamba_status_str.argtypes = [ctypes.c_int]
    lib.twomamba_fwd_workspace_size.restype = ctypes.c_int
    lib.twomamba_fwd_workspace_size.argtypes = [ctypes.POINTER(FwdDesc), ctypes.POINTER(ctypes.c_size_t)]
    lib.twomamba_fwd.restype = ctypes.c_int
    lib.twomamba_fwd.argtypes = [ctypes.POINTER(FwdDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                 ctypes.c_size_t, vp]
    lib.twomamba_fwd_stats.restype = ctypes.c_int
    lib.twomamba_fwd_stats.argtypes = [ctypes.POINTER(FwdDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       ctypes.c_size_t, vp]
    lib.twomamba_fwd_timed.restype = ctypes.c_int
    lib.twomamba_fwd_timed.argtypes = [ctypes.POINTER(FwdDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       ctypes.c_size_t, vp, ctypes.POINTER(ctypes.c_float),
                                       ctypes.POINTER(ctypes.c_char_p), ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.twomamba_step.restype = ctypes.c_int
    lib.twomamba_step.argtypes = [ctypes.POINTER(StepDesc), vp, vp, vp, vp, vp, vp, vp, vp]
    lib.twomamba_exp_cache_fill.restype = ctypes.c_int
    lib.twomamba_exp_cache_fill.argtypes = [ctypes.POINTER(ExpCacheDesc), vp, vp, vp, vp, vp, vp, vp]
    lib.twomamba_exp_step_workspace_size.restype = ctypes.c_int
    lib.twomamba_exp_step_workspace_size.argtypes = [ctypes.POINTER(ExpCacheDesc), ctypes.POINTER(ctypes.c_size_t)]
    lib.twomamba_exp_step.restype = ctypes.c_int
    lib.twomamba_exp_step.argtypes = [ctypes.POINTER(ExpCacheDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      ctypes.c_size_t, vp]
    lib.twomamba_bwd_workspace_size.restype = ctypes.c_int
    lib.twomamba_bwd_workspace_size.argtypes = [ctypes.POINTER(FwdDesc), ctypes.POINTER(ctypes.c_size_t)]
    lib.twomamba_bwd.restype = ctypes.c_int
    lib.twomamba_bwd.argtypes = [ctypes.POINTER(FwdDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                 ctypes.c_size_t, vp]
    lib.twomamba_bwd_timed.restype = ctypes.c_int
    lib.twomamba_bwd_timed.argtypes = [ctypes.POINTER(FwdDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       ctypes.c_size_t, vp, ctypes.POINTER(ctypes.c_float),
                                       ctypes.POINTER(ctypes.c_char_p), ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.twomamba_fwd_conv_workspace_size.restype = ctypes.c_int
    lib.twomamba_fwd_conv_workspace_size.argtypes = [ctypes.POINTER(FwdDesc), ctypes.POINTER(ctypes.c_size_t)]
    lib.twomamba_fwd_conv.restype = ctypes.c_int
    lib.twomamba_fwd_conv.argtypes = [ctypes.POINTER(FwdDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, ctypes.c_size_t, vp]
    lib.twomamba_fwd_noalloc.restype = ctypes.c_int
    lib.twomamba_fwd_noalloc.argtypes = [ctypes.POINTER(FwdDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.twomamba_ceiling_copy.restype = ctypes.c_int
    lib.twomamba_ceiling_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
    lib.twomamba_ceiling_mfma.restype = ctypes.c_int
    lib.twomamba_ceiling_mfma.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp]
    lib.twomamba_conv2.restype = ctypes.c_int
    lib.twomamba_conv2.argtypes = [ctypes.POINTER(ConvDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.twomamba_step_conv.restype = ctypes.c_int
    lib.twomamba_step_conv.argtypes = [ctypes.POINTER(StepDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    if path is None:
        _lib = lib
    return lib


def bwd_workspace_size(desc: FwdDesc) -> int:
    n = ctypes.c_size_t(0)
    s = load().twomamba_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if s != 0:
        raise TwoMambaError(s, "twomamba_bwd_workspace_size")
    return n.value


def abi_version() -> int:
    return load().twomamba_abi_version()


def status_str(status: int) -> str:
    return load().twomamba_status_str(status).decode()


def num_pairs(d: int) -> int:
    return d * (d + 1) // 2


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_desc(B, H, T, dk, dv, *, variant="sq", dtype=torch.bfloat16, scale=1.0, chunk=0, flags=0) -> FwdDesc:
    return FwdDesc(B, H, T, dk, dv, chunk, scale, _VARIANT[variant] if isinstance(variant, str) else variant,
                   _DT[dtype] if isinstance(dtype, torch.dtype) else dtype, flags)


def workspace_size(desc: FwdDesc) -> int:
    n = ctypes.c_size_t(0)
    s = load().twomamba_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if s != 0:
        raise TwoMambaError(s, "twomamba_fwd_workspace_size")
    return n.value


def _check(t, shape, dtype, name):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


def fwd(q, k, v, z, *, variant="sq", scale=1.0, chunk=0, no_norm=False, reference_kernels=False,
        state_in=None, norm_in=None, want_state=False, out=None, state_out=None, norm_out=None, workspace=None,
        kernel_times=None, want_stats=False, row_stat=None, noalloc=False):
    """Chunked forward.  Returns out, or (out, state_out, norm_out) with want_state.

    With ``want_stats`` (or a ``row_stat`` tensor [B, H, T] fp32 to fill) the
    call goes through twomamba_fwd_stats and the per-row statistic (the 2Mamba
    weight sum, the 2Mamba-E log-sum-exp) is appended to what is returned:
    (out, row_stat) or (out, state_out, norm_out, row_stat); bwd takes it.
    With ``kernel_times`` (a list), the call goes through twomamba_fwd_timed:
    it waits for completion and appends (kernel name, milliseconds) per launch.
    """
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    flags = (FLAG_NO_NORM if no_norm else 0) | (FLAG_REFERENCE_KERNELS if reference_kernels else 0)
    desc = make_desc(B, H, T, dk, dv, variant=variant, dtype=q.dtype, scale=scale, chunk=chunk, flags=flags)
    _check(q, (B, H, T, dk), q.dtype, "q")
    _check(k, (B, H, T, dk), q.dtype, "k")
    _check(v, (B, H, T, dv), q.dtype, "v")
    _check(z, (B, H, T), torch.float32, "z")
    lin = desc.variant == LIN     # first order: dk x dv state, no normaliser
    D = dk if lin else num_pairs(dk)
    if state_in is not None:
        _check(state_in, (B, H, D, dv), torch.float32, "state_in")
        if not lin:
            _check(norm_in, (B, H, D), torch.float32, "norm_in")
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if want_state and state_out is None:
        state_out = torch.empty((B, H, D, dv), dtype=torch.float32, device=q.device)
        if not lin:
            norm_out = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    stats = want_stats or row_stat is not None
    if stats:
        if kernel_times is not None:
            raise ValueError("kernel_times is not available with row statistics")
        if row_stat is None:
            row_stat = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
        _check(row_stat, (B, H, T), torch.float32, "row_stat")
    head = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(state_in), _ptr(norm_in),
            _ptr(out), _ptr(state_out), _ptr(norm_out))
    if noalloc:
        if stats or kernel_times is not None or workspace is not None:
            raise ValueError("noalloc takes no workspace, row statistics or kernel timings")
        s = load().twomamba_fwd_noalloc(*head, _stream())
        if s != 0:
            raise TwoMambaError(s, "twomamba_fwd_noalloc")
        return (out, state_out, norm_out) if want_state or state_out is not None else out
    nbytes = workspace_size(desc)
    if nbytes and (workspace is None or workspace.numel() * workspace.element_size() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    tail = (_ptr(workspace) if nbytes else None, ctypes.c_size_t(nbytes), _stream())
    args = head + tail
    if stats:
        s = load().twomamba_fwd_stats(*head, _ptr(row_stat), *tail)
    elif kernel_times is None:
        s = load().twomamba_fwd(*args)
    else:
        cap = 24
        ms = (ctypes.c_float * cap)()
        names = (ctypes.c_char_p * cap)()
        cnt = ctypes.c_int(0)
        s = load().twomamba_fwd_timed(*args, ms, names, cap, ctypes.byref(cnt))
        for i in range(min(cnt.value, cap)):
            kernel_times.append((names[i].decode(), float(ms[i])))
    if s != 0:
        raise TwoMambaError(s, "twomamba_fwd_stats" if stats else "twomamba_fwd")
    res = (out, state_out, norm_out) if want_state or state_out is not None else (out,)
    if stats:
        res += (row_stat,)
    return res if len(res) > 1 else out


def ceiling_copy(src, dst):
    """Streaming device copy of src into dst (measurement aid, twomamba_ceiling_copy)."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst sizes differ")
    s = load().twomamba_ceiling_copy(_ptr(src), _ptr(dst), ctypes.c_size_t(n), _stream())
    if s != 0:
        raise TwoMambaError(s, "twomamba_ceiling_copy")


def ceiling_mfma(workgroups, iters, sink, clocks=None):
    """MFMA-loop microbenchmark (measurement aid, twomamba_ceiling_mfma); sink is a
    float32 device tensor of workgroups * 256 elements, clocks None or an int64
    device tensor [workgroups, 2] (shader cycles, 100 MHz ticks)."""
    if sink.dtype != torch.float32 or sink.numel() < workgroups * 256 or not sink.is_contiguous():
        raise ValueError("sink must be a contiguous float32 tensor of workgroups * 256 elements")
    if clocks is not None and (clocks.dtype != torch.int64 or clocks.numel() < 2 * workgroups):
        raise ValueError("clocks must be an int64 tensor of workgroups x 2 elements")
    s = load().twomamba_ceiling_mfma(int(workgroups), int(iters), _ptr(sink), _ptr(clocks), _stream())
    if s != 0:
        raise TwoMambaError(s, "twomamba_ceiling_mfma")


def fwd_noalloc(q, k, v, z, **kw):
    """fwd through twomamba_fwd_noalloc: the library's static scratch instead of a
    workspace (output and state tensors are still allocated here unless passed)."""
    return fwd(q, k, v, z, noalloc=True, **kw)


def step(q, k, v, z, state, norm, *, scale=1.0, no_norm=False, first_order=False, out=None):
    """One decode step; state [B,H,D,dv] and norm [B,H,D] (fp32) are updated in
    place.  first_order: the Mamba-2S step on a [B,H,dk,dv] state, norm None."""
    B, H, dk = q.shape
    dv = v.shape[-1]
    _check(q, (B, H, dk), q.dtype, "q")
    _check(k, (B, H, dk), q.dtype, "k")
    _check(v, (B, H, dv), q.dtype, "v")
    _check(z, (B, H), torch.float32, "z")
    D = dk if first_order else num_pairs(dk)
    _check(state, (B, H, D, dv), torch.float32, "state")
    if not first_order:
        _check(norm, (B, H, D), torch.float32, "norm")
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    flags = (FLAG_NO_NORM if no_norm else 0) | (FLAG_FIRST_ORDER if first_order else 0)
    desc = StepDesc(B, H, dk, dv, scale, _DT[q.dtype], flags)
    s = load().twomamba_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(state), _ptr(norm),
                             _ptr(out), _stream())
    if s != 0:
        raise TwoMambaError(s, "twomamba_step")
    return out


# ---------------------------------------------------------------------------
# 2Mamba-E decoding over a key/value cache

def exp_cache(B, H, d, max_len, dtype=torch.bfloat16, device="cuda"):
    """Empty caches: k [B,H,max_len,d], v [B,H,max_len,d] (dtype), g [B,H,max_len] (fp64)."""
    kc = torch.empty((B, H, max_len, d), dtype=dtype, device=device)
    vc = torch.empty((B, H, max_len, d), dtype=dtype, device=device)
    gc = torch.empty((B, H, max_len), dtype=torch.float64, device=device)
    return kc, vc, gc


def _cache_desc(B, H, dk, dv, max_len, pos, scale, dtype):
    return ExpCacheDesc(B, H, dk, dv, max_len, pos, scale, _DT[dtype], 0)


def exp_cache_fill(k, v, z, k_cache, v_cache, g_cache):
    """Write a prompt k, v [B,H,T,d], z [B,H,T] into cache positions 0..T-1."""
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    L = k_cache.shape[2]
    _check(k, (B, H, T, dk), k.dtype, "k")
    _check(v, (B, H, T, dv), k.dtype, "v")
    _check(z, (B, H, T), torch.float32, "z")
    _check(k_cache, (B, H, L, dk), k.dtype, "k_cache")
    _check(v_cache, (B, H, L, dv), k.dtype, "v_cache")
    _check(g_cache, (B, H, L), torch.float64, "g_cache")
    desc = _cache_desc(B, H, dk, dv, L, T, 1.0, k.dtype)
    s = load().twomamba_exp_cache_fill(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(z), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(g_cache), _stream())
    if s != 0:
        raise TwoMambaError(s, "twomamba_exp_cache_fill")


def exp_step_workspace_size(B, H, d, max_len, pos, dtype=torch.bfloat16) -> int:
    desc = _cache_desc(B, H, d, d, max_len, pos, 1.0, dtype)
    n = ctypes.c_size_t(0)
    s = load().twomamba_exp_step_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if s != 0:
        raise TwoMambaError(s, "twomamba_exp_step_workspace_size")
    return n.value


def exp_step(q, k, v, z, k_cache, v_cache, g_cache, pos, *, scale=1.0, out=None, workspace=None):
    """2Mamba-E decode at position `pos` (caches hold tokens 0..pos-1; row pos is appended)."""
    B, H, dk = q.shape
    dv = v.shape[-1]
    L = k_cache.shape[2]
    _check(q, (B, H, dk), q.dtype, "q")
    _check(k, (B, H, dk), q.dtype, "k")
    _check(v, (B, H, dv), q.dtype, "v")
    _check(z, (B, H), torch.float32, "z")
    _check(k_cache, (B, H, L, dk), q.dtype, "k_cache")
    _check(v_cache, (B, H, L, dv), q.dtype, "v_cache")
    _check(g_cache, (B, H, L), torch.float64, "g_cache")
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    desc = _cache_desc(B, H, dk, dv, L, pos, scale, q.dtype)
    if workspace is None:
        n = ctypes.c_size_t(0)
        s = load().twomamba_exp_step_workspace_size(ctypes.byref(desc), ctypes.byref(n))
        if s != 0:
            raise TwoMambaError(s, "twomamba_exp_step_workspace_size")
        workspace = torch.empty(max(n.value, 1), dtype=torch.uint8, device=q.device)
    s = load().twomamba_exp_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(g_cache), _ptr(out), _ptr(workspace), workspace.numel(), _stream())
    if s != 0:
        raise TwoMambaError(s, "twomamba_exp_step")
    return out


def bwd(q, k, v, z, out, dout, *, variant="sq", scale=1.0, no_norm=False, reference_kernels=False,
        attention_form=False, chunked_form=False, grads=None, workspace=None, kernel_times=None, row_stat=None):
    """Backward of fwd (no initial state): returns (dq, dk, dv, dz).

    ``out`` is the forward output for the same inputs; ``row_stat`` the
    forward's row statistics (fwd(..., want_stats=True)), or None to have the
    backward recompute them; ``grads`` may supply the four output tensors.  With ``kernel_times`` (a list) the call goes through
    twomamba_bwd_timed and appends (kernel name, milliseconds) per launch.  ``attention_form``: the
    quadratic form instead of the linear-in-T one (first order at any T, 2Mamba from 20480 tokens on);
    ``chunked_form``: 2Mamba's linear-in-T form at any T.
    """
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    flags = ((FLAG_NO_NORM if no_norm else 0) | (FLAG_REFERENCE_KERNELS if reference_kernels else 0)
             | (FLAG_ATTENTION_FORM if attention_form else 0) | (FLAG_CHUNKED_FORM if chunked_form else 0))
    desc = make_desc(B, H, T, dk, dv, variant=variant, dtype=q.dtype, scale=scale, flags=flags)
    _check(q, (B, H, T, dk), q.dtype, "q")
    _check(k, (B, H, T, dk), q.dtype, "k")
    _check(v, (B, H, T, dv), q.dtype, "v")
    _check(z, (B, H, T), torch.float32, "z")
    _check(out, (B, H, T, dv), q.dtype, "out")
    _check(dout, (B, H, T, dv), q.dtype, "dout")
    if row_stat is not None:
        _check(row_stat, (B, H, T), torch.float32, "row_stat")
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(z))
    gq, gk, gv, gz = grads
    _check(gq, (B, H, T, dk), q.dtype, "dq")
    _check(gk, (B, H, T, dk), q.dtype, "dk")
    _check(gv, (B, H, T, dv), q.dtype, "dv")
    _check(gz, (B, H, T), torch.float32, "dz")
    nbytes = bwd_workspace_size(desc)
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    args = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(out), _ptr(dout), _ptr(row_stat),
            _ptr(gq), _ptr(gk), _ptr(gv), _ptr(gz), _ptr(workspace), ctypes.c_size_t(nbytes), _stream())
    if kernel_times is None:
        s = load().twomamba_bwd(*args)
    else:
        cap = 24
        ms = (ctypes.c_float * cap)()
        names = (ctypes.c_char_p * cap)()
        cnt = ctypes.c_int(0)
        s = load().twomamba_bwd_timed(*args, ms, names, cap, ctypes.byref(cnt))
        for i in range(min(cnt.value, cap)):
            kernel_times.append((names[i].decode(), float(ms[i])))
    if s != 0:
        raise TwoMambaError(s, "twomamba_bwd")
    return gq, gk, gv, gz


def conv2(q, k, v, weight, bias=None, state_in=None, *, outs=None, want_state=False, state_out=None):
    """Size-2 causal input convolution of q, k, v.  Returns (q', k', v') or,
    with ``want_state``, (q', k', v', conv_state_out)."""
    B, H, T, d = q.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, (B, H, T, d), q.dtype, n)
    _check(weight, (3, H, d, 2), torch.float32, "weight")
    if bias is not None:
        _check(bias, (3, H, d), torch.float32, "bias")
    if state_in is not None:
        _check(state_in, (B, H, 3, d), q.dtype, "state_in")
    if outs is None:
        outs = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    if want_state and state_out is None:
        state_out = torch.empty((B, H, 3, d), dtype=q.dtype, device=q.device)
    desc = ConvDesc(B, H, T, d, _DT[q.dtype], 0)
    s = load().twomamba_conv2(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(weight), _ptr(bias),
                              _ptr(state_in), _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]), _ptr(state_out),
                              _stream())
    if s != 0:
        raise TwoMambaError(s, "twomamba_conv2")
    return (*outs, state_out) if (want_state or state_out is not None) else tuple(outs)


def conv_workspace_size(desc: FwdDesc) -> int:
    n = ctypes.c_size_t(0)
    s = load().twomamba_fwd_conv_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if s != 0:
        raise TwoMambaError(s, "twomamba_fwd_conv_workspace_size")
    return n.value


def fwd_conv(q, k, v, z, weight, bias=None, conv_state_in=None, *, variant="sq", scale=1.0, chunk=0, no_norm=False,
             reference_kernels=False, state_in=None, norm_in=None, want_state=False, out=None, state_out=None,
             norm_out=None, want_conv_state=False, conv_state_out=None, workspace=None):
    """The forward with the size-2 input convolution in front (twomamba_fwd_conv):
    q, k, v are the raw inputs.  Returns out, then (state_out, norm_out) with
    ``want_state``, then conv_state_out with ``want_conv_state``."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    flags = (FLAG_NO_NORM if no_norm else 0) | (FLAG_REFERENCE_KERNELS if reference_kernels else 0)
    desc = make_desc(B, H, T, dk, dv, variant=variant, dtype=q.dtype, scale=scale, chunk=chunk, flags=flags)
    _check(q, (B, H, T, dk), q.dtype, "q")
    _check(k, (B, H, T, dk), q.dtype, "k")
    _check(v, (B, H, T, dv), q.dtype, "v")
    _check(z, (B, H, T), torch.float32, "z")
    _check(weight, (3, H, dk, 2), torch.float32, "weight")
    if bias is not None:
        _check(bias, (3, H, dk), torch.float32, "bias")
    if conv_state_in is not None:
        _check(conv_state_in, (B, H, 3, dk), q.dtype, "conv_state_in")
    lin = desc.variant == LIN
    D = dk if lin else num_pairs(dk)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if want_state and state_out is None:
        state_out = torch.empty((B, H, D, dv), dtype=torch.float32, device=q.device)
        if not lin:
            norm_out = torch.empty((B, H, D), dtype=torch.float32, device=q.device)
    if want_conv_state and conv_state_out is None:
        conv_state_out = torch.empty((B, H, 3, dk), dtype=q.dtype, device=q.device)
    nbytes = conv_workspace_size(desc)
    if nbytes and (workspace is None or workspace.numel() * workspace.element_size() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    s = load().twomamba_fwd_conv(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(weight), _ptr(bias),
                                 _ptr(conv_state_in), _ptr(conv_state_out), _ptr(state_in), _ptr(norm_in), _ptr(out),
                                 _ptr(state_out), _ptr(norm_out), _ptr(workspace) if nbytes else None,
                                 ctypes.c_size_t(nbytes), _stream())
    if s != 0:
        raise TwoMambaError(s, "twomamba_fwd_conv")
    res = (out,)
    if want_state or state_out is not None:
        res += (state_out, norm_out)
    if want_conv_state or conv_state_out is not None:
        res += (conv_state_out,)
    return res if len(res) > 1 else out


def step_conv(q, k, v, z, weight, bias, conv_state, state, norm, *, scale=1.0, no_norm=False, first_order=False,
              out=None):
    """Decode step with the size-2 input convolution; conv_state, state and
    norm are updated in place (first_order: [B,H,d,d] state, norm None)."""
    B, H, d = q.shape
    _check(k, (B, H, d), q.dtype, "k")
    _check(v, (B, H, d), q.dtype, "v")
    _check(z, (B, H), torch.float32, "z")
    _check(weight, (3, H, d, 2), torch.float32, "weight")
    if bias is not None:
        _check(bias, (3, H, d), torch.float32, "bias")
    _check(conv_state, (B, H, 3, d), q.dtype, "conv_state")
    D = d if first_order else num_pairs(d)
    _check(state, (B, H, D, d), torch.float32, "state")
    if not first_order:
        _check(norm, (B, H, D), torch.float32, "norm")
    if out is None:
        out = torch.empty((B, H, d), dtype=q.dtype, device=q.device)
    flags = (FLAG_NO_NORM if no_norm else 0) | (FLAG_FIRST_ORDER if first_order else 0)
    desc = StepDesc(B, H, d, d, scale, _DT[q.dtype], flags)
    s = load().twomamba_step_conv(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(weight),
                                  _ptr(bias), _ptr(conv_state), _ptr(state), _ptr(norm), _ptr(out), _stream())
    if s != 0:
        raise TwoMambaError(s, "twomamba_step_conv")
    return out


# ---------------------------------------------------------------------------
# autograd: the forward keeps its row statistics for the backward

class _TwoMambaFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, z, variant, scale, no_norm):
        q, k, v, z = (t.contiguous() for t in (q, k, v, z))
        if variant == "lin":
            out = fwd(q, k, v, z, variant=variant, scale=scale, no_norm=no_norm)
            stat = None
        else:
            out, stat = fwd(q, k, v, z, variant=variant, scale=scale, no_norm=no_norm, want_stats=True)
        ctx.save_for_backward(q, k, v, z, out, stat)
        ctx.opts = (variant, scale, no_norm)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, z, out, stat = ctx.saved_tensors
        variant, scale, no_norm = ctx.opts
        dq, dk, dv, dz = bwd(q, k, v, z, out, dout.contiguous(), variant=variant, scale=scale, no_norm=no_norm,
                             row_stat=stat)
        return dq, dk, dv, dz, None, None, None


def twomamba(q, k, v, z, *, variant="sq", scale=1.0, no_norm=False):
    """Differentiable operator: out = fwd(q, k, v, z); the backward runs
    twomamba_bwd with the forward's row statistics.  q, k, v [B,H,T,d] (bf16 or
    fp32, d = 16 or 64), z [B,H,T] fp32, no initial state."""
    return _TwoMambaFn.apply(q, k, v, z, variant, scale, no_norm)
