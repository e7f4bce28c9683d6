"""Gated delta rule on AMD MI355X (gfx950): Python binding of libgdr.so.

This module only marshals arguments: it checks torch tensors, allocates the
outputs with torch (PyTorch provides device memory and the stream), and calls
the C ABI declared in ``include/gdr.h`` through ctypes.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  If the
library has not been built (``python -m gated_delta_rule_68_amd.build``) every
call raises.

Entry points (same names as the C ABI):
  gates(q, k, a, b, A_log, dt_bias)             -> q_hat, k_hat, g, beta
  recurrent_fwd(q, k, v, a, b, A_log, dt_bias, initial_state=None, ...) -> o, final_state
  chunked_fwd(q, k, v, a, b, A_log, dt_bias, initial_state=None, chunk=32, ...) -> o, final_state
  fwd(...)  picks the form on the step count, as the GatedDeltaRule.ixx File
            Reference ("Detailed Description") describes the backend doing:
            sequences no longer than one chunk run the recurrence, longer
            ones the chunked form.
  conv_silu(x, weight, H_k, H_v, d_k, d_v, bias=None, conv_state=None, ...)
            -> q, k, v, final_conv_state   (the layer's step before the rule)
  gated_rmsnorm(o, z, weight, eps=1e-6)  -> out   (the layer's step after it)
  chunked_fwd_gated_rmsnorm(q, k, v, a, b, A_log, dt_bias, z, norm_weight, ...)
            -> out, final_state   (the chunked form, then that norm)
  chunked_fwd_split(..., segment_len)    -> o, final_state   (segments of each
            sequence in parallel: a two-level scan for long, few-head prefill)

Layouts: q, k [total, H_k, d_k]; v [total, H_v, d_v]; a, b [total, H_v]
(all fp32 or all bf16); A_log, dt_bias [H_v] fp32; states
[N, H_v, d_k, d_v] fp32; o [total, H_v, d_v] in the input dtype.  A dense
batch passes num_seqs (equal-length sequences back to back) or 4-D
[N, T, H, d] / 3-D [N, T, H] tensors; a packed batch passes cu_seqlens
(int32 [N + 1] on the device).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["gates", "recurrent_fwd", "chunked_fwd", "chunked_fwd_split", "fwd", "chunked_path", "conv_silu",
           "chunked_workspace", "chunked_workspace_bytes", "workspace_error",
           "gated_rmsnorm", "library_path", "lib", "GdrError", "abi_version",
           "chunked_fwd_noalloc", "NOALLOC_SCRATCH_BYTES", "chunked_fwd_gated_rmsnorm",
           "ssd_recurrent_fwd", "ssd_chunked_fwd", "ssd_chunked_fwd_split", "kda_recurrent_fwd",
           "kda_chunked_fwd",
           "kda_chunked_fwd_split"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgdr.so")

GDR_F32, GDR_BF16 = 0, 1
_STATUS = {0: "GDR_OK", 1: "GDR_ERR_NULL", 2: "GDR_ERR_SHAPE", 3: "GDR_ERR_UNSUPPORTED",
           4: "GDR_ERR_ALIGN", 5: "GDR_ERR_WORKSPACE", 6: "GDR_ERR_LAUNCH", 7: "GDR_ERR_ALIAS"}


class GdrError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {_STATUS.get(status, status)} ({msg})")
        self.status = status


class GdrShape(ctypes.Structure):
    """Mirror of ``gdr_shape`` in include/gdr.h."""
    _fields_ = [("num_seqs", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("total_tokens", ctypes.c_int64), ("cu_seqlens", ctypes.c_void_p),
                ("H_k", ctypes.c_int32), ("H_v", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("dtype", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("scale", ctypes.c_float), ("l2_eps", ctypes.c_float)]


_lib = None
_load_error: Optional[str] = None


def library_path() -> str:
    return _LIB_PATH


def _bind(lib):
    vp = ctypes.c_void_p
    sp = ctypes.POINTER(GdrShape)
    lib.gdr_gates.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdr_gates.restype = ctypes.c_int
    lib.gdr_recurrent_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdr_recurrent_fwd.restype = ctypes.c_int
    lib.gdr_chunked_fwd.argtypes = [sp] + [vp] * 10 + [vp, ctypes.c_size_t, vp]
    lib.gdr_chunked_fwd.restype = ctypes.c_int
    lib.gdr_chunked_fwd_gated_rmsnorm.argtypes = ([sp] + [vp] * 10 + [ctypes.c_float] +
                                                  [vp, vp, vp, ctypes.c_size_t, vp])
    lib.gdr_chunked_fwd_gated_rmsnorm.restype = ctypes.c_int
    lib.gdr_chunked_fwd_noalloc.argtypes = [sp] + [vp] * 10 + [vp]
    lib.gdr_chunked_fwd_noalloc.restype = ctypes.c_int
    lib.gdr_chunked_workspace_bytes.argtypes = [sp]
    lib.gdr_chunked_workspace_bytes.restype = ctypes.c_size_t
    lib.gdr_status_string.argtypes = [ctypes.c_int]
    lib.gdr_status_string.restype = ctypes.c_char_p
    lib.gdr_chunked_path.argtypes = [sp]
    lib.gdr_chunked_path.restype = ctypes.c_int
    lib.gdr_abi_version.argtypes = []
    lib.gdr_abi_version.restype = ctypes.c_int
    lib.gdr_conv_silu.argtypes = [sp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdr_conv_silu.restype = ctypes.c_int
    lib.gdr_gated_rmsnorm.argtypes = [sp, vp, vp, vp, ctypes.c_float, vp, vp]
    lib.gdr_gated_rmsnorm.restype = ctypes.c_int
    for name in ("gdr_chunked_fwd_split", "gdr_kda_chunked_fwd_split"):
        getattr(lib, name).argtypes = [sp, ctypes.c_int32] + [vp] * 10 + [vp, ctypes.c_size_t, vp]
        getattr(lib, name).restype = ctypes.c_int
    lib.gdr_ssd_chunked_fwd_split.argtypes = [sp, ctypes.c_int32] + [vp] * 9 + [vp, ctypes.c_size_t, vp]
    lib.gdr_ssd_chunked_fwd_split.restype = ctypes.c_int
    for name in ("gdr_chunked_split_workspace", "gdr_kda_chunked_split_workspace",
                 "gdr_ssd_chunked_split_workspace"):
        getattr(lib, name).argtypes = [sp, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
        getattr(lib, name).restype = ctypes.c_int
    lib.gdr_kda_recurrent_fwd.argtypes = [sp] + [vp] * 11
    lib.gdr_kda_recurrent_fwd.restype = ctypes.c_int
    lib.gdr_kda_chunked_fwd.argtypes = [sp] + [vp] * 10 + [vp, ctypes.c_size_t, vp]
    lib.gdr_kda_chunked_fwd.restype = ctypes.c_int
    lib.gdr_kda_chunked_workspace.argtypes = [sp, ctypes.POINTER(ctypes.c_size_t)]
    lib.gdr_kda_chunked_workspace.restype = ctypes.c_int
    for name in ("gdr_ssd_recurrent_fwd", "gdr_ssd_chunked_fwd"):
        getattr(lib, name).argtypes = [sp] + [vp] * 10
        getattr(lib, name).restype = ctypes.c_int
    return lib


def lib():
    """The loaded libgdr.so; raises if it is missing or fails to load."""
    global _lib, _load_error
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"libgdr.so is not built ({_LIB_PATH} missing): run "
                "`python -m gated_delta_rule_68_amd.build` (there is no non-HIP fallback)")
        try:
            _lib = _bind(ctypes.CDLL(_LIB_PATH))
        except OSError as e:  # pragma: no cover - depends on the box
            _load_error = str(e)
            raise RuntimeError(f"failed to load {_LIB_PATH}: {e}") from e
    return _lib


def abi_version() -> int:
    return int(lib().gdr_abi_version())


# ------------------------------------------------------------------ marshalling
def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return GDR_F32
    if dt == torch.bfloat16:
        return GDR_BF16
    raise TypeError(f"unsupported dtype {dt}: q, k, v, a, b must be float32 or bfloat16")


def _check(t: torch.Tensor, name: str, device, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _flatten(x: torch.Tensor, tail: int) -> torch.Tensor:
    """[N, T, ...] -> [N*T, ...] for dense 4-D/3-D inputs (view, no copy)."""
    if x.dim() == tail + 2:
        return x.reshape((-1,) + tuple(x.shape[2:]))
    return x


def _make_shape(total, H_k, H_v, d_k, d_v, cu_seqlens, num_seqs, dtype_code, chunk, scale,
                l2_eps, dense_T=None):
    s = GdrShape()
    if cu_seqlens is not None:
        s.num_seqs = cu_seqlens.numel() - 1
        s.seq_len = 0
        s.cu_seqlens = cu_seqlens.data_ptr()
    else:
        if num_seqs is None:
            num_seqs = 1 if dense_T is None else total // dense_T
        if num_seqs < 0 or (num_seqs > 0 and total % num_seqs != 0) or (num_seqs == 0 and total):
            raise ValueError(f"total tokens {total} is not a multiple of num_seqs {num_seqs}")
        s.num_seqs = num_seqs
        s.seq_len = total // num_seqs if num_seqs else 0
        s.cu_seqlens = None
    s.total_tokens = total
    s.H_k, s.H_v, s.d_k, s.d_v = H_k, H_v, d_k, d_v
    s.dtype = dtype_code
    s.chunk = chunk
    s.scale = 0.0 if scale is None else float(scale)
    s.l2_eps = float(l2_eps)
    return s


def _raise(fn: str, rc: int):
    if rc != 0:
        msg = lib().gdr_status_string(rc).decode()
        raise GdrError(fn, rc, msg)


def gates(q, k, a, b, A_log, dt_bias, *, scale=None, l2_eps=1e-6, num_seqs=None,
          outputs=("q_hat", "k_hat", "g", "beta")) -> Tuple:
    """beta = sigmoid(b), g = -exp(A_log)*softplus(a + dt_bias) (fp32) and the
    normalised q (times scale) and k (input dtype).  Outputs not named in
    ``outputs`` are returned as None and not computed."""
    dense_T = q.shape[1] if q.dim() == 4 else None
    q, k = _flatten(q, 2), _flatten(k, 2)
    a, b = _flatten(a, 1), _flatten(b, 1)
    dev = q.device
    dt = q.dtype
    code = _dtype_code(dt)
    total, H_k, d_k = q.shape
    H_v = a.shape[1]
    for t, n in ((q, "q"), (k, "k")):
        _check(t, n, dev, dt, (total, H_k, d_k))
    for t, n in ((a, "a"), (b, "b")):
        _check(t, n, dev, dt, (total, H_v))
    _check(A_log, "A_log", dev, torch.float32, (H_v,))
    _check(dt_bias, "dt_bias", dev, torch.float32, (H_v,))
    q_hat = torch.empty_like(q) if "q_hat" in outputs else None
    k_hat = torch.empty_like(k) if "k_hat" in outputs else None
    g = torch.empty((total, H_v), dtype=torch.float32, device=dev) if "g" in outputs else None
    beta = torch.empty((total, H_v), dtype=torch.float32, device=dev) if "beta" in outputs else None
    shape = _make_shape(total, H_k, H_v, d_k, d_k, None, num_seqs, code, 32, scale, l2_eps,
                        dense_T)
    rc = lib().gdr_gates(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(a), _ptr(b), _ptr(A_log),
                         _ptr(dt_bias), _ptr(q_hat), _ptr(k_hat), _ptr(g), _ptr(beta),
                         _stream(dev))
    _raise("gdr_gates", rc)
    return q_hat, k_hat, g, beta


def _fwd(fn_name, q, k, v, a, b, A_log, dt_bias, initial_state, cu_seqlens, num_seqs, chunk,
         scale, l2_eps, o, final_state, output_final_state, inplace, kda=False, fused=None,
         workspace=None, norm=None):
    dense_T = q.shape[1] if q.dim() == 4 else None
    q, k, v = _flatten(q, 2), _flatten(k, 2), _flatten(v, 2)
    a, b = _flatten(a, 2 if kda else 1), _flatten(b, 1)
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(f"{fn_name}: tensors must be on a GPU (got {dev})")
    dt = q.dtype
    code = _dtype_code(dt)
    total, H_k, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    _check(q, "q", dev, dt)
    _check(k, "k", dev, dt, (total, H_k, d_k))
    _check(v, "v", dev, dt, (total, H_v, d_v))
    # KDA: one gate value per key channel
    _check(a, "a", dev, dt, (total, H_v, d_k) if kda else (total, H_v))
    _check(b, "b", dev, dt, (total, H_v))
    _check(A_log, "A_log", dev, torch.float32, (H_v,))
    _check(dt_bias, "dt_bias", dev, torch.float32, (H_v, d_k) if kda else (H_v,))
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", dev, torch.int32)
    shape = _make_shape(total, H_k, H_v, d_k, d_v, cu_seqlens, num_seqs, code, chunk, scale,
                        l2_eps, dense_T)
    N = shape.num_seqs
    st_shape = (N, H_v, d_k, d_v)
    if initial_state is not None:
        _check(initial_state, "initial_state", dev, torch.float32, st_shape)
    if o is None:
        o = torch.empty((total, H_v, d_v), dtype=dt, device=dev)
    else:
        _check(o, "o", dev, dt, (total, H_v, d_v))
    if inplace:
        if initial_state is None:
            raise ValueError("inplace=True needs an initial_state to update")
        final_state = initial_state
    elif final_state is None and output_final_state:
        final_state = torch.empty(st_shape, dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check(final_state, "final_state", dev, torch.float32, st_shape)
    fn = getattr(lib(), fn_name)
    if norm is not None:
        # gdr_chunked_fwd_gated_rmsnorm: z, the weight and eps before out
        z, nw, neps = norm
        z = _flatten(z, 2)
        _check(z, "z", dev, dt, (total, H_v, d_v))
        _check(nw, "norm_weight", dev, torch.float32, (d_v,))
        args = [ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log),
                _ptr(dt_bias), _ptr(initial_state), _ptr(z), _ptr(nw), ctypes.c_float(neps),
                _ptr(o), _ptr(final_state)]
    else:
        args = [ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(A_log),
                _ptr(dt_bias), _ptr(initial_state), _ptr(o), _ptr(final_state)]
    if fused is not None:
        # gdr_kda_chunked_fwd: a workspace from torch selects the two-launch form
        nbytes = ctypes.c_size_t(0)
        if not fused:
            _raise("gdr_kda_chunked_workspace",
                   lib().gdr_kda_chunked_workspace(ctypes.byref(shape), ctypes.byref(nbytes)))
        ws = torch.empty(nbytes.value, dtype=torch.uint8, device=dev) if nbytes.value else None
        args += [_ptr(ws), ctypes.c_size_t(nbytes.value)]
    elif fn_name in ("gdr_chunked_fwd", "gdr_chunked_fwd_gated_rmsnorm"):
        # the cooperative form's workspace: "auto" allocates a zero-filled one
        # of the size the library reports (none when that is 0)
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError(f"workspace must be 'auto', None or a tensor, not {workspace!r}")
            nb = int(lib().gdr_chunked_workspace_bytes(ctypes.byref(shape)))
            workspace = torch.zeros(nb, dtype=torch.uint8, device=dev) if nb else None
        if workspace is not None:
            _check(workspace, "workspace", dev, torch.uint8)
        args += [_ptr(workspace), ctypes.c_size_t(0 if workspace is None else workspace.numel())]
    rc = fn(*args, _stream(dev))
    _raise(fn_name, rc)
    if dense_T is not None:
        o = o.view(N, dense_T, H_v, d_v)
    return o, final_state


def chunked_path(H_k, H_v, d_k, d_v, dtype, chunk=32) -> str:
    """Name of the kernel gdr_chunked_fwd runs for this shape: "matrix_bf16"
    (matrix cores, bf16 operands, fp32 accumulation), "matrix_f32" (matrix
    cores on fp32 operands) or "vector_f32"."""
    code = _dtype_code(dtype) if isinstance(dtype, torch.dtype) else (
        GDR_F32 if dtype in ("f32", "float32") else GDR_BF16)
    s = _make_shape(1, H_k, H_v, d_k, d_v, None, 1, code, chunk, None, 1e-6)
    rc = lib().gdr_chunked_path(ctypes.byref(s))
    if rc < 0:
        _raise("gdr_chunked_path", -rc)
    return {0: "vector_f32", 1: "matrix_bf16", 2: "matrix_f32"}[rc]


def recurrent_fwd(q, k, v, a, b, A_log, dt_bias, initial_state=None, *, cu_seqlens=None,
                  num_seqs=None, scale=None, l2_eps=1e-6, o=None, final_state=None,
                  output_final_state=True, inplace=False):
    """Sequential (decode) form; ``inplace=True`` updates initial_state."""
    return _fwd("gdr_recurrent_fwd", q, k, v, a, b, A_log, dt_bias, initial_state, cu_seqlens,
                num_seqs, 32, scale, l2_eps, o, final_state, output_final_state, inplace)


def chunked_fwd(q, k, v, a, b, A_log, dt_bias, initial_state=None, *, chunk=32, cu_seqlens=None,
                num_seqs=None, scale=None, l2_eps=1e-6, o=None, final_state=None,
                output_final_state=True, inplace=False, workspace="auto"):
    """Chunked (prefill) form with ``chunk`` tokens per triangular solve.

    ``workspace``: "auto" (a zero-filled uint8 tensor of the size
    gdr_chunked_workspace_bytes reports, allocated for this call), a tensor
    from ``chunked_workspace`` that the caller keeps across calls, or None (no
    workspace: the chain workgroups form every chunk's triangular inverse and
    output mask themselves)."""
    return _fwd("gdr_chunked_fwd", q, k, v, a, b, A_log, dt_bias, initial_state, cu_seqlens,
                num_seqs, chunk, scale, l2_eps, o, final_state, output_final_state, inplace,
                workspace=workspace)


def chunked_fwd_gated_rmsnorm(q, k, v, a, b, A_log, dt_bias, z, norm_weight, initial_state=None, *,
                              norm_eps=1e-6, chunk=32, cu_seqlens=None, num_seqs=None, scale=None,
                              l2_eps=1e-6, out=None, final_state=None, output_final_state=True,
                              inplace=False, workspace="auto"):
    """The chunked form followed by the gated RMSNorm of its output,
    out = o / sqrt(mean(o^2) + norm_eps) * norm_weight * SiLU(z) per (token,
    value head) row: gdr_chunked_fwd into out (``workspace`` as there), then
    gdr_gated_rmsnorm in place.  z [total, H_v, d_v] (or [N, T, H_v, d_v]) in
    the input dtype, norm_weight fp32 [d_v]; returns out (shaped as
    chunked_fwd's o) and final_state."""
    return _fwd("gdr_chunked_fwd_gated_rmsnorm", q, k, v, a, b, A_log, dt_bias, initial_state,
                cu_seqlens, num_seqs, chunk, scale, l2_eps, out, final_state, output_final_state,
                inplace, workspace=workspace, norm=(z, norm_weight, float(norm_eps)))


def chunked_fwd_noalloc(q, k, v, a, b, A_log, dt_bias, initial_state=None, *, chunk=32,
                        cu_seqlens=None, num_seqs=None, scale=None, l2_eps=1e-6, o=None,
                        final_state=None, output_final_state=True, inplace=False):
    """gdr_chunked_fwd_noalloc: the chunked form with the library's own
    per-device scratch as its cooperative workspace (no device allocation in
    the library; pass ``o`` and ``final_state`` to allocate nothing here
    either)."""
    return _fwd("gdr_chunked_fwd_noalloc", q, k, v, a, b, A_log, dt_bias, initial_state,
                cu_seqlens, num_seqs, chunk, scale, l2_eps, o, final_state, output_final_state,
                inplace)


NOALLOC_SCRATCH_BYTES = 6 << 20  # GDR_NOALLOC_SCRATCH_BYTES


def chunked_workspace_bytes(H_k, H_v, d_k, d_v, dtype, num_seqs=1, chunk=32) -> int:
    """gdr_chunked_workspace_bytes for a batch of ``num_seqs`` sequences of
    this head shape (independent of their lengths)."""
    code = _dtype_code(dtype) if isinstance(dtype, torch.dtype) else (
        GDR_F32 if dtype in ("f32", "float32") else GDR_BF16)
    s = _make_shape(num_seqs, H_k, H_v, d_k, d_v, None, num_seqs, code, chunk, None, 1e-6)
    return int(lib().gdr_chunked_workspace_bytes(ctypes.byref(s)))


def chunked_workspace(H_k, H_v, d_k, d_v, dtype, num_seqs=1, chunk=32, device="cuda"):
    """A zero-filled workspace for chunked_fwd on batches of this shape, to
    keep across calls (the library leaves it zero-filled after each call);
    None when the shape has no cooperative form.  Calls sharing one
    workspace must not overlap in time."""
    nb = chunked_workspace_bytes(H_k, H_v, d_k, d_v, dtype, num_seqs, chunk)
    return torch.zeros(nb, dtype=torch.uint8, device=device) if nb else None


def workspace_error(workspace) -> int:
    """The error words of a chunked_fwd workspace, ORed (synchronises): nonzero
    if a wait of the cooperative form ran out (its results are then invalid)."""
    if workspace is None:
        return 0
    # one 128-byte line per XCD: arrival and completion counters, error word
    acc = 0
    for v in workspace[:2048].view(torch.int32).view(16, 32)[:, 2].cpu().tolist():
        acc |= int(v)
    return acc


def fwd(q, k, v, a, b, A_log, dt_bias, initial_state=None, *, chunk=32, cu_seqlens=None,
        num_seqs=None, max_seqlen=None, **kw):
    """Pick the form on the step count: recurrent when no sequence is longer
    than one chunk, chunked otherwise.  For a packed batch pass ``max_seqlen``
    to avoid reading cu_seqlens back to the host."""
    if max_seqlen is None:
        if cu_seqlens is not None:
            cu = cu_seqlens.detach().to("cpu")
            max_seqlen = int((cu[1:] - cu[:-1]).max()) if cu.numel() > 1 else 0
        elif q.dim() == 4:
            max_seqlen = q.shape[1]
        else:
            n = 1 if num_seqs is None else num_seqs
            max_seqlen = q.shape[0] // n if n else 0
    if max_seqlen <= chunk:
        return recurrent_fwd(q, k, v, a, b, A_log, dt_bias, initial_state, cu_seqlens=cu_seqlens,
                             num_seqs=num_seqs, **kw)
    return chunked_fwd(q, k, v, a, b, A_log, dt_bias, initial_state, chunk=chunk,
                       cu_seqlens=cu_seqlens, num_seqs=num_seqs, **kw)


def conv_silu(x, weight, H_k, H_v, d_k, d_v, *, bias=None, conv_state=None, cu_seqlens=None,
              num_seqs=None, final_conv_state=None, output_final_state=True, inplace=False):
    """Short causal convolution + SiLU over the channels q | k | v of the
    in_proj output x [total, 2 H_k d_k + H_v d_v] (fp32 or bf16); weight
    [C, width] fp32, bias [C] fp32 or None; conv_state [N, C, width-1] in x's
    dtype or None.  Returns q [total, H_k, d_k], k, v [total, H_v, d_v] and
    the new history (or None); ``inplace=True`` updates conv_state."""
    dev = x.device
    if dev.type != "cuda":
        raise ValueError(f"gdr_conv_silu: tensors must be on a GPU (got {dev})")
    dt = x.dtype
    code = _dtype_code(dt)
    total = x.shape[0]
    C = 2 * H_k * d_k + H_v * d_v
    _check(x, "x", dev, dt, (total, C))
    if weight.dim() != 2 or weight.shape[0] != C:
        raise ValueError(f"weight has shape {tuple(weight.shape)}, expected ({C}, width)")
    width = weight.shape[1]
    _check(weight, "weight", dev, torch.float32, (C, width))
    if bias is not None:
        _check(bias, "bias", dev, torch.float32, (C,))
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", dev, torch.int32)
    shape = _make_shape(total, H_k, H_v, d_k, d_v, cu_seqlens, num_seqs, code, 32, None, 1e-6)
    N = shape.num_seqs
    st_shape = (N, C, width - 1)
    if conv_state is not None:
        _check(conv_state, "conv_state", dev, dt, st_shape)
    if inplace:
        if conv_state is None:
            raise ValueError("inplace=True needs a conv_state to update")
        final_conv_state = conv_state
    elif final_conv_state is None and output_final_state:
        final_conv_state = torch.empty(st_shape, dtype=dt, device=dev)
    elif final_conv_state is not None:
        _check(final_conv_state, "final_conv_state", dev, dt, st_shape)
    q = torch.empty((total, H_k, d_k), dtype=dt, device=dev)
    k = torch.empty((total, H_k, d_k), dtype=dt, device=dev)
    v = torch.empty((total, H_v, d_v), dtype=dt, device=dev)
    rc = lib().gdr_conv_silu(ctypes.byref(shape), width, _ptr(x), _ptr(weight), _ptr(bias),
                             _ptr(conv_state), _ptr(q), _ptr(k), _ptr(v), _ptr(final_conv_state),
                             _stream(dev))
    _raise("gdr_conv_silu", rc)
    return q, k, v, final_conv_state


def gated_rmsnorm(o, z, weight, eps=1e-6, *, out=None):
    """out = o / sqrt(mean(o^2) + eps) * weight * SiLU(z) per (token, head)
    row; o, z [total, H_v, d_v] (or [N, T, H_v, d_v]) fp32 or bf16, weight
    [d_v] fp32.  ``out`` may be o or z."""
    shape4 = o.shape if o.dim() == 4 else None
    o, z = _flatten(o, 2), _flatten(z, 2)
    dev = o.device
    if dev.type != "cuda":
        raise ValueError(f"gdr_gated_rmsnorm: tensors must be on a GPU (got {dev})")
    dt = o.dtype
    code = _dtype_code(dt)
    total, H_v, d_v = o.shape
    _check(o, "o", dev, dt)
    _check(z, "z", dev, dt, (total, H_v, d_v))
    _check(weight, "weight", dev, torch.float32, (d_v,))
    if out is None:
        out = torch.empty_like(o)
    else:
        out = _flatten(out, 2)
        _check(out, "out", dev, dt, (total, H_v, d_v))
    shape = _make_shape(total, 1, H_v, d_v, d_v, None, 1, code, 32, None, 1e-6)
    rc = lib().gdr_gated_rmsnorm(ctypes.byref(shape), _ptr(o), _ptr(z), _ptr(weight),
                                 float(eps), _ptr(out), _stream(dev))
    _raise("gdr_gated_rmsnorm", rc)
    return out.view(shape4) if shape4 is not None else out


def chunked_fwd_split(q, k, v, a, b, A_log, dt_bias, initial_state=None, *, segment_len,
                      chunk=32, cu_seqlens=None, num_seqs=None, scale=None, l2_eps=1e-6,
                      o=None, final_state=None, output_final_state=True, inplace=False):
    """Chunked form with every sequence cut into segments of ``segment_len``
    tokens run in parallel (two-level scan).  Dense batches (sequence length a
    multiple of segment_len) or packed ones (cu_seqlens: any lengths, the last
    segment of a sequence partial); the workspace is allocated here with
    torch."""
    return _split("gdr_chunked_fwd_split", q, k, v, a, b, A_log, dt_bias, initial_state,
                  segment_len, chunk, cu_seqlens, num_seqs, scale, l2_eps, o, final_state,
                  output_final_state, inplace, kda=False)


def kda_chunked_fwd_split(q, k, v, a, b, A_log, dt_bias, initial_state=None, *, segment_len,
                          chunk=32, cu_seqlens=None, num_seqs=None, scale=None, l2_eps=1e-6,
                          o=None, final_state=None, output_final_state=True, inplace=False):
    """The segmented chunked form for KDA (a [.., H_v, d_k], dt_bias [H_v, d_k])."""
    return _split("gdr_kda_chunked_fwd_split", q, k, v, a, b, A_log, dt_bias, initial_state,
                  segment_len, chunk, cu_seqlens, num_seqs, scale, l2_eps, o, final_state,
                  output_final_state, inplace, kda=True)


def _split(fn_name, q, k, v, a, b, A_log, dt_bias, initial_state, segment_len, chunk, cu_seqlens,
           num_seqs, scale, l2_eps, o, final_state, output_final_state, inplace, kda):
    dense_T = q.shape[1] if q.dim() == 4 else None
    q, k, v = _flatten(q, 2), _flatten(k, 2), _flatten(v, 2)
    a, b = _flatten(a, 2 if kda else 1), _flatten(b, 1)
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(f"{fn_name}: tensors must be on a GPU (got {dev})")
    dt = q.dtype
    code = _dtype_code(dt)
    total, H_k, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    _check(q, "q", dev, dt)
    _check(k, "k", dev, dt, (total, H_k, d_k))
    _check(v, "v", dev, dt, (total, H_v, d_v))
    _check(a, "a", dev, dt, (total, H_v, d_k) if kda else (total, H_v))
    _check(b, "b", dev, dt, (total, H_v))
    _check(A_log, "A_log", dev, torch.float32, (H_v,))
    _check(dt_bias, "dt_bias", dev, torch.float32, (H_v, d_k) if kda else (H_v,))
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", dev, torch.int32)
    shape = _make_shape(total, H_k, H_v, d_k, d_v, cu_seqlens, num_seqs, code, chunk, scale,
                        l2_eps, dense_T)
    N = shape.num_seqs
    st_shape = (N, H_v, d_k, d_v)
    if initial_state is not None:
        _check(initial_state, "initial_state", dev, torch.float32, st_shape)
    if o is None:
        o = torch.empty((total, H_v, d_v), dtype=dt, device=dev)
    else:
        _check(o, "o", dev, dt, (total, H_v, d_v))
    if inplace:
        if initial_state is None:
            raise ValueError("inplace=True needs an initial_state to update")
        final_state = initial_state
    elif final_state is None and output_final_state:
        final_state = torch.empty(st_shape, dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check(final_state, "final_state", dev, torch.float32, st_shape)
    nbytes = ctypes.c_size_t(0)
    wsq = "gdr_kda_chunked_split_workspace" if fn_name.startswith("gdr_kda") else "gdr_chunked_split_workspace"
    _raise(wsq, getattr(lib(), wsq)(ctypes.byref(shape), int(segment_len), ctypes.byref(nbytes)))
    ws = torch.empty(max(int(nbytes.value), 1), dtype=torch.uint8, device=dev)
    rc = getattr(lib(), fn_name)(ctypes.byref(shape), int(segment_len), _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
                                 _ptr(initial_state), _ptr(o), _ptr(final_state),
                                 _ptr(ws) if nbytes.value else None, int(nbytes.value),
                                 _stream(dev))
    _raise(fn_name, rc)
    if dense_T is not None:
        o = o.view(N, dense_T, H_v, d_v)
    return o, final_state


def _ssd(fn_name, x, delta, A, B, C, initial_state, z, cu_seqlens, num_seqs, chunk, y,
         final_state, output_final_state, inplace, segment_len=None):
    dense_T = x.shape[1] if x.dim() == 4 else None
    x, B, C = _flatten(x, 2), _flatten(B, 2), _flatten(C, 2)
    delta = _flatten(delta, 1)
    z = None if z is None else _flatten(z, 2)
    dev = x.device
    if dev.type != "cuda":
        raise ValueError(f"{fn_name}: tensors must be on a GPU (got {dev})")
    dt = x.dtype
    code = _dtype_code(dt)
    total, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    _check(x, "x", dev, dt)
    _check(delta, "delta", dev, dt, (total, H))
    _check(A, "A", dev, torch.float32, (H,))
    _check(B, "B", dev, dt, (total, G, N))
    _check(C, "C", dev, dt, (total, G, N))
    if z is not None:
        _check(z, "z", dev, dt, (total, H, P))
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", dev, torch.int32)
    shape = _make_shape(total, G, H, N, P, cu_seqlens, num_seqs, code, chunk, 1.0, 0.0, dense_T)
    S = shape.num_seqs
    st_shape = (S, H, N, P)
    if initial_state is not None:
        _check(initial_state, "initial_state", dev, torch.float32, st_shape)
    if y is None:
        y = torch.empty((total, H, P), dtype=dt, device=dev)
    else:
        _check(y, "y", dev, dt, (total, H, P))
    if inplace:
        if initial_state is None:
            raise ValueError("inplace=True needs an initial_state to update")
        final_state = initial_state
    elif final_state is None and output_final_state:
        final_state = torch.empty(st_shape, dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check(final_state, "final_state", dev, torch.float32, st_shape)
    ptrs = [_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(initial_state), _ptr(z),
            _ptr(y), _ptr(final_state)]
    if segment_len is None:
        rc = getattr(lib(), fn_name)(ctypes.byref(shape), *ptrs, _stream(dev))
    else:
        nbytes = ctypes.c_size_t(0)
        _raise("gdr_ssd_chunked_split_workspace",
               lib().gdr_ssd_chunked_split_workspace(ctypes.byref(shape), int(segment_len),
                                                     ctypes.byref(nbytes)))
        ws = torch.empty(max(int(nbytes.value), 1), dtype=torch.uint8, device=dev)
        rc = getattr(lib(), fn_name)(ctypes.byref(shape), int(segment_len), *ptrs,
                                     _ptr(ws) if nbytes.value else None, int(nbytes.value),
                                     _stream(dev))
    _raise(fn_name, rc)
    if dense_T is not None:
        y = y.view(S, dense_T, H, P)
    return y, final_state


def ssd_recurrent_fwd(x, delta, A, B, C, initial_state=None, *, z=None, cu_seqlens=None,
                      num_seqs=None, y=None, final_state=None, output_final_state=True,
                      inplace=False):
    """Mamba-2 SSD recurrence, sequential form: x [total, H, P], delta
    [total, H], A fp32 [H], B and C [total, G, N], states fp32 [S, H, N, P];
    ``z`` gates y by SiLU(z)."""
    return _ssd("gdr_ssd_recurrent_fwd", x, delta, A, B, C, initial_state, z, cu_seqlens,
                num_seqs, 32, y, final_state, output_final_state, inplace)


def ssd_chunked_fwd(x, delta, A, B, C, initial_state=None, *, z=None, chunk=32,
                    cu_seqlens=None, num_seqs=None, y=None, final_state=None,
                    output_final_state=True, inplace=False):
    """Mamba-2 SSD recurrence, chunked form (same arguments plus ``chunk``)."""
    return _ssd("gdr_ssd_chunked_fwd", x, delta, A, B, C, initial_state, z, cu_seqlens,
                num_seqs, chunk, y, final_state, output_final_state, inplace)


def ssd_chunked_fwd_split(x, delta, A, B, C, initial_state=None, *, segment_len, z=None,
                          chunk=32, cu_seqlens=None, num_seqs=None, y=None, final_state=None,
                          output_final_state=True, inplace=False):
    """Mamba-2 SSD recurrence in the segmented chunked form (two-level scan;
    arguments as ssd_chunked_fwd plus ``segment_len``, batches as
    chunked_fwd_split); the workspace is allocated here with torch."""
    return _ssd("gdr_ssd_chunked_fwd_split", x, delta, A, B, C, initial_state, z, cu_seqlens,
                num_seqs, chunk, y, final_state, output_final_state, inplace,
                segment_len=segment_len)


def kda_recurrent_fwd(q, k, v, a, b, A_log, dt_bias, initial_state=None, *, cu_seqlens=None,
                      num_seqs=None, scale=None, l2_eps=1e-6, o=None, final_state=None,
                      output_final_state=True, inplace=False):
    """The rule with one decay per key channel (KDA), sequential form:
    a [total, H_v, d_k] and dt_bias fp32 [H_v, d_k]; the rest as recurrent_fwd."""
    return _fwd("gdr_kda_recurrent_fwd", q, k, v, a, b, A_log, dt_bias, initial_state,
                cu_seqlens, num_seqs, 32, scale, l2_eps, o, final_state, output_final_state,
                inplace, kda=True)


def kda_chunked_fwd(q, k, v, a, b, A_log, dt_bias, initial_state=None, *, chunk=32,
                    cu_seqlens=None, num_seqs=None, scale=None, l2_eps=1e-6, o=None,
                    final_state=None, output_final_state=True, inplace=False, fused=False):
    """KDA, chunked form (chunk 16 or 32).  By default the workspace the
    library asks for is allocated here, which selects its two-launch form;
    ``fused=True`` passes none and runs the one-launch form."""
    return _fwd("gdr_kda_chunked_fwd", q, k, v, a, b, A_log, dt_bias, initial_state, cu_seqlens,
                num_seqs, chunk, scale, l2_eps, o, final_state, output_final_state, inplace,
                kda=True, fused=bool(fused))
