"""MI355X-native chunkwise KDA forward -- thin Python binding over libkda.so.

Every step of the forward pass runs in the HIP kernels of `libkda.so`; this
module only checks tensors, allocates outputs and workspace with torch, and
passes raw pointers and the current HIP stream through the C ABI declared in
include/kda.h.  There is no CPU or PyTorch fallback: if the library is
missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["chunk_fwd", "chunk_fwd_profile", "chunk_fwd_ckpt", "ckpt_slots", "ckpt_size", "chunk_bwd", "chunk_bwd_profile", "chunk_fwd_train", "train_context_size", "output_gate", "bwd_stage_names", "bwd_workspace_size", "recurrent_fwd", "validate_inputs", "chunk_transition",
           "compose_states", "sequence_parallel_fwd", "stage_names", "workspace_size", "status_string", "lib_path",
           "KDA_F32", "KDA_BF16", "KdaError"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libkda.so")
_lib = None

KDA_F32, KDA_BF16 = 0, 1
CHUNK = 64


class KdaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libkda.so is not built (%s); run gated_delta_rule_30_amd/build.py "
                               "or __graft_entry__.build()" % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lib.kda_chunk_fwd_workspace_size.argtypes = [I64, I32, I32, I32, I32, I32, ctypes.c_int]
        lib.kda_chunk_fwd_workspace_size.restype = SZ
        lib.kda_chunk_fwd.argtypes = [ctypes.c_int, I64, I32, I32, I32, I32, I32,
                                      P, P, P, P, P, P, P, P, P, P, SZ, P]
        lib.kda_chunk_fwd.restype = ctypes.c_int
        lib.kda_status_string.argtypes = [ctypes.c_int]
        lib.kda_status_string.restype = ctypes.c_char_p
        lib.kda_version.restype = ctypes.c_char_p
        lib.kda_chunk_fwd_profile.argtypes = lib.kda_chunk_fwd.argtypes + [P]
        lib.kda_chunk_fwd_profile.restype = ctypes.c_int
        lib.kda_profile_num_stages.restype = ctypes.c_int32
        lib.kda_profile_stage_name.argtypes = [ctypes.c_int32]
        lib.kda_profile_stage_name.restype = ctypes.c_char_p
        lib.kda_recurrent_fwd.argtypes = [ctypes.c_int, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P, P]
        lib.kda_recurrent_fwd.restype = ctypes.c_int
        lib.kda_recurrent_commit.argtypes = [ctypes.c_int, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P, P, P]
        lib.kda_recurrent_commit.restype = ctypes.c_int
        lib.kda_validate_inputs.argtypes = [ctypes.c_int, I64, I32, I32, I32, P, P, P, P, P]
        lib.kda_validate_inputs.restype = ctypes.c_int
        lib.kda_chunk_transition.argtypes = [ctypes.c_int, I64, I32, I32, I32, I32, P, P, P, P, P, P, SZ, P]
        lib.kda_chunk_transition.restype = ctypes.c_int
        lib.kda_compose_states.argtypes = [I32, I32, I32, P, P, P, P, P]
        lib.kda_compose_states.restype = ctypes.c_int
        lib.kda_chunk_bwd_workspace_size.argtypes = [I64, I32, I32, I32, I32, I32, ctypes.c_int]
        lib.kda_chunk_bwd_workspace_size.restype = SZ
        lib.kda_chunk_bwd.argtypes = [ctypes.c_int, I64, I32, I32, I32, I32, I32,
                                      P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
        lib.kda_chunk_bwd.restype = ctypes.c_int
        lib.kda_chunk_bwd_profile.argtypes = lib.kda_chunk_bwd.argtypes + [P]
        lib.kda_chunk_bwd_profile.restype = ctypes.c_int
        lib.kda_profile_bwd_num_stages.restype = ctypes.c_int32
        lib.kda_profile_bwd_stage_name.argtypes = [ctypes.c_int32]
        lib.kda_profile_bwd_stage_name.restype = ctypes.c_char_p
        lib.kda_chunk_train_context_size.argtypes = [I64, I32, I32, I32, I32, I32, ctypes.c_int]
        lib.kda_chunk_train_context_size.restype = SZ
        lib.kda_chunk_bwd_ctx_workspace_size.argtypes = [I64, I32, I32, I32, I32, I32, ctypes.c_int]
        lib.kda_chunk_bwd_ctx_workspace_size.restype = SZ
        lib.kda_chunk_fwd_train.argtypes = [ctypes.c_int, I64, I32, I32, I32, I32, I32,
                                            P, P, P, P, P, P, P, P, P, P, SZ, P, SZ, P]
        lib.kda_chunk_fwd_train.restype = ctypes.c_int
        lib.kda_chunk_bwd_ctx.argtypes = [ctypes.c_int, I64, I32, I32, I32, I32, I32,
                                          P, P, P, P, P, P, P, SZ, P, P, P, P, P, P, P, P, P, SZ, P]
        lib.kda_chunk_bwd_ctx.restype = ctypes.c_int
        lib.kda_output_gate.argtypes = [ctypes.c_int, I64, I32, P, P, P, ctypes.c_float, P, P]
        lib.kda_output_gate.restype = ctypes.c_int
        lib.kda_chunk_ckpt_size.argtypes = [I64, I32, I32, I32, I32, I32]
        lib.kda_chunk_ckpt_size.restype = SZ
        lib.kda_chunk_fwd_ckpt.argtypes = [ctypes.c_int, I64, I32, I32, I32, I32, I32,
                                           P, P, P, P, P, P, P, P, P, I32, P, SZ, P, SZ, P]
        lib.kda_chunk_fwd_ckpt.restype = ctypes.c_int
        _lib = lib
    return _lib


def status_string(code: int) -> str:
    return _load().kda_status_string(int(code)).decode()


def workspace_size(total_tokens: int, n_seqs: int, n_heads: int, d_k: int, d_v: int,
                   chunk: int = CHUNK, dtype_code: int = KDA_BF16) -> int:
    return int(_load().kda_chunk_fwd_workspace_size(int(total_tokens), int(n_seqs), int(n_heads), int(d_k),
                                                    int(d_v), int(chunk), int(dtype_code)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def stage_names():
    lib = _load()
    return [lib.kda_profile_stage_name(i).decode() for i in range(lib.kda_profile_num_stages())]


def _nbytes(t):
    return t.numel() * t.element_size()


def _fwd_problem(q, k, v, beta, log_alpha, S0=None, cu_seqlens=None, n_seqs=None, dtypes=None):
    """Checks the forward-shaped arguments every entry point shares, before
    anything is launched: one float dtype (in `dtypes` when given); q, k,
    log_alpha [T, H, d_k] and v [T, H, d_v], beta [T, H] (or the same with a
    leading batch axis B); cu_seqlens a contiguous 1-D int32 tensor of N + 1
    offsets; S0 contiguous float32 [N, H, d_k, d_v]; everything contiguous
    on one GPU.  The C ABI sees only pointers, so an extent it cannot check
    would become an out-of-bounds access on the device.  Extents and dtypes
    are checked before devices.  Returns a namespace with the flattened 3-D
    tensors, dt, dev, T, H, dk, dv, N, batched and B."""
    import torch
    from types import SimpleNamespace
    dt = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}.get(q.dtype)
    if dt is None or (dtypes is not None and q.dtype not in dtypes):
        raise TypeError("q has unsupported dtype %s" % q.dtype)
    for name, t in (("k", k), ("v", v), ("beta", beta), ("log_alpha", log_alpha)):
        if t.dtype != q.dtype:
            raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, q.dtype))
    if q.dim() not in (3, 4):
        raise ValueError("q must be [T, H, d_k] or [B, T, H, d_k], got shape %s" % (tuple(q.shape),))
    batched = q.dim() == 4
    B = q.shape[0] if batched else 1
    if batched:
        if v.dim() != 4 or beta.dim() != 3 or k.dim() != 4 or log_alpha.dim() != 4:
            raise ValueError("4-D q needs 4-D k, v, log_alpha and 3-D beta (shape)")
        q, k, v, log_alpha = (t.reshape(-1, *t.shape[2:]) for t in (q, k, v, log_alpha))
        beta = beta.reshape(-1, beta.shape[-1])
    T, H, dk = q.shape
    if v.dim() != 3:
        raise ValueError("v must have as many axes as q (shape %s)" % (tuple(v.shape),))
    dv = v.shape[-1]
    if k.shape != (T, H, dk) or log_alpha.shape != (T, H, dk) or v.shape != (T, H, dv) or beta.shape != (T, H):
        raise ValueError("inconsistent shapes q%s k%s v%s beta%s log_alpha%s"
                         % (tuple(q.shape), tuple(k.shape), tuple(v.shape), tuple(beta.shape),
                            tuple(log_alpha.shape)))
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous() \
                or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor of N + 1 >= 2 offsets")
        N = cu_seqlens.numel() - 1
    else:
        N = int(n_seqs) if n_seqs is not None else B
    if S0 is not None and (S0.dtype != torch.float32 or S0.shape != (N, H, dk, dv) or not S0.is_contiguous()):
        raise ValueError("S0 must be contiguous float32 [%d, %d, %d, %d]" % (N, H, dk, dv))
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("log_alpha", log_alpha),
                    ("cu_seqlens", cu_seqlens), ("S0", S0)):
        if t is not None and (t.device != dev or not t.is_contiguous()):
            raise ValueError("%s must be contiguous on %s" % (name, dev))
    return SimpleNamespace(q=q, k=k, v=v, beta=beta, log_alpha=log_alpha, dt=dt, dev=dev, T=T, H=H, dk=dk,
                           dv=dv, N=N, batched=batched, B=B)


def _check_out(name, t, shape, dtype, dev):
    if t is not None and (tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != dev
                          or not t.is_contiguous()):
        raise ValueError("%s must be contiguous %s %s on %s" % (name, dtype, list(shape), dev))


def _check_buffer(name, t, nbytes, dev):
    if t is not None and (t.device != dev or not t.is_contiguous() or _nbytes(t) < nbytes):
        raise ValueError("%s must be a contiguous tensor of at least %d bytes on %s" % (name, nbytes, dev))


def chunk_fwd_profile(*args, **kw):
    """Same as chunk_fwd, but through the measurement entry point: blocks until
    done and returns (o, S_T, {kernel name: milliseconds})."""
    ms = (ctypes.c_float * _load().kda_profile_num_stages())()
    o, ST = chunk_fwd(*args, _stage_ms=ms, **kw)
    return o, ST, dict(zip(stage_names(), [float(x) for x in ms]))


def chunk_fwd(q, k, v, beta, log_alpha, S0=None, cu_seqlens=None, chunk: int = CHUNK,
              output_final_state: bool = True, o=None, S_T=None, workspace=None, n_seqs=None, _stage_ms=None,
              _ckpt=None):
    """KDA chunkwise forward on the GPU.

    q, k, log_alpha: [T_total, H, d_k] or [B, T, H, d_k]; v: [..., H, d_v];
    beta: [..., H] -- all float32 or all bfloat16, contiguous, on one GPU.
    S0: [N, H, d_k, d_v] float32 or None.  cu_seqlens: int32 device tensor
    [N+1] (packed variable-length batch) or None (B equal sequences for 4-D
    inputs, one sequence for 3-D inputs; `n_seqs` overrides).  Optional
    preallocated `o`, `S_T` and `workspace` (uint8) tensors are used as given.
    `chunk`: 16, 32, 64 or 128 tokens; d_k, d_v: 64 or 128.  Chunk 64 with
    d_k == d_v (bf16 at 64 or 128, fp32 at 64) runs the tuned kernels, every
    other supported size the generic fp32 ones (same results to rounding).
    Returns (o, S_T) with o shaped like v and S_T None unless requested.
    """
    import torch
    lib = _load()
    P = _fwd_problem(q, k, v, beta, log_alpha, S0, cu_seqlens, n_seqs)
    q, k, v, beta, log_alpha = P.q, P.k, P.v, P.beta, P.log_alpha
    dt, dev, T, H, dk, dv, N, batched, B = P.dt, P.dev, P.T, P.H, P.dk, P.dv, P.N, P.batched, P.B
    ws_bytes = int(lib.kda_chunk_fwd_workspace_size(T, N, H, dk, dv, chunk, dt))
    if ws_bytes == 0:
        code = lib.kda_chunk_fwd(dt, T, N, H, dk, dv, chunk, None, None, None, None, None, None, None,
                                 None, None, None, 0, None)
        raise KdaError(code, lib.kda_status_string(code).decode())
    _check_buffer("workspace", workspace, ws_bytes, dev)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _check_out("o", o, (T, H, dv), q.dtype, dev)
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    _check_out("S_T", S_T, (N, H, dk, dv), torch.float32, dev)
    if output_final_state and S_T is None:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (dt, T, N, H, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha),
            _ptr(S0), _ptr(cu_seqlens), _ptr(o), _ptr(S_T), _ptr(workspace),
            _nbytes(workspace), ctypes.c_void_p(stream))
    if _ckpt is not None:
        every, S_ckpt = _ckpt
        code = lib.kda_chunk_fwd_ckpt(*args[:16], int(every), _ptr(S_ckpt), _nbytes(S_ckpt), *args[16:])
    elif _stage_ms is None:
        code = lib.kda_chunk_fwd(*args)
    else:
        code = lib.kda_chunk_fwd_profile(*args, _stage_ms)
    if code != 0:
        raise KdaError(code, lib.kda_status_string(code).decode())
    if batched:
        o = o.reshape(B, -1, H, dv)
    return o, (S_T if output_final_state else None)


def ckpt_slots(lengths, every: int, chunk: int = CHUNK):
    """Where chunk_fwd_ckpt puts each sequence's checkpoints: for sequence n a
    list of (tokens, slot) -- the state after its first `tokens` tokens is
    S_ckpt[slot].  The checkpoints are packed in sequence order.  `lengths`
    are the sequence lengths (host integers)."""
    out, slot = [], 0
    for L in lengths:
        nch = (int(L) + chunk - 1) // chunk
        lst = []
        for j in range(nch):
            if (j + 1) % every == 0:
                lst.append((min((j + 1) * chunk, int(L)), slot))
                slot += 1
        out.append(lst)
    return out


def ckpt_size(total_tokens: int, n_seqs: int, n_heads: int, d_k: int, d_v: int, every: int) -> int:
    """Bytes of the checkpoint buffer for kda_chunk_fwd_ckpt (an upper bound
    over all splits of total_tokens into n_seqs sequences)."""
    return int(_load().kda_chunk_ckpt_size(int(total_tokens), int(n_seqs), int(n_heads), int(d_k), int(d_v),
                                           int(every)))


def chunk_fwd_ckpt(q, k, v, beta, log_alpha, every: int, S_ckpt=None, **kw):
    """chunk_fwd that also writes the state after every `every`-th chunk of each
    sequence (prefix-cache checkpoints) into S_ckpt, float32 [slots, H, d_k,
    d_v] (allocated when None; see ckpt_slots for the slot of each).  bf16
    only.  Returns (o, S_T, S_ckpt)."""
    import torch
    P = _fwd_problem(q, k, v, beta, log_alpha, kw.get("S0"), kw.get("cu_seqlens"), kw.get("n_seqs"))
    if int(every) < 1:
        raise ValueError("every must be >= 1")
    nbytes = ckpt_size(P.T, P.N, P.H, P.dk, P.dv, every)
    if nbytes == 0:
        raise KdaError(4, "unsupported sizes for checkpoints")
    if S_ckpt is None:
        S_ckpt = torch.empty(nbytes // 4, dtype=torch.float32, device=P.dev).view(-1, P.H, P.dk, P.dv)
    elif (S_ckpt.dtype != torch.float32 or _nbytes(S_ckpt) < nbytes or not S_ckpt.is_contiguous()
          or S_ckpt.device != P.dev):
        raise ValueError("S_ckpt must be contiguous float32 with at least %d bytes on %s" % (nbytes, P.dev))
    o, S_T = chunk_fwd(q, k, v, beta, log_alpha, _ckpt=(every, S_ckpt), **kw)
    return o, S_T, S_ckpt


def bwd_workspace_size(total_tokens: int, n_seqs: int, n_heads: int, d_k: int, d_v: int,
                       chunk: int = CHUNK, dtype_code: int = KDA_BF16) -> int:
    return int(_load().kda_chunk_bwd_workspace_size(int(total_tokens), int(n_seqs), int(n_heads), int(d_k),
                                                    int(d_v), int(chunk), int(dtype_code)))


def bwd_stage_names():
    lib = _load()
    return [lib.kda_profile_bwd_stage_name(i).decode() for i in range(lib.kda_profile_bwd_num_stages())]


def chunk_bwd_profile(*args, **kw):
    """Same as chunk_bwd, through the measurement entry point: blocks until
    done and returns (grads, {kernel name: milliseconds})."""
    ms = (ctypes.c_float * _load().kda_profile_bwd_num_stages())()
    grads = chunk_bwd(*args, _stage_ms=ms, **kw)
    return grads, dict(zip(bwd_stage_names(), [float(x) for x in ms]))


def train_context_size(total_tokens: int, n_seqs: int, n_heads: int, d_k: int, d_v: int,
                       chunk: int = CHUNK, dtype_code: int = KDA_BF16) -> int:
    return int(_load().kda_chunk_train_context_size(int(total_tokens), int(n_seqs), int(n_heads), int(d_k),
                                                    int(d_v), int(chunk), int(dtype_code)))


def chunk_fwd_train(q, k, v, beta, log_alpha, S0=None, cu_seqlens=None, chunk: int = CHUNK, n_seqs=None,
                    context=None, o=None, S_T=None, workspace=None):
    """Forward for training (kda_chunk_fwd_train): chunk_fwd plus a context
    (uint8 device tensor, allocated when None) that chunk_bwd(..., context=)
    turns into the gradients without evaluating the forward again.  bfloat16,
    3-D packed inputs.  Returns (o, S_T, context)."""
    import torch
    lib = _load()
    if q.dim() != 3:
        raise ValueError("chunk_fwd_train takes 3-D packed inputs [T, H, d], got shape %s" % (tuple(q.shape),))
    P = _fwd_problem(q, k, v, beta, log_alpha, S0, cu_seqlens, n_seqs, dtypes=(torch.bfloat16,))
    dt, dev, T, H, dk, dv, N = P.dt, P.dev, P.T, P.H, P.dk, P.dv, P.N
    cb = int(lib.kda_chunk_train_context_size(T, N, H, dk, dv, chunk, dt))
    wb = int(lib.kda_chunk_fwd_workspace_size(T, N, H, dk, dv, chunk, dt))
    if cb == 0 or wb == 0:
        raise KdaError(4, "KDA_ERR_UNSUPPORTED: sizes or dtype not supported by the training pair")
    _check_buffer("context", context, cb, dev)
    _check_buffer("workspace", workspace, wb, dev)
    _check_out("o", o, (T, H, dv), q.dtype, dev)
    _check_out("S_T", S_T, (N, H, dk, dv), torch.float32, dev)
    if context is None:
        context = torch.empty(cb, dtype=torch.uint8, device=dev)
    if workspace is None:
        workspace = torch.empty(wb, dtype=torch.uint8, device=dev)
    if o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    if S_T is None:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    code = lib.kda_chunk_fwd_train(dt, T, N, H, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                   _ptr(log_alpha), _ptr(S0), _ptr(cu_seqlens), _ptr(o), _ptr(S_T), _ptr(context),
                                   _nbytes(context), _ptr(workspace), _nbytes(workspace), ctypes.c_void_p(stream))
    if code != 0:
        raise KdaError(code, lib.kda_status_string(code).decode())
    return o, S_T, context


def chunk_bwd(q, k, v, beta, log_alpha, dO, S0=None, dS_T=None, cu_seqlens=None, chunk: int = CHUNK,
              n_seqs=None, workspace=None, context=None, _stage_ms=None):
    """KDA chunkwise backward on the GPU (kda_chunk_bwd, or kda_chunk_bwd_ctx
    when `context` comes from chunk_fwd_train on the same inputs).

    Inputs as for chunk_fwd (bfloat16, 3-D packed [T, H, d] or 4-D [B, T, H, d]);
    dO shaped like v; dS_T [N, H, d_k, d_v] float32 or None.  Returns a dict
    with dq, dk, dv, dbeta, dg (gradient of log_alpha; shapes and dtype of the
    inputs) and dS0 ([N, H, d_k, d_v] float32)."""
    import torch
    lib = _load()
    shape_q, shape_v, shape_b = q.shape, v.shape, beta.shape
    P = _fwd_problem(q, k, v, beta, log_alpha, S0, cu_seqlens, n_seqs, dtypes=(torch.bfloat16,))
    q, k, v, beta, log_alpha = P.q, P.k, P.v, P.beta, P.log_alpha
    dt, dev, T, H, dk, dv, N, batched = P.dt, P.dev, P.T, P.H, P.dk, P.dv, P.N, P.batched
    if batched:
        dO = dO.reshape(-1, *dO.shape[2:])
    if dO.shape != (T, H, dv) or dO.dtype != q.dtype or dO.device != dev or not dO.is_contiguous():
        raise ValueError("dO must be contiguous %s shaped like v on %s" % (q.dtype, dev))
    _check_out("dS_T", dS_T, (N, H, dk, dv), torch.float32, dev)
    size_fn = lib.kda_chunk_bwd_workspace_size if context is None else lib.kda_chunk_bwd_ctx_workspace_size
    ws_bytes = int(size_fn(T, N, H, dk, dv, chunk, dt))
    if ws_bytes == 0:
        code = lib.kda_chunk_bwd(dt, T, N, H, dk, dv, chunk, *([None] * 15), 0, None)
        raise KdaError(code, lib.kda_status_string(code).decode())
    _check_buffer("workspace", workspace, ws_bytes, dev)
    if context is not None:
        _check_buffer("context", context, int(lib.kda_chunk_train_context_size(T, N, H, dk, dv, chunk, dt)), dev)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dbeta=torch.empty_like(beta), dg=torch.empty_like(log_alpha),
               dS0=torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev))
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (dt, T, N, H, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha), _ptr(S0),
            _ptr(cu_seqlens), _ptr(dO), _ptr(dS_T), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
            _ptr(out["dbeta"]), _ptr(out["dg"]), _ptr(out["dS0"]), _ptr(workspace),
            _nbytes(workspace), ctypes.c_void_p(stream))
    if context is not None:
        if _stage_ms is not None:
            raise ValueError("the context form has no per-kernel measurement entry point")
        code = lib.kda_chunk_bwd_ctx(dt, T, N, H, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
                                     _ptr(log_alpha), _ptr(cu_seqlens), _ptr(context), _nbytes(context), _ptr(dO),
                                     _ptr(dS_T),
                                     _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dbeta"]),
                                     _ptr(out["dg"]), _ptr(out["dS0"]), _ptr(workspace),
                                     _nbytes(workspace), ctypes.c_void_p(stream))
    else:
        code = lib.kda_chunk_bwd(*args) if _stage_ms is None else lib.kda_chunk_bwd_profile(*args, _stage_ms)
    if code != 0:
        raise KdaError(code, lib.kda_status_string(code).decode())
    if batched:
        for key, shp in (("dq", shape_q), ("dk", shape_q), ("dg", shape_q), ("dv", shape_v), ("dbeta", shape_b)):
            out[key] = out[key].reshape(shp)
    return out


def output_gate(o, gate, weight=None, eps: float = 1e-6, out=None):
    """Output epilogue (kda_output_gate): RMSNorm(o) * weight * sigmoid(gate)
    per row of the last dimension.  o, gate: same shape [..., d_v], float32 or
    bfloat16, contiguous, on one GPU; weight: [d_v] float32 or None; out:
    preallocated result (may be o) or None."""
    import torch
    lib = _load()
    dt = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}.get(o.dtype)
    if dt is None:
        raise TypeError("o must be float32 or bfloat16, got %s" % o.dtype)
    if gate.shape != o.shape or gate.dtype != o.dtype:
        raise ValueError("gate must match o in shape and dtype")
    dev = o.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    for name, t in (("o", o), ("gate", gate)):
        if t.device != dev or not t.is_contiguous():
            raise ValueError("%s must be contiguous on %s" % (name, dev))
    d = o.shape[-1]
    if weight is not None and (weight.dtype != torch.float32 or weight.shape != (d,) or weight.device != dev
                               or not weight.is_contiguous()):
        raise ValueError("weight must be contiguous float32 [%d] on %s" % (d, dev))
    if out is None:
        out = torch.empty_like(o)
    elif out.shape != o.shape or out.dtype != o.dtype or out.device != dev or not out.is_contiguous():
        raise ValueError("out must match o")
    n_rows = o.numel() // d if d else 0
    code = lib.kda_output_gate(dt, n_rows, d, _ptr(o), _ptr(gate), _ptr(weight), float(eps), _ptr(out),
                               ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    if code != 0:
        raise KdaError(code, lib.kda_status_string(code).decode())
    return out


def _check_common(q, k, v, beta, log_alpha):
    import torch
    dt = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}.get(q.dtype)
    if dt is None:
        raise TypeError("q must be float32 or bfloat16, got %s" % q.dtype)
    for name, t in (("k", k), ("v", v), ("beta", beta), ("log_alpha", log_alpha)):
        if t.dtype != q.dtype:
            raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, q.dtype))
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU device")
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("log_alpha", log_alpha)):
        if t.device != dev or not t.is_contiguous():
            raise ValueError("%s must be contiguous on %s" % (name, dev))
    return dt, dev


def recurrent_fwd(q, k, v, beta, log_alpha, S_in=None, S_out=None, n_seqs=None, o=None, n_accept=None,
                  want_o=True):
    """Token-by-token KDA update for decoding (kda_recurrent_fwd).

    q, k, log_alpha: [N*n, H, d_k] or [N, n, H, d_k]; v: [..., H, d_v];
    beta: [..., H] -- n tokens for each of N sequences (N from the 4-D shape
    or `n_seqs`, default 1).  S_in: [N, H, d_k, d_v] float32 or None (zeros).
    S_out: preallocated output state (may be S_in itself for an in-place
    update) or None (allocated).  Returns (o, S_out).

    With n_accept (int32 [N] on the device) the call goes to
    kda_recurrent_commit: sequence i takes only its first n_accept[i] token
    slots (clamped to [0, n]); o rows of the other slots are left as they
    were, and with want_o=False no o is written at all (returned as None).
    """
    import torch
    lib = _load()
    dt, dev = _check_common(q, k, v, beta, log_alpha)
    batched = q.dim() == 4
    if batched:
        N = q.shape[0]
        q, k, v, log_alpha = (t.reshape(-1, *t.shape[2:]) for t in (q, k, v, log_alpha))
        beta = beta.reshape(-1, beta.shape[-1])
    else:
        N = 1 if n_seqs is None else int(n_seqs)
    T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != (T, H, dk) or log_alpha.shape != (T, H, dk) or v.shape != (T, H, dv) or beta.shape != (T, H):
        raise ValueError("inconsistent shapes")
    if N < 1 or T % N != 0:
        raise ValueError("%d tokens do not split into %d equal sequences" % (T, N))
    for name, t in (("S_in", S_in), ("S_out", S_out)):
        if t is not None and (t.dtype != torch.float32 or t.shape != (N, H, dk, dv) or t.device != dev
                              or not t.is_contiguous()):
            raise ValueError("%s must be contiguous float32 [%d, %d, %d, %d] on %s" % (name, N, H, dk, dv, dev))
    if n_accept is not None and (n_accept.dtype != torch.int32 or n_accept.shape != (N,) or n_accept.device != dev
                                 or not n_accept.is_contiguous()):
        raise ValueError("n_accept must be contiguous int32 [%d] on %s" % (N, dev))
    if not want_o and n_accept is None:
        raise ValueError("want_o=False needs n_accept")
    if S_out is None:
        S_out = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    if not want_o:
        o = None
    elif o is None:
        o = torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    elif o.shape != (T, H, dv) or o.dtype != q.dtype or o.device != dev or not o.is_contiguous():
        raise ValueError("o must be contiguous %s [%d, %d, %d] on %s" % (q.dtype, T, H, dv, dev))
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    args = (dt, N, T // N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(log_alpha))
    if n_accept is None:
        code = lib.kda_recurrent_fwd(*args, _ptr(S_in), _ptr(S_out), _ptr(o), stream)
    else:
        code = lib.kda_recurrent_commit(*args, _ptr(n_accept), _ptr(S_in), _ptr(S_out), _ptr(o), stream)
    if code != 0:
        raise KdaError(code, lib.kda_status_string(code).decode())
    if batched and o is not None:
        o = o.reshape(N, -1, H, dv)
    return o, S_out


def validate_inputs(beta, log_alpha, cu_seqlens=None, n_seqs=None):
    """Counts value-range violations on the GPU (kda_validate_inputs) and
    returns {"log_alpha": n, "beta": n, "cu_seqlens": n}; synchronises the
    current stream to read the counts."""
    import torch
    lib = _load()
    dt = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}.get(log_alpha.dtype)
    if dt is None or beta.dtype != log_alpha.dtype:
        raise TypeError("beta and log_alpha must both be float32 or bfloat16")
    if log_alpha.dim() == 4:
        log_alpha = log_alpha.reshape(-1, *log_alpha.shape[2:])
        beta = beta.reshape(-1, beta.shape[-1])
    T, H, dk = log_alpha.shape
    dev = log_alpha.device
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != dev or cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be a 1-D int32 tensor on %s" % dev)
        N = cu_seqlens.numel() - 1
    else:
        N = 1 if n_seqs is None else int(n_seqs)
    counts = torch.empty(3, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    code = lib.kda_validate_inputs(dt, T, N, H, dk, _ptr(beta.contiguous()), _ptr(log_alpha.contiguous()),
                                   _ptr(cu_seqlens), _ptr(counts), ctypes.c_void_p(stream.cuda_stream))
    if code != 0:
        raise KdaError(code, lib.kda_status_string(code).decode())
    c = counts.cpu().tolist()
    return {"log_alpha": c[0], "beta": c[1], "cu_seqlens": c[2]}


def chunk_transition(k, beta, log_alpha, cu_seqlens=None, n_seqs=None, workspace=None):
    """Transition matrices P [N, H, d, d] (kda_chunk_transition): each
    sequence maps an incoming state S to P S + Z (Z its zero-start state)."""
    import torch
    lib = _load()
    if k.dtype != torch.bfloat16:
        raise TypeError("chunk_transition takes bfloat16 k, beta, log_alpha")
    # k stands in for q and v in the shared checks (the transition reads neither)
    P = _fwd_problem(k, k, k, beta, log_alpha, None, cu_seqlens, n_seqs, dtypes=(torch.bfloat16,))
    k, beta, log_alpha = P.k, P.beta, P.log_alpha
    T, H, d, N, dev = P.T, P.H, P.dk, P.N, P.dev
    ws_bytes = int(lib.kda_chunk_fwd_workspace_size(T, N, H, d, d, CHUNK, KDA_BF16))
    _check_buffer("workspace", workspace, ws_bytes, dev)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    P_out = torch.empty((N, H, d, d), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    code = lib.kda_chunk_transition(KDA_BF16, T, N, H, d, CHUNK, _ptr(k), _ptr(beta), _ptr(log_alpha),
                                    _ptr(cu_seqlens), _ptr(P_out), _ptr(workspace),
                                    0 if workspace is None else _nbytes(workspace), ctypes.c_void_p(stream))
    if code != 0:
        raise KdaError(code, lib.kda_status_string(code).decode())
    return P_out


def compose_states(P, Z, S0=None):
    """States entering consecutive segments (kda_compose_states):
    S_in[0] = S0, S_in[g+1] = P[g] S_in[g] + Z[g]; returns [G+1, H, d, d]."""
    import torch
    lib = _load()
    G, H, d, _ = P.shape
    for name, t in (("P", P), ("Z", Z)):
        if t.dtype != torch.float32 or t.shape != (G, H, d, d) or not t.is_contiguous():
            raise ValueError("%s must be contiguous float32 [%d, %d, %d, %d]" % (name, G, H, d, d))
    if S0 is not None and (S0.dtype != torch.float32 or S0.shape != (H, d, d) or not S0.is_contiguous()):
        raise ValueError("S0 must be contiguous float32 [%d, %d, %d]" % (H, d, d))
    S_in = torch.empty((G + 1, H, d, d), dtype=torch.float32, device=P.device)
    stream = torch.cuda.current_stream(P.device).cuda_stream
    code = lib.kda_compose_states(G, H, d, _ptr(P), _ptr(Z), _ptr(S0), _ptr(S_in), ctypes.c_void_p(stream))
    if code != 0:
        raise KdaError(code, lib.kda_status_string(code).decode())
    return S_in


def sequence_parallel_fwd(q, k, v, beta, log_alpha, S0=None, n_segments=4):
    """One long sequence ([T, H, d] bf16) by sequence-parallel state passing,
    on one GPU: the token axis is cut into `n_segments` segments; per segment
    the zero-start final state Z_g (kda_chunk_fwd, S0 = 0) and the transition
    P_g (kda_chunk_transition) -- the work each device would do on its own
    segment --, then the incoming states by composition (kda_compose_states;
    across devices this is where the one all-gather of (P_g, Z_g) goes), then
    every segment's outputs from its incoming state.  Returns (o, S_T) equal,
    to rounding, to chunk_fwd over the whole sequence."""
    import torch
    T, H, d = q.shape
    G = max(1, min(int(n_segments), T))
    bounds = [round(i * T / G) for i in range(G + 1)]
    cu = torch.tensor(bounds, dtype=torch.int32, device=q.device)
    _, Z = chunk_fwd(q, k, v, beta, log_alpha, S0=None, cu_seqlens=cu)
    P = chunk_transition(k, beta, log_alpha, cu_seqlens=cu)
    S_in = compose_states(P, Z, None if S0 is None else S0.reshape(H, d, d).contiguous())
    o, _ = chunk_fwd(q, k, v, beta, log_alpha, S0=S_in[:G].contiguous(), cu_seqlens=cu, output_final_state=False)
    return o, S_in[G].reshape(1, H, d, d)
