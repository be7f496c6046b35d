"""kda_chunk_fwd_noalloc (the forward with its workspace in the library's
fixed device array) called through the C ABI: two calls in a row, the second
smaller, each bit for bit equal to kda_chunk_fwd on the same inputs (same
kernels) and within the bf16 bar of the fp64 oracle, for the tuned sizes and
for sizes that run the generic kernels; sizes past the array are rejected
before anything is launched."""
import ctypes
import sys

import numpy as np
import pytest

import kda_inputs as ki
import oracle

pytestmark = pytest.mark.gpu

KDA_OK, KDA_ERR_WORKSPACE = 0, 5


def _say(msg):
    print("[gpu-noalloc] %s" % msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_delta_rule_30_amd as kda
    lib = kda._load()
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.kda_chunk_fwd_noalloc.argtypes = [ctypes.c_int, I64, I32, I32, I32, I32, I32,
                                          P, P, P, P, P, P, P, P, P, P]
    lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    return torch, kda, lib, torch.device("cuda:0")


def _call(torch, kda, lib, dev, lengths, H, d, seed, dv=None, C=64):
    dk, dv = d, (d if dv is None else dv)
    spec = ki.Spec("noalloc", "bf16", tuple(lengths), H, dk, dv, s0_std=0.02, varlen=True, seed=seed)
    inp = ki.generate_numpy(spec)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)
    q, k, v, beta, g = (t(a) for a in (inp.q, inp.k, inp.v, inp.beta, inp.g))
    S0 = torch.from_numpy(inp.S0).to(dev)
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev)
    T, N = spec.total_tokens, spec.n_seqs
    need = kda.workspace_size(T, N, H, dk, dv, C)
    o = torch.full((T, H, dv), float("nan"), dtype=torch.bfloat16, device=dev)
    S_T = torch.full((N, H, dk, dv), float("nan"), dtype=torch.float32, device=dev)
    ptr = lambda x: ctypes.c_void_p(x.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    _say("lengths %s H=%d d_k=%d d_v=%d chunk %d: workspace %.1f MiB of %d MiB"
         % (lengths, H, dk, dv, C, need / 2 ** 20, 64))
    rc = lib.kda_chunk_fwd_noalloc(kda.KDA_BF16, T, N, H, dk, dv, C, ptr(q), ptr(k), ptr(v), ptr(beta), ptr(g),
                                   ptr(S0), ptr(cu), ptr(o), ptr(S_T), stream)
    assert rc == KDA_OK, kda.status_string(rc)
    o_ref, S_ref = kda.chunk_fwd(q, k, v, beta, g, S0=S0, cu_seqlens=cu, chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S_T, S_ref), "noalloc differs from kda_chunk_fwd"
    o64, S64 = oracle.forward(inp.q, inp.k, inp.v, inp.beta, inp.g, inp.S0, inp.cu_seqlens)
    eo = oracle.parity_error(o.float().cpu().numpy(), o64, inp.cu_seqlens)
    es = oracle.parity_error(S_T.cpu().numpy(), S64)
    _say("  o %.2e S_T %.2e (bit-identical to kda_chunk_fwd)" % (eo, es))
    assert eo <= 2e-2 and es <= 2e-2


def test_noalloc_two_calls_second_smaller(env):
    torch, kda, lib, dev = env
    _call(torch, kda, lib, dev, (700, 64, 1100, 0, 513), 4, 128, seed=31)
    _call(torch, kda, lib, dev, (150, 77), 2, 64, seed=32)


def test_noalloc_generic_sizes(env):
    """The sizes that run the generic kernels (chunk 32 with d_k != d_v, then
    chunk 128): same two-call pattern, the second smaller."""
    torch, kda, lib, dev = env
    _call(torch, kda, lib, dev, (300, 45, 0, 129), 2, 64, seed=33, dv=128, C=32)
    _call(torch, kda, lib, dev, (200,), 2, 128, seed=34, dv=64, C=128)


def test_noalloc_rejects_sizes_past_the_array(env):
    torch, kda, lib, dev = env
    T, N, H, d = 65536, 1, 32, 128
    assert kda.workspace_size(T, N, H, d, d) > 64 << 20
    fake = ctypes.c_void_p(1 << 20)   # 16-byte aligned, never dereferenced: the size check comes first
    rc = lib.kda_chunk_fwd_noalloc(kda.KDA_BF16, T, N, H, d, d, 64, fake, fake, fake, fake, fake, None, None,
                                   fake, None, None)
    assert rc == KDA_ERR_WORKSPACE, kda.status_string(rc)
    rc = lib.kda_chunk_fwd_noalloc(kda.KDA_BF16, T, N, H, 96, 96, 64, fake, fake, fake, fake, fake, None, None,
                                   fake, None, None)
    assert rc == 4, kda.status_string(rc)   # unsupported sizes: as kda_chunk_fwd
