"""The C-ABI library: it loads, exports every function include/kda.h declares,
sizes its workspace, and rejects bad arguments on the host with the
documented status before anything is enqueued.  No GPU needed: every call
here fails validation, so no kernel is ever launched."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_30_amd as kda

ROOT = os.path.abspath(os.path.join(os.path.dirname(__file__), ".."))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(7)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.lib_path()):
        pytest.fail("libkda.so not built; run __graft_entry__.build()")
    return kda._load()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) >= {"kda_chunk_fwd", "kda_chunk_fwd_workspace_size", "kda_status_string", "kda_version"}
    for n in names:
        assert hasattr(lib, n), "libkda.so does not export %s" % n


def test_status_strings(lib):
    for code in range(7):
        s = kda.status_string(code)
        assert s.startswith("KDA_")
    assert "unknown" in kda.status_string(99)
    assert lib.kda_version().decode().count(".") == 2


def test_workspace_size():
    a = kda.workspace_size(65536, 1, 32, 128, 128, 64, kda.KDA_BF16)
    b = kda.workspace_size(65536, 1, 32, 128, 128, 64, kda.KDA_F32)
    assert a > 0 and b > 0                     # fp32 at d = 128: the generic kernels
    assert kda.workspace_size(256, 1, 2, 64, 64, 64, kda.KDA_F32) > 0
    assert kda.workspace_size(256, 1, 2, 96, 96, 64, kda.KDA_BF16) == 0
    assert kda.workspace_size(256, 1, 2, 64, 96, 64, kda.KDA_BF16) == 0
    for C in (16, 32, 128):
        assert kda.workspace_size(256, 1, 2, 64, 64, C, kda.KDA_BF16) > 0
    for C in (0, 8, 48, 96, 256):
        assert kda.workspace_size(256, 1, 2, 64, 64, C, kda.KDA_BF16) == 0
    assert kda.workspace_size(-1, 1, 2, 64, 64, 64, kda.KDA_BF16) == 0
    assert kda.workspace_size(1 << 31, 1, 2, 64, 64, 64, kda.KDA_BF16) == 0
    # monotone in tokens and heads; 256-byte granularity
    s1 = kda.workspace_size(1000, 3, 4, 64, 64, 64, kda.KDA_BF16)
    s2 = kda.workspace_size(2000, 3, 4, 64, 64, 64, kda.KDA_BF16)
    s3 = kda.workspace_size(1000, 3, 8, 64, 64, 64, kda.KDA_BF16)
    assert s1 < s2 and s1 < s3 and s1 % 256 == 0
    assert kda.workspace_size(0, 2, 4, 128, 128, 64, kda.KDA_BF16) > 0


@pytest.mark.parametrize("T,N,H,dk,dv,C,dt", [(1000, 3, 4, 64, 128, 32, kda.KDA_BF16),
                                              (65536, 1, 32, 128, 128, 128, kda.KDA_BF16),
                                              (4096, 2, 2, 128, 64, 16, kda.KDA_F32),
                                              (777, 5, 3, 128, 128, 64, kda.KDA_F32)])
def test_generic_workspace_size(T, N, H, dk, dv, C, dt):
    """The sizes outside the tuned ones take fp32 operands: per chunk slot
    and head, Q.e^b, K.e^b, K.e^{b_L-b} (C x d_k each), T diag(beta) and M
    (C x C each) and e^{b_L} (d_k), plus the chunk table; every region
    rounded up to 256 bytes."""
    mc = T // C + N
    up = lambda x: (x + 255) // 256 * 256
    expect = up(4) + up(4 * (N + 1)) + up(16 * mc)
    expect += 3 * up(4 * mc * H * C * dk) + 2 * up(4 * mc * H * C * C) + up(4 * mc * H * dk)
    assert kda.workspace_size(T, N, H, dk, dv, C, dt) == expect


def _call(lib, dt=kda.KDA_BF16, T=128, N=1, H=2, dk=64, dv=64, C=64, ptrs=None, S0=None, cu=None,
          ST=None, ws=0x100000, ws_bytes=None):
    P = ctypes.c_void_p
    fake = 0x7f0000000000          # never dereferenced: every case below fails validation
    p = dict(q=fake, k=fake, v=fake, beta=fake, g=fake, o=fake)
    if ptrs:
        p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = 0
    return lib.kda_chunk_fwd(dt, T, N, H, dk, dv, C, P(p["q"]), P(p["k"]), P(p["v"]), P(p["beta"]), P(p["g"]),
                             P(S0), P(cu), P(p["o"]), P(ST), P(ws), ws_bytes, None)


def test_rejects_bad_arguments(lib):
    assert _call(lib, dt=7) == ERR_DTYPE
    assert _call(lib, T=-5) == ERR_SHAPE
    assert _call(lib, N=0) == ERR_SHAPE
    assert _call(lib, H=0) == ERR_SHAPE
    assert _call(lib, T=100, N=3) == ERR_SHAPE              # equal lengths must divide
    assert _call(lib, dk=96, dv=96) == ERR_UNSUPPORTED
    assert _call(lib, dk=64, dv=32) == ERR_UNSUPPORTED
    for C in (0, 8, 48, 256):
        assert _call(lib, C=C) == (ERR_SHAPE if C == 0 else ERR_UNSUPPORTED), C
    # the generic sizes are accepted (and fail here on the missing workspace)
    assert _call(lib, dk=64, dv=128) == ERR_WORKSPACE
    assert _call(lib, C=128) == ERR_WORKSPACE
    assert _call(lib, C=16, dk=128) == ERR_WORKSPACE
    assert _call(lib, dt=kda.KDA_F32, dk=128, dv=128) == ERR_WORKSPACE
    assert _call(lib, T=1 << 31) == ERR_UNSUPPORTED
    assert _call(lib, H=70000) == ERR_UNSUPPORTED
    for name in ("q", "k", "v", "beta", "g", "o"):
        assert _call(lib, ptrs={name: None}) == ERR_NULL, name
    assert _call(lib, ptrs={"q": 0x7f0000000008}) == ERR_SHAPE   # misaligned
    assert _call(lib, S0=0x7f0000000004) == ERR_SHAPE
    assert _call(lib, ws=None) == ERR_WORKSPACE
    assert _call(lib, ws=0x100010, ws_bytes=1 << 40) == ERR_WORKSPACE   # misaligned workspace
    need = kda.workspace_size(128, 1, 2, 64, 64, 64, kda.KDA_BF16)
    assert _call(lib, ws_bytes=need - 1) == ERR_WORKSPACE
    # varlen sizing: the workspace for N sequences covers any split of the tokens
    assert _call(lib, T=100, N=3, cu=0x7f0000001000, ws_bytes=10) == ERR_WORKSPACE


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(4, 2, 64)
    with pytest.raises(ValueError):
        kda.chunk_fwd(x, x, x, torch.zeros(4, 2), x)
    with pytest.raises(TypeError):
        kda.chunk_fwd(x.double(), x, x, torch.zeros(4, 2), x)


def test_recurrent_rejects_bad_arguments(lib):
    P = ctypes.c_void_p
    fake = 0x7f0000000000          # never dereferenced: every case fails validation

    def call(dt=kda.KDA_BF16, N=2, n=1, H=2, dk=64, dv=64, q=fake, S_in=None, S_out=fake, o=fake):
        return lib.kda_recurrent_fwd(dt, N, n, H, dk, dv, P(q), P(fake), P(fake), P(fake), P(fake),
                                     P(S_in), P(S_out), P(o), None)
    assert call(dt=5) == ERR_DTYPE
    assert call(N=0) == ERR_SHAPE
    assert call(n=0) == ERR_SHAPE
    assert call(dk=96, dv=96) == ERR_UNSUPPORTED
    assert call(dk=64, dv=128) == ERR_UNSUPPORTED
    assert call(N=1 << 20, n=1 << 12) == ERR_UNSUPPORTED
    assert call(q=None) == ERR_NULL
    assert call(S_out=None) == ERR_NULL
    assert call(o=None) == ERR_NULL
    assert call(o=fake + 4) == ERR_SHAPE
    assert call(S_in=fake + 8) == ERR_SHAPE


def test_recurrent_commit_rejects_bad_arguments(lib):
    P = ctypes.c_void_p
    fake = 0x7f0000000000          # never dereferenced: every case fails validation

    def call(dt=kda.KDA_BF16, N=2, n=3, H=2, dk=64, dv=64, acc=fake, S_out=fake, o=None):
        return lib.kda_recurrent_commit(dt, N, n, H, dk, dv, P(fake), P(fake), P(fake), P(fake), P(fake),
                                        P(acc), None, P(S_out), P(o), None)
    assert call(dt=7) == ERR_DTYPE
    assert call(n=0) == ERR_SHAPE
    assert call(dk=32, dv=32) == ERR_UNSUPPORTED
    assert call(acc=None) == ERR_NULL          # the accepted counts are required
    assert call(S_out=None) == ERR_NULL
    assert call(acc=fake + 2) == ERR_SHAPE     # int32 alignment
    assert call(o=fake + 4) == ERR_SHAPE


def test_validate_rejects_bad_arguments(lib):
    P = ctypes.c_void_p
    fake = 0x7f0000000000

    def call(dt=kda.KDA_BF16, T=16, N=1, H=2, dk=64, beta=fake, g=fake, counts=fake):
        return lib.kda_validate_inputs(dt, T, N, H, dk, P(beta), P(g), None, P(counts), None)
    assert call(dt=9) == ERR_DTYPE
    assert call(T=-1) == ERR_SHAPE
    assert call(N=0) == ERR_SHAPE
    assert call(counts=None) == ERR_NULL
    assert call(beta=None) == ERR_NULL
    assert call(counts=fake + 4) == ERR_SHAPE


def test_transition_and_compose_reject_bad_arguments(lib):
    P = ctypes.c_void_p
    fake = 0x7f0000000000

    def tr(dt=kda.KDA_BF16, T=128, N=1, H=2, d=64, C=64, Pout=fake, ws=0x100000, ws_bytes=0):
        return lib.kda_chunk_transition(dt, T, N, H, d, C, P(fake), P(fake), P(fake), None, P(Pout), P(ws),
                                        ws_bytes, None)
    assert tr(dt=kda.KDA_F32) == ERR_UNSUPPORTED
    assert tr(Pout=None) == ERR_NULL
    assert tr(d=96) == ERR_UNSUPPORTED
    assert tr(C=32) == ERR_UNSUPPORTED
    assert tr(ws_bytes=16) == ERR_WORKSPACE

    def comp(G=2, H=2, d=64, Pp=fake, Z=fake, S0=None, S=fake):
        return lib.kda_compose_states(G, H, d, P(Pp), P(Z), P(S0), P(S), None)
    assert comp(G=0) == ERR_SHAPE
    assert comp(d=96) == ERR_UNSUPPORTED
    assert comp(Pp=None) == ERR_NULL
    assert comp(S=None) == ERR_NULL
    assert comp(Z=fake + 4) == ERR_SHAPE


def test_backward_workspace_and_rejections(lib):
    P = ctypes.c_void_p
    fake = 0x7f0000000000          # never dereferenced: every case below fails validation
    fwd = kda.workspace_size(65536, 1, 32, 128, 128, 64, kda.KDA_BF16)
    bwd = kda.bwd_workspace_size(65536, 1, 32, 128, 128, 64, kda.KDA_BF16)
    # the backward keeps two d x d bf16 states per chunk and head and three v-sized bf16 tensors
    assert bwd >= fwd + 2 * 1024 * 32 * 128 * 128 * 2 + 3 * 65536 * 32 * 128 * 2
    assert kda.bwd_workspace_size(65536, 1, 32, 128, 128, 64, kda.KDA_F32) == 0
    assert kda.bwd_workspace_size(256, 1, 2, 96, 96, 64, kda.KDA_BF16) == 0
    assert kda.bwd_workspace_size(0, 3, 2, 64, 64, 64, kda.KDA_BF16) > 0
    assert kda.bwd_workspace_size(1000, 3, 4, 64, 64, 64, kda.KDA_BF16) % 256 == 0

    def bw(dt=kda.KDA_BF16, T=128, N=1, H=2, d=64, C=64, ptrs=None, ws=0x100000, ws_bytes=0):
        p = dict(q=fake, k=fake, v=fake, beta=fake, g=fake, S0=None, cu=None, dO=fake, dST=None,
                 dq=fake, dk=fake, dv=fake, dbeta=fake, dg=fake, dS0=None)
        if ptrs:
            p.update(ptrs)
        return lib.kda_chunk_bwd(dt, T, N, H, d, d, C, *(P(p[n]) for n in (
            "q", "k", "v", "beta", "g", "S0", "cu", "dO", "dST", "dq", "dk", "dv", "dbeta", "dg", "dS0")),
            P(ws), ws_bytes, None)
    assert bw(dt=kda.KDA_F32) == ERR_UNSUPPORTED
    assert bw(dt=9) == ERR_DTYPE
    assert bw(d=96) == ERR_UNSUPPORTED
    assert bw(C=32) == ERR_UNSUPPORTED
    assert bw(T=100, N=3) == ERR_SHAPE
    for name in ("q", "k", "v", "beta", "g", "dO", "dq", "dk", "dv", "dbeta", "dg"):
        assert bw(ptrs={name: None}) == ERR_NULL, name
    assert bw(ptrs={"dS0": fake + 4}) == ERR_SHAPE
    assert bw(ptrs={"dST": fake + 8}) == ERR_SHAPE
    assert bw(ws=None) == ERR_WORKSPACE
    need = kda.bwd_workspace_size(128, 1, 2, 64, 64, 64, kda.KDA_BF16)
    assert bw(ws_bytes=need - 1) == ERR_WORKSPACE
    # the forward's workspace is not enough for the backward
    assert bw(ws_bytes=kda.workspace_size(128, 1, 2, 64, 64, 64, kda.KDA_BF16)) == ERR_WORKSPACE
    ms = (ctypes.c_float * 6)()
    assert lib.kda_chunk_bwd_profile(kda.KDA_F32, 128, 1, 2, 64, 64, 64, *([None] * 15), None, 0, None,
                                     ms) == ERR_UNSUPPORTED
    assert kda.bwd_stage_names() == ["k_chunk_table", "k_prep<fwd+bwd>", "k_recur_lds<ckpt>",
                                     "k_recur_lds<bwd>", "k_grad", "k_dbeta_sum"]


def test_backward_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kda.chunk_bwd(x, x, x, torch.zeros(4, 2, dtype=torch.bfloat16), x, x)


def test_output_gate_rejects_bad_arguments(lib):
    P = ctypes.c_void_p
    fake = 0x7f0000000000

    def og(dt=kda.KDA_BF16, n=10, d=128, o=fake, z=fake, w=None, eps=1e-6, y=fake):
        return lib.kda_output_gate(dt, n, d, P(o), P(z), P(w), eps, P(y), None)
    assert og(dt=5) == ERR_DTYPE
    assert og(n=-1) == ERR_SHAPE
    assert og(d=96) == ERR_UNSUPPORTED
    assert og(eps=float("nan")) == ERR_SHAPE
    assert og(eps=-1.0) == ERR_SHAPE
    assert og(o=None) == ERR_NULL
    assert og(z=None) == ERR_NULL
    assert og(y=None) == ERR_NULL
    assert og(w=fake + 4) == ERR_SHAPE
    assert og(n=0, o=None, z=None, y=None) == OK      # nothing to do, nothing launched


def test_training_pair_rejects_bad_arguments(lib):
    P = ctypes.c_void_p
    fake = 0x7f0000000000
    assert kda.train_context_size(65536, 1, 32, 128, 128) > 0
    assert kda.train_context_size(256, 1, 2, 64, 64, 64, kda.KDA_F32) == 0
    assert lib.kda_chunk_bwd_ctx_workspace_size(256, 1, 2, 64, 64, 64, kda.KDA_BF16) > 0
    need_ws = kda.workspace_size(128, 1, 2, 64, 64, 64, kda.KDA_BF16)
    need_ctx = kda.train_context_size(128, 1, 2, 64, 64)

    def ft(dt=kda.KDA_BF16, ctx=0x200000, ctx_bytes=None, ws_bytes=None, o=fake):
        return lib.kda_chunk_fwd_train(dt, 128, 1, 2, 64, 64, 64, P(fake), P(fake), P(fake), P(fake), P(fake), None,
                                       None, P(o), None, P(ctx), need_ctx if ctx_bytes is None else ctx_bytes,
                                       P(0x100000), need_ws if ws_bytes is None else ws_bytes, None)
    assert ft(dt=kda.KDA_F32) == ERR_UNSUPPORTED
    assert ft(o=None) == ERR_NULL
    assert ft(ctx=None) == ERR_WORKSPACE
    assert ft(ctx=0x200010) == ERR_WORKSPACE
    assert ft(ctx_bytes=need_ctx - 1) == ERR_WORKSPACE
    assert ft(ws_bytes=need_ws - 1) == ERR_WORKSPACE

    need_bws = lib.kda_chunk_bwd_ctx_workspace_size(128, 1, 2, 64, 64, 64, kda.KDA_BF16)

    def bc(dt=kda.KDA_BF16, ctx=0x200000, ctx_bytes=None, ws_bytes=None, dO=fake, v=fake):
        return lib.kda_chunk_bwd_ctx(dt, 128, 1, 2, 64, 64, 64, P(fake), P(fake), P(v), P(fake), P(fake), None,
                                     P(ctx), need_ctx if ctx_bytes is None else ctx_bytes, P(dO), None, P(fake), P(fake),
                                     P(fake), P(fake), P(fake), None, P(0x100000),
                                     need_bws if ws_bytes is None else ws_bytes, None)
    assert bc(dt=kda.KDA_F32) == ERR_UNSUPPORTED
    assert bc(dO=None) == ERR_NULL
    assert bc(v=None) == ERR_NULL
    assert bc(ctx=None) == ERR_WORKSPACE
    assert bc(ctx_bytes=16) == ERR_WORKSPACE
    assert bc(ws_bytes=need_bws - 1) == ERR_WORKSPACE


def test_checkpoint_size_and_rejections(lib):
    P = ctypes.c_void_p
    # slots = (total_tokens / 64 + n_seqs) / every, each n_heads x d_k x d_v float32
    assert lib.kda_chunk_ckpt_size(65536, 1, 32, 128, 128, 1) == (65536 // 64 + 1) * 32 * 128 * 128 * 4
    assert lib.kda_chunk_ckpt_size(65536, 1, 32, 128, 128, 8) == (1025 // 8) * 32 * 128 * 128 * 4
    assert lib.kda_chunk_ckpt_size(100, 3, 2, 64, 64, 1) == (100 // 64 + 3) * 2 * 64 * 64 * 4
    assert lib.kda_chunk_ckpt_size(100, 3, 2, 64, 64, 3) == 1 * 2 * 64 * 64 * 4
    assert lib.kda_chunk_ckpt_size(100, 3, 2, 96, 96, 1) == 0
    assert lib.kda_chunk_ckpt_size(-1, 3, 2, 64, 64, 1) == 0
    assert lib.kda_chunk_ckpt_size(100, 3, 2, 64, 64, 0) == 0
    buf = (ctypes.c_byte * 4096)()
    a = ctypes.addressof(buf)
    a16 = P(a + (-a) % 16)
    need = lib.kda_chunk_ckpt_size(128, 1, 2, 64, 64, 2)

    def call(dt=kda.KDA_BF16, every=2, sck=a16, sck_bytes=need, ws=a16, ws_bytes=1 << 40):
        return lib.kda_chunk_fwd_ckpt(dt, 128, 1, 2, 64, 64, 64, a16, a16, a16, a16, a16, None, None,
                                      a16, None, every, sck, sck_bytes, ws, ws_bytes, None)
    assert call(dt=kda.KDA_F32) == ERR_UNSUPPORTED
    for C in (16, 32, 128):   # the generic sizes are the plain forward's only
        assert lib.kda_chunk_fwd_ckpt(kda.KDA_BF16, 128, 1, 2, 64, 64, C, a16, a16, a16, a16, a16, None, None,
                                      a16, None, 2, a16, need, a16, 1 << 40, None) == ERR_UNSUPPORTED
        assert kda.bwd_workspace_size(128, 1, 2, 64, 64, C, kda.KDA_BF16) == 0
    assert kda.bwd_workspace_size(128, 1, 2, 64, 128, 64, kda.KDA_BF16) == 0
    assert call(every=0) == ERR_SHAPE
    assert call(every=-3) == ERR_SHAPE
    assert call(sck=None) == ERR_NULL
    assert call(sck=P(a16.value + 4)) == ERR_SHAPE
    assert call(ws=None) == ERR_WORKSPACE
    assert call(sck_bytes=need - 1) == ERR_WORKSPACE


def test_checkpoint_slots_helper():
    got = kda.ckpt_slots([700, 64, 1100, 0, 513], 2)
    # packed in sequence order: sequence 0 (11 chunks) has checkpoints after
    # chunks 1, 3, 5, 7, 9 in slots 0-4; sequence 1 (one chunk) none;
    # sequence 2 (18 chunks, the last partial, ending at token 1100) 9 in
    # slots 5-13; sequence 4 (9 chunks) 4 in slots 14-17
    assert got[0] == [(128, 0), (256, 1), (384, 2), (512, 3), (640, 4)]
    assert got[1] == [] and got[3] == []
    assert got[2][0] == (128, 5) and got[2][-1] == (1100, 13) and len(got[2]) == 9
    assert got[4] == [(128, 14), (256, 15), (384, 16), (512, 17)]
    assert kda.ckpt_slots([512], 8) == [[(512, 0)]]
    # every split fits the size the library reports
    for lengths, every in (([700, 64, 1100, 0, 513], 2), ([63] * 7, 1), ([65] * 5, 2), ([512], 8)):
        n = sum(len(x) for x in got) if lengths == [700, 64, 1100, 0, 513] else \
            sum(len(x) for x in kda.ckpt_slots(lengths, every))
        assert n <= (sum(lengths) // 64 + len(lengths)) // every


def _cpu(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


@pytest.mark.parametrize("entry", ["chunk_fwd", "chunk_fwd_train", "chunk_bwd", "chunk_fwd_ckpt"])
def test_bad_shapes_rejected_before_launch(entry):
    """The binding checks every shape the C ABI cannot see (it takes only
    pointers) before anything is launched: a wrong extent raises ValueError
    (these CPU tensors never reach the device)."""
    import torch
    T, H, d = 70, 2, 64
    good = dict(q=_cpu(T, H, d), k=_cpu(T, H, d), v=_cpu(T, H, d), beta=_cpu(T, H), log_alpha=_cpu(T, H, d))
    bad = [dict(good, beta=_cpu(T)), dict(good, beta=_cpu(T, H + 1)), dict(good, k=_cpu(T, H, d + 1)),
           dict(good, log_alpha=_cpu(T - 1, H, d)), dict(good, v=_cpu(T, H + 1, d)), dict(good, q=_cpu(T, d))]

    def call(a, **kw):
        if entry == "chunk_fwd":
            return kda.chunk_fwd(**a, **kw)
        if entry == "chunk_fwd_train":
            return kda.chunk_fwd_train(**a, **kw)
        if entry == "chunk_fwd_ckpt":
            return kda.chunk_fwd_ckpt(**a, every=2, **kw)
        return kda.chunk_bwd(**a, dO=_cpu(T, H, d), **kw)
    for a in bad:
        with pytest.raises(ValueError, match="shape|must be"):
            call(a)
    # well-shaped CPU tensors get as far as the device check
    with pytest.raises(ValueError, match="GPU"):
        call(good)


def test_bad_state_and_offsets_rejected():
    """S0 of the wrong dtype or extent, and cu_seqlens of the wrong dtype or
    rank, are rejected by the shared check before its device check (so CPU
    tensors show it)."""
    import torch
    T, H, d = 70, 2, 64
    good = dict(q=_cpu(T, H, d), k=_cpu(T, H, d), v=_cpu(T, H, d), beta=_cpu(T, H), log_alpha=_cpu(T, H, d))
    with pytest.raises(ValueError, match="GPU"):
        kda._fwd_problem(**good, S0=_cpu(1, H, d, d, dtype=torch.float32),
                         cu_seqlens=torch.tensor([0, 70], dtype=torch.int32))
    for kw in (dict(S0=_cpu(1, H, d, d)),                                   # bf16 state
               dict(S0=_cpu(2, H, d, d, dtype=torch.float32)),              # wrong N
               dict(cu_seqlens=torch.tensor([0, 30, 70], dtype=torch.int64)),
               dict(cu_seqlens=torch.tensor([[0, 70]], dtype=torch.int32)),
               dict(cu_seqlens=torch.tensor([0], dtype=torch.int32))):
        with pytest.raises(ValueError):
            try:
                kda._fwd_problem(**good, **kw)
            except ValueError as e:
                assert "GPU" not in str(e), "the device check came first: %s" % e
                raise
