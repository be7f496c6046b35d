"""Stage tests: the GPU's per-chunk intermediates against the chunkwise fp64
model's (oracle/chunked.py, stages=True), chunk by chunk.

After a forward pass the workspace holds every chunk's operands (Q . Gamma,
K . Gamma, (K . exp(b_L - b))^T, T diag(beta), M, Gamma_L); after the
training forward the context holds the backward operand set (T^T, M^T,
K . exp(b_L - b), (Q . Gamma)^T, (K . Gamma)^T, beta), the state entering
every chunk, and per token U~ = T diag(beta) (V - (K . Gamma) S).  The regions are
found from the published workspace sizes and the library's documented carve
order, and the fragment-major tiles are decoded here.  Every stage is
compared per chunk as max|gpu - ref| / max|ref| <= 1e-2 (bf16 storage),
and the triangular inverse is checked directly: (I + A) T diag(beta) =
diag(beta) with A from the model.  The halves of the triangular tiles that
are zero by structure are not stored and are left out of the comparison.
"""
import sys

import numpy as np
import pytest

import kda_inputs as ki
from oracle import chunked

pytestmark = pytest.mark.gpu

C = 64
TOL = 1e-2


def _say(msg):
    print("[gpu-stages] %s" % msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import gated_delta_rule_30_amd  # noqa: F401
    return torch, torch.device("cuda:0")


def _align(x):
    return (x + 255) // 256 * 256


def _carve(sizes):
    """Byte offsets of consecutive 256-byte aligned regions."""
    offs, at = [], 0
    for s in sizes:
        offs.append(at)
        at = _align(at + s)
    return offs, at


def _bf16_view(buf, off, count):
    import torch
    return buf[off:off + 2 * count].view(torch.bfloat16).float().cpu().numpy()


def _f32_view(buf, off, count):
    import torch
    return buf[off:off + 4 * count].view(torch.float32).cpu().numpy()


def _tiles_rows_over_tokens(raw):
    """[tiles][NV=2][64 lanes][8] fragment-major -> [16 * tiles, 64] (row, token)."""
    n_t = raw.size // (2 * 64 * 8)
    a = raw.reshape(n_t, 2, 4, 16, 8)              # tile, v, lg, li, e
    # token = 32 v + 8 lg + e, row = 16 tile + li
    return a.transpose(0, 3, 1, 2, 4).reshape(16 * n_t, 64)


def _tiles_rows_over_channels(raw, D):
    """[4 tiles][VPL][64 lanes][8] -> [64, D] (token row, channel): lane (li, lg)
    holds channels lg * D/4 + 8 v + e."""
    vpl = D // 32
    a = raw.reshape(4, vpl, 4, 16, 8)               # tile, v, lg, li, e
    return a.transpose(0, 3, 2, 1, 4).reshape(64, D)


def _chunks(cu):
    out = []
    for n in range(len(cu) - 1):
        for c0 in range(int(cu[n]), int(cu[n + 1]), C):
            out.append((n, c0, min(c0 + C, int(cu[n + 1]))))
    return out


def _err(x, ref):
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-30))


def _pad(m, rows, cols):
    out = np.zeros((rows, cols))
    out[:m.shape[0], :m.shape[1]] = m
    return out


@pytest.mark.parametrize("lengths,H,d", [((150, 77, 64), 2, 64), ((200, 33), 2, 128)], ids=["d64", "d128"])
def test_stages_match_chunked_model(torch_dev, lengths, H, d):
    torch, dev = torch_dev
    import gated_delta_rule_30_amd as kda
    spec = ki.Spec("stages", "bf16", tuple(lengths), H, d, d, s0_std=0.02, pin_frac=0.25, varlen=True, seed=5)
    inp = ki.generate_numpy(spec)
    T, N = spec.total_tokens, spec.n_seqs
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16)
    q, k, v, beta, g = (t(a) for a in (inp.q, inp.k, inp.v, inp.beta, inp.g))
    S0 = torch.from_numpy(inp.S0).to(dev)
    cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev)
    mc = T // C + N
    # forward workspace: n_chunks, seq_chunk0, chunk table, TB, M, Qg, Kg, KhT, Gamma_L, the two states
    # between pipelined blocks, the first checkpoint slot per sequence, and last the recurrence's
    # per-workgroup step counts
    sizes = [4, 4 * (N + 1), 16 * mc, 2 * mc * H * C * C, 2 * mc * H * C * C, 2 * mc * H * C * d,
             2 * mc * H * C * d, 2 * mc * H * d * C, 4 * mc * H * d, 4 * 2 * N * H * d * d, 4 * (N + 1),
             4 * N * H * (d // 16)]
    offs, total = _carve(sizes)
    assert total == kda.workspace_size(T, N, H, d, d)
    ws = torch.zeros(total, dtype=torch.uint8, device=dev)
    kda.chunk_fwd(q, k, v, beta, g, S0=S0, cu_seqlens=cu, workspace=ws)
    # training forward: its context holds the backward set, states and U~
    csz = [4 * mc * H * d, 4 * mc * H * C, 2 * mc * H * C * C, 2 * mc * H * C * C, 2 * mc * H * C * d,
           2 * mc * H * d * C, 2 * mc * H * d * C, 2 * mc * H * d * d, 2 * T * H * d]
    coffs, ctotal = _carve(csz)
    assert ctotal == kda.train_context_size(T, N, H, d, d)
    _, _, ctx = kda.chunk_fwd_train(q, k, v, beta, g, S0=S0, cu_seqlens=cu)
    torch.cuda.synchronize()

    _, _, rec = chunked.forward_chunked(inp.q, inp.k, inp.v, inp.beta, inp.g, inp.S0, inp.cu_seqlens, stages=True)
    Ug = _bf16_view(ctx, coffs[8], T * H * d).reshape(T, H, d)
    worst = {}
    for ci, (n, c0, c1) in enumerate(_chunks(inp.cu_seqlens)):
        L = c1 - c0
        for h in range(H):
            r = next(x for x in rec if x["seq"] == n and x["head"] == h and x["start"] == c0)
            slot = h * mc + ci
            bt = inp.beta[c0:c1, h].astype(np.float64)
            Qv, Kv = (a[c0:c1, h].astype(np.float64) for a in (inp.q, inp.k))
            Gam = np.exp(r["b"])
            Kh = Kv * np.exp(r["b"][-1][None, :] - r["b"])
            TB_ref = r["T"] * bt[None, :]
            M_ref = r["M"]
            got = {}
            got["TB"] = _tiles_rows_over_tokens(_bf16_view(ws, offs[3] + 2 * slot * C * C, C * C))
            got["M"] = _tiles_rows_over_tokens(_bf16_view(ws, offs[4] + 2 * slot * C * C, C * C))
            got["Qg"] = _tiles_rows_over_channels(_bf16_view(ws, offs[5] + 2 * slot * C * d, C * d), d)
            got["Kg"] = _tiles_rows_over_channels(_bf16_view(ws, offs[6] + 2 * slot * C * d, C * d), d)
            got["KhT"] = _tiles_rows_over_tokens(_bf16_view(ws, offs[7] + 2 * slot * d * C, d * C))
            got["gam"] = _f32_view(ws, offs[8] + 4 * slot * d, d)
            ref = {"TB": _pad(TB_ref, C, C), "M": _pad(M_ref, C, C), "Qg": _pad(Qv * Gam, C, d),
                   "Kg": _pad(Kv * Gam, C, d), "KhT": _pad(Kh.T, d, C), "gam": np.exp(r["b"][-1])}
            # backward set in the context
            got["bTT"] = _tiles_rows_over_tokens(_bf16_view(ctx, coffs[2] + 2 * slot * C * C, C * C))
            got["bMT"] = _tiles_rows_over_tokens(_bf16_view(ctx, coffs[3] + 2 * slot * C * C, C * C))
            got["bKh"] = _tiles_rows_over_channels(_bf16_view(ctx, coffs[4] + 2 * slot * C * d, C * d), d)
            got["bQgT"] = _tiles_rows_over_tokens(_bf16_view(ctx, coffs[5] + 2 * slot * d * C, d * C))
            got["bKgT"] = _tiles_rows_over_tokens(_bf16_view(ctx, coffs[6] + 2 * slot * d * C, d * C))
            got["bet"] = _f32_view(ctx, coffs[1] + 4 * slot * C, C)[:L]
            # past the chunk end A is zero, so T continues as the identity there
            T_full = np.eye(C)
            T_full[:L, :L] = r["T"]
            ref.update({"bTT": T_full.T, "bMT": _pad(M_ref.T, C, C), "bKh": _pad(Kh, C, d),
                        "bQgT": _pad((Qv * Gam).T, d, C), "bKgT": _pad((Kv * Gam).T, d, C), "bet": bt})
            # state entering the chunk (state_swz layout: 16-byte vectors of row c permuted by c mod d/8)
            raw = _bf16_view(ctx, coffs[7] + 2 * slot * d * d, d * d).reshape(d, d // 8, 8)
            perm = (np.arange(d // 8)[None, :] ^ (np.arange(d)[:, None] % (d // 8)))
            got["S_in"] = np.take_along_axis(raw, perm[:, :, None], axis=1).reshape(d, d)
            ref["S_in"] = r["S_in"]
            got["Ut"] = Ug[c0:c1, h]
            ref["Ut"] = r["Ut"]
            # bf16 tiles: the 32-token halves that are zero by structure are
            # not stored (rows 0..31 x tokens 32..63 of the lower-triangular
            # T diag(beta) and M; rows 32..63 x tokens 0..31 of T^T and M^T);
            # the reference is zero there, so the unwritten bytes are left out
            for key in ("TB", "M"):
                got[key][:32, 32:] = 0.0
                assert not np.any(ref[key][:32, 32:])
            for key in ("bTT", "bMT"):
                got[key][32:, :32] = 0.0
                assert not np.any(ref[key][32:, :32])
            for key in ref:
                worst[key] = max(worst.get(key, 0.0), _err(got[key], ref[key]))
            # the inverse itself: (I + A) (T diag(beta)) = diag(beta)
            resid = (np.eye(L) + r["A"]) @ got["TB"][:L, :L] - np.diag(bt)
            worst["(I+A)TB-diag(beta)"] = max(worst.get("(I+A)TB-diag(beta)", 0.0),
                                              float(np.max(np.abs(resid)) / max(np.max(np.abs(bt)), 1e-30)))
    _say("%s H=%d d=%d: " % (lengths, H, d) + " ".join("%s=%.1e" % kv for kv in worst.items()))
    for key, e in worst.items():
        assert e <= TOL, "%s: %.3e > %.0e" % (key, e, TOL)
