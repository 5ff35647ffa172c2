"""Kernel-level GPU checks: the bf16 GEMM family (matrix-core tiles, split-K, epilogues) against
plain float64 arithmetic, and the fused readout (LM head + ExitGate + commit) against the oracle
at the 8B LM-head shape."""
import numpy as np
import pytest
import torch

from adaptive_looped_denoising_amd import synth
from oracle import alodlm_oracle as orc
from tests.parity import log

pytestmark = pytest.mark.gpu

N_TILES = 65  # matrix-core tiles in the library's table (alodlm_diag_gemm force_tile 0 .. N_TILES - 1)
SHAPES = [(32, 4096, 2048), (256, 6144, 4096), (200, 1024, 512), (1, 128, 64), (77, 640, 384), (2048, 1024, 4096),
          (130, 4096, 12288), (32, 2048, 6144)]


def _bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


def _gemm(epi, A, Bm, C=None, act=None, splits=0, generic=0, tile=-1):
    from adaptive_looped_denoising_amd import binding as B
    M, K = A.shape
    N = Bm.shape[0]
    scratch = torch.empty(max(8 * M * N, 1), dtype=torch.float32, device="cuda")
    B.diag_gemm(epi, M, N, K, A.data_ptr(), Bm.data_ptr(), 0 if C is None else C.data_ptr(),
                0 if act is None else act.data_ptr(), scratch.data_ptr(), scratch.numel(), splits, generic,
                torch.cuda.current_stream().cuda_stream, tile)
    torch.cuda.synchronize()


def _ref(A, Bm):
    return A.double().numpy() @ Bm.double().numpy().T


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_store_and_resid(gpu_lib, M, N, K):
    log("gemm M=%d N=%d K=%d" % (M, N, K))
    A, Bm = _bf16((M, K), 1), _bf16((N, K), 2, 0.02)
    ref = _ref(A, Bm)
    scale = np.sqrt(K) * 0.02
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    _gemm(0, A.cuda(), Bm.cuda(), C=C)
    err = np.abs(C.cpu().numpy() - ref).max() / scale
    assert err < 2e-5, err
    C0 = torch.randn((M, N), generator=torch.Generator().manual_seed(3)).cuda()
    C1 = C0.clone()
    _gemm(1, A.cuda(), Bm.cuda(), C=C1)
    err = np.abs(C1.cpu().numpy() - (C0.cpu().double().numpy() + ref)).max() / scale
    assert err < 2e-5, err


@pytest.mark.parametrize("tile", range(N_TILES))
def test_gemm_every_tile(gpu_lib, tile):
    M, N, K = 300, 1024, 1024
    A, Bm = _bf16((M, K), 10), _bf16((N, K), 11, 0.02)
    ref = _ref(A, Bm)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    _gemm(0, A.cuda(), Bm.cuda(), C=C, tile=tile)
    assert np.abs(C.cpu().numpy() - ref).max() / (np.sqrt(K) * 0.02) < 2e-5
    F = 512
    Bg = _bf16((2 * F, K), 12, 0.05)
    act = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    _gemm(3, A.cuda(), Bg.cuda(), act=act, tile=tile, splits=1)  # the single-pass SwiGLU epilogue
    gu = _ref(A, Bg)
    g, u = gu[:, :F], gu[:, F:]
    refa = g / (1 + np.exp(-g)) * u
    err = np.abs(act.cpu().float().numpy() - refa) / (np.abs(refa) + 1e-2 * np.abs(refa).max())
    assert err.max() < 1.6e-2


@pytest.mark.parametrize("tile", range(N_TILES))
def test_softstat_every_tile(gpu_lib, tile):
    """LM-head readout statistics (entropy, log-sum-exp, argmax over the columns) of every tile,
    on a ragged shape, against float64 arithmetic on the same bf16 operands."""
    from adaptive_looped_denoising_amd import binding as B
    M, N, K = 77, 1000, 256
    A, Bm = _bf16((M, K), 20), _bf16((N, K), 21, 0.1)
    z = _ref(A, Bm)
    zmax = z.max(axis=1, keepdims=True)
    p = np.exp(z - zmax)
    S = p.sum(axis=1)
    lse = zmax[:, 0] + np.log(S)
    H = lse - (p * z).sum(axis=1) / S
    out = torch.empty((2, M), dtype=torch.float32, device="cuda")
    tok = torch.empty(M, dtype=torch.int32, device="cuda")
    scratch = torch.empty(4 * M * ((N + 63) // 64), dtype=torch.float32, device="cuda")
    Ad, Bd = A.cuda(), Bm.cuda()  # held until the asynchronous launch has finished
    B.diag_gemm(B.DIAG_SOFTSTAT, M, N, K, Ad.data_ptr(), Bd.data_ptr(), out.data_ptr(), tok.data_ptr(),
                scratch.data_ptr(), scratch.numel(), 0, 0, torch.cuda.current_stream().cuda_stream, tile)
    torch.cuda.synchronize()
    gH, glse = out.cpu().numpy()
    assert np.abs(gH - H).max() < 1e-4 and np.abs(glse - lse).max() < 1e-4
    top2 = np.sort(z, axis=1)[:, -2:]
    ok = (tok.cpu().numpy() == z.argmax(axis=1)) | (top2[:, 1] - top2[:, 0] < 1e-4)
    assert ok.all()


@pytest.mark.parametrize("M", [128, 129, 256, 257, 300, 384, 385])
def test_softstat_auto_tile_across_row_thresholds(gpu_lib, M):
    """The readout's automatic tile choice around its row thresholds (128 / 256 / 384)."""
    from adaptive_looped_denoising_amd import binding as B
    N, K = 1000, 256
    A, Bm = _bf16((M, K), 22), _bf16((N, K), 23, 0.1)
    z = _ref(A, Bm)
    zmax = z.max(axis=1, keepdims=True)
    p = np.exp(z - zmax)
    S = p.sum(axis=1)
    lse = zmax[:, 0] + np.log(S)
    H = lse - (p * z).sum(axis=1) / S
    out = torch.empty((2, M), dtype=torch.float32, device="cuda")
    tok = torch.empty(M, dtype=torch.int32, device="cuda")
    scratch = torch.empty(4 * M * ((N + 63) // 64), dtype=torch.float32, device="cuda")
    Ad, Bd = A.cuda(), Bm.cuda()
    B.diag_gemm(B.DIAG_SOFTSTAT, M, N, K, Ad.data_ptr(), Bd.data_ptr(), out.data_ptr(), tok.data_ptr(),
                scratch.data_ptr(), scratch.numel(), 0, 0, torch.cuda.current_stream().cuda_stream, -1)
    torch.cuda.synchronize()
    gH, glse = out.cpu().numpy()
    assert np.abs(gH - H).max() < 1e-4 and np.abs(glse - lse).max() < 1e-4
    top2 = np.sort(z, axis=1)[:, -2:]
    assert ((tok.cpu().numpy() == z.argmax(axis=1)) | (top2[:, 1] - top2[:, 0] < 1e-4)).all()


@pytest.mark.parametrize("tile", list(range(N_TILES)) + ["generic"])
def test_readout_sample_every_tile(gpu_lib, tile):
    """Gumbel-max draws of the LM-head kernel (every tile and the vector-ALU path), on a ragged
    shape, against argmax(z + g) with z in float64 on the same bf16 operands and g the oracle's own
    noise at the same counters.  A draw may differ only where the top two of z + g are within the
    fp32 accumulation error."""
    from adaptive_looped_denoising_amd import binding as B
    M, N, K = 77, 1000, 256
    seed, loop, step = 0x0123456789ABCDEF, 3, 41
    A, Bm = _bf16((M, K), 22), _bf16((N, K), 23, 0.1)
    z = _ref(A, Bm)
    bi = [(m // 50 + 1, (7 * m) % 50) for m in range(M)]
    G = np.stack([orc.gumbel_noise(seed, step, b, i, loop, N) for b, i in bi])
    want, gap = orc.gumbel_sample(z, G)
    rk = torch.tensor([64 * b + i for b, i in bi], dtype=torch.int32, device="cuda")
    tok = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    scratch = torch.empty(6 * M * ((N + 63) // 64) + 3 * M, dtype=torch.float32, device="cuda")
    Ad, Bd = A.cuda(), Bm.cuda()  # held until the asynchronous launch has finished
    B.diag_readout_sample(M, N, K, Ad.data_ptr(), Bd.data_ptr(), rk.data_ptr(), seed, loop, step, tok.data_ptr(),
                          scratch.data_ptr(), scratch.numel(), 1 if tile == "generic" else 0,
                          torch.cuda.current_stream().cuda_stream, -1 if tile == "generic" else tile)
    torch.cuda.synchronize()
    got = tok.cpu().numpy()
    ok = (got == want) | (gap < 1e-4)
    assert ok.all(), (np.nonzero(~ok)[0][:8], got[~ok][:8], want[~ok][:8])
    assert (got != z.argmax(axis=1)).sum() > M // 4   # the draws are not the argmax


@pytest.mark.parametrize("splits", [2, 4, 8])
def test_gemm_split_k_matches_single_pass(gpu_lib, splits):
    M, N, K = 96, 2048, 4096
    A, Bm = _bf16((M, K), 4).cuda(), _bf16((N, K), 5, 0.02).cuda()
    C1 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    C2 = torch.empty_like(C1)
    _gemm(0, A, Bm, C=C1, splits=1)
    _gemm(0, A, Bm, C=C2, splits=splits)
    ref = _ref(A.cpu(), Bm.cpu())
    for C in (C1, C2):
        assert np.abs(C.cpu().numpy() - ref).max() / (np.sqrt(K) * 0.02) < 2e-5
    # the fixed-order reduction is deterministic
    C3 = torch.empty_like(C1)
    _gemm(0, A, Bm, C=C3, splits=splits)
    assert torch.equal(C2, C3)


@pytest.mark.parametrize("M,F,K,splits", [(32, 6144, 2048, 0), (256, 12288, 4096, 0), (50, 384, 128, 0),
                                          (64, 1024, 4096, 4)])
def test_gemm_swiglu(gpu_lib, M, F, K, splits):
    A, Bm = _bf16((M, K), 6), _bf16((2 * F, K), 7, 0.05)
    act = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    _gemm(3, A.cuda(), Bm.cuda(), act=act, splits=splits)
    gu = _ref(A, Bm)
    g, u = gu[:, :F], gu[:, F:]
    ref = g / (1 + np.exp(-g)) * u
    got = act.cpu().float().numpy()
    err = np.abs(got - ref) / (np.abs(ref) + 1e-2 * np.abs(ref).max())
    assert err.max() < 1.6e-2, err.max()


def test_gemm_generic_matches(gpu_lib):
    M, N, K = 70, 300, 256
    A, Bm = _bf16((M, K), 8).cuda(), _bf16((N, K), 9, 0.02).cuda()
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    _gemm(0, A, Bm, C=C, generic=1)
    assert np.abs(C.cpu().numpy() - _ref(A.cpu(), Bm.cpu())).max() / (16 * 0.02) < 2e-5


@pytest.mark.parametrize("n_rows", synth.READOUT_ROWS)
def test_readout_commit_at_8b_vocab(gpu_lib, n_rows):
    """LM head 4096 x 151936 + ExitGate + commit rule on rows standing for post-RMSNorm states,
    grouped into sequences of 32; every row of the first group and a row sample of the rest is
    recomputed by the oracle in float64."""
    from adaptive_looped_denoising_amd.engine import Engine
    w = synth.readout_workload(n_rows)
    log("readout n_rows=%d" % n_rows)
    e = Engine(w)
    rows = synth.readout_rows(n_rows)
    bt, bv = synth.boosts(w)
    bt, bv = bt.reshape(-1), bv.reshape(-1)
    rows_d = torch.from_numpy(rows.view(np.int16)).cuda().view(torch.bfloat16)
    bt_d, bv_d = torch.from_numpy(bt).cuda(), torch.from_numpy(bv).cuda()  # alive until the launch finishes
    out = e.readout_commit(rows_d, synth.READOUT_GROUP if n_rows >= 32 else n_rows, w.tau_ent, w.tau_halt, bt_d, bv_d)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in out.items()}
    W = {k: synth.as_f32(v) for k, v in synth.host_weights(w, ["lm_head", "embed", "exit_w"]).items()}
    r = synth.as_f32(rows)
    group = list(range(min(32, n_rows)))
    sample = sorted(set(group) | set(range(0, n_rows, max(1, n_rows // 16))))
    og = orc.readout_commit_group(r[group], W["lm_head"], W["embed"], W["exit_w"], e.exit_b, w.tau_ent,
                                  w.tau_halt, bt[group], bv[group])
    H, tok, lse, gap = orc.readout(r[sample], W["lm_head"], bt[sample], bv[sample])
    lam = orc.exit_gate(r[sample], W["exit_w"], e.exit_b)
    assert np.abs(got["entropy"][sample] - H).max() < 1e-2
    assert np.abs(got["lse"][sample] - lse).max() < 1e-3 * np.abs(lse).max()
    assert np.abs(got["lam"][sample] - lam).max() < 1e-4
    mism = got["argmax"][sample] != tok
    assert (gap[mism] < 1e-2).all()
    # the first group's decisions: commits, forced progress, Eq. 3 rows
    near = (np.abs(og["H"] - w.tau_ent) < 1e-2).any() or (og["forced"] >= 0 and np.sort(og["H"])[1] -
                                                           np.sort(og["H"])[0] < 1e-2)
    if not near:
        assert np.array_equal(got["commit_loop"][group], og["commit_loop"])
        committed = og["commit_loop"] != 0
        assert np.array_equal(got["tokens"][group][committed], og["tok"][committed])
        np.testing.assert_array_equal(got["embed"][group], og["embed_rows"].astype(np.float32))
        np.testing.assert_allclose(got["halt"][group], og["a"], atol=1e-4)
    log("readout n=%d: H err %.2e, commits %d, forced %d" % (n_rows, np.abs(got["entropy"][sample] - H).max(),
                                                               int((got["commit_loop"] > 0).sum()),
                                                               int((got["commit_loop"] < 0).sum())))
