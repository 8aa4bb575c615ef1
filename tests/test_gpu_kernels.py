"""Single-kernel parity on the GPU: the MFMA GEMMs (every epilogue, ragged
tiles, the decode-row kernel) and prefill attention on ragged packed
batches, each against a plain float64 definition on the same bf16 inputs."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import bf16_round, to_dev_bf16, torch

pytestmark = pytest.mark.gpu

B = pytest.importorskip("gpt_block_fwd_amd.binding")

GEMM_SHAPES = [
    # (M, N, K): several 256x256 tiles with ragged M, N = 4.5 tiles, odd tile counts
    # (the residual add takes 256x192 tiles where N splits into 192 columns)
    (300, 384, 192),
    (1000, 1152, 768),
    (513, 1920, 1664),
    # residual add on 192-column tiles (N = 768, 1152, 384), ragged M
    (700, 768, 3072),
    # 1, 2, 4 and 5 k-tiles of 64: every way the k loop can end (its
    # two-k-tile steady state, the tested tail pair, the last single
    # k-tile); N = 768 and 384 also take 192-column tiles for epilogues 2, 3
    (300, 256, 64),
    (520, 512, 128),
    (600, 768, 256),
    (260, 384, 320),
    # decode-row kernel (M <= 64): 1, 2, 3 and 4 row blocks, ragged M; 32-column
    # tiles where 64-column ones would number fewer than 128
    (1, 128, 64),
    (33, 768, 768),
    (64, 1024, 3072),
    (64, 1920, 1664),
    (17, 6656, 1664),
    (40, 384, 1152),
    # 64-column tiles: 160 and 512 of them
    (48, 10240, 768),
    (8, 32768, 256),
    # more 256x256 tiles than CUs, ragged in M and N: 9 x 33 tiles of 2
    # k-tiles, 6 x 50 of 5
    (2100, 8320, 128),
    (1300, 12800, 320),
]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
@pytest.mark.parametrize("epi", [0, 1, 2, 3])
def test_gemm_matches_float64(M, N, K, epi):
    t = torch()
    rng = np.random.default_rng(M * 7 + N + K + epi)
    A = bf16_round(rng.standard_normal((M, K)))
    W = bf16_round(rng.standard_normal((N, K)) * 0.05)
    ref = A.astype(np.float64) @ W.astype(np.float64).T
    dA, dW = to_dev_bf16(A), to_dev_bf16(W)
    if epi in (0, 1):
        C = t.empty((M, N), dtype=t.bfloat16, device="cuda")
    else:
        init = rng.standard_normal((M, N)).astype(np.float32) if epi == 2 else np.zeros((M, N), np.float32)
        C = t.from_numpy(init).cuda()
    B.gpt_debug_gemm(dA, dW, M, N, K, C, epi)
    t.cuda.synchronize()
    out = C.float().cpu().numpy().astype(np.float64)
    scale = np.sqrt(K) * 0.05
    if epi == 0:
        np.testing.assert_allclose(out, ref, rtol=2 ** -8, atol=1e-5 * scale)
    elif epi == 1:
        r2 = np.maximum(ref, 0) ** 2
        np.testing.assert_allclose(out, r2, rtol=2 ** -7, atol=1e-5 * scale ** 2)
    elif epi == 2:
        np.testing.assert_allclose(out, init + ref, rtol=1e-5, atol=1e-5 * scale)
    else:
        np.testing.assert_allclose(out, ref, rtol=1e-5, atol=1e-5 * scale)


@pytest.mark.parametrize("M,N,K,ks", [(32, 768, 768, 6), (64, 1664, 6656, 12), (17, 1024, 320, 2),
                                      (5, 128, 1024, 16), (64, 1920, 1664, 11)])
def test_gemm_rows_split_slabs(M, N, K, ks):
    """k split over workgroups: the slabs are partial products over disjoint k
    ranges (ragged: ranges differ by one 64-deep chunk) that sum to A W^T."""
    t = torch()
    rng = np.random.default_rng(M + N + K + ks)
    A = bf16_round(rng.standard_normal((M, K)))
    W = bf16_round(rng.standard_normal((N, K)) * 0.05)
    C = t.full((ks, M, N), float("nan"), dtype=t.float32, device="cuda")
    B.gpt_debug_gemm(to_dev_bf16(A), to_dev_bf16(W), M, N, K, C, 3, ks)
    t.cuda.synchronize()
    slabs = C.cpu().numpy().astype(np.float64)
    assert np.isfinite(slabs).all()  # every slab element written
    chunks = K // 64
    bounds = [kz * chunks // ks * 64 for kz in range(ks + 1)]
    for kz in range(ks):  # each slab is exactly its own k range
        k0, k1 = bounds[kz], bounds[kz + 1]
        ref = A[:, k0:k1].astype(np.float64) @ W[:, k0:k1].astype(np.float64).T
        np.testing.assert_allclose(slabs[kz], ref, rtol=1e-5, atol=1e-5 * np.sqrt(k1 - k0) * 0.05)
    ref = A.astype(np.float64) @ W.astype(np.float64).T
    np.testing.assert_allclose(slabs.sum(0), ref, rtol=1e-5, atol=1e-5 * np.sqrt(K) * 0.05)


def test_gemm_is_deterministic():
    t = torch()
    rng = np.random.default_rng(3)
    M, N, K = 777, 1024, 768
    dA = to_dev_bf16(bf16_round(rng.standard_normal((M, K))))
    dW = to_dev_bf16(bf16_round(rng.standard_normal((N, K)) * 0.05))
    outs = []
    for _ in range(2):
        C = t.empty((M, N), dtype=t.float32, device="cuda")
        B.gpt_debug_gemm(dA, dW, M, N, K, C, 3)
        outs.append(C.cpu().numpy())
    np.testing.assert_array_equal(outs[0], outs[1])


def _attn_case(lens, H, seed, qk_norm):
    rng = np.random.default_rng(seed)
    total = int(np.sum(lens))
    if qk_norm:  # unit-RMS q and k, as QK-norm leaves them
        q = oracle.rmsnorm(rng.standard_normal((total, H, 128)), 1e-6)
        k = oracle.rmsnorm(rng.standard_normal((total, 1, 128)), 1e-6)
    else:  # larger scores, and a drift along the sequence that keeps raising the row maxima
        q = rng.standard_normal((total, H, 128)) * 2.0
        k = rng.standard_normal((total, 1, 128)) * 2.0 + np.linspace(0, 3, total)[:, None, None]
    v = rng.standard_normal((total, 1, 128)) * 0.5
    return bf16_round(q), bf16_round(k), bf16_round(v)


@pytest.mark.parametrize("qk_norm", [1, 0])
@pytest.mark.parametrize("lens,H", [([1, 63, 64, 65, 300], 6), ([2048], 6), ([129, 7, 1000], 13),
                                    ([256], 1)])
def test_prefill_attention_matches_oracle(lens, H, qk_norm):
    t = torch()
    q, k, v = _attn_case(lens, H, seed=sum(lens) + H, qk_norm=qk_norm)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pads = [(L + 63) // 64 * 64 for L in lens]
    cu_pad = np.concatenate([[0], np.cumsum(pads)]).astype(np.int64)
    ldvt = int(cu_pad[-1])
    vt = np.full((128, ldvt), np.nan, np.float32)  # padding must never be read as data
    for b, L in enumerate(lens):
        # position i at column cu_pad[b] + (i with bits 2 and 3 swapped)
        i = np.arange(L)
        col = (i & ~15) | (((i >> 2) & 1) << 3) | (((i >> 3) & 1) << 2) | (i & 3)
        vt[:, cu_pad[b] + col] = v[cu[b]:cu[b + 1], 0, :].T
    dq = to_dev_bf16(q.reshape(len(q), -1))
    dk = to_dev_bf16(k.reshape(len(k), -1))
    dvt = to_dev_bf16(vt)
    cu_dev = t.zeros(2 * (len(lens) + 1), dtype=t.int32, device="cuda")
    o = t.empty((len(q), H * 128), dtype=t.bfloat16, device="cuda")
    B.gpt_debug_attn_prefill(dq, dk, dvt, ldvt, cu, len(lens), H, cu_dev, o, qk_norm=qk_norm)
    t.cuda.synchronize()
    got = o.float().cpu().numpy().reshape(len(q), H, 128)
    assert np.isfinite(got).all()
    for b in range(len(lens)):
        s = slice(cu[b], cu[b + 1])
        ref = oracle.causal_attention(q[s].astype(np.float64), k[s].astype(np.float64),
                                      v[s].astype(np.float64), 0)
        # error budget: P rounded to bf16 (2^-9 relative) and the bf16 output
        np.testing.assert_allclose(got[s], ref, atol=1.5e-2, rtol=1e-2)


# ---------------------------------------------------------------- Adam

@pytest.mark.parametrize("n,copy", [(1, True), (3, False), (4, True), (1_000_003, True), (4096, False)])
def test_adam_matches_oracle(n, copy):
    """Three chained Adam steps against the float64 oracle; the bf16 copy is
    the nearest-even rounding of the updated fp32 parameters."""
    t = torch()
    rng = np.random.default_rng(n)
    p = rng.normal(size=n).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    dp, dm_, dv = (t.from_numpy(a.copy()).cuda() for a in (p, m, v))
    pb = t.empty(n, dtype=t.bfloat16, device="cuda") if copy else None
    lr, b1, b2, eps = 2e-3, 0.85, 0.99, 1e-8
    rp, rm, rv = p.astype(np.float64), m.astype(np.float64), v.astype(np.float64)
    sm = np.zeros(n)  # the same running mean over |g|: the scale of m's terms where they cancel
    for step in (1, 2, 3):
        g = (rng.normal(size=n) * 10.0 ** rng.uniform(-4, 1, n)).astype(np.float32)
        B.gpt_adam_step(dp, t.from_numpy(g).cuda(), dm_, dv, pb, n, step, lr, b1, b2, eps)
        rp, rm, rv = oracle.adam_step(rp, g, rm, rv, step, lr, b1, b2, eps)
        sm = b1 * sm + (1 - b1) * np.abs(g.astype(np.float64))
    t.cuda.synchronize()
    gp, gm, gv = (a.cpu().numpy().astype(np.float64) for a in (dp, dm_, dv))
    assert np.all(np.abs(gm - rm) <= 2e-6 * sm)
    np.testing.assert_allclose(gv, rv, rtol=2e-6, atol=1e-30)  # positive terms: no cancellation
    # fp32 storage of p: a few ulps of p plus a relative error of the step
    np.testing.assert_allclose(gp, rp, rtol=0, atol=float(np.max(4 * np.spacing(np.abs(rp).astype(np.float32)))) + 1e-5 * lr)
    if copy:
        np.testing.assert_array_equal(pb.float().cpu().numpy(), oracle.round_bf16(gp).astype(np.float32))
