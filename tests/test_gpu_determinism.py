"""Bitwise repeat-run determinism of the kernels whose results combine
partial work from several workgroups or lanes: prefill attention, the whole
prefill (GEMMs, attention, LSE), decode attention with its cross-chunk
merge, argmax and sampling.  Each case runs twice on identical inputs and
the outputs must be bit-identical (no atomics or arrival-order-dependent
sums decide a value)."""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import bf16_round, to_dev, to_dev_bf16, torch

pytestmark = pytest.mark.gpu

B = pytest.importorskip("gpt_block_fwd_amd.binding")


def test_prefill_attention_bitwise_repeatable():
    """Ragged sequences up to 2048 positions, 13 query heads on one K/V head."""
    t = torch()
    rng = np.random.default_rng(21)
    lens = [2048, 1000, 129, 1]
    H = 13
    total = int(np.sum(lens))
    # unit-RMS heads, as QK-norm leaves them
    q = bf16_round(oracle.rmsnorm(rng.standard_normal((total, H, 128)), 1e-6))
    k = bf16_round(oracle.rmsnorm(rng.standard_normal((total, 128)), 1e-6))
    v = rng.standard_normal((total, 128)) * 0.5
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pad = sum((n + 63) // 64 * 64 for n in lens)
    vt = np.zeros((128, pad), np.float32)
    col = 0
    for b, n in enumerate(lens):
        # columns of a sequence in the kernel's V^T order (bits 2 and 3 of
        # the position swapped within each 16-position group)
        p = np.arange(n)
        perm = (p & ~15) | (((p >> 2) & 1) << 3) | (((p >> 3) & 1) << 2) | (p & 3)
        vt[:, col + perm] = v[cu[b]:cu[b + 1]].T
        col += (n + 63) // 64 * 64
    dq, dk, dvt = to_dev_bf16(q.reshape(total, -1)), to_dev_bf16(k), to_dev_bf16(bf16_round(vt))
    cu_dev = t.empty(2 * len(lens) + 2, dtype=t.int32, device="cuda")
    outs = []
    for _ in range(2):
        o = t.empty((total, H * 128), dtype=t.bfloat16, device="cuda")
        B.gpt_debug_attn_prefill(dq, dk, dvt, pad, cu, len(lens), H, cu_dev, o)
        t.cuda.synchronize()
        outs.append(o.view(t.int16).cpu().numpy())
    np.testing.assert_array_equal(outs[0], outs[1])


def test_whole_prefill_bitwise_repeatable():
    """GEMMs (large-M tiles, fused epilogues), attention, LM-head partials and
    the LSE merge over 3 ragged sequences of a 2-layer bf16 model."""
    t = torch()
    cfg = wl.small_model(2, 6, vocab=8192, max_seq=2048)
    w = wl.ragged_prefill(cfg, [700, 1500, 65], seed=3)
    dm = B.DeviceModel(cfg, wl.make_weights(cfg, 3))
    M = int(w.cu_seqlens[-1])
    tok = to_dev(w.tokens)
    res = []
    for _ in range(2):
        lg = t.empty((M, cfg.vocab), dtype=t.float32, device="cuda")
        lse = t.empty(M, dtype=t.float32, device="cuda")
        dm.prefill(tok, w.cu_seqlens, lg, lse)
        t.cuda.synchronize()
        res.append((lg.cpu().numpy(), lse.cpu().numpy()))
    np.testing.assert_array_equal(res[0][0], res[1][0])
    np.testing.assert_array_equal(res[0][1], res[1][1])


@pytest.mark.parametrize("temperature", [0.0, 0.7])
def test_decode_step_bitwise_repeatable(temperature):
    """64 sequences of 64 to 2400 cached positions (several chunks per
    sequence, merged by the last chunk to finish, whose identity varies from
    run to run): re-prefilling the same prompts and decoding two steps gives
    bit-identical logits and tokens."""
    t = torch()
    cfg = wl.small_model(2, 13, vocab=4096, max_seq=2560)
    rng = np.random.default_rng(17)
    lens = rng.integers(64, 2401, size=64)
    lens[0], lens[1] = 2400, 64
    w = wl.ragged_prefill(cfg, lens, seed=5)
    dm = B.DeviceModel(cfg, wl.make_weights(cfg, 5))
    n = w.n_seqs
    kv = B.DeviceKV(dm, n, 2560)
    tok = to_dev(w.tokens)
    U = to_dev(rng.random((3, n)).astype(np.float32))
    pws, dws = dm.workspace(int(w.cu_seqlens[-1]), n), dm.workspace(n, n)
    runs = []
    for _ in range(2):
        first = t.empty((n, cfg.vocab), dtype=t.float32, device="cuda")
        dm.prefill(tok, w.cu_seqlens, first, kv=kv.handle, logits_rows=B.ROWS_LAST, workspace=pws)
        ids = t.empty(n, dtype=t.int32, device="cuda")
        B.gpt_select_tokens(first, n, cfg.vocab, temperature, U[0] if temperature > 0 else None, ids)
        out = []
        for s in range(2):
            lg = t.empty((n, cfg.vocab), dtype=t.float32, device="cuda")
            nxt = t.empty(n, dtype=t.int32, device="cuda")
            dm.decode_step(kv.handle, ids, nxt, temperature=temperature,
                           uniforms=U[s + 1] if temperature > 0 else None, logits=lg, workspace=dws)
            ids = nxt
            out.append((lg.cpu().numpy(), nxt.cpu().numpy()))
        t.cuda.synchronize()
        runs.append(out)
    for s in range(2):
        np.testing.assert_array_equal(runs[0][s][0], runs[1][s][0])
        np.testing.assert_array_equal(runs[0][s][1], runs[1][s][1])
    kv.close()


@pytest.mark.parametrize("temperature", [0.0, 0.7])
def test_selection_bitwise_repeatable(temperature):
    t = torch()
    rng = np.random.default_rng(4)
    rows, V = 96, 65536
    lg = t.from_numpy((rng.standard_normal((rows, V)) * 0.8).astype(np.float32)).cuda()
    U = t.from_numpy(rng.random(rows).astype(np.float32)).cuda()
    outs = []
    for _ in range(2):
        o = t.empty(rows, dtype=t.int32, device="cuda")
        B.gpt_select_tokens(lg, rows, V, temperature, U if temperature > 0 else None, o)
        outs.append(o.cpu().numpy())
    np.testing.assert_array_equal(outs[0], outs[1])
