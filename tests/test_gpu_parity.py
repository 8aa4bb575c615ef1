"""End-to-end parity of the HIP path (through the C ABI) against the oracle.

fp32 tiny model: max |logit diff| <= 1e-4 and greedy ids bit-exact.
bf16 models: max |logit diff| <= 3e-2; top-1 agreement is reported, and
every row where the GPU's choice differs from the oracle's argmax must be
explained by that row's own logit errors (the bf16 storage noise floor on
near-flat random-weight logits makes a literal 99.9% top-1 bar unreachable
for any bf16-operand path; tests/test_gpu_fullsize.py measures that floor).
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import logit_stats, to_dev, torch

pytestmark = pytest.mark.gpu

B = pytest.importorskip("gpt_block_fwd_amd.binding")

_models = {}


def device_model(cfg, seed=0):
    key = (cfg, seed)
    if key not in _models:
        W = wl.make_weights(cfg, seed)
        _models[key] = (W, B.DeviceModel(cfg, W))
    return _models[key]


def gpu_prefill(dm, tokens, seqlens, rows=B.ROWS_ALL, kv=None, want_probs=False):
    t = torch()
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    n_rows = int(cu[-1]) if rows == B.ROWS_ALL else len(seqlens)
    V = dm.model.vocab
    logits = t.empty((n_rows, V), dtype=t.float32, device="cuda")
    lse = t.empty(n_rows, dtype=t.float32, device="cuda")
    probs = t.empty((n_rows, V), dtype=t.float32, device="cuda") if want_probs else None
    dtok = to_dev(np.asarray(tokens, np.int32))
    dm.prefill(dtok, cu, logits, lse, probs, kv=kv, logits_rows=rows)
    t.cuda.synchronize()
    out = (logits.cpu().numpy(), lse.cpu().numpy())
    if want_probs:
        out = out + (probs.cpu().numpy(),)
    return out


# ---------------------------------------------------------------- fp32 tiny

def test_tiny_prefill_fp32():
    w = wl.tiny_workload()
    W, dm = device_model(w.model)
    logits, lse, probs = gpu_prefill(dm, w.tokens, w.seqlens, want_probs=True)
    ref, _ = oracle.prefill(w.model, W, w.tokens, w.seqlens)
    ref = np.concatenate(ref)
    assert np.max(np.abs(logits - ref)) <= 1e-4
    # greedy ids: both decisions taken on fp32 logits
    np.testing.assert_array_equal(np.argmax(logits, -1), np.argmax(ref.astype(np.float32), -1))
    np.testing.assert_allclose(lse, oracle.logsumexp(ref), atol=1e-4)
    np.testing.assert_allclose(probs, oracle.softmax(ref), atol=1e-5)
    np.testing.assert_allclose(probs.sum(-1), 1.0, atol=1e-5)


def test_tiny_greedy_decode_fp32():
    """Prefill the BOS-started prompts' first 4 tokens, then greedy-decode to
    16 positions; ids must equal the oracle's bit for bit."""
    t = torch()
    w = wl.tiny_workload()
    cfg = w.model
    W, dm = device_model(cfg)
    n, p0, steps = 8, 4, 11
    prompts = w.tokens.reshape(8, 16)[:, :p0].reshape(-1)
    seqlens = np.full(n, p0)
    kv = B.DeviceKV(dm, n, 16)
    logits, _ = gpu_prefill(dm, prompts, seqlens, rows=B.ROWS_LAST, kv=kv.handle)
    assert (kv.lengths() == p0).all()
    dlog = t.from_numpy(logits).cuda()
    toks = t.empty(n, dtype=t.int32, device="cuda")
    B.gpt_select_tokens(dlog, n, cfg.vocab, 0.0, None, toks)
    ws = dm.workspace(n, n)
    got_tok = [toks.cpu().numpy().copy()]
    got_logits = [logits]
    step_logits = t.empty((n, cfg.vocab), dtype=t.float32, device="cuda")
    for _ in range(steps):
        dm.decode_step(kv.handle, toks, toks, logits=step_logits, workspace=ws)
        got_tok.append(toks.cpu().numpy().copy())
        got_logits.append(step_logits.cpu().numpy().copy())
    assert (kv.lengths() == p0 + steps).all()
    chosen, ref_logits = oracle.run_serving(cfg, W, prompts, seqlens, steps)
    np.testing.assert_array_equal(np.stack(got_tok), chosen)
    assert np.max(np.abs(np.stack(got_logits) - ref_logits)) <= 1e-4
    kv.close()


# ---------------------------------------------------------------- bf16 small models

@pytest.mark.parametrize("n_layer,n_head,lens", [(1, 1, [64]), (2, 2, [300, 173, 64, 1]),
                                                (2, 6, [513, 70])])
def test_small_bf16_prefill(n_layer, n_head, lens):
    cfg = wl.small_model(n_layer, n_head, vocab=4096)
    w = wl.ragged_prefill(cfg, lens, seed=n_layer + n_head)
    W, dm = device_model(cfg)
    logits, lse, probs = gpu_prefill(dm, w.tokens, w.seqlens, want_probs=True)
    ref, _ = oracle.prefill(cfg, W, w.tokens, w.seqlens)
    ref = np.concatenate(ref)
    st = logit_stats(logits, ref)
    print(st)
    assert st["max_abs"] <= 3e-2
    assert st["rows_explained"], st
    np.testing.assert_allclose(lse, oracle.logsumexp(ref), atol=3e-2)
    # the softmax outputs are distributions consistent with the GPU's own logits
    lg = logits.astype(np.float64)
    np.testing.assert_allclose(lse, oracle.logsumexp(lg), atol=2e-5)
    np.testing.assert_allclose(probs, oracle.softmax(lg), atol=2e-6)
    np.testing.assert_allclose(probs.sum(-1), 1.0, atol=1e-4)


def test_small_bf16_prefill_last_rows_and_cache():
    """ROWS_LAST returns each sequence's last row of the ROWS_ALL logits (up to
    fp32 summation order: few rows run the LM head on the decode-row GEMM),
    and writing the cache changes nothing."""
    cfg = wl.small_model(2, 2, vocab=4096)
    w = wl.ragged_prefill(cfg, [100, 37, 200], seed=5)
    W, dm = device_model(cfg)
    full, _ = gpu_prefill(dm, w.tokens, w.seqlens)
    kv = B.DeviceKV(dm, 3, 256)
    last, _ = gpu_prefill(dm, w.tokens, w.seqlens, rows=B.ROWS_LAST, kv=kv.handle)
    cu = w.cu_seqlens
    np.testing.assert_allclose(last, full[cu[1:] - 1], rtol=0, atol=2e-6)
    np.testing.assert_array_equal(kv.lengths(), w.seqlens)
    kv.close()


# ---------------------------------------------------------------- next-token cross-entropy

def gpu_loss(dm, tokens, seqlens, targets):
    t = torch()
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    M = int(cu[-1])
    loss = t.full((M,), float("nan"), dtype=t.float32, device="cuda")
    lse = t.empty(M, dtype=t.float32, device="cuda")
    mean = t.empty(1, dtype=t.float32, device="cuda")
    dm.prefill_loss(to_dev(np.asarray(tokens, np.int32)), to_dev(np.asarray(targets, np.int32)), cu,
                    loss, lse, mean)
    t.cuda.synchronize()
    return loss.cpu().numpy(), lse.cpu().numpy(), float(mean.cpu().numpy()[0])


def test_tiny_loss_fp32():
    """Per-row losses, lse and the mean of the tiny model against the oracle,
    with each sequence's last row (no next token) left out."""
    w = wl.tiny_workload()
    W, dm = device_model(w.model)
    tg = w.next_token_targets()
    loss, lse, mean = gpu_loss(dm, w.tokens, w.seqlens, tg)
    ref = np.concatenate(oracle.prefill(w.model, W, w.tokens, w.seqlens)[0])
    rl = oracle.token_losses(ref, tg)
    assert np.max(np.abs(loss - rl)) <= 1e-4
    assert (loss[tg < 0] == 0).all()
    np.testing.assert_allclose(lse, oracle.logsumexp(ref), atol=1e-4)
    assert abs(mean - oracle.mean_loss(rl, tg, w.model.vocab)) <= 1e-4


@pytest.mark.parametrize("n_layer,n_head,lens", [(2, 2, [300, 173, 64, 1]), (1, 1, [40, 9]),
                                                (2, 6, [513, 70])])
def test_small_bf16_loss(n_layer, n_head, lens):
    """bf16: losses within the logit bar of the oracle's, and equal to
    lse - logit[target] of the same prefill's materialised logits (the fused
    epilogue keeps the very accumulators the logits path stores).  Rows with
    a target of -1, -5 or vocab are skipped; 49 rows take the unfused path."""
    cfg = wl.small_model(n_layer, n_head, vocab=4096)
    w = wl.ragged_prefill(cfg, lens, seed=n_layer + 3 * n_head)
    W, dm = device_model(cfg)
    tg = w.next_token_targets()
    tg[3] = cfg.vocab
    tg[5] = -5
    loss, lse, mean = gpu_loss(dm, w.tokens, w.seqlens, tg)
    ok = (tg >= 0) & (tg < cfg.vocab)
    assert (loss[~ok] == 0).all()
    ref = np.concatenate(oracle.prefill(cfg, W, w.tokens, w.seqlens)[0])
    rl = oracle.token_losses(ref, tg)
    d = np.abs(loss - rl)
    print("loss max |diff|", float(d.max()), "std", float(np.std(loss[ok] - rl[ok])))
    assert d.max() <= 3e-2
    logits, lse2 = gpu_prefill(dm, w.tokens, w.seqlens)
    np.testing.assert_array_equal(lse, lse2)
    rows = np.nonzero(ok)[0]
    own = lse2[rows].astype(np.float64) - logits[rows, tg[rows]]
    np.testing.assert_allclose(loss[rows], own, rtol=0, atol=2e-6)
    assert abs(mean - float(np.mean(loss[rows].astype(np.float64)))) <= 1e-6
    # no counted row: the mean is 0
    _, _, m0 = gpu_loss(dm, w.tokens, w.seqlens, np.full_like(tg, -1))
    assert m0 == 0.0


def test_lm_head_persistent_ragged_tiles():
    """The LM head's persistent grid (one workgroup per CU walking the tiles,
    each tile's first loads issued before the previous tile's epilogue):
    2229 rows and a 16512-entry vocabulary give 9 x 65 = 585 tiles of
    256 x 256, with a partial last row of tiles and a half-empty last column
    of tiles, so workgroups take two or three tiles and some follow a
    partial one.  Logits, lse and softmax against the oracle; the fused
    cross-entropy against the same prefill's logits."""
    cfg = wl.small_model(1, 1, vocab=16512)
    w = wl.ragged_prefill(cfg, [1500, 700, 29], seed=11)
    W, dm = device_model(cfg)
    logits, lse, probs = gpu_prefill(dm, w.tokens, w.seqlens, want_probs=True)
    ref = np.concatenate(oracle.prefill(cfg, W, w.tokens, w.seqlens)[0])
    st = logit_stats(logits, ref)
    print(st)
    assert st["max_abs"] <= 3e-2
    assert st["rows_explained"], st
    lg = logits.astype(np.float64)
    np.testing.assert_allclose(lse, oracle.logsumexp(lg), atol=2e-5)
    np.testing.assert_allclose(probs, oracle.softmax(lg), atol=2e-6)
    tg = w.next_token_targets()
    tg[7] = cfg.vocab - 1          # the last column, in the half-empty tile
    tg[2228 - 1] = 16384           # the first column of that tile
    loss, lse2, _ = gpu_loss(dm, w.tokens, w.seqlens, tg)
    np.testing.assert_array_equal(lse, lse2)
    rows = np.nonzero(tg >= 0)[0]
    own = lse2[rows].astype(np.float64) - logits[rows, tg[rows]]
    np.testing.assert_allclose(loss[rows], own, rtol=0, atol=2e-6)


@pytest.mark.parametrize("temperature", [0.0, 0.7])
def test_small_bf16_decode_teacher_forced(temperature):
    """Prefill ragged prompts into the paged cache, decode 40 steps crossing
    page and chunk boundaries; the oracle consumes the GPU's tokens."""
    t = torch()
    cfg = wl.small_model(2, 2, vocab=4096)
    lens = [250, 63, 1, 130]
    w = wl.ragged_prefill(cfg, lens, seed=9)
    W, dm = device_model(cfg)
    n, steps = len(lens), 40
    kv = B.DeviceKV(dm, n, 320)
    logits0, _ = gpu_prefill(dm, w.tokens, w.seqlens, rows=B.ROWS_LAST, kv=kv.handle)
    rng = np.random.default_rng(4)
    U = rng.random((steps + 1, n)).astype(np.float32)
    toks = t.empty(n, dtype=t.int32, device="cuda")
    dU = t.from_numpy(U).cuda()
    B.gpt_select_tokens(t.from_numpy(logits0).cuda(), n, cfg.vocab, temperature, dU[0], toks)
    ws = dm.workspace(n, n)
    step_logits = t.empty((n, cfg.vocab), dtype=t.float32, device="cuda")
    got_tok, got_logits = [toks.cpu().numpy().copy()], [logits0]
    for s in range(steps):
        dm.decode_step(kv.handle, toks, toks, temperature=temperature, uniforms=dU[s + 1],
                       logits=step_logits, workspace=ws)
        got_tok.append(toks.cpu().numpy().copy())
        got_logits.append(step_logits.cpu().numpy().copy())
    got_tok = np.stack(got_tok)
    _, ref_logits = oracle.run_serving(cfg, W, w.tokens, w.seqlens, steps, forced=got_tok)
    st = logit_stats(np.stack(got_logits), ref_logits, chosen=got_tok if temperature <= 0 else None)
    print(st)
    assert st["max_abs"] <= 3e-2
    assert st["rows_explained"], st
    # every chosen token is a valid choice for the GPU's own logits
    for s in range(steps + 1):
        for j in range(n):
            lg = np.asarray(got_logits[s][j], np.float64)
            if temperature <= 0:
                assert got_tok[s, j] == int(np.argmax(got_logits[s][j]))
            else:
                c = np.cumsum(oracle.softmax(lg / temperature))
                k = got_tok[s, j]
                lo = c[k - 1] if k > 0 else 0.0
                assert lo - 1e-5 <= U[s, j] <= c[k] + 1e-5
    np.testing.assert_array_equal(kv.lengths(), np.asarray(lens) + steps)
    kv.close()


# ---------------------------------------------------------------- grouped-query attention

@pytest.mark.parametrize("n_head,n_kv,lens", [(6, 2, [300, 173, 64, 1]), (4, 4, [257, 90]),
                                              (6, 3, [40, 9]), (2, 2, [700])])
def test_small_bf16_gqa_prefill(n_head, n_kv, lens):
    """Grouped-query attention (n_kv K/V heads, each shared by n_head / n_kv
    query heads; n_kv = n_head is multi-head) through the whole prefill;
    49 rows take the small-M path with its separate RoPE/norm scatter."""
    cfg = wl.small_model(2, n_head, vocab=4096, n_kv_head=n_kv)
    w = wl.ragged_prefill(cfg, lens, seed=n_head + 7 * n_kv)
    W, dm = device_model(cfg)
    logits, lse = gpu_prefill(dm, w.tokens, w.seqlens)
    ref = np.concatenate(oracle.prefill(cfg, W, w.tokens, w.seqlens)[0])
    st = logit_stats(logits, ref)
    print(st)
    assert st["max_abs"] <= 3e-2
    assert st["rows_explained"], st
    np.testing.assert_allclose(lse, oracle.logsumexp(ref), atol=3e-2)


@pytest.mark.parametrize("n_head,n_kv,n_seqs", [(6, 2, 4), (4, 4, 3), (6, 3, 40)])
def test_small_bf16_gqa_decode_teacher_forced(n_head, n_kv, n_seqs):
    """Prefill into the paged cache, then 20 greedy decode steps with GQA; the
    oracle consumes the GPU's tokens.  (6, 3, 40): 240 decode-attention
    workgroups of one page per wave."""
    t = torch()
    cfg = wl.small_model(2, n_head, vocab=4096, n_kv_head=n_kv)
    rng = np.random.default_rng(n_seqs)
    lens = [int(x) for x in rng.integers(1, 300, n_seqs)]
    lens[0] = 255  # the first decode position opens a new page
    w = wl.ragged_prefill(cfg, lens, seed=n_head * n_kv)
    W, dm = device_model(cfg)
    n, steps = n_seqs, 20
    kv = B.DeviceKV(dm, n, 320)
    logits0, _ = gpu_prefill(dm, w.tokens, w.seqlens, rows=B.ROWS_LAST, kv=kv.handle)
    toks = t.empty(n, dtype=t.int32, device="cuda")
    B.gpt_select_tokens(t.from_numpy(logits0).cuda(), n, cfg.vocab, 0.0, None, toks)
    ws = dm.workspace(n, n)
    step_logits = t.empty((n, cfg.vocab), dtype=t.float32, device="cuda")
    got_tok, got_logits = [toks.cpu().numpy().copy()], [logits0]
    for s in range(steps):
        dm.decode_step(kv.handle, toks, toks, logits=step_logits, workspace=ws)
        got_tok.append(toks.cpu().numpy().copy())
        got_logits.append(step_logits.cpu().numpy().copy())
    got_tok = np.stack(got_tok)
    sample = [0, n - 1]
    _, ref_logits = oracle.run_serving(cfg, W, w.tokens, w.seqlens, steps, forced=got_tok,
                                       seqs=sample)
    st = logit_stats(np.stack(got_logits)[:, sample], ref_logits, chosen=got_tok[:, sample])
    print(st)
    assert st["max_abs"] <= 3e-2
    assert st["rows_explained"], st
    for s in range(steps + 1):
        np.testing.assert_array_equal(got_tok[s], np.argmax(got_logits[s], axis=-1))
    np.testing.assert_array_equal(kv.lengths(), np.asarray(lens) + steps)
    kv.close()


def decode_chunk_pages(lens, n_kv_head=1):
    """The decode step's chunk size for these cached lengths, as the library
    picks it: the fewest pages per chunk (1 .. 16) for which the chunks that
    hold positions (the new one included) number at most 256.  (The library
    also keeps at least ceil(longest / partial-buffer splits) pages, at most
    2 with max_seq >= the longest sequence, which these cases never reach.)"""
    pages = [(int(n) + 1 + 63) // 64 for n in lens]
    chunk = 1
    while chunk < 16 and sum(-(-p // chunk) for p in pages) * n_kv_head > 256:
        chunk += 1
    return chunk


@pytest.mark.parametrize("n_head,n_kv,cap,chunk", [(7, 1, 1250, 4), (2, 1, 2100, 6), (2, 1, 2900, 8),
                                                   (2, 1, 3600, 9), (2, 1, 6400, 16), (4, 2, 1100, 7),
                                                   (4, 2, 1650, 10)])
def test_small_bf16_decode_many_sequences(n_head, n_kv, cap, chunk):
    """64 sequences of up to `cap` positions: the decode-attention chunks
    grow with the total length.  Chunks of up to 4 pages run on four waves
    that stage K and V^T in LDS (cap 1250: every wave busy); 5 to 8 pages on
    eight waves that stage K and hold V^T in registers (cap 2100: two waves
    idle; cap 2900: all busy), and 9 to 16 pages on those eight waves in two
    rounds with the online softmax across them (cap 3600: one wave takes a
    second page; cap 6400: all do).  7 heads (cap 1250): the 9 q/k/v slots of
    the owning chunk take two passes of the four waves' 8 half-waves.  Two
    K/V heads (4 query heads): a workgroup per chunk and K/V head, so the
    chunks double in count and the eight-wave shapes are reached at shorter
    lengths, one and two rounds.  3 greedy steps, the longest and the
    shortest sequence teacher-forced through the oracle."""
    t = torch()
    cfg = wl.small_model(2, n_head, vocab=4096, max_seq=max(cap, 4096), n_kv_head=n_kv)
    rng = np.random.default_rng(21)
    lens = rng.integers(1, cap - 10, size=64)
    lens[0], lens[1] = cap - 11, 1
    # the chunk size this case is meant to reach, on every step
    for s_ in range(3):
        assert decode_chunk_pages(lens + s_, n_kv) == chunk
    w = wl.ragged_prefill(cfg, lens, seed=21)
    W, dm = device_model(cfg)
    n, steps = len(lens), 3
    kv = B.DeviceKV(dm, n, cap)
    logits0, _ = gpu_prefill(dm, w.tokens, w.seqlens, rows=B.ROWS_LAST, kv=kv.handle)
    toks = t.empty(n, dtype=t.int32, device="cuda")
    B.gpt_select_tokens(t.from_numpy(logits0).cuda(), n, cfg.vocab, 0.0, None, toks)
    ws = dm.workspace(n, n)
    step_logits = t.empty((n, cfg.vocab), dtype=t.float32, device="cuda")
    got_tok, got_logits = [toks.cpu().numpy().copy()], [logits0]
    for _ in range(steps):
        dm.decode_step(kv.handle, toks, toks, logits=step_logits, workspace=ws)
        got_tok.append(toks.cpu().numpy().copy())
        got_logits.append(step_logits.cpu().numpy().copy())
    np.testing.assert_array_equal(kv.lengths(), w.seqlens + steps)
    kv.close()
    got_tok = np.stack(got_tok)
    sample = [0, 1]
    _, ref = oracle.run_serving(cfg, W, w.tokens, w.seqlens, steps, forced=got_tok, seqs=sample)
    st = logit_stats(np.stack(got_logits)[:, sample], ref, chosen=got_tok[:, sample])
    print(st)
    assert st["max_abs"] <= 3e-2
    assert st["rows_explained"], st
    for s_ in range(1, steps + 1):  # greedy: every sequence's token is its own argmax
        np.testing.assert_array_equal(got_tok[s_], np.argmax(got_logits[s_], axis=-1))


@pytest.mark.parametrize("n_seqs", [65, 130])
def test_small_bf16_decode_beyond_64_sequences(n_seqs):
    """More than 64 sequences per step take the large-tile GEMMs (residual
    adds in the GEMM epilogue, RMSNorm on its own, the large-M LM head) and
    feed decode attention an unsplit QKV projection.  6 greedy steps; the
    first, the 65th and the last sequence are teacher-forced through the
    oracle."""
    t = torch()
    cfg = wl.small_model(2, 2, vocab=4096)
    rng = np.random.default_rng(n_seqs)
    lens = rng.integers(1, 600, size=n_seqs)
    lens[0], lens[64] = 599, 1
    w = wl.ragged_prefill(cfg, lens, seed=n_seqs)
    W, dm = device_model(cfg)
    n, steps = n_seqs, 6
    kv = B.DeviceKV(dm, n, 640)
    logits0, _ = gpu_prefill(dm, w.tokens, w.seqlens, rows=B.ROWS_LAST, kv=kv.handle)
    toks = t.empty(n, dtype=t.int32, device="cuda")
    B.gpt_select_tokens(t.from_numpy(logits0).cuda(), n, cfg.vocab, 0.0, None, toks)
    ws = dm.workspace(n, n)
    step_logits = t.empty((n, cfg.vocab), dtype=t.float32, device="cuda")
    got_tok, got_logits = [toks.cpu().numpy().copy()], [logits0]
    for _ in range(steps):
        dm.decode_step(kv.handle, toks, toks, logits=step_logits, workspace=ws)
        got_tok.append(toks.cpu().numpy().copy())
        got_logits.append(step_logits.cpu().numpy().copy())
    np.testing.assert_array_equal(kv.lengths(), w.seqlens + steps)
    kv.close()
    got_tok = np.stack(got_tok)
    sample = [0, 64, n - 1]
    _, ref = oracle.run_serving(cfg, W, w.tokens, w.seqlens, steps, forced=got_tok, seqs=sample)
    st = logit_stats(np.stack(got_logits)[:, sample], ref, chosen=got_tok[:, sample])
    print(st)
    assert st["max_abs"] <= 3e-2
    assert st["rows_explained"], st
    for s_ in range(1, steps + 1):
        np.testing.assert_array_equal(got_tok[s_], np.argmax(got_logits[s_], axis=-1))


def test_decode_capacity_error():
    t = torch()
    cfg = wl.small_model(1, 1, vocab=1024)
    W, dm = device_model(cfg)
    kv = B.DeviceKV(dm, 1, 64)
    gpu_prefill(dm, np.arange(64, dtype=np.int32), [64], rows=B.ROWS_LAST, kv=kv.handle)
    toks = t.zeros(1, dtype=t.int32, device="cuda")
    with pytest.raises(B.GptError) as e:
        dm.decode_step(kv.handle, toks, toks, workspace=dm.workspace(1, 1))
    assert e.value.status == B.GPT_ERR_CAPACITY
    assert (kv.lengths() == 64).all()
    kv.close()


# ---------------------------------------------------------------- selection kernels

def test_argmax_lowest_index_on_ties():
    t = torch()
    lg = np.zeros((3, 65536), np.float32)
    lg[0, [5, 9, 60000]] = 2.0
    lg[1, :] = -1.0
    lg[2, 65535] = 1.0
    out = t.empty(3, dtype=t.int32, device="cuda")
    B.gpt_select_tokens(t.from_numpy(lg).cuda(), 3, 65536, 0.0, None, out)
    np.testing.assert_array_equal(out.cpu().numpy(), [5, 0, 65535])


@pytest.mark.parametrize("V", [65536, 27, 70000, 70001])
def test_sampling_inverse_cdf(V):
    """Whole 8192-entry super-tiles, a vocabulary under one tile, a ragged
    last tile, and a width that is not a multiple of four (scalar loads)."""
    t = torch()
    rng = np.random.default_rng(8 + V)
    rows = 64
    lg = (rng.standard_normal((rows, V)) * 0.8).astype(np.float32)
    U = rng.random(rows).astype(np.float32)
    U[0], U[1] = 0.0, np.float32(1.0 - 2 ** -24)
    out = t.empty(rows, dtype=t.int32, device="cuda")
    B.gpt_select_tokens(t.from_numpy(lg).cuda(), rows, V, 0.7, t.from_numpy(U).cuda(), out)
    got = out.cpu().numpy()
    for j in range(rows):
        c = np.cumsum(oracle.softmax(lg[j].astype(np.float64) / 0.7))
        k = got[j]
        lo = c[k - 1] if k > 0 else 0.0
        assert lo - 1e-5 <= U[j] <= c[k] + 1e-5, (j, k, lo, c[k], U[j])


def _boundary_rows(rng, rows, V, spread):
    """Rows of logits and uniforms aimed at the cumulative weight just before
    or after an entry index that starts a thread's 8 entries, a wave's 512 or
    a super-tile's 8192 (where the kernel's partial sums meet), plus plain
    draws; with a large spread most weights underflow to zero."""
    lg = (rng.standard_normal((rows, V)) * spread).astype(np.float32)
    U = np.empty(rows, np.float32)
    cdfs = []
    for j in range(rows):
        c = np.cumsum(oracle.softmax(lg[j].astype(np.float64) / 0.7))
        cdfs.append(c)
        b = [8, 512, 8192][j % 3]
        k = int(rng.integers(1, V // b)) * b
        eps = (1 if j % 2 else -1) * 10.0 ** rng.uniform(-9, -6)
        U[j] = np.float32(min(max(c[k - 1] + eps, 0.0), 1 - 2 ** -24)) if j % 4 else rng.random()
    return lg, U, cdfs


@pytest.mark.parametrize("V,spread", [(65536, 0.8), (65536, 40.0), (100000, 0.8)])
def test_sampling_at_range_boundaries(V, spread):
    """512 rows with uniforms aimed at the boundaries between the kernel's
    per-thread, per-wave and per-super-tile partial sums, for the
    register-resident kernel (V = 65536) and the three-pass one (V = 100000):
    every pick lies at the float64 inverse-CDF crossing within 1e-5
    (Microgpt, "Inference")."""
    t = torch()
    rng = np.random.default_rng(int(V + spread))
    rows = 512
    lg, U, cdfs = _boundary_rows(rng, rows, V, spread)
    out = t.empty(rows, dtype=t.int32, device="cuda")
    B.gpt_select_tokens(t.from_numpy(lg).cuda(), rows, V, 0.7, t.from_numpy(U).cuda(), out)
    got = out.cpu().numpy()
    for j in range(rows):
        c, k = cdfs[j], got[j]
        lo = c[k - 1] if k > 0 else 0.0
        assert lo - 1e-5 <= U[j] <= c[k] + 1e-5, (j, k, lo, c[k], U[j])


# ---------------------------------------------------------------- loss backward

def gpu_loss_grads(cfg, dm, w, targets):
    t = torch()
    M = int(w.cu_seqlens[-1])
    g = B.DeviceGrads(dm)
    loss = t.empty(M, dtype=t.float32, device="cuda")
    mean = t.empty(1, dtype=t.float32, device="cuda")
    dm.loss_grads(to_dev(np.asarray(w.tokens, np.int32)), to_dev(np.asarray(targets, np.int32)),
                  w.cu_seqlens, g, loss, mean)
    t.cuda.synchronize()
    return {k: v.cpu().numpy().astype(np.float64) for k, v in g.flat()}, loss.cpu().numpy(), \
        float(mean.cpu().numpy()[0])


def test_tiny_loss_grads_fp32():
    """Every weight gradient of the tiny fp32 model's mean loss against the
    float64 oracle backward (itself pinned by finite differences)."""
    w = wl.tiny_workload()
    cfg = w.model
    W, dm = device_model(cfg)
    tg = w.next_token_targets()
    g, loss, mean = gpu_loss_grads(cfg, dm, w, tg)
    ref_mean, ref = oracle.loss_and_grads(cfg, W, w.tokens, w.seqlens, tg)
    assert abs(mean - ref_mean) <= 1e-5
    lg = np.concatenate(oracle.prefill(cfg, W, w.tokens, w.seqlens)[0])
    assert np.max(np.abs(loss - oracle.token_losses(lg, tg))) <= 1e-4
    for k, r in ref.items():
        err = np.max(np.abs(g[k] - r))
        assert err <= 1e-4 * np.max(np.abs(r)) + 1e-7, (k, err, np.max(np.abs(r)))


# Per-entry bound on bf16-model weight gradients:
#   |g - r| <= GRAD_REL |r| + GRAD_ABS max(rms(row of r), rms(r)).
# Every GEMM of the backward takes bf16 operands, each rounded with a
# relative error of at most 2^-9, so a product's entry errs by at most 2^-8
# of the sum of its terms' magnitudes; the chain through the layers
# compounds the operand errors to the 1.2-1.5% relative Frobenius error
# measured on these models.  An entry dominated by one term errs by about
# that fraction of itself, hence 3% of the entry.  An entry that sums many
# terms of both signs can err by much more than its own size, but not by
# more than a few times that 1.5% of the typical entry around it: 0.1 of an
# RMS.  The row's RMS is the scale where a row shares one large upstream
# factor (the LM head's rows of target tokens are about V times its other
# rows); the tensor's where a row is small only because its upstream factor
# nearly vanishes (an MLP feature whose ReLU^2 derivative 2 max(z, 0) is
# near zero for every token, and is itself moved by the forward's rounding
# of z at the scale of the other features).
GRAD_REL, GRAD_ABS = 0.03, 0.1


@pytest.mark.parametrize("n_head,n_kv,lens", [(2, 1, [150, 70, 33]), (4, 2, [40, 9]), (2, 2, [130]),
                                              (2, 1, [700, 452])])
def test_small_bf16_loss_grads(n_head, n_kv, lens):
    """bf16 models (MQA, GQA, MHA; 253 rows on the large-M GEMMs, 49 on the
    decode-row ones, 1152 rows with the weight-gradient GEMMs split over k):
    each weight gradient within 5% (relative Frobenius
    norm) of the float64 oracle's, pointing the same way (cosine >=
    0.998), and every entry within GRAD_REL of itself plus GRAD_ABS of the larger of its row's and its tensor's RMS.  The bf16 operands of the forward and of the gradient GEMMs set
    that floor; the loss matches the fused-loss prefill."""
    cfg = wl.small_model(2, n_head, vocab=2048, max_seq=1024, n_kv_head=n_kv)
    w = wl.ragged_prefill(cfg, lens, seed=11 + n_head)
    W, dm = device_model(cfg)
    tg = w.next_token_targets()
    g, loss, mean = gpu_loss_grads(cfg, dm, w, tg)
    ref_mean, ref = oracle.loss_and_grads(cfg, W, w.tokens, w.seqlens, tg)
    assert abs(mean - ref_mean) <= 1e-3
    l2, _, m2 = gpu_loss(dm, w.tokens, w.seqlens, tg)
    assert abs(mean - m2) <= 1e-5
    worst, worst_el = 0.0, 0.0
    for k, r in ref.items():
        nr = np.linalg.norm(r)
        if nr == 0:
            assert np.all(g[k] == 0), k
            continue
        rel = np.linalg.norm(g[k] - r) / nr
        cos = float(np.sum(g[k] * r) / (np.linalg.norm(g[k]) * nr))
        worst = max(worst, rel)
        assert rel <= 5e-2 and cos >= 0.998, (k, rel, cos)
        # element by element (the token table's rows that no token reads
        # stay exactly zero)
        live = np.any(r != 0, axis=1)
        assert np.all(g[k][~live] == 0), k
        rms = np.maximum(np.sqrt(np.mean(r[live] ** 2, axis=1, keepdims=True)), np.sqrt(np.mean(r[live] ** 2)))
        el = float(np.max(np.abs(g[k][live] - r[live]) / (GRAD_REL * np.abs(r[live]) + GRAD_ABS * rms)))
        worst_el = max(worst_el, el)
        assert el <= 1.0, (k, el)
    print("worst relative gradient error", worst, "worst entry error / its bound", worst_el)
