"""gpt_decode_step_noalloc (the decode step on the library's own device
scratch, for callers that cannot allocate) against gpt_decode_step with a
caller workspace: two calls in a row on fresh caches, the second with fewer
sequences, greedy and sampled, must give bit-identical logits, tokens and
cache lengths; a step that needs more scratch than the library holds is
refused before anything is enqueued."""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import to_dev, torch

pytestmark = pytest.mark.gpu

B = pytest.importorskip("gpt_block_fwd_amd.binding")


def _prefilled(dm, w, cap):
    t = torch()
    kv = B.DeviceKV(dm, w.n_seqs, cap)
    lg = t.empty((w.n_seqs, dm.model.vocab), dtype=t.float32, device="cuda")
    dm.prefill(to_dev(w.tokens), w.cu_seqlens, lg, kv=kv.handle, logits_rows=B.ROWS_LAST)
    return kv, lg


@pytest.mark.parametrize("temperature", [0.0, 0.7])
def test_noalloc_decode_matches_workspace_decode(temperature):
    t = torch()
    cfg = wl.small_model(2, 6, vocab=4096, max_seq=1024)
    dm = B.DeviceModel(cfg, wl.make_weights(cfg, 8))
    rng = np.random.default_rng(31)
    for n in (40, 5):  # the second call is smaller than the first
        lens = rng.integers(1, 700, size=n)
        w = wl.ragged_prefill(cfg, lens, seed=n)
        kv_a, lg0 = _prefilled(dm, w, 800)
        kv_b, _ = _prefilled(dm, w, 800)
        U = to_dev(rng.random((3, n)).astype(np.float32))
        first = t.empty(n, dtype=t.int32, device="cuda")
        B.gpt_select_tokens(lg0, n, cfg.vocab, temperature, U[0] if temperature > 0 else None, first)
        ta, tb = first.clone(), first.clone()
        ws = dm.workspace(n, n)
        for s in range(2):
            la = t.empty((n, cfg.vocab), dtype=t.float32, device="cuda")
            lb = t.full((n, cfg.vocab), float("nan"), dtype=t.float32, device="cuda")
            u = U[s + 1] if temperature > 0 else None
            dm.decode_step(kv_a.handle, ta, ta, temperature=temperature, uniforms=u, logits=la, workspace=ws)
            B.gpt_decode_step_noalloc(dm.cfg, dm.weights, dm.rope_cos, dm.rope_sin, kv_b.handle, tb,
                                      temperature, u, tb, lb)
            t.cuda.synchronize()
            np.testing.assert_array_equal(la.cpu().numpy(), lb.cpu().numpy())
            np.testing.assert_array_equal(ta.cpu().numpy(), tb.cpu().numpy())
        np.testing.assert_array_equal(kv_a.lengths(), kv_b.lengths())
        np.testing.assert_array_equal(kv_b.lengths(), lens + 2)
        kv_a.close()
        kv_b.close()


def test_noalloc_refuses_steps_beyond_its_scratch():
    """256 sequences of a 65536-token vocabulary need 64 MiB of logits alone."""
    t = torch()
    cfg = wl.small_model(1, 2, vocab=65536, max_seq=128)
    dm = B.DeviceModel(cfg, wl.make_weights(cfg, 9))
    n = 256
    assert B.gpt_workspace_bytes(dm.cfg, n, n) > 64 << 20
    kv = B.DeviceKV(dm, n, 64)
    toks = t.zeros(n, dtype=t.int32, device="cuda")
    with pytest.raises(B.GptError) as e:
        B.gpt_decode_step_noalloc(dm.cfg, dm.weights, dm.rope_cos, dm.rope_sin, kv.handle, toks, 0.0,
                                  None, toks, None)
    assert e.value.status == B.GPT_ERR_CAPACITY
    assert (kv.lengths() == 0).all()
    kv.close()
