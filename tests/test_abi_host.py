"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function the headers declare, answers size queries, and rejects bad
arguments before touching the device."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

import workloads as wl

g = pytest.importorskip("gpt_block_fwd_amd")
from gpt_block_fwd_amd import binding as B  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?(?:gpt_status|size_t|char|void)\s*\*?\s*(\w+)\s*\(",
                             text, flags=re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"gpt_prefill", "gpt_decode_step", "kv_cache_alloc", "rope_tables"} <= names
    L = B.lib()
    missing = [n for n in sorted(names) if not hasattr(L, n)]
    assert not missing, missing
    assert names == set(B.EXPORTS)


def test_workspace_and_cache_size_queries():
    cfg = B.make_config(wl.depth_model(12))
    ws = B.gpt_workspace_bytes(cfg, 16384, 8)
    assert ws > 16384 * 768 * 4  # at least the fp32 residual stream
    assert ws % 256 == 0
    nb = B.kv_cache_bytes(cfg, 32, 768)
    pages = 32 * 12
    assert nb >= 12 * pages * 2 * 64 * 128 * 2 + pages * 4 + 32 * 4
    # capacity rounds up to whole 64-position pages
    assert B.kv_cache_bytes(cfg, 32, 705) == nb
    assert B.kv_cache_bytes(cfg, 32, 704) < nb
    assert B.gpt_workspace_bytes(cfg, 0, 1) == 0


def _bad(fn, status):
    with pytest.raises(B.GptError) as e:
        fn()
    assert e.value.status == status, str(e.value)
    return str(e.value)


def test_unsupported_configs_are_reported():
    m = wl.depth_model(12)
    import dataclasses
    for change in ({"head_dim": 64, "d_model": 384}, {"n_head": 18, "d_model": 18 * 128},
                   {"pos_kind": 0}, {"vocab": 1000}, {"act": 0}):
        cfg = B.make_config(dataclasses.replace(m, **change))
        _bad(lambda: B.kv_cache_bytes(cfg, 4, 64), B.GPT_ERR_UNSUPPORTED)
    # grouped-query attention is supported; a K/V head count that does not
    # divide the query heads is an argument error
    gqa = B.make_config(dataclasses.replace(m, n_kv_head=2))
    assert B.kv_cache_bytes(gqa, 4, 64) > B.kv_cache_bytes(B.make_config(m), 4, 64)
    _bad(lambda: B.kv_cache_bytes(B.make_config(dataclasses.replace(m, n_kv_head=4)), 4, 64),
         B.GPT_ERR_ARG)
    bad = B.make_config(dataclasses.replace(m, n_head=5))  # 6 % ... n_kv divides, d != H*dh
    _bad(lambda: B.kv_cache_bytes(bad, 4, 64), B.GPT_ERR_UNSUPPORTED)
    neg = B.make_config(dataclasses.replace(m, n_layer=0))
    _bad(lambda: B.kv_cache_bytes(neg, 4, 64), B.GPT_ERR_ARG)


def test_cache_argument_errors():
    cfg = B.make_config(wl.depth_model(12, max_seq=1024))
    _bad(lambda: B.kv_cache_bytes(cfg, 0, 64), B.GPT_ERR_ARG)
    _bad(lambda: B.kv_cache_bytes(cfg, 4, 2048), B.GPT_ERR_ARG)  # beyond max_seq
    _bad(lambda: B.kv_cache_bytes(cfg, 4, 64, page_size=32), B.GPT_ERR_UNSUPPORTED)
    # a buffer that is too small is refused before any device call
    _bad(lambda: B.kv_cache_alloc(cfg, 4, 64, 0x100000, 16), B.GPT_ERR_ARG)


def _weights_struct(L=2):
    arr = (ctypes.c_void_p * L)(*([0x1000] * L))
    pp = ctypes.cast(arr, B._PP)
    return B.GptWeights(0x1000, None, 0x1000, pp, pp, pp, pp, pp, pp), arr


def test_prefill_validation_runs_before_device_work():
    m = wl.small_model(2, 2, vocab=256)
    cfg = B.make_config(m)
    w, keep = _weights_struct()
    good_cu = np.array([0, 5, 9], np.int32)
    ws = B.gpt_workspace_bytes(cfg, 9, 2)

    def call(cu=good_cu, n=2, logits=0x2000, tokens=0x3000, ws_bytes=ws, rows=B.ROWS_ALL,
             cos=0x4000, wsp=0x100000):
        B.gpt_prefill(cfg, w, cos, cos, tokens, cu, n, None, rows, logits, None, None, wsp,
                      ws_bytes, 0)

    _bad(lambda: call(tokens=None), B.GPT_ERR_ARG)
    _bad(lambda: call(logits=None), B.GPT_ERR_ARG)
    assert "decreases" in _bad(lambda: call(cu=np.array([0, 5, 4], np.int32)), B.GPT_ERR_ARG)
    _bad(lambda: call(cu=np.array([1, 5, 9], np.int32)), B.GPT_ERR_ARG)
    assert "workspace" in _bad(lambda: call(ws_bytes=ws - 256), B.GPT_ERR_ARG)
    _bad(lambda: call(wsp=0x100010), B.GPT_ERR_ARG)  # not 256-byte aligned
    _bad(lambda: call(rows=7), B.GPT_ERR_ARG)
    _bad(lambda: call(cos=None), B.GPT_ERR_ARG)
    _bad(lambda: call(n=0), B.GPT_ERR_ARG)
    _bad(lambda: call(cu=np.array([0, 5000, 5001], np.int32)), B.GPT_ERR_ARG)  # > max_seq


def test_prefill_rows_beyond_32bit_offsets_rejected():
    """The GEMMs address activation rows with 32-bit element offsets: a
    depth-26 prefill whose rows x widest activation (d_ff = 6656) reaches
    2^31 is refused before any launch, for logits and for the loss, while
    one row fewer than the limit passes that check (and then fails only on
    the deliberately short workspace)."""
    m = wl.depth_model(26, max_seq=4096)
    cfg = B.make_config(m)
    w, keep = _weights_struct(m.n_layer)
    limit = (1 << 31) // m.d_ff          # first row count that overflows is limit + 1
    n = (limit + 1 + 4095) // 4096
    lens = np.full(n, 4096, np.int64)
    lens[-1] -= n * 4096 - (limit + 1)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    assert int(cu[-1]) * m.d_ff >= 1 << 31 and (int(cu[-1]) - 1) * m.d_ff < 1 << 31
    msg = _bad(lambda: B.gpt_prefill(cfg, w, 0x4000, 0x4000, 0x3000, cu, n, None, B.ROWS_LAST,
                                     0x2000, None, None, 0x100000, 1 << 40, 0), B.GPT_ERR_UNSUPPORTED)
    assert "32-bit" in msg
    _bad(lambda: B.gpt_prefill_loss(cfg, w, 0x4000, 0x4000, 0x3000, 0x5000, cu, n, None, 0x6000,
                                    None, None, 0x100000, 1 << 40, 0), B.GPT_ERR_UNSUPPORTED)
    cu2 = cu.copy()
    cu2[-1] -= 1
    msg = _bad(lambda: B.gpt_prefill(cfg, w, 0x4000, 0x4000, 0x3000, cu2, n, None, B.ROWS_LAST,
                                     0x2000, None, None, 0x100000, 256, 0), B.GPT_ERR_ARG)
    assert "workspace" in msg


def test_weights_beyond_32bit_offsets_rejected():
    """An LM head of 2^20 x 2048 entries is refused by every entry point."""
    cfg = B.make_config(wl.small_model(1, 16, vocab=1 << 20))
    assert B.gpt_workspace_bytes(cfg, 1, 1) == 0
    assert "2^31" in B.last_error()
    assert "2^31" in _bad(lambda: B.kv_cache_bytes(cfg, 1, 64), B.GPT_ERR_UNSUPPORTED)


def test_prefill_loss_validation():
    m = wl.small_model(2, 2, vocab=256)
    cfg = B.make_config(m)
    w, keep = _weights_struct()
    cu = np.array([0, 5, 9], np.int32)
    ws = B.gpt_workspace_bytes(cfg, 9, 2)

    def call(targets=0x5000, loss=0x6000, cu=cu):
        B.gpt_prefill_loss(cfg, w, 0x4000, 0x4000, 0x3000, targets, cu, 2, None, loss, None, None,
                           0x100000, ws, 0)

    _bad(lambda: call(targets=None), B.GPT_ERR_ARG)
    _bad(lambda: call(loss=None), B.GPT_ERR_ARG)
    _bad(lambda: call(cu=np.array([0, 5, 4], np.int32)), B.GPT_ERR_ARG)


def test_adam_validation():
    def call(p=0x1000, g=0x2000, m=0x3000, v=0x4000, pb=None, n=100, step=1, lr=1e-3, b1=0.9,
             b2=0.999, eps=1e-8):
        B.gpt_adam_step(p, g, m, v, pb, n, step, lr, b1, b2, eps, 0)

    _bad(lambda: call(p=None), B.GPT_ERR_ARG)
    _bad(lambda: call(v=None), B.GPT_ERR_ARG)
    _bad(lambda: call(g=0x2004), B.GPT_ERR_ARG)
    _bad(lambda: call(pb=0x5002), B.GPT_ERR_ARG)
    _bad(lambda: call(n=-1), B.GPT_ERR_ARG)
    _bad(lambda: call(step=0), B.GPT_ERR_ARG)
    _bad(lambda: call(b1=1.0), B.GPT_ERR_ARG)
    _bad(lambda: call(b2=-0.1), B.GPT_ERR_ARG)
    _bad(lambda: call(eps=-1.0), B.GPT_ERR_ARG)
    _bad(lambda: call(eps=float("nan")), B.GPT_ERR_ARG)
    _bad(lambda: call(lr=float("inf")), B.GPT_ERR_ARG)
    call(n=0)  # nothing to do: no device work, no error


def test_misaligned_weights_rejected():
    m = wl.small_model(2, 2, vocab=256)
    cfg = B.make_config(m)
    arr = (ctypes.c_void_p * 2)(0x1000, 0x1008)
    pp = ctypes.cast(arr, B._PP)
    w = B.GptWeights(0x1000, None, 0x1000, pp, pp, pp, pp, pp, pp)
    cu = np.array([0, 4], np.int32)
    ws = B.gpt_workspace_bytes(cfg, 4, 1)
    _bad(lambda: B.gpt_prefill(cfg, w, 0x4000, 0x4000, 0x3000, cu, 1, None, 0, 0x2000, None,
                               None, 0x100000, ws, 0), B.GPT_ERR_ARG)


def test_select_and_rope_validation():
    _bad(lambda: B.gpt_select_tokens(0x1000, 2, 100, 0.7, None, 0x2000, 0), B.GPT_ERR_ARG)
    _bad(lambda: B.gpt_select_tokens(0x1000, 0, 100, 0.0, None, 0x2000, 0), B.GPT_ERR_ARG)
    _bad(lambda: B.rope_tables(16, 7, 10000.0, 0x1000, 0x2000, 0), B.GPT_ERR_ARG)
    _bad(lambda: B.rope_tables(0, 8, 10000.0, 0x1000, 0x2000, 0), B.GPT_ERR_ARG)
    _bad(lambda: B.rope_tables(16, 8, -1.0, 0x1000, 0x2000, 0), B.GPT_ERR_ARG)


def test_debug_entry_validation():
    _bad(lambda: B.gpt_debug_gemm(0x1000, 0x2000, 10, 100, 64, 0x3000, 0, 1, 0), B.GPT_ERR_ARG)
    _bad(lambda: B.gpt_debug_gemm(0x1000, 0x2000, 10, 128, 60, 0x3000, 0, 1, 0), B.GPT_ERR_ARG)
    _bad(lambda: B.gpt_debug_gemm(0x1000, 0x2000, 10, 128, 64, 0x3000, 9, 1, 0), B.GPT_ERR_ARG)
    # k split: fp32 slabs only, M <= 64, 2 .. 16 ranges of at least 64
    _bad(lambda: B.gpt_debug_gemm(0x1000, 0x2000, 10, 128, 256, 0x3000, 0, 2, 0), B.GPT_ERR_ARG)
    _bad(lambda: B.gpt_debug_gemm(0x1000, 0x2000, 100, 128, 256, 0x3000, 3, 2, 0), B.GPT_ERR_ARG)
    _bad(lambda: B.gpt_debug_gemm(0x1000, 0x2000, 10, 128, 256, 0x3000, 3, 5, 0), B.GPT_ERR_ARG)
    _bad(lambda: B.gpt_debug_gemm(0x1000, 0x2000, 10, 128, 64 * 32, 0x3000, 3, 17, 0), B.GPT_ERR_ARG)
    _bad(lambda: B.gpt_debug_gemm(0x1000, 0x2000, 10, 128, 256, 0x3000, 3, 0, 0), B.GPT_ERR_ARG)
