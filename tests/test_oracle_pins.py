"""Pins of the CPU oracle to facts fixed by the source pages and by mathematics.

Each test checks the oracle against something other than itself: a value
the pages print (tests/golden/microgpt_facts.json), a closed form, an
invariant, a reduction to a textbook routine, or a brute-force scalar loop
on a tiny input.  None of these needs a GPU.
"""
import cmath
import json
import math
import os
import struct

import numpy as np
import pytest

import oracle
import workloads as wl

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "microgpt_facts.json")))


def tiny_rope_model(vocab=11):
    """A RoPE + QK-norm + MQA + ReLU^2 model small enough for scalar loops."""
    return wl.ModelConfig(vocab=vocab, n_layer=2, d_model=8, n_head=2, n_kv_head=1,
                          head_dim=4, d_ff=32, max_seq=16, rope_base=10000.0,
                          norm_eps=1e-6, pos_kind=1, act=1, qk_norm=1, dtype=0,
                          init_std=0.3)


# ---------------------------------------------------------------- layout

def test_tiny_layout_has_4192_parameters():
    W = wl.make_weights(wl.tiny_model())
    assert oracle.param_count(W) == GOLDEN["n_params"]["value"]


def test_every_tiny_parameter_is_read():
    """The 4,192 count only pins the layout if the forward reads every tensor."""
    cfg = wl.tiny_model()
    W = wl.make_weights(cfg)
    toks = np.array([26, 3, 7, 1, 0, 25, 26, 4], np.int64)
    base = oracle.forward(cfg, W, toks)
    for name, a in list(W.flat()):
        flat = a.reshape(-1)
        # bump the largest entry of this tensor that the tokens/positions reach
        if name == "wte":
            idx = toks[0] * cfg.d_model
        elif name == "wpe":
            idx = 0
        else:
            idx = int(np.argmax(np.abs(flat)))
        old = flat[idx]
        flat[idx] = old + 0.5
        changed = not np.array_equal(oracle.forward(cfg, W, toks), base)
        flat[idx] = old
        assert changed, f"{name} does not influence the logits"


def test_tiny_vocab_is_letters_plus_bos():
    cfg = wl.tiny_model()
    assert cfg.vocab == GOLDEN["vocab"]["value"] == GOLDEN["letters"]["value"] + 1
    w = wl.tiny_workload()
    toks = w.tokens.reshape(8, 16)
    assert (toks[:, 0] == 26).all() and toks.max() < 27 and toks.min() >= 0


def test_depth_param_counts_derived():
    """Derived (not printed by the pages): depth 12 and depth 26 sizes."""
    def count(cfg):
        return sum(int(np.prod(s)) for _, s in wl.weight_shapes(cfg))
    assert count(wl.depth_model(12)) == 173_801_472
    assert count(wl.depth_model(26)) == 949_092_352


def test_init_loss_near_3_3():
    """Random-init next-token loss sits near 3.3 (Microgpt, 'Training')."""
    w = wl.tiny_workload()
    cfg = w.model
    W = wl.make_weights(cfg)
    losses = []
    for b in range(w.n_seqs):
        t = w.seq_tokens(b).astype(np.int64)
        lg = oracle.forward(cfg, W, t)
        losses.append(oracle.cross_entropy(lg[:-1], t[1:]))
    g = GOLDEN["init_loss"]
    assert abs(np.mean(losses) - g["value"]) <= g["tol"]
    # and it exceeds uniform guessing, ln 27, by about half the logit variance
    assert np.mean(losses) > math.log(27) - 0.05


# ---------------------------------------------------------------- cross-entropy

def test_token_losses_closed_forms():
    """Uniform logits cost ln V for any target; shifting a row changes
    nothing; a target far ahead of the rest costs ~(V-1) e^-gap."""
    V = 37
    lg = np.zeros((3, V))
    np.testing.assert_allclose(oracle.token_losses(lg, [0, 5, 36]), math.log(V), rtol=0, atol=1e-15)
    rng = np.random.default_rng(11)
    lg = rng.normal(size=(5, V)) * 4
    t = rng.integers(0, V, 5)
    np.testing.assert_allclose(oracle.token_losses(lg + rng.normal(size=(5, 1)) * 50, t),
                               oracle.token_losses(lg, t), rtol=0, atol=1e-12)
    one = np.zeros((1, V))
    one[0, 7] = 30.0
    # lse - 30 cancels in float64: absolute error ~ 30 * 2^-52
    np.testing.assert_allclose(oracle.token_losses(one, [7]), (V - 1) * math.exp(-30.0), rtol=0, atol=2e-14)
    # and the wrong target pays the gap
    np.testing.assert_allclose(oracle.token_losses(one, [8]), 30.0 + (V - 1) * math.exp(-30.0), rtol=1e-12)


def test_token_losses_match_scalar_loop():
    """-log(softmax) written out with math.exp per entry, on a small vocabulary."""
    rng = np.random.default_rng(12)
    V = 9
    lg = rng.normal(size=(6, V)) * 3
    t = rng.integers(0, V, 6)
    ref = []
    for r in range(6):
        z = sum(math.exp(float(v)) for v in lg[r])
        ref.append(-math.log(math.exp(float(lg[r, t[r]])) / z))
    np.testing.assert_allclose(oracle.token_losses(lg, t), ref, rtol=0, atol=1e-12)


def test_ignored_targets_and_mean():
    rng = np.random.default_rng(13)
    V = 10
    lg = rng.normal(size=(5, V))
    t = np.array([3, -1, 9, 10, 0])   # rows 1 and 3 have no target
    loss = oracle.token_losses(lg, t)
    assert loss[1] == 0.0 and loss[3] == 0.0
    full = oracle.token_losses(lg[[0, 2, 4]], t[[0, 2, 4]])
    np.testing.assert_array_equal(loss[[0, 2, 4]], full)
    assert oracle.mean_loss(loss, t, V) == pytest.approx(float(np.mean(full)), abs=1e-15)
    assert oracle.mean_loss(loss, np.full(5, -1), V) == 0.0


def test_init_token_loss_near_3_3():
    """The per-row losses of the tiny model at init, averaged over every row
    with a next token, sit near 3.3 (Microgpt, 'Training process')."""
    w = wl.tiny_workload()
    W = wl.make_weights(w.model)
    lg = np.concatenate(oracle.prefill(w.model, W, w.tokens, w.seqlens)[0])
    t = w.next_token_targets()
    assert (t.reshape(8, 16)[:, -1] == -1).all()
    np.testing.assert_array_equal(t.reshape(8, 16)[:, :-1], w.tokens.reshape(8, 16)[:, 1:])
    m = oracle.mean_loss(oracle.token_losses(lg, t), t, w.model.vocab)
    g = GOLDEN["init_loss"]
    assert abs(m - g["value"]) <= g["tol"]


# ---------------------------------------------------------------- Adam

def test_adam_first_step_moves_by_lr_times_sign():
    """From zero moments the bias-corrected means are g and g^2, so the
    first step is lr * g / (|g| + eps): about lr against the gradient."""
    rng = np.random.default_rng(21)
    p = rng.normal(size=50)
    g = rng.normal(size=50) * 10.0 ** rng.uniform(-3, 3, 50)
    z = np.zeros(50)
    lr, eps = 0.01, 1e-8
    p1, m1, v1 = oracle.adam_step(p, g, z, z, 1, lr, 0.85, 0.99, eps)
    np.testing.assert_allclose(p1, p - lr * g / (np.abs(g) + eps), rtol=0, atol=1e-15)
    np.testing.assert_allclose(m1, 0.15 * g, rtol=1e-14)  # 1 - 0.85 is not exactly 0.15 in float64
    np.testing.assert_allclose(v1, 0.01 * g * g, rtol=1e-14)


def test_adam_constant_gradient_has_exact_bias_correction():
    """With a constant gradient the corrected means stay exactly g and g^2,
    so every step moves the parameter by the same lr * g / (|g| + eps)."""
    g = np.array([0.3, -2.0, 1e-4, 7.0])
    p = np.array([1.0, -1.0, 0.5, 0.0])
    m = np.zeros(4)
    v = np.zeros(4)
    lr, eps = 1e-3, 1e-8
    for t in range(1, 40):
        p, m, v = oracle.adam_step(p, g, m, v, t, lr, 0.9, 0.999, eps)
        np.testing.assert_allclose(m / (1 - 0.9 ** t), g, rtol=1e-12)
        np.testing.assert_allclose(v / (1 - 0.999 ** t), g * g, rtol=1e-12)
    np.testing.assert_allclose(p, np.array([1.0, -1.0, 0.5, 0.0]) - 39 * lr * g / (np.abs(g) + eps),
                               rtol=0, atol=1e-12)


def test_adam_is_invariant_to_gradient_scale_and_still_at_zero():
    rng = np.random.default_rng(22)
    p, g = rng.normal(size=20), rng.normal(size=20)
    m, v = rng.normal(size=20) * 0.1, rng.uniform(0.0, 1.0, 20)
    a = oracle.adam_step(p, g, m, v, 5, 0.02, 0.9, 0.95, 0.0)
    b = oracle.adam_step(p, 1000.0 * g, 1000.0 * m, 1e6 * v, 5, 0.02, 0.9, 0.95, 0.0)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-13)
    z = np.zeros(20)
    np.testing.assert_array_equal(oracle.adam_step(p, z, z, z, 3, 0.1, 0.9, 0.99, 1e-8)[0], p)


# ---------------------------------------------------------------- backward

def _f64_weights(W):
    import dataclasses
    return dataclasses.replace(
        W, wte=W.wte.astype(np.float64),
        wpe=None if W.wpe is None else W.wpe.astype(np.float64),
        lm_head=W.lm_head.astype(np.float64),
        layers=[{k: v.astype(np.float64) for k, v in lw.items()} for lw in W.layers])


@pytest.mark.parametrize("which", ["tiny", "rope_mqa", "rope_gqa"])
def test_loss_gradients_match_finite_differences(which):
    """Every weight tensor's gradient of the mean next-token loss, at sampled
    entries, against central differences of the oracle's own forward loss
    (float64 weights, step 1e-5: truncation ~1e-10 relative, roundoff
    ~2e-16 * loss / step ~ 1e-10 absolute)."""
    if which == "tiny":
        w = wl.tiny_workload()
        cfg = w.model
    else:
        import dataclasses
        cfg = tiny_rope_model()
        if which == "rope_gqa":
            cfg = dataclasses.replace(cfg, n_head=4, n_kv_head=2, d_model=16)
        w = wl.ragged_prefill(cfg, [9, 5, 12], seed=3)
    W = _f64_weights(wl.make_weights(cfg))
    tg = w.next_token_targets()
    tg[2] = -1  # a skipped row in the middle of a sequence
    loss, g = oracle.loss_and_grads(cfg, W, w.tokens, w.seqlens, tg)
    lg = np.concatenate(oracle.prefill(cfg, W, w.tokens, w.seqlens)[0])
    assert loss == pytest.approx(oracle.mean_loss(oracle.token_losses(lg, tg), tg, cfg.vocab), abs=1e-12)
    rng = np.random.default_rng(len(which))
    tensors = list(W.flat()) + [("lm_head", W.lm_head)]
    for name, arr in tensors:
        assert g[name].shape == arr.shape
        for _ in range(3):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            if name == "wte":
                idx = (int(w.tokens[rng.integers(0, len(w.tokens))]), idx[1])  # a row that is read
            old = arr[idx]
            arr[idx] = old + 1e-5
            lp = oracle.loss_and_grads(cfg, W, w.tokens, w.seqlens, tg)[0]
            arr[idx] = old - 1e-5
            lm = oracle.loss_and_grads(cfg, W, w.tokens, w.seqlens, tg)[0]
            arr[idx] = old
            fd = (lp - lm) / 2e-5
            assert abs(g[name][idx] - fd) <= 1e-6 * (abs(fd) + abs(g[name][idx])) + 1e-9, (name, idx)
    # rows of the token table that no position reads get no gradient
    unused = np.setdiff1d(np.arange(cfg.vocab), w.tokens)
    assert np.all(g["wte"][unused] == 0.0)


# ---------------------------------------------------------------- softmax

def test_vocab_softmax_rows_are_distributions():
    cfg = wl.tiny_model()
    W = wl.make_weights(cfg)
    lg = oracle.forward(cfg, W, wl.tiny_workload().seq_tokens(0))
    p = oracle.softmax(lg)
    r = GOLDEN["softmax_range"]
    assert p.min() >= r["lo"] and p.max() <= r["hi"]
    np.testing.assert_allclose(p.sum(-1), r["sum"], atol=1e-12)
    np.testing.assert_allclose(np.exp(lg - oracle.logsumexp(lg)[:, None]), p, atol=1e-15)


def test_attention_weights_are_distributions():
    rng = np.random.default_rng(5)
    s = rng.normal(size=(7, 7)) * 3
    s = np.where(np.tril(np.ones((7, 7), bool)), s, -np.inf)
    p = oracle.softmax(s)
    assert p.min() >= 0 and p.max() <= 1
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)
    assert (p[np.triu_indices(7, 1)] == 0).all()


# ---------------------------------------------------------------- RoPE

def test_rope_preserves_norm_and_is_identity_at_zero():
    rng = np.random.default_rng(0)
    cos, sin = oracle.rope_tables(64, 128, 10000.0)
    u = rng.normal(size=(64, 3, 128))
    r = oracle.apply_rope(u, cos, sin)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(u, axis=-1), rtol=1e-12)
    np.testing.assert_array_equal(r[0], u[0])


def test_rope_scores_depend_only_on_offset():
    rng = np.random.default_rng(1)
    cos, sin = oracle.rope_tables(40, 8, 10000.0)
    q = rng.normal(size=(1, 1, 8))
    k = rng.normal(size=(1, 1, 8))

    def score(t, s):
        qt = oracle.apply_rope(q, cos[t:t + 1], sin[t:t + 1])
        ks = oracle.apply_rope(k, cos[s:s + 1], sin[s:s + 1])
        return float((qt * ks).sum())

    for off in (0, 1, 5, 17):
        vals = [score(t + off, t) for t in (0, 3, 11, 20)]
        np.testing.assert_allclose(vals, vals[0], rtol=1e-10, atol=1e-12)


def test_rope_equals_complex_multiplication():
    """Half-split rotation = multiplying z_i = u_i + j u_{i+dh/2} by e^{j t theta_i}."""
    rng = np.random.default_rng(2)
    dh, base = 8, 10000.0
    cos, sin = oracle.rope_tables(10, dh, base)
    u = rng.normal(size=(10, 1, dh))
    r = oracle.apply_rope(u, cos, sin)
    for t in range(10):
        for i in range(dh // 2):
            theta = base ** (-(2 * i) / dh)
            z = complex(u[t, 0, i], u[t, 0, i + dh // 2]) * cmath.exp(1j * t * theta)
            assert abs(r[t, 0, i] - z.real) < 1e-12
            assert abs(r[t, 0, i + dh // 2] - z.imag) < 1e-12


def test_rope_frequency_ladder():
    """Pair 0 turns by one radian per position; frequencies fall geometrically
    and would reach 1/base at pair dh/2."""
    ang = oracle.rope_angles(3, 128, 10000.0)
    assert ang[1, 0] == 1.0 and (ang[0] == 0).all()
    ratios = ang[1, 1:] / ang[1, :-1]
    np.testing.assert_allclose(ratios, ratios[0], rtol=1e-12)
    np.testing.assert_allclose(ang[1, 0] * ratios[0] ** 64, 1e-4, rtol=1e-10)


def test_qknorm_commutes_with_rope():
    rng = np.random.default_rng(3)
    cos, sin = oracle.rope_tables(16, 128, 10000.0)
    u = rng.normal(size=(16, 2, 128))
    a = oracle.rmsnorm(oracle.apply_rope(u, cos, sin), 1e-6)
    b = oracle.apply_rope(oracle.rmsnorm(u, 1e-6), cos, sin)
    np.testing.assert_allclose(a, b, atol=1e-12)


# ---------------------------------------------------------------- norm / act

def test_rmsnorm_closed_form_and_scale_invariance():
    rng = np.random.default_rng(4)
    z = rng.normal(size=(5, 96)) * 3
    y = oracle.rmsnorm(z, 1e-6)
    ms = np.mean(z * z, -1)
    np.testing.assert_allclose(np.mean(y * y, -1), ms / (ms + 1e-6), rtol=1e-12)
    np.testing.assert_allclose(oracle.rmsnorm(7.5 * z, 0.0), oracle.rmsnorm(z, 0.0), rtol=1e-12)
    assert np.all(np.sign(y) == np.sign(z))


def test_activations_special_values():
    z = np.array([-2.0, -0.0, 0.0, 0.5, 3.0])
    np.testing.assert_array_equal(oracle.relu(z), [0, 0, 0, 0.5, 3.0])
    np.testing.assert_array_equal(oracle.relu2(z), [0, 0, 0, 0.25, 9.0])


def test_round_bf16_known_values():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 1 + 2 ** -7], np.float64)
    np.testing.assert_array_equal(oracle.round_bf16(x), [1.0, 1.0, 1 + 2 ** -6, -2.5, 1 + 2 ** -7])


# ---------------------------------------------------------------- attention

def brute_attention(q, k, v, q_start):
    tq, H, dh = q.shape
    tk, Hkv, _ = k.shape
    out = np.zeros_like(q)
    for i in range(tq):
        for h in range(H):
            g = h * Hkv // H
            n = q_start + i + 1
            s = [sum(q[i, h, c] * k[j, g, c] for c in range(dh)) / math.sqrt(dh) for j in range(n)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for c in range(dh):
                out[i, h, c] = sum(e[j] * v[j, g, c] for j in range(n)) / z
    return out


@pytest.mark.parametrize("n_kv", [1, 2, 4])
@pytest.mark.parametrize("tq,tk", [(8, 8), (1, 5), (3, 7)])
def test_attention_matches_brute_force(n_kv, tq, tk):
    rng = np.random.default_rng(10 + n_kv)
    q = rng.normal(size=(tq, 4, 4))
    k = rng.normal(size=(tk, n_kv, 4))
    v = rng.normal(size=(tk, n_kv, 4))
    start = tk - tq
    np.testing.assert_allclose(oracle.causal_attention(q, k, v, start),
                               brute_attention(q, k, v, start), atol=1e-12)


def test_attention_single_position_returns_v0():
    rng = np.random.default_rng(6)
    q = rng.normal(size=(1, 3, 16))
    k = rng.normal(size=(1, 1, 16))
    v = rng.normal(size=(1, 1, 16))
    o = oracle.causal_attention(q, k, v, 0)
    for h in range(3):
        np.testing.assert_array_equal(o[0, h], v[0, 0])


def test_attention_zero_query_is_causal_prefix_mean():
    rng = np.random.default_rng(7)
    k = rng.normal(size=(9, 1, 8))
    v = rng.normal(size=(9, 1, 8))
    q = np.zeros((9, 2, 8))
    o = oracle.causal_attention(q, k, v, 0)
    mean = np.cumsum(v[:, 0], axis=0) / np.arange(1, 10)[:, None]
    for h in range(2):
        np.testing.assert_allclose(o[:, h], mean, atol=1e-12)


def test_mqa_equals_mha_with_replicated_kv():
    rng = np.random.default_rng(8)
    q = rng.normal(size=(6, 4, 8))
    k = rng.normal(size=(6, 1, 8))
    v = rng.normal(size=(6, 1, 8))
    a = oracle.causal_attention(q, k, v, 0)
    b = oracle.causal_attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0)
    np.testing.assert_allclose(a, b, atol=1e-14)


# ---------------------------------------------------------------- whole model

def bf16_scalar(x):
    """Round a Python float to float32 (ties to even, through the C cast of
    struct) and then to the nearest bfloat16 value (8 significant bits, ties
    to even via Python's round): the value a float32 GPU register holds after
    conversion to bf16.  Written independently of oracle.round_bf16."""
    x32 = struct.unpack("f", struct.pack("f", x))[0]
    if x32 == 0.0 or not math.isfinite(x32):
        return x32
    m, e = math.frexp(x32)
    return math.ldexp(round(m * 256.0), e - 8)


def scalar_forward(cfg, W, tokens, bf16=False):
    """Pure-Python scalar loops over one sequence, written independently of
    the vectorised oracle (pre-norm blocks, learned or rotary positions).

    ``bf16`` rounds to bf16 where a bf16-operand GPU path stores its GEMM
    operands: each normed input (h, h2 and the final hf), q, k and v after
    RoPE and QK-norm, the unnormalised attention weights exp(s - max) that
    multiply V (the sum that divides stays unrounded), the attention output o
    and the MLP activation u."""
    d, H, Hkv, dh = cfg.d_model, cfg.n_head, cfg.n_kv_head, cfg.head_dim
    T = len(tokens)
    rb = (lambda vec: [bf16_scalar(a) for a in vec]) if bf16 else (lambda vec: vec)

    def rms(vec):
        ms = sum(a * a for a in vec) / len(vec)
        r = 1.0 / math.sqrt(ms + cfg.norm_eps)
        return [a * r for a in vec]

    def matvec(Wm, vec):
        return [sum(float(Wm[o, i]) * vec[i] for i in range(len(vec))) for o in range(Wm.shape[0])]

    def rot(vec, t):
        half = dh // 2
        out = list(vec)
        for i in range(half):
            ang = t * cfg.rope_base ** (-2.0 * i / dh)
            a, b = vec[i], vec[i + half]
            out[i] = a * math.cos(ang) - b * math.sin(ang)
            out[i + half] = a * math.sin(ang) + b * math.cos(ang)
        return out

    xs = []
    for t, tok in enumerate(tokens):
        x = [float(W.wte[tok, c]) for c in range(d)]
        if cfg.pos_kind == 0:
            x = [x[c] + float(W.wpe[t, c]) for c in range(d)]
        xs.append(x)
    for lw in W.layers:
        Ks, Vs, Qs = [], [], []
        for t in range(T):
            h = rb(rms(xs[t]))
            q, k, v = matvec(lw["wq"], h), matvec(lw["wk"], h), matvec(lw["wv"], h)
            qh = [q[i * dh:(i + 1) * dh] for i in range(H)]
            kh = [k[i * dh:(i + 1) * dh] for i in range(Hkv)]
            vh = [v[i * dh:(i + 1) * dh] for i in range(Hkv)]
            if cfg.pos_kind == 1:
                qh = [rot(a, t) for a in qh]
                kh = [rot(a, t) for a in kh]
            if cfg.qk_norm:
                qh = [rms(a) for a in qh]
                kh = [rms(a) for a in kh]
            Qs.append([rb(a) for a in qh]), Ks.append([rb(a) for a in kh]), Vs.append([rb(a) for a in vh])
        new = []
        for t in range(T):
            o = []
            for hh in range(H):
                g = hh * Hkv // H
                s = [sum(Qs[t][hh][c] * Ks[j][g][c] for c in range(dh)) / math.sqrt(dh)
                     for j in range(t + 1)]
                m = max(s)
                e = [math.exp(a - m) for a in s]
                z = sum(e)
                ew = rb(e)
                o += [sum(ew[j] * Vs[j][g][c] for j in range(t + 1)) / z for c in range(dh)]
            a = matvec(lw["wo"], rb(o))
            x = [xs[t][c] + a[c] for c in range(d)]
            zz = matvec(lw["w1"], rb(rms(x)))
            act = rb([max(a, 0.0) ** 2 if cfg.act == 1 else max(a, 0.0) for a in zz])
            m2 = matvec(lw["w2"], act)
            new.append([x[c] + m2[c] for c in range(d)])
        xs = new
    return np.array([matvec(W.lm_head, rb(rms(x))) for x in xs])


def test_tiny_forward_matches_scalar_loops():
    cfg = wl.tiny_model()
    W = wl.make_weights(cfg)
    toks = wl.tiny_workload().seq_tokens(3)
    np.testing.assert_allclose(oracle.forward(cfg, W, toks), scalar_forward(cfg, W, toks),
                               atol=1e-12)


def test_rope_model_forward_matches_scalar_loops():
    cfg = tiny_rope_model()
    W = wl.make_weights(cfg, seed=3)
    toks = np.array([1, 5, 5, 0, 10, 2, 7], np.int64)
    np.testing.assert_allclose(oracle.forward(cfg, W, toks), scalar_forward(cfg, W, toks),
                               atol=1e-12)


def test_bf16_scalar_rounding_known_values():
    assert bf16_scalar(1.0) == 1.0
    assert bf16_scalar(1.0 + 2 ** -8) == 1.0                 # tie to even (down)
    assert bf16_scalar(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6   # tie to even (up)
    assert bf16_scalar(1.0 + 2 ** -8 + 2 ** -20) == 1.0 + 2 ** -7
    assert bf16_scalar(-3.0) == -3.0
    assert bf16_scalar(0.1) == 0.10009765625


@pytest.mark.parametrize("which", ["tiny", "rope"])
def test_bf16_storage_mode_matches_scalar_loops(which):
    """The oracle's bf16-storage mode (used only to measure the bf16 noise
    floor) rounds at exactly the points the scalar loop rounds, on the
    microgpt layout and on a RoPE + QK-norm + MQA + ReLU^2 model: agreement
    to 1e-12, far below one bf16 step, so a rounding point added, dropped or
    moved anywhere would fail.  It also differs from the exact mode."""
    if which == "tiny":
        cfg, W = wl.tiny_model(), wl.make_weights(wl.tiny_model())
        toks = wl.tiny_workload().seq_tokens(2)[:9]
    else:
        cfg = tiny_rope_model()
        W = wl.make_weights(cfg, seed=4)
        toks = np.array([3, 9, 9, 1, 0, 7, 2, 10], np.int64)
    got = oracle.forward(cfg, W, toks, bf16_points=True)
    np.testing.assert_allclose(got, scalar_forward(cfg, W, toks, bf16=True), atol=1e-12, rtol=0)
    assert np.max(np.abs(got - oracle.forward(cfg, W, toks))) > 1e-4


def test_bf16_storage_mode_decode_equals_recompute():
    """In bf16-storage mode the cache holds the rounded k and v, so decoding
    position by position reproduces the full forward (1e-12)."""
    cfg = tiny_rope_model()
    W = wl.make_weights(cfg, seed=4)
    toks = np.array([3, 9, 9, 1, 0, 7, 2, 10, 4], np.int64)
    full = oracle.forward(cfg, W, toks, bf16_points=True)
    cache = oracle.KVCache(cfg.n_layer)
    part = [oracle.forward(cfg, W, toks[:4], cache, bf16_points=True)]
    for t in range(4, len(toks)):
        part.append(oracle.forward(cfg, W, toks[t:t + 1], cache, bf16_points=True))
    np.testing.assert_allclose(np.concatenate(part), full, atol=1e-12, rtol=0)


def test_prefill_packing_matches_per_sequence_forward():
    """oracle.prefill slices packed tokens by the cumulative lengths: each
    sequence's logits (all rows, or the last row) equal a forward of that
    sequence alone, also for a subset of sequences in any order."""
    cfg = tiny_rope_model()
    W = wl.make_weights(cfg, seed=6)
    lens = np.array([5, 1, 9, 3])
    rng = np.random.default_rng(13)
    toks = rng.integers(0, cfg.vocab, size=int(lens.sum()))
    cu = np.concatenate([[0], np.cumsum(lens)])
    outs, _ = oracle.prefill(cfg, W, toks, lens)
    last, _ = oracle.prefill(cfg, W, toks, lens, rows="last", seqs=[3, 0, 2])
    for b in range(len(lens)):
        ref = oracle.forward(cfg, W, toks[cu[b]:cu[b + 1]])
        np.testing.assert_array_equal(outs[b], ref)
    for j, b in enumerate([3, 0, 2]):
        np.testing.assert_allclose(last[j], oracle.forward(cfg, W, toks[cu[b]:cu[b + 1]])[-1:],
                                   atol=1e-12, rtol=0)


@pytest.mark.parametrize("mode", ["greedy", "forced", "sampled"])
def test_run_serving_matches_forward_on_the_whole_sequence(mode):
    """Serving (prefill a prompt into the cache, choose a token from the last
    logits, feed it back at the next position) equals one forward over the
    prompt followed by the fed tokens: the logits of every step are the rows
    of that forward from the prompt's last position on (1e-12), each choice
    is the selection rule applied to its row (with the uniform of its step
    and sequence), and teacher forcing feeds the given tokens instead."""
    cfg = tiny_rope_model()
    W = wl.make_weights(cfg, seed=7)
    lens = np.array([3, 6, 1])
    rng = np.random.default_rng(14)
    toks = rng.integers(0, cfg.vocab, size=int(lens.sum()))
    cu = np.concatenate([[0], np.cumsum(lens)])
    steps, seqs = 5, [2, 0]
    U = rng.random((steps + 1, len(lens)))
    forced = rng.integers(0, cfg.vocab, size=(steps + 1, len(lens)))
    T = 0.7 if mode == "sampled" else 0.0
    chosen, logits = oracle.run_serving(cfg, W, toks, lens, steps, temperature=T,
                                        uniforms=U if T else None,
                                        forced=forced if mode == "forced" else None, seqs=seqs)
    for j, b in enumerate(seqs):
        fed = (forced[:steps, b] if mode == "forced" else chosen[:steps, j])
        seq = np.concatenate([toks[cu[b]:cu[b + 1]], fed])
        ref = oracle.forward(cfg, W, seq)[lens[b] - 1:]
        np.testing.assert_allclose(logits[:, j], ref, atol=1e-12, rtol=0)
        for s_ in range(steps + 1):
            want = oracle.sample(ref[s_], T, U[s_, b]) if T else int(np.argmax(ref[s_]))
            assert chosen[s_, j] == want


@pytest.mark.parametrize("cfg_fn", [wl.tiny_model, tiny_rope_model])
def test_causality_bit_exact(cfg_fn):
    cfg = cfg_fn()
    W = wl.make_weights(cfg, seed=1)
    rng = np.random.default_rng(9)
    toks = rng.integers(0, cfg.vocab, size=12)
    base = oracle.forward(cfg, W, toks)
    for t in (0, 4, 11):
        pert = toks.copy()
        pert[t] = (pert[t] + 1) % cfg.vocab
        out = oracle.forward(cfg, W, pert)
        np.testing.assert_array_equal(out[:t], base[:t])
        assert not np.array_equal(out[t], base[t])


@pytest.mark.parametrize("cfg_fn", [wl.tiny_model, tiny_rope_model])
@pytest.mark.parametrize("k", [1, 5, 11])
def test_decode_equals_recompute(cfg_fn, k):
    cfg = cfg_fn()
    W = wl.make_weights(cfg, seed=2)
    rng = np.random.default_rng(11)
    toks = rng.integers(0, cfg.vocab, size=12)
    full = oracle.forward(cfg, W, toks)
    cache = oracle.KVCache(cfg.n_layer)
    part = [oracle.forward(cfg, W, toks[:k], cache)]
    for t in range(k, 12):
        part.append(oracle.decode_step(cfg, W, cache, toks[t])[None])
    np.testing.assert_allclose(np.concatenate(part), full, atol=1e-12)
    assert cache.length == 12


# ---------------------------------------------------------------- selection

def test_greedy_ties_lowest_index():
    assert oracle.greedy(np.array([0.0, 2.0, 1.0, 2.0])) == 1


def test_inverse_cdf_sampling_closed_form():
    lg = np.log(np.array([0.1, 0.2, 0.7]))
    assert oracle.sample(lg, 1.0, 0.05) == 0
    assert oracle.sample(lg, 1.0, 0.15) == 1
    assert oracle.sample(lg, 1.0, 0.2999) == 1
    assert oracle.sample(lg, 1.0, 0.31) == 2
    assert oracle.sample(lg, 1.0, 0.9999999) == 2
    # a uniform at or beyond the total falls back to the last index with p > 0
    assert oracle.sample(np.array([0.0, 0.0, -np.inf]), 1.0, 1.0) == 1


def test_temperature_limits():
    """Low temperature tends to argmax; entropy grows with temperature."""
    rng = np.random.default_rng(12)
    lg = rng.normal(size=200)
    top = int(np.argmax(lg))
    for u in (0.0, 0.3, 0.97):
        assert oracle.sample(lg, 1e-4, u) == top
    ent = []
    for T in (0.2, 0.5, 0.7, 1.0, 2.0):
        p = oracle.softmax(lg / T)
        ent.append(-(p * np.log(p)).sum())
    assert all(a < b for a, b in zip(ent, ent[1:]))
