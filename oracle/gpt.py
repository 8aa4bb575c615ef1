"""Plain numpy oracle of the decoder-block forward pass (prefill and decode).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Shares no code with
the HIP path.

Notation: ``d`` model width, ``H`` query heads, ``Hkv`` key/value heads,
``dh`` head width, ``F`` MLP width, ``V`` vocabulary, ``T`` positions.
Linear weights are ``[out, in]`` so a projection is ``y = W x``.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "READINGS", "rmsnorm", "rope_angles", "rope_tables", "apply_rope",
    "relu", "relu2", "softmax", "logsumexp", "causal_attention", "KVCache",
    "embed", "block", "final_logits", "forward", "prefill", "decode_step",
    "greedy", "sample", "cross_entropy", "token_losses", "mean_loss", "adam_step",
    "loss_and_grads", "param_count",
    "round_bf16",
    "run_serving",
]

# Points the pages leave open, and the reading taken for each.  Both sides
# implement these independently.
READINGS = {
    "layout": "microgpt: learned token and position embeddings, untied LM head, "
              "MHA with as many K/V heads as query heads, ReLU MLP 4x wide, no "
              "biases and no norm gains -- the only layout giving 4,192 parameters",
    "norm_placement": "pre-norm: RMSNorm before attention, before the MLP and "
                      "before the LM head; none right after the embedding",
    "norm_eps": "1e-6 inside the square root, for every norm including QK-norm",
    "rope": "half-split pairs (i, i + dh/2) rotated counter-clockwise by "
            "t * base**(-2i/dh), t the 0-based absolute position",
    "qk_norm_order": "RoPE then a weightless RMSNorm over each head vector "
                     "(the two commute up to rounding)",
    "attention": "scale 1/sqrt(dh), key j visible from position t iff j <= t, "
                 "no softcap, no dropout; query head h reads K/V head "
                 "floor(h * Hkv / H)",
    "argmax_ties": "lowest index wins",
    "sampling": "p = softmax(logits / T); token = min{i : cumsum(p)_i > u}; if "
                "rounding leaves sum(p) <= u, the last index with p > 0",
}


# ------------------------------------------------------------------ pieces

def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 value, ties to even (returns float64).

    Used only to measure the bf16 storage noise floor: the oracle proper
    never rounds activations.
    """
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def rmsnorm(z: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm with no learnable gain over the last axis.

    Microgpt, section "Core architecture": RMSNorm replaces LayerNorm and
    there are no bias terms; with no room for gains in the 4,192-parameter
    count, the norm has no weight.  ``z / sqrt(mean(z^2) + eps)``.
    """
    ms = np.mean(z * z, axis=-1, keepdims=True)
    return z / np.sqrt(ms + eps)


def rope_angles(max_seq: int, head_dim: int, base: float) -> np.ndarray:
    """Rotation angle of pair i at position t: ``t * base**(-2 i / head_dim)``.

    NanoChat launch, tricks section: rotary embeddings are precomputed once
    as cos/sin tables because they depend on no trained parameter.  The
    frequency ladder is the standard rotary one (a reading: the pages give no
    formula).  Returns float64 ``[max_seq, head_dim // 2]``.
    """
    half = head_dim // 2
    inv_freq = np.power(float(base), -2.0 * np.arange(half, dtype=np.float64) / head_dim)
    t = np.arange(max_seq, dtype=np.float64)
    return np.outer(t, inv_freq)


def rope_tables(max_seq: int, head_dim: int, base: float):
    """cos and sin of ``rope_angles`` in float64 (tricks section, NanoChat launch)."""
    ang = rope_angles(max_seq, head_dim, base)
    return np.cos(ang), np.sin(ang)


def apply_rope(u: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Half-split rotary embedding of head vectors.

    NanoChat launch, tricks section: the vector is split into two halves, the
    halves are rotated with a rotation matrix, and the result is concatenated
    back.  Pair i is ``(u[i], u[i + dh/2])`` and is turned counter-clockwise
    by its angle: ``(a, b) -> (a cos - b sin, a sin + b cos)``.

    ``u``: ``[T, heads, dh]``; ``cos``/``sin``: ``[T, dh/2]`` (rows already
    selected for the positions of ``u``).
    """
    half = u.shape[-1] // 2
    a, b = u[..., :half], u[..., half:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def relu(z: np.ndarray) -> np.ndarray:
    """ReLU, used instead of GeLU (Microgpt, section "Core architecture")."""
    return np.maximum(z, 0.0)


def relu2(z: np.ndarray) -> np.ndarray:
    """ReLU squared (NanoChat launch, tricks section): ``max(z, 0)^2``."""
    r = np.maximum(z, 0.0)
    return r * r


def logsumexp(s: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(s, axis=axis, keepdims=True)
    return (m + np.log(np.sum(np.exp(s - m), axis=axis, keepdims=True))).squeeze(axis)


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    """Softmax: values in [0, 1] that sum to 1 (Microgpt, "Core architecture", item 2).

    Written with the usual max shift, which leaves the result unchanged.
    """
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_start: int,
                     bf16_p: bool = False) -> np.ndarray:
    """Causal multi-query / multi-head attention for one sequence.

    Microgpt, "Core architecture", item 4: the token at the current position
    reads information from earlier positions through query, key and value
    vectors.  nanochat hand-written page: multi-query attention, one K/V head
    shared by every query head.  Query head ``h`` uses K/V head
    ``h * Hkv // H``; query row ``i`` sits at absolute position
    ``q_start + i`` and sees keys ``j <= q_start + i``; scores are scaled by
    ``1/sqrt(dh)`` and normalised with ``softmax``.

    ``q``: ``[Tq, H, dh]``, ``k``/``v``: ``[Tk, Hkv, dh]`` -> ``[Tq, H, dh]``.
    ``bf16_p`` (noise-floor probe only) rounds the unnormalised
    probabilities to bf16 before they weight V, as a bf16 MFMA path does.
    """
    tq, n_head, dh = q.shape
    tk, n_kv, _ = k.shape
    out = np.empty_like(q)
    scale = 1.0 / math.sqrt(dh)
    pos_q = q_start + np.arange(tq)
    visible = np.arange(tk)[None, :] <= pos_q[:, None]          # [Tq, Tk]
    for h in range(n_head):
        g = h * n_kv // n_head
        s = (q[:, h, :] @ k[:, g, :].T) * scale                 # [Tq, Tk]
        s = np.where(visible, s, -np.inf)
        if bf16_p:
            m = np.max(s, axis=-1, keepdims=True)
            e = np.exp(s - m)
            out[:, h, :] = (round_bf16(e).astype(q.dtype) @ v[:, g, :]) / np.sum(e, -1, keepdims=True)
        else:
            out[:, h, :] = softmax(s, axis=-1) @ v[:, g, :]
    return out


class KVCache:
    """Per-layer keys and values of the positions seen so far.

    NanoChat launch, tricks section: a KV cache speeds up inference, and the
    code branches on whether the cache is present.  Microgpt, "Core
    architecture", item 7: cached states of earlier positions.  Keys are
    stored after RoPE and QK-norm, exactly as attention reads them.
    """

    def __init__(self, n_layer: int):
        self.k: List[Optional[np.ndarray]] = [None] * n_layer
        self.v: List[Optional[np.ndarray]] = [None] * n_layer

    @property
    def length(self) -> int:
        return 0 if self.k[0] is None else int(self.k[0].shape[0])


# ------------------------------------------------------------------ model

def _linear(x: np.ndarray, w: np.ndarray, dtype) -> np.ndarray:
    """``y = W x`` for each row of ``x`` with ``W`` stored ``[out, in]``."""
    return x @ w.astype(dtype, copy=False).T


def embed(cfg, W, tokens: np.ndarray, positions: np.ndarray, dtype=np.float64):
    """Token embedding plus learned position embedding when the layout has one.

    Microgpt, "Core architecture", item 3: token ids and position ids are
    turned into vectors that carry what the token is and where it sits.
    The nanochat blocks use rotary embeddings instead of a position table.
    """
    x = W.wte[tokens].astype(dtype)
    if cfg.pos_kind == 0:
        x = x + W.wpe[positions].astype(dtype)
    return x


def block(cfg, lw: dict, x: np.ndarray, positions: np.ndarray, cache: Optional[KVCache],
          layer: int, tables, dtype=np.float64, bf16_points: bool = False) -> np.ndarray:
    """One pre-norm decoder block: ``x += Attn(rms(x)); x += MLP(rms(x))``.

    * Microgpt, "Core architecture": RMSNorm, no biases, residual
      connections around attention and the MLP (items 6), a two-layer MLP
      (item 5) with ReLU.
    * NanoChat launch, tricks section: separate Q, K, V linear layers;
      ReLU^2 in the MLP; precomputed rotary tables.
    * nanochat hand-written page: rotary positions, QK normalisation,
      multi-query attention.

    ``positions`` are the absolute positions of the rows of ``x`` (one
    sequence); when ``cache`` is given the new K/V rows are appended to it
    and attention reads the whole cache (decode equals recompute).
    ``bf16_points`` rounds to bf16 where a bf16 GPU path stores operands
    (noise-floor probe only).
    """
    rb = (lambda a: round_bf16(a).astype(dtype)) if bf16_points else (lambda a: a)
    t = x.shape[0]
    n_head, n_kv, dh = cfg.n_head, cfg.n_kv_head, cfg.head_dim
    h = rb(rmsnorm(x, cfg.norm_eps))
    q = _linear(h, lw["wq"], dtype).reshape(t, n_head, dh)
    k = _linear(h, lw["wk"], dtype).reshape(t, n_kv, dh)
    v = _linear(h, lw["wv"], dtype).reshape(t, n_kv, dh)
    if cfg.pos_kind == 1:
        cos, sin = tables
        q = apply_rope(q, cos[positions].astype(dtype), sin[positions].astype(dtype))
        k = apply_rope(k, cos[positions].astype(dtype), sin[positions].astype(dtype))
    if cfg.qk_norm:
        q = rmsnorm(q, cfg.norm_eps)
        k = rmsnorm(k, cfg.norm_eps)
    q, k, v = rb(q), rb(k), rb(v)
    if cache is not None:
        if cache.k[layer] is not None:
            k = np.concatenate([cache.k[layer], k], axis=0)
            v = np.concatenate([cache.v[layer], v], axis=0)
        cache.k[layer], cache.v[layer] = k, v
    o = causal_attention(q, k, v, int(positions[0]), bf16_p=bf16_points)
    x = x + _linear(rb(o.reshape(t, n_head * dh)), lw["wo"], dtype)
    h2 = rb(rmsnorm(x, cfg.norm_eps))
    z = _linear(h2, lw["w1"], dtype)
    u = rb(relu2(z) if cfg.act == 1 else relu(z))
    return x + _linear(u, lw["w2"], dtype)


def final_logits(cfg, W, x: np.ndarray, dtype=np.float64, bf16_points: bool = False):
    """Final RMSNorm then the untied LM head, ``logits = W_lm rms(x)``.

    Microgpt, "Model parameters": a final output projection separate from
    the embedding table (the 4,192 count needs it untied); NanoChat launch,
    tricks section: the LM head is its own optimiser group.
    """
    hf = rmsnorm(x, cfg.norm_eps)
    if bf16_points:
        hf = round_bf16(hf).astype(dtype)
    return _linear(hf, W.lm_head, dtype)


def forward(cfg, W, tokens: Sequence[int], cache: Optional[KVCache] = None,
            dtype=np.float64, bf16_points: bool = False, rows: str = "all",
            tables=None) -> np.ndarray:
    """Logits of one sequence chunk ``tokens`` at positions ``cache.length + i``.

    With ``cache=None`` this is a full-sequence forward from position 0;
    with a cache it continues from the cached length (prefill into a cache,
    or one decode step).  ``rows="last"`` returns only the last row.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    start = 0 if cache is None else cache.length
    positions = start + np.arange(len(tokens))
    if tables is None and cfg.pos_kind == 1:
        tables = rope_tables(max(int(positions[-1]) + 1, 1), cfg.head_dim, cfg.rope_base)
    x = embed(cfg, W, tokens, positions, dtype)
    for i, lw in enumerate(W.layers):
        x = block(cfg, lw, x, positions, cache, i, tables, dtype, bf16_points)
    if rows == "last":
        x = x[-1:]
    return final_logits(cfg, W, x, dtype, bf16_points)


def prefill(cfg, W, tokens, seqlens, dtype=np.float64, rows: str = "all",
            with_cache: bool = False, seqs: Optional[Sequence[int]] = None,
            bf16_points: bool = False):
    """Run ``forward`` for each packed sequence (or the subset ``seqs``).

    Returns ``(logits_list, caches)``; ``caches`` is None unless requested.
    """
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64)
    idx = range(len(seqlens)) if seqs is None else seqs
    tables = None
    if cfg.pos_kind == 1:
        tables = rope_tables(cfg.max_seq, cfg.head_dim, cfg.rope_base)
    out, caches = [], []
    for b in idx:
        cache = KVCache(cfg.n_layer) if with_cache else None
        out.append(forward(cfg, W, tokens[cu[b]:cu[b + 1]], cache, dtype, bf16_points,
                           rows, tables))
        caches.append(cache)
    return out, (caches if with_cache else None)


def decode_step(cfg, W, cache: KVCache, token: int, dtype=np.float64, tables=None):
    """One KV-cache decode step: the logits of the next position.

    CSDN walkthrough: a custom Engine with a KV cache and separate prefill
    and decode; Microgpt, "Inference": feed the sampled token back in.
    """
    return forward(cfg, W, [int(token)], cache, dtype, tables=tables)[0]


def greedy(logits: np.ndarray) -> np.ndarray:
    """Argmax over the vocabulary; ties go to the lowest index."""
    return np.argmax(logits, axis=-1)


def sample(logits: np.ndarray, temperature: float, u: float) -> int:
    """Temperature sampling by inverse CDF with a given uniform ``u``.

    Microgpt, "Inference": sample the next token from the predicted
    distribution; a lower temperature sharpens it.  ``p = softmax(logits/T)``
    in float64, ``token = min{i : sum_{j<=i} p_j > u}``.
    """
    p = softmax(np.asarray(logits, np.float64) / float(temperature))
    c = np.cumsum(p)
    hit = np.nonzero(c > float(u))[0]
    if len(hit):
        return int(hit[0])
    return int(np.nonzero(p > 0)[0][-1])


def cross_entropy(logits: np.ndarray, targets: np.ndarray) -> float:
    """Mean next-token cross-entropy (Microgpt, "Training"): how surprised the
    model is by the real next token."""
    lse = logsumexp(logits, axis=-1)
    return float(np.mean(lse - logits[np.arange(len(targets)), targets]))


def token_losses(logits: np.ndarray, targets: np.ndarray) -> np.ndarray:
    """Per-row next-token cross-entropy (Microgpt, "Training process", item 2):
    the negative log-probability the model gives the real next token,
    ``loss[r] = logsumexp(logits[r]) - logits[r, targets[r]]``, in float64.

    A target outside ``[0, V)`` marks a row with no next token (a sequence's
    last position); its loss is 0.
    """
    lg = np.asarray(logits, np.float64)
    t = np.asarray(targets, np.int64)
    V = lg.shape[-1]
    ok = (t >= 0) & (t < V)
    out = np.zeros(len(t), np.float64)
    rows = np.nonzero(ok)[0]
    out[rows] = logsumexp(lg[rows], axis=-1) - lg[rows, t[rows]]
    return out


def mean_loss(losses: np.ndarray, targets: np.ndarray, vocab: int) -> float:
    """Mean of ``token_losses`` over the rows that have a target (0 if none)."""
    t = np.asarray(targets, np.int64)
    ok = (t >= 0) & (t < vocab)
    return float(np.mean(np.asarray(losses, np.float64)[ok])) if ok.any() else 0.0


def adam_step(param: np.ndarray, grad: np.ndarray, m: np.ndarray, v: np.ndarray, step: int,
              lr: float, beta1: float, beta2: float, eps: float):
    """One Adam update (Microgpt, "Training process", item 4): running means
    of the gradient (momentum) and of its square (a per-parameter step
    size), each divided by its start-up bias ``1 - beta**step``, in float64.

    Returns ``(param, m, v)`` after the step; the inputs are not modified.
    """
    p = np.asarray(param, np.float64)
    g = np.asarray(grad, np.float64)
    m1 = beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * g
    v1 = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * g * g
    mhat = m1 / (1.0 - beta1 ** step)
    vhat = v1 / (1.0 - beta2 ** step)
    return p - lr * mhat / (np.sqrt(vhat) + eps), m1, v1


# ------------------------------------------------------------------ backward

def _rms_backward(x: np.ndarray, dy: np.ndarray, eps: float) -> np.ndarray:
    """Gradient through ``y = x / sqrt(mean(x^2) + eps)`` over the last axis:
    ``dx = (dy - y * mean(dy * y)) / r``."""
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    y = x / r
    return (dy - y * np.mean(dy * y, axis=-1, keepdims=True)) / r


def _rope_backward(du: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Gradient through ``apply_rope``: the transpose of a rotation turns the
    pair back by the same angle."""
    half = du.shape[-1] // 2
    a, b = du[..., :half], du[..., half:]
    c, s = cos[:, None, :], sin[:, None, :]
    return np.concatenate([a * c + b * s, -a * s + b * c], axis=-1)


def loss_and_grads(cfg, W, tokens, seqlens, targets):
    """Mean next-token cross-entropy of packed sequences and its gradient
    with respect to every weight, in float64 (Microgpt, "Training process",
    items 2 and 3: the forward pass and its loss, then the chain rule run
    backwards from the loss to every parameter).

    The loss is ``mean_loss(token_losses(logits, targets))`` over the rows
    whose target lies in ``[0, V)``; its gradient with respect to row r's
    logits is ``(softmax(logits[r]) - onehot(target)) / count``.  The backward
    retraces ``block``: RMSNorm, the three projections, RoPE, QK-norm,
    attention with each query head on K/V head ``h * Hkv // H``, the output
    projection, the MLP and the residual adds, then the final norm and the
    LM head.  Returns ``(mean_loss, grads)`` with ``grads`` keyed like
    ``W.flat()`` plus ``"lm_head"``.
    """
    f = np.float64
    eps = cfg.norm_eps
    n_head, n_kv, dh = cfg.n_head, cfg.n_kv_head, cfg.head_dim
    tables = rope_tables(cfg.max_seq, dh, cfg.rope_base) if cfg.pos_kind == 1 else None
    targets = np.asarray(targets, np.int64)
    V = cfg.vocab
    count = int(np.sum((targets >= 0) & (targets < V)))
    g = {"wte": np.zeros(W.wte.shape), "lm_head": np.zeros(W.lm_head.shape)}
    if W.wpe is not None:
        g["wpe"] = np.zeros(W.wpe.shape)
    for i, lw in enumerate(W.layers):
        for k in ("wq", "wk", "wv", "wo", "w1", "w2"):
            g[f"layer{i}.{k}"] = np.zeros(lw[k].shape)
    total = 0.0
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64)
    for b in range(len(seqlens)):
        tok = np.asarray(tokens[cu[b]:cu[b + 1]], np.int64)
        tg = targets[cu[b]:cu[b + 1]]
        t = len(tok)
        pos = np.arange(t)
        x = embed(cfg, W, tok, pos, f)
        saved = []
        for lw in W.layers:
            c = {"x": x}
            h = rmsnorm(x, eps)
            qr = _linear(h, lw["wq"], f).reshape(t, n_head, dh)
            kr = _linear(h, lw["wk"], f).reshape(t, n_kv, dh)
            v = _linear(h, lw["wv"], f).reshape(t, n_kv, dh)
            if tables is not None:
                cs, sn = tables[0][pos], tables[1][pos]
                qr, kr = apply_rope(qr, cs, sn), apply_rope(kr, cs, sn)
            q = rmsnorm(qr, eps) if cfg.qk_norm else qr
            k = rmsnorm(kr, eps) if cfg.qk_norm else kr
            o = causal_attention(q, k, v, 0)
            c.update(h=h, qr=qr, kr=kr, q=q, k=k, v=v, o=o.reshape(t, n_head * dh))
            x = x + _linear(c["o"], lw["wo"], f)
            c["xm"] = x
            h2 = rmsnorm(x, eps)
            z = _linear(h2, lw["w1"], f)
            u = relu2(z) if cfg.act == 1 else relu(z)
            c.update(h2=h2, z=z, u=u)
            x = x + _linear(u, lw["w2"], f)
            saved.append(c)
        hf = rmsnorm(x, eps)
        logits = _linear(hf, W.lm_head, f)
        losses = token_losses(logits, tg)
        total += float(np.sum(losses))
        ok = (tg >= 0) & (tg < V)
        dlog = softmax(logits)
        dlog[np.nonzero(ok)[0], tg[ok]] -= 1.0
        dlog[~ok] = 0.0
        dlog /= max(count, 1)
        g["lm_head"] += dlog.T @ hf
        dx = _rms_backward(x, dlog @ W.lm_head.astype(f), eps)
        scale = 1.0 / math.sqrt(dh)
        visible = pos[None, :] <= pos[:, None]
        for i in reversed(range(len(W.layers))):
            lw, c = W.layers[i], saved[i]
            # MLP: x += W2 act(W1 rms(xm))
            g[f"layer{i}.w2"] += dx.T @ c["u"]
            du = dx @ lw["w2"].astype(f)
            dz = du * (2.0 * np.maximum(c["z"], 0.0) if cfg.act == 1 else (c["z"] > 0).astype(f))
            g[f"layer{i}.w1"] += dz.T @ c["h2"]
            dx = dx + _rms_backward(c["xm"], dz @ lw["w1"].astype(f), eps)
            # attention: x += Wo o
            g[f"layer{i}.wo"] += dx.T @ c["o"]
            do = (dx @ lw["wo"].astype(f)).reshape(t, n_head, dh)
            q, k, v = c["q"], c["k"], c["v"]
            dq = np.zeros_like(q)
            dk = np.zeros_like(k)
            dv = np.zeros_like(v)
            for hh in range(n_head):
                gk = hh * n_kv // n_head
                sc = np.where(visible, (q[:, hh] @ k[:, gk].T) * scale, -np.inf)
                p = softmax(sc, axis=-1)
                dp = do[:, hh] @ v[:, gk].T
                ds = p * (dp - np.sum(dp * p, axis=-1, keepdims=True))
                dq[:, hh] = ds @ k[:, gk] * scale
                dk[:, gk] += ds.T @ q[:, hh] * scale
                dv[:, gk] += p.T @ do[:, hh]
            if cfg.qk_norm:
                dq = _rms_backward(c["qr"], dq, eps)
                dk = _rms_backward(c["kr"], dk, eps)
            if tables is not None:
                cs, sn = tables[0][pos], tables[1][pos]
                dq, dk = _rope_backward(dq, cs, sn), _rope_backward(dk, cs, sn)
            dq, dk, dv = dq.reshape(t, -1), dk.reshape(t, -1), dv.reshape(t, -1)
            h = c["h"]
            g[f"layer{i}.wq"] += dq.T @ h
            g[f"layer{i}.wk"] += dk.T @ h
            g[f"layer{i}.wv"] += dv.T @ h
            dh_ = dq @ lw["wq"].astype(f) + dk @ lw["wk"].astype(f) + dv @ lw["wv"].astype(f)
            dx = dx + _rms_backward(c["x"], dh_, eps)
        np.add.at(g["wte"], tok, dx)
        if W.wpe is not None:
            np.add.at(g["wpe"], pos, dx)
    return total / max(count, 1), g


def param_count(W) -> int:
    """Number of scalars the oracle's forward reads from ``W``."""
    n = W.wte.size + W.lm_head.size + (W.wpe.size if W.wpe is not None else 0)
    for lw in W.layers:
        n += sum(lw[k].size for k in ("wq", "wk", "wv", "wo", "w1", "w2"))
    return int(n)


def run_serving(cfg, W, tokens, seqlens, steps: int, temperature: float = 0.0,
                uniforms: Optional[np.ndarray] = None, forced: Optional[np.ndarray] = None,
                dtype=np.float64, seqs: Optional[Sequence[int]] = None,
                bf16_points: bool = False):
    """Prefill each prompt into a cache, then decode ``steps`` tokens.

    The first new token comes from the last prompt position's logits; each
    step feeds the previous token back at the next position.  With
    ``forced`` (``[steps + 1, n_seqs]``) the oracle consumes those tokens
    instead of its own choices (teacher forcing), so per-step logits stay
    comparable with another implementation after a near-tie.

    Returns ``(chosen [steps+1, n], logits [steps+1, n, V])`` for the
    selected sequences.  ``bf16_points`` (noise-floor probe only) rounds at the
    bf16 storage points as in ``block``.
    """
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int64)
    idx = list(range(len(seqlens)) if seqs is None else seqs)
    tables = None
    if cfg.pos_kind == 1:
        tables = rope_tables(cfg.max_seq, cfg.head_dim, cfg.rope_base)
    caches = []
    last = []
    for b in idx:
        c = KVCache(cfg.n_layer)
        last.append(forward(cfg, W, tokens[cu[b]:cu[b + 1]], c, dtype, bf16_points, rows="last",
                            tables=tables)[0])
        caches.append(c)
    chosen = np.zeros((steps + 1, len(idx)), np.int64)
    all_logits = np.zeros((steps + 1, len(idx), cfg.vocab), dtype)
    cur = np.stack(last)
    for s in range(steps + 1):
        all_logits[s] = cur
        for j in range(len(idx)):
            if temperature <= 0:
                chosen[s, j] = greedy(cur[j])
            else:
                chosen[s, j] = sample(cur[j], temperature, float(uniforms[s, idx[j]]))
        if s == steps:
            break
        feed = chosen[s] if forced is None else forced[s, idx]
        cur = np.stack([forward(cfg, W, [int(feed[j])], caches[j], dtype, bf16_points, rows="last",
                                tables=tables)[0] for j in range(len(idx))])
    return chosen, all_logits
