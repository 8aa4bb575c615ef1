"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds no step of the decoder-block computation.  It only
describes model shapes, draws random weights and token streams from numpy's
PCG64 generator (``numpy.random.default_rng``), and rounds the drawn weights
to the storage precision of the model (bfloat16, round-to-nearest-even) so
that both sides start from bit-identical parameter values.

Shapes follow the five workloads of the build:

* ``tiny``       -- the microgpt layout: vocabulary 27 (26 lowercase letters
  plus BOS, microgpt HN summary, section "Tokenizer"), one layer, width 16,
  4 heads of 4, MLP 16->64->16 with ReLU, learned positions, 16 positions,
  batch 8, fp32 weights drawn N(0, 0.08).
* ``d12_prefill`` / ``d12_decode`` -- the depth-12 nanochat block
  (d_model 768, 6 query heads of 128, one K/V head, ReLU^2 MLP 768->3072),
  vocabulary 65536, bf16 weights N(0, 0.02).
* ``d26_prefill`` / ``d26_serving`` -- the depth-26 block (d_model 1664,
  13 query heads, MLP 1664->6656).

Weights are drawn in the fixed order WTE, WPE (learned positions only),
[Wq, Wk, Wv, Wo, W1, W2] for each layer, LM head, each as
``standard_normal(shape, float32) * sigma`` from ``default_rng(seed)``.
Token ids, prompt lengths and sampling uniforms come from
``default_rng(seed + 1)``.  Linear weights use the ``[out, in]`` row-major
convention (``y = W x``).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

POS_LEARNED = 0
POS_ROPE = 1
ACT_RELU = 0
ACT_RELU2 = 1
DTYPE_F32 = 0
DTYPE_BF16 = 1


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    """Field-for-field mirror of the C ``gpt_config`` struct."""

    vocab: int
    n_layer: int
    d_model: int
    n_head: int
    n_kv_head: int
    head_dim: int
    d_ff: int
    max_seq: int
    rope_base: float
    norm_eps: float
    pos_kind: int
    act: int
    qk_norm: int
    dtype: int
    init_std: float  # not part of the C struct: sigma of the weight draw

    @property
    def name(self) -> str:
        if self.dtype == DTYPE_F32:
            return f"tiny-v{self.vocab}-d{self.d_model}"
        return f"depth{self.d_model // 64}"


def tiny_model() -> ModelConfig:
    """microgpt layout: 4,192 parameters with learned positions, MHA, ReLU."""
    return ModelConfig(vocab=27, n_layer=1, d_model=16, n_head=4, n_kv_head=4,
                       head_dim=4, d_ff=64, max_seq=16, rope_base=10000.0,
                       norm_eps=1e-6, pos_kind=POS_LEARNED, act=ACT_RELU,
                       qk_norm=0, dtype=DTYPE_F32, init_std=0.08)


def depth_model(depth: int, max_seq: int = 4096, vocab: int = 65536) -> ModelConfig:
    """nanochat block sized by the single depth knob.

    Width is 64 per layer of depth and heads are 128 wide, which gives the
    768/6 and 1664/13 shapes of the depth-12 and depth-26 workloads.
    """
    d = 64 * depth
    if d % 128:
        raise ValueError("depth must be even so that d_model is a multiple of 128")
    return ModelConfig(vocab=vocab, n_layer=depth, d_model=d, n_head=d // 128,
                       n_kv_head=1, head_dim=128, d_ff=4 * d, max_seq=max_seq,
                       rope_base=10000.0, norm_eps=1e-6, pos_kind=POS_ROPE,
                       act=ACT_RELU2, qk_norm=1, dtype=DTYPE_BF16, init_std=0.02)


def small_model(n_layer: int, n_head: int, vocab: int = 65536,
                max_seq: int = 4096, n_kv_head: int = 1) -> ModelConfig:
    """A nanochat-style block with free layer/head counts for quick tests
    (n_kv_head > 1: grouped-query attention)."""
    d = 128 * n_head
    return ModelConfig(vocab=vocab, n_layer=n_layer, d_model=d, n_head=n_head,
                       n_kv_head=n_kv_head, head_dim=128, d_ff=4 * d, max_seq=max_seq,
                       rope_base=10000.0, norm_eps=1e-6, pos_kind=POS_ROPE,
                       act=ACT_RELU2, qk_norm=1, dtype=DTYPE_BF16, init_std=0.02)


# ---------------------------------------------------------------- weights

def round_to_bf16_(a: np.ndarray) -> np.ndarray:
    """Round a float32 array in place to the nearest bfloat16 value (ties to even)."""
    assert a.dtype == np.float32 and a.flags.c_contiguous
    u = a.view(np.uint32)
    bias = (u >> np.uint32(16)) & np.uint32(1)
    bias += np.uint32(0x7FFF)
    u += bias
    u &= np.uint32(0xFFFF0000)
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of a float32 array whose values are bf16-exact."""
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def weight_shapes(cfg: ModelConfig):
    """(name, shape) list in draw order."""
    d, dh = cfg.d_model, cfg.head_dim
    out = [("wte", (cfg.vocab, d))]
    if cfg.pos_kind == POS_LEARNED:
        out.append(("wpe", (cfg.max_seq, d)))
    for i in range(cfg.n_layer):
        out += [(f"layer{i}.wq", (cfg.n_head * dh, d)),
                (f"layer{i}.wk", (cfg.n_kv_head * dh, d)),
                (f"layer{i}.wv", (cfg.n_kv_head * dh, d)),
                (f"layer{i}.wo", (d, cfg.n_head * dh)),
                (f"layer{i}.w1", (cfg.d_ff, d)),
                (f"layer{i}.w2", (d, cfg.d_ff))]
    out.append(("lm_head", (cfg.vocab, d)))
    return out


@dataclasses.dataclass
class Weights:
    wte: np.ndarray
    wpe: Optional[np.ndarray]
    layers: List[dict]
    lm_head: np.ndarray

    def flat(self):
        yield "wte", self.wte
        if self.wpe is not None:
            yield "wpe", self.wpe
        for i, lw in enumerate(self.layers):
            for k in ("wq", "wk", "wv", "wo", "w1", "w2"):
                yield f"layer{i}.{k}", lw[k]
        yield "lm_head", self.lm_head


def make_weights(cfg: ModelConfig, seed: int = 0) -> Weights:
    rng = np.random.default_rng(seed)
    sigma = np.float32(cfg.init_std)
    arrays = {}
    for name, shape in weight_shapes(cfg):
        a = rng.standard_normal(size=shape, dtype=np.float32)
        a *= sigma
        if cfg.dtype == DTYPE_BF16:
            round_to_bf16_(a)
        arrays[name] = a
    layers = [{k: arrays[f"layer{i}.{k}"] for k in ("wq", "wk", "wv", "wo", "w1", "w2")}
              for i in range(cfg.n_layer)]
    return Weights(wte=arrays["wte"], wpe=arrays.get("wpe"), layers=layers,
                   lm_head=arrays["lm_head"])


# ---------------------------------------------------------------- workloads

@dataclasses.dataclass
class Workload:
    name: str
    model: ModelConfig
    seqlens: np.ndarray            # int64 [n_seqs], prompt lengths
    tokens: np.ndarray             # int32 [sum(seqlens)], packed prompts
    decode_steps: int = 0
    temperature: float = 0.0       # <= 0: greedy
    uniforms: Optional[np.ndarray] = None   # float32 [decode_steps + 1, n_seqs]
    logits_rows: str = "all"       # "all" positions or "last" per sequence

    @property
    def n_seqs(self) -> int:
        return int(len(self.seqlens))

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)

    def seq_tokens(self, b: int) -> np.ndarray:
        cu = self.cu_seqlens
        return self.tokens[cu[b]:cu[b + 1]]

    def next_token_targets(self) -> np.ndarray:
        """int32 [sum(seqlens)]: the token that follows each position within
        its sequence, -1 at each sequence's last position."""
        t = np.full(len(self.tokens), -1, np.int32)
        cu = self.cu_seqlens
        for b in range(self.n_seqs):
            t[cu[b]:cu[b + 1] - 1] = self.tokens[cu[b] + 1:cu[b + 1]]
        return t


def tiny_workload(seed: int = 0) -> Workload:
    """8 sequences of 16: position 0 is BOS (id 26), the rest uniform on [0, 27)."""
    cfg = tiny_model()
    rng = np.random.default_rng(seed + 1)
    toks = rng.integers(0, cfg.vocab, size=(8, 16)).astype(np.int32)
    toks[:, 0] = 26
    return Workload("tiny", cfg, np.full(8, 16, np.int64), toks.reshape(-1))


def uniform_prefill(cfg: ModelConfig, batch: int, seq: int, seed: int = 0,
                    name: str = "prefill") -> Workload:
    rng = np.random.default_rng(seed + 1)
    toks = rng.integers(0, cfg.vocab, size=(batch, seq)).astype(np.int32)
    return Workload(name, cfg, np.full(batch, seq, np.int64), toks.reshape(-1))


def ragged_prefill(cfg: ModelConfig, seqlens, seed: int = 0,
                   name: str = "ragged") -> Workload:
    rng = np.random.default_rng(seed + 1)
    lens = np.asarray(seqlens, np.int64)
    toks = rng.integers(0, cfg.vocab, size=int(lens.sum())).astype(np.int32)
    return Workload(name, cfg, lens, toks)


def d12_prefill(seed: int = 0) -> Workload:
    """Depth-12 prefill: 8 sequences of 2048 uniform tokens, logits at every position."""
    return uniform_prefill(depth_model(12), 8, 2048, seed, "d12_prefill")


def d12_decode(seed: int = 0, steps: int = 256) -> Workload:
    """Depth-12 decode: 32 prompts of 512, then greedy steps of one token each."""
    w = uniform_prefill(depth_model(12), 32, 512, seed, "d12_decode")
    w.decode_steps = steps
    w.logits_rows = "last"
    return w


def d26_prefill(seed: int = 0) -> Workload:
    """Depth-26 prefill: 16 sequences of 2048 uniform tokens."""
    return uniform_prefill(depth_model(26), 16, 2048, seed, "d26_prefill")


def d26_serving(seed: int = 0, steps: int = 512) -> Workload:
    """Depth-26 serving: 64 prompts with lengths uniform on [64, 2048], then
    ``steps`` sampled decode steps at temperature 0.7 from pre-drawn uniforms."""
    cfg = depth_model(26)
    rng = np.random.default_rng(seed + 1)
    lens = rng.integers(64, 2049, size=64).astype(np.int64)
    toks = rng.integers(0, cfg.vocab, size=int(lens.sum())).astype(np.int32)
    # one uniform per token choice: row 0 picks the token after the prompt,
    # row s + 1 the token after decode step s
    u = rng.random((513, 64)).astype(np.float32)[:steps + 1]
    return Workload("d26_serving", cfg, lens, toks, decode_steps=steps,
                    temperature=0.7, uniforms=np.ascontiguousarray(u),
                    logits_rows="last")


WORKLOADS = {
    "tiny": tiny_workload,
    "d12_prefill": d12_prefill,
    "d12_decode": d12_decode,
    "d26_prefill": d26_prefill,
    "d26_serving": d26_serving,
}
