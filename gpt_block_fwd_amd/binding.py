"""ctypes binding of libgpt.so (include/gpt.h, include/gpt_profile.h).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels of libgpt.so.  PyTorch is used for device memory and streams; the
library must be built (``python -m gpt_block_fwd_amd.build``) and a missing
library is an error, never a silent fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgpt.so")

GPT_OK, GPT_ERR_ARG, GPT_ERR_CAPACITY, GPT_ERR_UNSUPPORTED, GPT_ERR_HIP = range(5)
ROWS_ALL, ROWS_LAST = 0, 1
STATUS_NAMES = {0: "GPT_OK", 1: "GPT_ERR_ARG", 2: "GPT_ERR_CAPACITY", 3: "GPT_ERR_UNSUPPORTED",
                4: "GPT_ERR_HIP"}

PROF_CLASSES = {"gemm": 0, "lmhead": 1, "attn": 2, "decode_attn": 3, "skinny": 4, "norm": 5,
                "softmax": 6, "optim": 7, "bwd_gemm": 8, "bwd_attn": 9, "bwd_other": 10}

#: every entry point declared by include/gpt.h and include/gpt_profile.h
EXPORTS = ("gpt_last_error", "rope_tables", "kv_cache_alloc", "kv_cache_free",
           "kv_cache_lengths", "gpt_workspace_bytes", "gpt_prefill", "gpt_prefill_loss",
           "gpt_decode_step", "gpt_decode_step_noalloc",
           "gpt_select_tokens", "gpt_train_workspace_bytes", "gpt_loss_grads", "gpt_adam_step",
           "gpt_profile_enable", "gpt_profile_mask", "gpt_profile_read", "gpt_profile_read_launch",
           "gpt_debug_gemm", "gpt_debug_attn_prefill")


class GptError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class GptConfig(ctypes.Structure):
    _fields_ = [("vocab", ctypes.c_int32), ("n_layer", ctypes.c_int32),
                ("d_model", ctypes.c_int32), ("n_head", ctypes.c_int32),
                ("n_kv_head", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("max_seq", ctypes.c_int32),
                ("rope_base", ctypes.c_float), ("norm_eps", ctypes.c_float),
                ("pos_kind", ctypes.c_int32), ("act", ctypes.c_int32),
                ("qk_norm", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_PP = ctypes.POINTER(ctypes.c_void_p)


class GptWeights(ctypes.Structure):
    _fields_ = [("wte", ctypes.c_void_p), ("wpe", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("wq", _PP), ("wk", _PP), ("wv", _PP), ("wo", _PP), ("w1", _PP), ("w2", _PP)]


class GptGrads(ctypes.Structure):
    _fields_ = [("wte", ctypes.c_void_p), ("wpe", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("wq", _PP), ("wk", _PP), ("wv", _PP), ("wo", _PP), ("w1", _PP), ("w2", _PP)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libgpt.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m gpt_block_fwd_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    cfgp = ctypes.POINTER(GptConfig)
    L.gpt_last_error.restype = ctypes.c_char_p
    L.rope_tables.argtypes = [i32, i32, f32, vp, vp, vp]
    L.kv_cache_alloc.argtypes = [cfgp, i32, i32, i32, vp, ctypes.POINTER(sz), ctypes.POINTER(vp)]
    L.kv_cache_free.argtypes = [vp]
    L.kv_cache_lengths.argtypes = [vp, vp]
    L.gpt_workspace_bytes.argtypes = [cfgp, i32, i32]
    L.gpt_workspace_bytes.restype = sz
    L.gpt_prefill.argtypes = [cfgp, ctypes.POINTER(GptWeights), vp, vp, vp, vp, i32, vp, i32,
                              vp, vp, vp, vp, sz, vp]
    L.gpt_prefill_loss.argtypes = [cfgp, ctypes.POINTER(GptWeights), vp, vp, vp, vp, vp, i32, vp,
                                   vp, vp, vp, vp, sz, vp]
    L.gpt_decode_step.argtypes = [cfgp, ctypes.POINTER(GptWeights), vp, vp, vp, vp, f32, vp, vp,
                                  vp, vp, sz, vp]
    L.gpt_decode_step_noalloc.argtypes = [cfgp, ctypes.POINTER(GptWeights), vp, vp, vp, vp, f32, vp,
                                          vp, vp, vp]
    L.gpt_select_tokens.argtypes = [vp, i32, i32, f32, vp, vp, vp]
    L.gpt_adam_step.argtypes = [vp, vp, vp, vp, vp, ctypes.c_int64, i32, f32, f32, f32, f32, vp]
    L.gpt_train_workspace_bytes.argtypes = [cfgp, i32, i32]
    L.gpt_train_workspace_bytes.restype = sz
    L.gpt_loss_grads.argtypes = [cfgp, ctypes.POINTER(GptWeights), vp, vp, vp, vp, vp, i32,
                                 ctypes.POINTER(GptGrads), vp, vp, vp, sz, vp]
    L.gpt_profile_enable.argtypes = [ctypes.c_uint32]
    L.gpt_profile_mask.argtypes = [ctypes.c_uint32]
    L.gpt_profile_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(ctypes.c_double)]
    L.gpt_profile_read_launch.argtypes = [i32, ctypes.c_int64, ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    L.gpt_debug_gemm.argtypes = [vp, vp, i32, i32, i32, vp, i32, i32, vp]
    L.gpt_debug_attn_prefill.argtypes = [vp, vp, vp, ctypes.c_int64, vp, i32, i32, i32, vp, vp, vp]
    for name in EXPORTS:
        if name not in ("gpt_last_error", "gpt_workspace_bytes", "gpt_train_workspace_bytes"):
            getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int):
    if status != GPT_OK:
        raise GptError(status, lib().gpt_last_error().decode())


def last_error() -> str:
    return lib().gpt_last_error().decode()


def make_config(m) -> GptConfig:
    """GptConfig from any object with the gpt_config field names."""
    return GptConfig(m.vocab, m.n_layer, m.d_model, m.n_head, m.n_kv_head, m.head_dim, m.d_ff,
                     m.max_seq, m.rope_base, m.norm_eps, m.pos_kind, m.act, m.qk_norm, m.dtype)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


# ------------------------------------------------------------------ entry points

def rope_tables(max_seq: int, head_dim: int, base: float, cos_out, sin_out, stream=None):
    _check(lib().rope_tables(max_seq, head_dim, base, _ptr(cos_out), _ptr(sin_out), _stream(stream)))


def kv_cache_bytes(cfg: GptConfig, n_seqs: int, capacity: int, page_size: int = 64) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().kv_cache_alloc(ctypes.byref(cfg), n_seqs, capacity, page_size, None,
                                ctypes.byref(n), None))
    return n.value


def kv_cache_alloc(cfg: GptConfig, n_seqs: int, capacity: int, device_buf, nbytes: int,
                   page_size: int = 64) -> int:
    n = ctypes.c_size_t(nbytes)
    h = ctypes.c_void_p()
    _check(lib().kv_cache_alloc(ctypes.byref(cfg), n_seqs, capacity, page_size, _ptr(device_buf),
                                ctypes.byref(n), ctypes.byref(h)))
    return h.value


def kv_cache_free(handle: int):
    _check(lib().kv_cache_free(handle))


def kv_cache_lengths(handle: int, n_seqs: int) -> np.ndarray:
    out = np.zeros(n_seqs, np.int32)
    _check(lib().kv_cache_lengths(handle, out.ctypes.data))
    return out


def gpt_workspace_bytes(cfg: GptConfig, max_tokens: int, max_seqs: int) -> int:
    return int(lib().gpt_workspace_bytes(ctypes.byref(cfg), max_tokens, max_seqs))


def gpt_prefill(cfg: GptConfig, weights: GptWeights, rope_cos, rope_sin, tokens,
                cu_seqlens: np.ndarray, n_seqs: int, kv: Optional[int], logits_rows: int, logits,
                lse, probs, workspace, workspace_bytes: int, stream=None):
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    _check(lib().gpt_prefill(ctypes.byref(cfg), ctypes.byref(weights), _ptr(rope_cos),
                             _ptr(rope_sin), _ptr(tokens), cu.ctypes.data, n_seqs, kv, logits_rows,
                             _ptr(logits), _ptr(lse), _ptr(probs), _ptr(workspace),
                             workspace_bytes, _stream(stream)))


def gpt_prefill_loss(cfg: GptConfig, weights: GptWeights, rope_cos, rope_sin, tokens, targets,
                     cu_seqlens: np.ndarray, n_seqs: int, kv: Optional[int], loss, lse, mean,
                     workspace, workspace_bytes: int, stream=None):
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    _check(lib().gpt_prefill_loss(ctypes.byref(cfg), ctypes.byref(weights), _ptr(rope_cos),
                                  _ptr(rope_sin), _ptr(tokens), _ptr(targets), cu.ctypes.data,
                                  n_seqs, kv, _ptr(loss), _ptr(lse), _ptr(mean), _ptr(workspace),
                                  workspace_bytes, _stream(stream)))


def gpt_decode_step(cfg: GptConfig, weights: GptWeights, rope_cos, rope_sin, kv: int, tokens_in,
                    temperature: float, uniforms, tokens_out, logits, workspace,
                    workspace_bytes: int, stream=None):
    _check(lib().gpt_decode_step(ctypes.byref(cfg), ctypes.byref(weights), _ptr(rope_cos),
                                 _ptr(rope_sin), kv, _ptr(tokens_in), temperature, _ptr(uniforms),
                                 _ptr(tokens_out), _ptr(logits), _ptr(workspace), workspace_bytes,
                                 _stream(stream)))


def gpt_decode_step_noalloc(cfg: GptConfig, weights: GptWeights, rope_cos, rope_sin, kv: int,
                            tokens_in, temperature: float, uniforms, tokens_out, logits, stream=None):
    _check(lib().gpt_decode_step_noalloc(ctypes.byref(cfg), ctypes.byref(weights), _ptr(rope_cos),
                                         _ptr(rope_sin), kv, _ptr(tokens_in), temperature,
                                         _ptr(uniforms), _ptr(tokens_out), _ptr(logits),
                                         _stream(stream)))


def gpt_select_tokens(logits, rows: int, vocab: int, temperature: float, uniforms, tokens_out,
                      stream=None):
    _check(lib().gpt_select_tokens(_ptr(logits), rows, vocab, temperature, _ptr(uniforms),
                                   _ptr(tokens_out), _stream(stream)))


def gpt_train_workspace_bytes(cfg: GptConfig, max_tokens: int, max_seqs: int) -> int:
    return int(lib().gpt_train_workspace_bytes(ctypes.byref(cfg), max_tokens, max_seqs))


def gpt_loss_grads(cfg: GptConfig, weights: GptWeights, rope_cos, rope_sin, tokens, targets,
                   cu_seqlens: np.ndarray, n_seqs: int, grads: GptGrads, loss, mean, workspace,
                   workspace_bytes: int, stream=None):
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    _check(lib().gpt_loss_grads(ctypes.byref(cfg), ctypes.byref(weights), _ptr(rope_cos),
                                _ptr(rope_sin), _ptr(tokens), _ptr(targets), cu.ctypes.data,
                                n_seqs, ctypes.byref(grads), _ptr(loss), _ptr(mean),
                                _ptr(workspace), workspace_bytes, _stream(stream)))


def gpt_adam_step(param, grad, m, v, param_bf16, n: int, step: int, lr: float, beta1: float,
                  beta2: float, eps: float, stream=None):
    _check(lib().gpt_adam_step(_ptr(param), _ptr(grad), _ptr(m), _ptr(v), _ptr(param_bf16), n, step,
                               lr, beta1, beta2, eps, _stream(stream)))


def gpt_profile_enable(mask: int):
    _check(lib().gpt_profile_enable(mask))


def gpt_profile_mask(mask: int):
    _check(lib().gpt_profile_mask(mask))


def gpt_profile_read(cls: int):
    ms, fl, by = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().gpt_profile_read(cls, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(fl),
                                  ctypes.byref(by)))
    return {"ms": ms.value, "launches": n.value, "flops": fl.value, "bytes": by.value}


def gpt_profile_read_launch(cls: int, i: int):
    ms, fl, by = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _check(lib().gpt_profile_read_launch(cls, i, ctypes.byref(ms), ctypes.byref(fl), ctypes.byref(by)))
    return {"ms": ms.value, "flops": fl.value, "bytes": by.value}


def gpt_debug_gemm(A, W, M: int, N: int, K: int, C, epi: int, ksplit: int = 1, stream=None):
    _check(lib().gpt_debug_gemm(_ptr(A), _ptr(W), M, N, K, _ptr(C), epi, ksplit, _stream(stream)))


def gpt_debug_attn_prefill(q, k, vt, ldvt: int, cu_seqlens, n_seqs: int, n_head: int, cu_dev, o,
                           qk_norm: int = 1, stream=None):
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    _check(lib().gpt_debug_attn_prefill(_ptr(q), _ptr(k), _ptr(vt), ldvt, cu.ctypes.data, n_seqs,
                                        n_head, qk_norm, _ptr(cu_dev), _ptr(o), _stream(stream)))


# ------------------------------------------------------------------ device weights

class DeviceModel:
    """Weights of one model resident in device memory plus the RoPE tables.

    ``W`` is any object with ``wte``, ``wpe``, ``lm_head`` and ``layers``
    (dicts with wq, wk, wv, wo, w1, w2) holding numpy float32 arrays whose
    values are exact in the model dtype.  The device copies are torch
    tensors; the GptWeights struct points at them.
    """

    def __init__(self, model_cfg, W, device="cuda"):
        import torch
        self.model = model_cfg
        self.cfg = make_config(model_cfg)
        dt = torch.bfloat16 if model_cfg.dtype == 1 else torch.float32
        self._keep = []

        def up(a):
            if a is None:
                return None
            t = torch.from_numpy(np.ascontiguousarray(a)).to(device).to(dt).contiguous()
            self._keep.append(t)
            return t

        self.wte = up(W.wte)
        self.wpe = up(W.wpe)
        self.lm_head = up(W.lm_head)
        L = model_cfg.n_layer
        self.layers = [{k: up(lw[k]) for k in ("wq", "wk", "wv", "wo", "w1", "w2")}
                       for lw in W.layers]
        arrs = {}
        for k in ("wq", "wk", "wv", "wo", "w1", "w2"):
            arrs[k] = (ctypes.c_void_p * L)(*[lw[k].data_ptr() for lw in self.layers])
        self._arrs = arrs
        self.weights = GptWeights(self.wte.data_ptr(), _ptr(self.wpe), self.lm_head.data_ptr(),
                                  *[ctypes.cast(arrs[k], _PP) for k in ("wq", "wk", "wv", "wo", "w1", "w2")])
        half = model_cfg.head_dim // 2
        self.rope_cos = torch.empty(model_cfg.max_seq * half, dtype=torch.float32, device=device)
        self.rope_sin = torch.empty_like(self.rope_cos)
        rope_tables(model_cfg.max_seq, model_cfg.head_dim, model_cfg.rope_base, self.rope_cos,
                    self.rope_sin)

    def workspace(self, max_tokens: int, max_seqs: int):
        import torch
        n = gpt_workspace_bytes(self.cfg, max_tokens, max_seqs)
        if n == 0:
            raise GptError(GPT_ERR_ARG, "gpt_workspace_bytes returned 0: " + last_error())
        return torch.empty(n, dtype=torch.uint8, device="cuda"), n

    def prefill(self, tokens, cu_seqlens, logits, lse=None, probs=None, kv=None,
                logits_rows=ROWS_ALL, workspace=None, stream=None):
        n = len(cu_seqlens) - 1
        total = int(cu_seqlens[-1])
        ws, nb = workspace if workspace is not None else self.workspace(total, n)
        gpt_prefill(self.cfg, self.weights, self.rope_cos, self.rope_sin, tokens, cu_seqlens, n,
                    kv, logits_rows, logits, lse, probs, ws, nb, stream)

    def prefill_loss(self, tokens, targets, cu_seqlens, loss, lse=None, mean=None, kv=None,
                     workspace=None, stream=None):
        n = len(cu_seqlens) - 1
        total = int(cu_seqlens[-1])
        ws, nb = workspace if workspace is not None else self.workspace(total, n)
        gpt_prefill_loss(self.cfg, self.weights, self.rope_cos, self.rope_sin, tokens, targets,
                         cu_seqlens, n, kv, loss, lse, mean, ws, nb, stream)

    def train_workspace(self, max_tokens: int, max_seqs: int):
        import torch
        n = gpt_train_workspace_bytes(self.cfg, max_tokens, max_seqs)
        if n == 0:
            raise GptError(GPT_ERR_ARG, "gpt_train_workspace_bytes returned 0: " + last_error())
        return torch.empty(n, dtype=torch.uint8, device="cuda"), n

    def loss_grads(self, tokens, targets, cu_seqlens, grads: "DeviceGrads", loss, mean=None,
                   workspace=None, stream=None):
        n = len(cu_seqlens) - 1
        total = int(cu_seqlens[-1])
        ws, nb = workspace if workspace is not None else self.train_workspace(total, n)
        gpt_loss_grads(self.cfg, self.weights, self.rope_cos, self.rope_sin, tokens, targets,
                       cu_seqlens, n, grads.struct, loss, mean, ws, nb, stream)

    def decode_step(self, kv: int, tokens_in, tokens_out, temperature=0.0, uniforms=None,
                    logits=None, workspace=None, stream=None):
        ws, nb = workspace
        gpt_decode_step(self.cfg, self.weights, self.rope_cos, self.rope_sin, kv, tokens_in,
                        temperature, uniforms, tokens_out, logits, ws, nb, stream)


class DeviceGrads:
    """fp32 gradient buffers shaped like a DeviceModel's weights."""

    def __init__(self, dm: "DeviceModel"):
        import torch

        def like(t):
            return None if t is None else torch.zeros(t.shape, dtype=torch.float32, device=t.device)

        self.wte, self.wpe, self.lm_head = like(dm.wte), like(dm.wpe), like(dm.lm_head)
        self.layers = [{k: like(lw[k]) for k in lw} for lw in dm.layers]
        L = len(self.layers)
        self._arrs = {k: (ctypes.c_void_p * L)(*[lw[k].data_ptr() for lw in self.layers])
                      for k in ("wq", "wk", "wv", "wo", "w1", "w2")}
        self.struct = GptGrads(self.wte.data_ptr(), _ptr(self.wpe), self.lm_head.data_ptr(),
                               *[ctypes.cast(self._arrs[k], _PP)
                                 for k in ("wq", "wk", "wv", "wo", "w1", "w2")])

    def flat(self):
        yield "wte", self.wte
        if self.wpe is not None:
            yield "wpe", self.wpe
        for i, lw in enumerate(self.layers):
            for k in ("wq", "wk", "wv", "wo", "w1", "w2"):
                yield f"layer{i}.{k}", lw[k]
        yield "lm_head", self.lm_head


class DeviceKV:
    """A paged KV cache in a torch-owned device buffer."""

    def __init__(self, dm: DeviceModel, n_seqs: int, capacity: int, page_size: int = 64):
        import torch
        self.n_seqs = n_seqs
        self.nbytes = kv_cache_bytes(dm.cfg, n_seqs, capacity, page_size)
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device="cuda")
        self.handle = kv_cache_alloc(dm.cfg, n_seqs, capacity, self.buf, self.nbytes, page_size)

    def lengths(self) -> np.ndarray:
        return kv_cache_lengths(self.handle, self.n_seqs)

    def close(self):
        if self.handle:
            kv_cache_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
