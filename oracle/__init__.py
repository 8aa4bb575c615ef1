"""CPU oracle for the nanochat-style decoder-block forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (``gpt_block_fwd_amd``); both sides receive the same seeded inputs from
``workloads``.

The oracle is a plain, slow transformer written in numpy, computed in
float64 unless the caller asks for float32 matmuls (allowed for the large
bf16 models, whose float32 and float64 logits differ by about 1e-6).  Every
function cites the passage of the source pages it follows.  Pages:

* "Microgpt" -- Hacker News summary of microgpt (telegra.ph); sections
  Tokenizer, Model parameters, Core architecture, Training, Inference,
  Differences from production models.
* "NanoChat launch" -- 復刻 ChatGPT 有多難？ (jxzklqfsx.com, article 827243);
  section on Karpathy's tricks (為什么可以訓練如此之快).
* "nanochat hand-written" -- hongdingcd.com thread 19501, the paragraphs on
  the model architecture.
* "nanochat CSDN walkthrough" -- wap.jaobe.com, show-85130.

Parity status of each function is stated in its docstring; the readings of
points the pages leave open are listed in ``gpt.READINGS``.
"""
from .gpt import *  # noqa: F401,F403
