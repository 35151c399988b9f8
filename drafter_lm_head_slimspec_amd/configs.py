"""Workload shapes.

Shapes follow the pages' model families (SlimSpec write-up section 六: Llama-3.1-8B,
GPT-OSS-20B, Qwen3-30B-A3B drafters with EAGLE-3 backbones, batch 1 and 64; SpecVocab
write-up section 2.2: d' = d/16, k = 2048) and the synthetic recipe stated with each
entry.  ``M`` is the number of hidden-state rows in one head call (sequences x draft
steps).  Seeds: weights 1000+c, hidden states 2000+c, logits 3000+c, draft tokens 4000+c,
accept uniforms 5000+c, Philox sampling seed 5000+c, for workload index c.
"""
from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class HeadWorkload:
    name: str
    index: int
    d: int
    V: int
    r: int
    dprime: int
    k: int
    Ms: Tuple[int, ...]
    dtype: str
    temperature: float = 1.0
    gamma: int = 0

    @property
    def seeds(self):
        c = self.index
        return {"weights": 1000 + c, "hidden": 2000 + c, "philox": 5000 + c}


@dataclass(frozen=True)
class VerifyWorkload:
    name: str
    index: int
    B: int
    gamma: int
    V: int
    sigmas: Tuple[float, ...]
    dtype: str
    temperature: float = 1.0
    target_std: float = 3.0

    @property
    def seeds(self):
        c = self.index
        return {"logits": 3000 + c, "tokens": 4000 + c, "uniforms": 5000 + c, "philox": 5000 + c}


# one sequence, gamma = 4 draft steps, fp32; SpecVocab parameters for this size are our own
TINY = HeadWorkload("tiny", 0, d=256, V=1024, r=32, dprime=16, k=64, Ms=(4,), dtype="f32", gamma=4)
TINY_VERIFY = VerifyWorkload("tiny-verify", 0, B=1, gamma=4, V=1024, sigmas=(1.0,), dtype="f32")

# Llama-3.1-8B-shaped drafter head: batch 1 and 8 sequences x gamma 6 rows; r = d/8.
# SpecVocab at the same shape uses d' = d/16 and k = 2048.
LLAMA = HeadWorkload("llama3.1-8b-head", 1, d=4096, V=128256, r=512, dprime=256, k=2048,
                     Ms=(6, 48), dtype="bf16", temperature=1.0, gamma=6)

# Qwen3-8B-shaped SpecVocab head, batch 1 and 16
QWEN = HeadWorkload("qwen3-8b-specvocab", 2, d=4096, V=151936, r=512, dprime=256, k=2048,
                    Ms=(1, 16), dtype="bf16")

# GPT-OSS-20B-shaped low-rank head: 32 sequences x gamma 6 = 192 rows, T = 0.7
GPTOSS = HeadWorkload("gpt-oss-20b-head", 3, d=2880, V=201088, r=360, dprime=180, k=2048,
                      Ms=(192,), dtype="bf16", temperature=0.7, gamma=6)

# batched verification: 64 sequences, gamma 5, V = 151936, target N(0, 3^2),
# draft = target + N(0, sigma^2)
VERIFY = VerifyWorkload("verify-b64-g5", 4, B=64, gamma=5, V=151936, sigmas=(0.5, 1.0, 2.0),
                        dtype="bf16")

HEADS = {w.name: w for w in (TINY, LLAMA, QWEN, GPTOSS)}
VERIFIES = {w.name: w for w in (TINY_VERIFY, VERIFY)}
