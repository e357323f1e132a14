"""The five synthetic workloads, by shape.

Head geometry follows the YOCO-3B family (head_dim 128, grouped KV heads) of
"YOCO 深度技术分析" (liuhc.cn), section 5.3.4 (model configuration table);
the shapes themselves are the benchmark's configurations:

* tiny fp32:   B=1, N=256, Hq=4, Hkv=1, d=64, 2 layers, entries N(0,1); rows 0..254
               are written directly, row 255 by one append
* prefill:     B=1, N=32768, Hq=16, Hkv=4, d=128, 16 layers, entries N(0,1)/sqrt(128)
* decode:      B=8, N=131072 after the step's append (131071 rows before it),
               Hq=16, Hkv=2, d=128, 16 layers
* long decode: B=1, N=1048576 at start, 64 steps of append + 16 layers
* ragged:      16 sequences, L = floor(4096 * 16**u), u ~ U[0,1), Hq=32, Hkv=8,
               d=128; prefill then 32 decode steps, one layer call per step

Seeds: workload c (0-based) uses seed c.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16": storage dtype of Q, K, V and O
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    layers: int
    seq_lens: tuple       # rows of each sequence's shared cache before any decode-step append
    value_std: float      # std of every entry of Q, K, V
    seed: int
    decode_steps: int = 0
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads


def ragged_lengths(seed: int, n: int = 16, lo: int = 4096, ratio: int = 16) -> tuple:
    """Lengths log-uniform in [lo, lo*ratio): L = floor(lo * ratio**u), u ~ U[0, 1)."""
    ss = np.random.SeedSequence(seed).spawn(8)[7]
    u = np.random.Generator(np.random.PCG64(ss)).random(n)
    return tuple(int(math.floor(lo * ratio ** x)) for x in u)


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", "f32", 1, 4, 1, 64, 2, (255,), 1.0, 0, 1,
                         "B=1 N=256 Hq=4 Hkv=1 d=64 fp32, 2 layers, prefill + decode of the last row"),
    "prefill_32k": Workload("prefill_32k", "bf16", 1, 16, 4, 128, 16, (32768,), 1.0 / math.sqrt(128), 1, 0,
                            "B=1 N=32768 Hq=16 Hkv=4 d=128 bf16 causal prefill, 16 layers"),
    "decode_128k": Workload("decode_128k", "bf16", 8, 16, 2, 128, 16, (131071,) * 8, 1.0 / math.sqrt(128), 2, 1,
                            "B=8 N=131072 Hq=16 Hkv=2 d=128 bf16 decode, 16 layers per step"),
    "decode_1m": Workload("decode_1m", "bf16", 1, 16, 2, 128, 16, (1048576,), 1.0 / math.sqrt(128), 3, 64,
                          "B=1 N=1048576 Hq=16 Hkv=2 d=128 bf16 decode, 64 steps x 16 layers"),
    "ragged": Workload("ragged", "bf16", 16, 32, 8, 128, 1, ragged_lengths(4), 1.0 / math.sqrt(128), 4, 32,
                       "16 seqs, L log-uniform [4096, 65536), Hq=32 Hkv=8 d=128 bf16; prefill + 32 decode steps"),
}
