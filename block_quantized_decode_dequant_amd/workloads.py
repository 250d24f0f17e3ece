"""The synthetic workloads: shapes, seeds and generator streams (no arithmetic).

The ntransformer write-up measured Llama 3.1 8B (Q8_0, "Roadmap") and 70B
(Q4_K_M / Q6_K, "Performance", "NVMe direct streaming") GGUF models, which are
not available here; these seeded stand-ins take their shapes.

* Q8_0 GEMV: 4096 x 4096, codes uniform on [-127, 127], fp16 scales
  |N(0,1)| * 0.01, x ~ N(0,1), seed 0.
* K-quant GEMV sweep on the 70B projection shapes: W fp32 N(0, 0.02) encoded to
  Q4_K or Q6_K, x ~ N(0,1), seed 0.  The two 235M-value shapes (28672 x 8192,
  8192 x 28672) draw their values from one stream.
* Llama-3-8B-shaped decode (Q8_0) and Llama-70B-shaped decode (Q4_K with Q6_K
  for attn_v, ffn_down and the output head), fp16 KV cache prefilled with
  N(0,1) values, norm gains 1.0.
"""
from __future__ import annotations

from dataclasses import dataclass

SEED = 0

Q8_0_GEMV = dict(name="q8_0 gemv 4096x4096", qtype="q8_0", rows=4096, cols=4096)

KQ_SHAPES = [(8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672)]
KQ_TYPES = ["q4_k", "q6_k"]


def kq_w_stream(shape_idx: int) -> int:
    rows, cols = KQ_SHAPES[shape_idx]
    return 100 + (2 if rows * cols == 28672 * 8192 else shape_idx)


def kq_x_stream(shape_idx: int) -> int:
    return 200 + shape_idx


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    ctx: int          # prefilled positions before the first decoded token
    n_tokens: int     # greedy tokens decoded
    weights: str      # "q8_0" or "mix" (Q4_K, Q6_K for attn_v / ffn_down / output)
    rms_eps: float = 1e-5
    rope_theta: float = 500000.0

    @property
    def ctx_cap(self) -> int:
        return self.ctx + self.n_tokens


LLAMA_8B_Q8_0 = ModelShape("llama3-8b-shaped q8_0", 32, 4096, 32, 8, 128, 14336, 128256,
                           1024, 128, "q8_0")
LLAMA_70B_MIX = ModelShape("llama-70b-shaped q4_k/q6_k", 80, 8192, 64, 8, 128, 28672, 128256,
                           4096, 64, "mix")
LLAMA_70B_Q6K = ModelShape("llama-70b-shaped q6_k (host-streamed)", 80, 8192, 64, 8, 128, 28672, 128256,
                           4096, 64, "q6_k")
