"""The five seeded synthetic workloads (shapes and knobs only, no arithmetic).

tiny             tiny fp32 decoder, 1024-token prompt, token-drop 4x (64 recent + top
                 192 by observed attention of the last 32 prompt queries), x = 8, 64 tokens.
gqa_layer        one GQA attention layer with Llama-3-8B head shapes, bf16, 16 x 32768,
                 K/V ~ N(0,1) with 4 outlier channels per head scaled x10, 4-bit KIVI-style
                 quantization with group 128, one draft decode step and a 32-row verify.
llama8b_tokdrop  32-layer Llama-3-8B-shaped decoder, bf16, 8 x 65536 prompts, 4x
                 token-dropped draft cache, full KV on the host, x = 32, 256 tokens per
                 request, staggered verification.
llama8b_q2       same model, 4 x 131072, 2-bit quantization with group 64, x = 40,
                 512 tokens per request.
llama8b_mixed    same model, 16 requests with log-uniform contexts in [8192, 131072],
                 3-bit quantization (group 128), x per request from {16, 24, 32, 40},
                 256 tokens per request, staggered.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rope_theta: float
    dtype: str            # "fp32" | "bf16"
    eps: float = 1e-5

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


@dataclass(frozen=True)
class CompressSpec:
    kind: str             # "tokdrop" | "quant" | "none"
    bits: int = 0
    group: int = 0
    keep_recent: int = 64
    ratio: int = 4        # token drop keeps T // ratio rows
    obs_window: int = 32
    score: str = "attn"   # token-drop ranking: "attn" (observed attention) | "keynorm"


@dataclass(frozen=True)
class Workload:
    name: str
    model: ModelShape | None
    compress: CompressSpec
    batch: int
    ctx: tuple = ()                    # per-request prompt lengths
    x: tuple = ()                      # per-request draft horizon
    n_tokens: int = 0                  # tokens emitted per request (counts g0)
    extra: dict = field(default_factory=dict)


TINY = ModelShape(n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=64, ffn=1024,
                  vocab=512, rope_theta=10000.0, dtype="fp32")
LLAMA8B = ModelShape(n_layers=32, d_model=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=14336,
                     vocab=128256, rope_theta=500000.0, dtype="bf16")


def tiny() -> Workload:
    return Workload("tiny_fp32_t1024_tokdrop4x_x8", TINY, CompressSpec("tokdrop", keep_recent=64, ratio=4, obs_window=32),
                    batch=1, ctx=(1024,), x=(8,), n_tokens=64)


def gqa_layer() -> Workload:
    return Workload("gqa_layer_bf16_b16_t32768_q4g128", None, CompressSpec("quant", bits=4, group=128),
                    batch=16, ctx=(32768,) * 16, x=(32,) * 16,
                    extra=dict(n_q_heads=32, n_kv_heads=8, head_dim=128, n_outlier=4, outlier_scale=10.0,
                               verify_rows=32))


def llama8b_tokdrop() -> Workload:
    return Workload("llama8b_bf16_b8_t65536_tokdrop4x_x32", LLAMA8B,
                    CompressSpec("tokdrop", keep_recent=64, ratio=4, obs_window=32),
                    batch=8, ctx=(65536,) * 8, x=(32,) * 8, n_tokens=256)


def llama8b_q2() -> Workload:
    return Workload("llama8b_bf16_b4_t131072_q2g64_x40", LLAMA8B, CompressSpec("quant", bits=2, group=64),
                    batch=4, ctx=(131072,) * 4, x=(40,) * 4, n_tokens=512)


def llama8b_mixed() -> Workload:
    from . import mixed_context_lengths, mixed_draft_horizons
    ctx = tuple(int(t) for t in mixed_context_lengths(16))
    xs = tuple(int(v) for v in mixed_draft_horizons(16))
    return Workload("llama8b_bf16_mixed16_q3g128", LLAMA8B, CompressSpec("quant", bits=3, group=128),
                    batch=16, ctx=ctx, x=xs, n_tokens=256)


ALL = {"tiny": tiny, "gqa_layer": gqa_layer, "llama8b_tokdrop": llama8b_tokdrop, "llama8b_q2": llama8b_q2,
       "llama8b_mixed": llama8b_mixed}


def scaled(w: Workload, **kw) -> Workload:
    return replace(w, **kw)
