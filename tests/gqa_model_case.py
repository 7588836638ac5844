"""The small bf16 GQA decoder with Llama-3-8B head shapes used for end-to-end parity:
2 layers, d_model 1024, 32 query heads over 8 KV heads of 128 (so a query row is 4096 wide),
SwiGLU 2048, vocab 2048, RoPE base 500000; a 2000-token prompt (ragged against every
quantization group and the 64-key tiles); draft length 8; 32 tokens.  Shapes and knobs only."""
from synth.configs import CompressSpec, ModelShape

SHAPE = ModelShape(n_layers=2, d_model=1024, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=2048, vocab=2048,
                   rope_theta=500000.0, dtype="bf16")
T = 2000
N = 32
X = 8
PROMPT_SEED = 9          # synth.prompt(PROMPT_SEED, T, vocab)
SPECS = {
    "tokdrop": CompressSpec("tokdrop", keep_recent=64, ratio=4, obs_window=32),
    "keynorm": CompressSpec("tokdrop", keep_recent=0, ratio=4, score="keynorm"),
    "q2g64": CompressSpec("quant", bits=2, group=64),
    "q3g128": CompressSpec("quant", bits=3, group=128),
    "q4g128": CompressSpec("quant", bits=4, group=128),
}
GOLDEN = "gqa_model_oracle.npz"


def keep_total(spec) -> int:
    """Rows a token-drop cache keeps (the engine's rule)."""
    return max(32, T // spec.ratio) if spec.score == "keynorm" else T // spec.ratio
