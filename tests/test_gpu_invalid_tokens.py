"""Token ids outside the vocabulary and rows without a finite logit (regression: an all-NaN row
used to make argmax emit 0x7fffffff, which the next step's embedding gather used as a row index
17 TB past the table).  An invalid input id must read nothing and give a NaN row whose argmax is
-1 (rows after it see its NaN keys and give -1 as well), and no memory outside the table is read."""
import numpy as np
import pytest

from gpu_helpers import log, need_gpu, torch
from synth.configs import ModelShape

pytestmark = pytest.mark.gpu

SHAPES = {"bf16": ModelShape(n_layers=1, d_model=512, n_q_heads=4, n_kv_heads=1, head_dim=128, ffn=1024,
                             vocab=1024, rope_theta=500000.0, dtype="bf16"),
          "fp32": ModelShape(n_layers=1, d_model=256, n_q_heads=4, n_kv_heads=4, head_dim=64, ffn=512,
                             vocab=512, rope_theta=10000.0, dtype="fp32")}


@pytest.mark.parametrize("name", list(SHAPES))
def test_invalid_token_ids_give_minus_one_without_reading_outside(name):
    need_gpu()
    from lossless_speculative_decoding_amd import Model
    from lossless_speculative_decoding_amd._vc import Req
    from lossless_speculative_decoding_amd.engine import make_weights
    s = SHAPES[name]
    W = make_weights(s)
    m = Model(s, W, max_pos=64)
    dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    toks = torch.tensor([5, 9, -1, s.vocab + 3, 2 ** 31 - 1, 7], dtype=torch.int32, device="cuda")
    n = toks.numel()
    ws = m.workspace(n, n)
    out = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    lg = torch.empty(n, s.vocab, dtype=torch.float32, device="cuda")
    vk = torch.empty(1, s.n_kv_heads, n, s.head_dim, dtype=dt, device="cuda")
    vv = torch.empty_like(vk)
    m.verify_raw(Req(ctx_len=0), 0, 0, 0, toks.data_ptr(), n, out.data_ptr(), vk.data_ptr(), vv.data_ptr(), n, ws,
                 lg.data_ptr())
    torch.cuda.synchronize()
    o = out.cpu().tolist()
    log(f"{name}: tokens {toks.cpu().tolist()} -> argmax {o}")
    # rows at or after an invalid one are NaN (rows before it may be too: the P.V product of a key
    # tile multiplies their zero weights into its NaN values)
    assert o[2:] == [-1, -1, -1, -1]
    assert torch.isnan(lg[2:]).all()
    # the same call with valid ids only: every row finite
    toks2 = torch.tensor([5, 9, 11, 3, 0, 7], dtype=torch.int32, device="cuda")
    m.verify_raw(Req(ctx_len=0), 0, 0, 0, toks2.data_ptr(), n, out.data_ptr(), vk.data_ptr(), vv.data_ptr(), n, ws,
                 lg.data_ptr())
    torch.cuda.synchronize()
    assert min(out.cpu().tolist()) >= 0 and torch.isfinite(lg).all()
