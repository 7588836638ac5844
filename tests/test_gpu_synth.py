"""The GPU input generator equals the host generator bit for bit."""
import numpy as np
import pytest

import synth
from gpu_helpers import log, need_gpu, torch

pytestmark = pytest.mark.gpu


def test_xavier_matches_host():
    need_gpu()
    from lossless_speculative_decoding_amd import synth_xavier
    for dt, tdt in (("bf16", torch.bfloat16), ("fp32", torch.float32)):
        log("xavier", dt)
        t = torch.empty(4096 * 3 + 17, dtype=tdt, device="cuda")
        synth_xavier(t, 1234, 4096, 6144, seed=0, start=1000)
        host = synth.xavier(1234, (t.numel(),), 4096, 6144, start=1000)
        if dt == "bf16":
            got = t.view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(got, synth.gen_bf16(host))
        else:
            assert np.array_equal(t.cpu().numpy(), synth.f32(host))


def test_normal_heads_with_outliers_matches_host():
    need_gpu()
    from lossless_speculative_decoding_amd import synth_normal_heads
    B, H, T, D = 3, 8, 96, 128
    outl = np.stack([synth.outlier_channels_for(b, j, H, D) for b in range(B) for j in range(H)]).astype(np.int32)
    t = torch.empty((B, H, T, D), dtype=torch.bfloat16, device="cuda")
    synth_normal_heads(t, synth.S_ATT_K, torch.from_numpy(outl).cuda(), 10.0)
    got = t.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(B):
        for j in range(H):
            want = synth.att_head(synth.S_ATT_K, b, j, T, H, D, outl[b * H + j], 10.0)
            assert np.array_equal(got[b, j], want), (b, j)


def test_ids_match_host():
    need_gpu()
    from lossless_speculative_decoding_amd import synth_ids
    t = torch.empty(70000, dtype=torch.int32, device="cuda")
    synth_ids(t, synth.S_PROMPT + 3, 128256)
    assert np.array_equal(t.cpu().numpy(), synth.prompt(3, 70000, 128256))
