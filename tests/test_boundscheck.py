"""The library's address-range checks, on the CPU (no GPU: the dry mode makes no HIP call).

Every model workload's exact sequence of library calls (bench.py --bounds-replay: weights,
prefill, compression and offload of every request, warmup and timed rounds under the staggered
scheduler, the compressed-only and comparator passes) is replayed at full size with every
launch's and copy's byte ranges checked against the buffers allocated for it; and the check is
shown to fire on planted mistakes (a tail or a staging slot smaller than the request claims)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _replay(config: str, *extra) -> dict:
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", config, "--bounds-replay",
                        "--steps", "16", "--warmup", "2", *extra], capture_output=True, text=True, timeout=600)
    line = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert line, r.stdout[-2000:] + r.stderr[-2000:]
    out = json.loads(line[-1])
    out["rc"] = r.returncode
    return out


@pytest.mark.parametrize("config", ["llama8b_q2", "llama8b_mixed", "llama8b_tokdrop"])
def test_full_size_workload_replay_stays_in_bounds(config):
    out = _replay(config)
    print(out)
    assert out["rc"] == 0 and out["ok"] and out["violations"] == 0
    assert out["launches"] > 500_000
    # pinned host memory stays under the budget the engine keeps (the driver limit is ~70.75 GB)
    assert out["pinned_peak"] <= 69e9


@pytest.mark.parametrize("config,extra", [("llama8b_tokdrop", ("--temperature", "0.8")),
                                          ("llama8b_q2", ("--temperature", "0.8", "--adaptive", "--fallback-after",
                                                          "2", "--plain-rounds", "3", "--replay-policy", "collapse")),
                                          ("llama8b_tokdrop", ("--adaptive", "--fallback-after", "2",
                                                               "--replay-policy", "collapse"))])
def test_sampled_and_fallback_replay_stays_in_bounds(config, extra):
    """Sampled decoding (draft distributions, verify logits, rejection sampling) and plain rounds
    (x = 0) add launches and buffers of their own: the same replay, with them."""
    out = _replay(config, "--no-whole-decode", *extra)
    print(out)
    assert out["rc"] == 0 and out["ok"] and out["violations"] == 0
    assert out["launches"] > 100_000
    if "--fallback-after" in extra:
        assert out["plain_round_share"] > 0.05          # plain rounds (x = 0) were replayed


def _dry_model():
    """A 1-layer bf16 model on host memory under the dry mode, and a quantized request."""
    import torch

    import lossless_speculative_decoding_amd as vc
    from lossless_speculative_decoding_amd import runtime
    from lossless_speculative_decoding_amd.engine import Engine, make_weights
    from synth.configs import CompressSpec, ModelShape
    runtime.use(runtime.DryRT())
    vc.debug_mode(vc.VC_DEBUG_DRY)
    s = ModelShape(n_layers=1, d_model=512, n_q_heads=4, n_kv_heads=1, head_dim=128, ffn=1024, vocab=1024,
                   rope_theta=500000.0, dtype="bf16")
    m = vc.Model(s, make_weights(s, device="cpu"), max_pos=2048)
    eng = Engine(m, CompressSpec("quant", bits=2, group=64), chunk=256, device="cpu")
    r = eng.add_request(torch.zeros(700, dtype=torch.int32), 4, 16)
    return vc, m, eng, r


@pytest.fixture
def dry():
    yield
    import lossless_speculative_decoding_amd as vc
    from lossless_speculative_decoding_amd import runtime
    vc.debug_mode(vc.VC_DEBUG_OFF)
    runtime.use(runtime.CudaRT())


def test_check_fires_on_a_tail_smaller_than_claimed(dry):
    import torch

    vc, m, eng, r = _dry_model()
    ws = m.workspace(1, 1024, device="cpu")
    m.draft_step([r.req], ws)                       # as allocated: in bounds
    # a tail buffer three rows shorter than the request's tail_cap says
    short = torch.empty(1, 1, r.req.tail_cap - 3, 128, dtype=torch.bfloat16)
    r.req.tail_k = short.data_ptr()
    vc.debug_register(short)
    with pytest.raises(vc._vc.VCError, match="bounds check: vc_draft_step: request tail K"):
        m.draft_step([r.req], ws)
    # and with the claim checked away, the write of row n_tail itself past the buffer's end
    r.req.tail_cap -= 3
    r.req.n_tail = r.req.tail_cap - 1
    m.draft_step([r.req], ws)                       # last row of the buffer: in bounds
    r.req.tail_cap += 3
    r.req.n_tail += 2
    with pytest.raises(vc._vc.VCError, match="bounds check"):
        m.draft_step([r.req], ws)
    assert vc.debug_stats()["violations"] >= 1


def test_check_fires_on_a_staging_slot_smaller_than_claimed(dry):
    import torch

    vc, m, eng, r = _dry_model()
    slot = torch.empty(1, 1, r.n_host - 1, 128, dtype=torch.bfloat16)
    vc.debug_register(slot)
    with pytest.raises(vc._vc.VCError, match="vc_stage"):      # the library's own argument check
        m.stage(r.req, slot, slot, 0, 1)
    big = torch.empty(1, 1, r.n_host, 128, dtype=torch.bfloat16)
    vc.debug_register(big)
    m.stage(r.req, big, big, 0, 1)                  # as large as claimed: in bounds
    small = torch.empty(8 * 128, dtype=torch.bfloat16)   # claimed to hold n_host rows
    vc.debug_register(small)
    from lossless_speculative_decoding_amd._vc import call
    with pytest.raises(vc._vc.VCError, match="bounds check: vc_stage: slot K"):
        call("vc_stage", m.h, __import__("ctypes").byref(r.req), small.data_ptr(), big.data_ptr(), r.n_host, 0, 1, 0)
