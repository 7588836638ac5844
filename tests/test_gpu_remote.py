"""Remote prefix caching on the GPU (tiny fp32 decoder): the compressed cache is wiped on the
device and shipped back over a paced link; drafting waits for it, and every round (drafts,
verifier tokens, accept count) equals that of a run whose cache was there from the start, so
no draft read the cache before it landed."""
import pytest

import synth
from gpu_helpers import log, need_gpu, torch
from synth.configs import tiny as tiny_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("polled", [False, True])
def test_drafting_waits_for_the_shipped_cache(polled):
    need_gpu()
    from lossless_speculative_decoding_amd import Model
    from lossless_speculative_decoding_amd.engine import Engine, make_weights
    from lossless_speculative_decoding_amd.remote import SlowLink
    w = tiny_workload()
    s = w.model
    m = Model(s, make_weights(s), max_pos=w.ctx[0] + w.n_tokens + 64)
    prompt = torch.from_numpy(synth.prompt(0, w.ctx[0], s.vocab)).cuda()
    ref = Engine(m, w.compress, record=True)
    ref.add_request(prompt, w.x[0], w.n_tokens)
    ref.run()
    eng = Engine(m, w.compress, record=True)
    r = eng.add_request(prompt, w.x[0], w.n_tokens)
    store = torch.empty(r.comp.numel(), dtype=torch.uint8, pin_memory=polled)
    store.copy_(r.comp)
    r.comp.zero_()
    torch.cuda.synchronize()
    secs = 0.3
    link = SlowLink(store.numel() / secs / 1e9, chunk_bytes=1 << 16)
    r.ready = (link.start if polled else link.ship)([(store, r.comp)])[0]
    eng.run()
    link.wait()
    log(f"cache of {store.numel()} bytes landed after {link.arrival[0]:.3f}s; first round done after "
        f"{r.t_first - link.t0:.3f}s")
    assert link.arrival[0] >= secs - 1e-3
    assert r.t_first - link.t0 >= link.arrival[0]
    assert torch.equal(r.comp.cpu(), store)
    assert r.emitted == ref.reqs[0].emitted
    assert [(g["pos"], g["draft"], g["verified"], g["a"]) for g in r.rounds] == \
           [(g["pos"], g["draft"], g["verified"], g["a"]) for g in ref.reqs[0].rounds]
