"""The rate-limited link of the remote-prefix workload and the engine's gating on it, on the
CPU: a transfer of n bytes lasts n / rate and lands intact (contiguous and strided
destinations), jobs arrive in order, and a request never drafts or stages before its
compressed cache has arrived."""
import threading
import time

import pytest
import torch

from lossless_speculative_decoding_amd import engine as E
from lossless_speculative_decoding_amd import runtime
from lossless_speculative_decoding_amd.remote import SlowLink

import test_host_scheduler as H


@pytest.fixture
def dry_rt(monkeypatch):
    monkeypatch.setattr(runtime, "RT", runtime.DryRT(seed=0))


def test_paced_transfers_take_bytes_over_rate(dry_rt):
    rate = 0.25                                            # GB/s
    srcs = [torch.arange(2_000_000, dtype=torch.int32) + k for k in range(3)]   # 8 MB each
    dsts = [torch.empty_like(s) for s in srcs]
    strided_src = torch.randn(4, 3, 1000, 64)
    big = torch.zeros(4, 3, 1500, 64)
    jobs = list(zip(srcs, dsts)) + [(strided_src, big[:, :, :1000])]
    link = SlowLink(rate, chunk_bytes=1 << 20, device="cpu")
    evs = link.ship(jobs)
    link.wait()
    assert all(e.is_set() for e in evs)
    total = 0
    for k, (s, d) in enumerate(jobs):
        total += s.numel() * s.element_size()
        want = total / (rate * 1e9)
        assert want - 1e-3 <= link.arrival[k] <= want + 0.05, (k, link.arrival[k], want)
        assert torch.equal(s, d)
    assert torch.count_nonzero(big[:, :, 1000:]) == 0      # nothing written past the destination view
    assert link.arrival == sorted(link.arrival)


def test_requests_wait_for_their_compressed_cache(monkeypatch):
    """Request 1's cache arrives after some scheduler iterations: until then it neither drafts
    nor stages, the others proceed; afterwards it decodes to the end like the rest."""
    eng = H.make_engine(monkeypatch, n_req=3, x=4, n_tokens=[30, 30, 30], lag=1)
    H.guard(monkeypatch, eng)
    gate = threading.Event()
    eng.reqs[1].ready = gate
    eng.start()
    for _ in range(40):
        eng.step()
    assert all(i != 1 for _, i in eng.m.log)
    assert any(i == 0 for _, i in eng.m.log) and any(i == 2 for _, i in eng.m.log)
    gate.set()
    while any(r.phase != E.DONE for r in eng.reqs):
        eng.step()
    eng.drain()
    assert len(eng.reqs[1].emitted) >= 30
    assert eng.reqs[1].t_first is not None
