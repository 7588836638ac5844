"""Where the host side gets its streams, events and synchronisation from.

On a GPU this is torch.cuda.  For a dry run of the library's address-range checks
(vc_debug_mode(VC_DEBUG_DRY): no HIP call at all, host memory standing in for device memory)
the same scheduler runs against stand-ins: streams with a null handle, events that are always
complete, and results the library does not compute supplied by a seeded policy (the accept
count of a round, the first token of a prefill), so that every code path a real run takes,
including the longest tails, is replayed."""
from __future__ import annotations

import random

import torch


class CudaRT:
    dry = False
    device = "cuda"
    pin = True

    Stream = staticmethod(lambda device=None: torch.cuda.Stream(device=device))
    Event = staticmethod(lambda: torch.cuda.Event())
    current_stream = staticmethod(lambda: torch.cuda.current_stream())
    synchronize = staticmethod(lambda: torch.cuda.synchronize())


class _DryStream:
    cuda_stream = 0

    def synchronize(self):
        pass

    def wait_event(self, ev):
        pass


class _DryEvent:
    cuda_event = None

    def record(self, stream=None):
        pass

    def query(self):
        return True

    def synchronize(self):
        pass


class DryRT:
    """Stand-ins for a dry run (see the module docstring).  accept_policy(request index, round,
    draft length) -> accept count; by default every other round accepts all drafts (the fastest
    growth of the committed tails) and the others a seeded count below x."""
    dry = True
    device = "cpu"
    pin = False

    def __init__(self, seed: int = 0, accept_policy=None):
        self.rng = random.Random(seed)
        self.accept_policy = accept_policy or (
            lambda idx, rnd, x: x if rnd % 2 == 0 else self.rng.randrange(0, x + 1))

    Stream = staticmethod(lambda device=None: _DryStream())
    Event = staticmethod(lambda: _DryEvent())
    current_stream = staticmethod(lambda: _DryStream())
    synchronize = staticmethod(lambda: None)

    def fill_accept(self, idx: int, rnd: int, x: int, result: torch.Tensor):
        """What vc_accept would have written: [a, a + 1 valid token ids]."""
        a = int(self.accept_policy(idx, rnd, x))
        result[0] = a
        result[1:a + 2] = torch.arange(a + 1, dtype=torch.int32) + 1


RT = CudaRT()


def use(rt) -> None:
    """Select the runtime the scheduler and the greedy drivers use."""
    global RT
    RT = rt
