"""Remote prefix caching on one GPU: a rate-limited link for shipping caches.

The setting ("VeriCache: Making Lossy KV Compression Exact", "Verifying Without
Giving Back the Speedup", the second serving setting; the study note's
"实践案例" case 3): a long shared prefix's KV cache is precomputed and stored
away from the serving GPU, behind a slow link.  Shipping the full cache before
decoding moves the cost from prefill to transfer; VeriCache ships only the
compressed cache over the slow link and starts drafting once it has landed,
while the exact state stays with the storage side and reaches verification
over a fast link.  On one GPU the two links are modelled as two paths into
the same device: the slow link is this module's paced copy, the fast link the
PCIe staging of host rows that every verification already does.

SlowLink copies host memory to the device in chunks, paced on the wall clock:
the chunk that starts at byte B of the link's whole schedule is issued no
earlier than t0 + B / rate, so a transfer of n bytes lasts n / rate (as long
as the rate is below what the copy engine reaches).  Jobs go out one after
another in the order given; each has an arrival flag (is_set()) that turns on
once its last byte is on the device.  Two ways to drive it: ship() runs the
schedule on a worker thread (blocking copies, any host memory), start() plus
pump() issues due chunks as asynchronous copies from the caller's own loop
(pinned sources; nothing blocks and no thread competes with the caller for the
interpreter).  All arithmetic of the method stays in the library; this is
plumbing (torch copies on a stream of the link's own).
"""
from __future__ import annotations

import threading
import time

import torch

from . import runtime


class SlowLink:
    def __init__(self, gbps: float, chunk_bytes: int = 64 << 20, device="cuda"):
        if gbps <= 0:
            raise ValueError("link rate must be positive")
        self.rate = gbps * 1e9
        self.chunk = int(chunk_bytes)
        self.device = device
        self.t0 = None
        self.arrival = []       # seconds after t0 at which each job's last byte landed
        self.error = None
        self._thread = None
        self._plan = None

    def ship(self, jobs):
        """jobs: [(src, dst)] with src a host tensor and dst a device tensor of the same bytes
        (dst may be a strided view; it is filled per leading index).  Returns one
        threading.Event per job, set when that job has fully arrived."""
        events = [threading.Event() for _ in jobs]
        self.arrival = [None] * len(jobs)
        self.t0 = time.perf_counter()

        def work():
            try:
                stream = runtime.RT.Stream(device=self.device) if not runtime.RT.dry else None
                sent = 0
                for k, (src, dst) in enumerate(jobs):
                    for s_part, d_part in _chunks(src, dst, self.chunk):
                        n = s_part.numel() * s_part.element_size()
                        wait = self.t0 + sent / self.rate - time.perf_counter()
                        if wait > 0:
                            time.sleep(wait)
                        if stream is None:
                            d_part.copy_(s_part)
                        else:
                            with torch.cuda.stream(stream):
                                d_part.copy_(s_part, non_blocking=True)
                        sent += n
                    # the job's last byte leaves the link at t0 + sent / rate
                    wait = self.t0 + sent / self.rate - time.perf_counter()
                    if wait > 0:
                        time.sleep(wait)
                    if stream is not None:
                        stream.synchronize()
                    self.arrival[k] = time.perf_counter() - self.t0
                    events[k].set()
            except BaseException as e:  # surfaced by wait(); every event is released
                self.error = e
                for ev in events:
                    ev.set()

        self._thread = threading.Thread(target=work, daemon=True)
        self._thread.start()
        return events

    # ---------------------------------------------------------------- polled mode
    def start(self, jobs):
        """Plan the schedule of jobs [(pinned src, dst)]; returns one arrival flag per job.  The
        caller calls pump() regularly (e.g. before every scheduler step) until done()."""
        self._plan = []                       # (due time offset, src piece, dst piece, job or -1)
        sent = 0
        for k, (src, dst) in enumerate(jobs):
            pieces = list(_chunks(src, dst, self.chunk))
            for i, (sp, dp) in enumerate(pieces):
                self._plan.append((sent / self.rate, sp, dp, k if i == len(pieces) - 1 else -1))
                sent += sp.numel() * sp.element_size()
        self._ends = [sum(sp.numel() * sp.element_size() for sp, _ in _chunks(s_, d_, self.chunk))
                      for s_, d_ in jobs]
        self._next = 0
        self._stream = torch.cuda.Stream(device=self.device)
        self._t0_ev = torch.cuda.Event(enable_timing=True)
        self._t0_ev.record(self._stream)
        self.t0 = time.perf_counter()
        self.arrival = [None] * len(jobs)
        self._flags = [_Arrival(self, k) for k in range(len(jobs))]
        self._job_ev = [None] * len(jobs)
        self._final = [sum(self._ends[:k + 1]) / self.rate for k in range(len(jobs))]
        self.pump()
        return self._flags

    def pump(self):
        """Issue every chunk whose time has come."""
        now = time.perf_counter() - self.t0
        while self._next < len(self._plan) and self._plan[self._next][0] <= now:
            _, sp, dp, k = self._plan[self._next]
            with torch.cuda.stream(self._stream):
                dp.copy_(sp, non_blocking=True)
                if k >= 0:
                    ev = torch.cuda.Event(enable_timing=True)
                    ev.record(self._stream)
                    self._job_ev[k] = ev
            self._next += 1

    def done(self) -> bool:
        return self._next == len(self._plan)

    def _landed(self, k: int) -> bool:
        ev = self._job_ev[k]
        # a job has landed once its last chunk's copy has completed and the link's schedule has
        # reached its last byte (a chunk's copy itself runs at the copy engine's rate)
        if ev is None or time.perf_counter() - self.t0 < self._final[k] or not ev.query():
            return False
        if self.arrival[k] is None:
            self.arrival[k] = max(self._t0_ev.elapsed_time(ev) / 1e3, self._final[k])
        return True

    def wait(self):
        """Until every job has landed (polled mode: keeps pumping)."""
        if self._thread is not None:
            self._thread.join()
        elif getattr(self, "_plan", None) is not None:
            while not all(f.is_set() for f in self._flags):
                time.sleep(0.001)
            self._stream.synchronize()
        if self.error is not None:
            raise self.error


class _Arrival:
    """is_set() of one job in polled mode."""

    def __init__(self, link: SlowLink, k: int):
        self.link, self.k = link, k

    def is_set(self) -> bool:
        self.link.pump()
        return self.link._landed(self.k)


def _chunks(src: torch.Tensor, dst: torch.Tensor, chunk_bytes: int):
    """(src piece, dst piece) pairs of about chunk_bytes each: whole slices along the leading
    index while they fit, flat pieces of a contiguous pair otherwise."""
    if src.shape != dst.shape and src.numel() != dst.numel():
        raise ValueError("source and destination sizes differ")
    if src.shape != dst.shape:
        src = src.reshape(dst.shape)
    per = src[0].numel() * src.element_size() if src.dim() > 1 else src.element_size()
    if src.dim() > 1 and per >= chunk_bytes // 4:
        for i in range(src.shape[0]):
            yield from _chunks(src[i], dst[i], chunk_bytes)
        return
    if src.dim() > 1 and not (src.is_contiguous() and dst.is_contiguous()):
        step = max(1, chunk_bytes // per)
        for i in range(0, src.shape[0], step):
            yield src[i:i + step], dst[i:i + step]
        return
    s, d = src.reshape(-1), dst.reshape(-1)
    step = max(1, chunk_bytes // src.element_size())
    for o in range(0, s.numel(), step):
        yield s[o:o + step], d[o:o + step]
