"""GPU timing helpers shared by the sweep and multi-chunk CLIs.

Modes are timed interleaved round-robin, so all of them see the same clock
and thermal state, with HBM and the caches flushed (a 1 GiB write) before
every call; times are HIP events on the current stream."""
from __future__ import annotations

import statistics


def interleaved_us(fns, steps: int, warmup: int, flush):
    """Median microseconds of each callable over `steps` interleaved rounds."""
    import torch
    for _ in range(warmup):
        for fn in fns:
            fn()
    ts = [[] for _ in fns]
    for _ in range(steps):
        for k, fn in enumerate(fns):
            flush.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            ts[k].append((e0, e1))
    torch.cuda.synchronize()
    return [statistics.median(a.elapsed_time(b) for a, b in t) * 1e3 for t in ts]


def on_two_streams(first, second, s1, s2):
    """Run first() on stream s1 and second() on s2, forked from and joined
    back into the current stream with events (the two-stream baseline)."""
    import torch
    main = torch.cuda.current_stream()
    fork = torch.cuda.Event()
    fork.record(main)
    s1.wait_event(fork)
    s2.wait_event(fork)
    first(s1)
    second(s2)
    j1, j2 = torch.cuda.Event(), torch.cuda.Event()
    j1.record(s1)
    j2.record(s2)
    main.wait_event(j1)
    main.wait_event(j2)
