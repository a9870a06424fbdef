"""The streaming-read reference runs through the C ABI and reports a rate in
a physically plausible range for one MI355X (HBM3E, 8 TB/s nominal)."""

import pytest
import torch

import kv_cache_vector_tq_amd as tqa

pytestmark = pytest.mark.gpu


def test_read_probe_rate():
    print("case read_probe 1 GiB", flush=True)
    buf = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ms = tqa.tq_read_probe(buf, sink, reps=3)
    rate = buf.numel() / (ms / 1e3) / 1e12
    print(f"streaming read {rate:.2f} TB/s", flush=True)
    assert 0.5 < rate < 12.0
    assert int(sink.item()) == 0  # the fold of all-ones bytes never equals the guard value
