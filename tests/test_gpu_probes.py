"""GPU runs of the two measurement hooks (the read ceiling and the issue-rate
probe): they complete, touch only what they document, and write what they
promise."""
import numpy as np
import pytest

from gpu_cases import q8, say, torch

pytestmark = pytest.mark.gpu


def test_stream_read_reads_without_writing_the_sink():
    # a buffer of 0x01 bytes folds to 0 (an even count of equal words), so the
    # sink, written only for one fixed value, keeps its contents
    t, m = torch(), q8()
    say("[probe] q8_stream_read")
    buf = t.ones(1 << 20, dtype=t.uint8, device="cuda")
    sink = t.full((1,), 7, dtype=t.int32, device="cuda")
    for wg in (1, 256, 1024):
        for nt in (False, True):
            m.stream_read(buf, wg, nt, sink)
    t.cuda.synchronize()
    assert int(sink.item()) == 7


@pytest.mark.parametrize("mode", [0, 1, 2, 3, 4])
def test_issue_probe_writes_every_lane(mode):
    t, m = torch(), q8()
    say(f"[probe] q8_issue_probe mode {mode}")
    wg = 8
    out = t.full((wg * 1024,), float("nan"), dtype=t.float32, device="cuda")
    m.issue_probe(out, mode, 16, 16, wg)
    got = out.cpu().numpy()
    lanes = wg * (1024 if mode == 4 else 512)
    assert np.all(np.isfinite(got[:lanes]))
    if mode != 4:   # workgroups of 512 lanes: the rest of the scratch is untouched
        assert np.all(np.isnan(got[lanes:]))
