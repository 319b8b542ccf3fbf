"""The scaling sweep's measurement helper on small points: it runs through the
library, reports finite times, and its memory accounting follows the layout
(state independent of L, workspace linear in the segment count)."""

import math

import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import compressive_memory_transformers_segment_amd as ia
    ia.load()
    yield
    ia.release_handles()


def test_sweep_points():
    from compressive_memory_transformers_segment_amd import scaling
    pts = [scaling.point(L, 512, "delta", heads=2, d=64, min_seconds=0.0, min_steps=2)
           for L in (1024, 4096)]
    full = scaling.point(4096, 4096, "delta", heads=2, d=64, min_seconds=0.0, min_steps=2)
    for p in pts + [full]:
        assert math.isfinite(p["ms_per_forward"]) and p["ms_per_forward"] > 0
        assert p["fused_ms"] > 0 and p["scan_ms"] > 0
    assert pts[0]["state_bytes"] == pts[1]["state_bytes"] == full["state_bytes"]
    # Per-segment snapshots and statistics: 4x the segments, 4x the workspace
    # (up to the 256-byte rounding of each region).
    assert abs(pts[1]["workspace_bytes"] - 4 * pts[0]["workspace_bytes"]) <= 5 * 4 * 256
    assert pts[0]["segments"] == 2 and pts[1]["segments"] == 8 and full["segments"] == 1
