"""Host logic of the step schedule (section 6, "Implementations": 50 steps, dense for the
first 20%, clustering and masks recomputed every R = 10 steps and reused in between)."""
import pytest

from block_sparse_attention_response_amd.schedule import ParkSchedule


def test_paper_schedule():
    s = ParkSchedule(1024, 10, 0.9, 8)
    kinds = [s.kind(t) for t in range(50)]
    assert kinds[:10] == ["dense"] * 10
    assert [t for t in range(50) if kinds[t] == "recompute"] == [10, 20, 30, 40]
    assert kinds.count("reuse") == 36


def test_no_dense_prefix_and_rounding():
    s = ParkSchedule(8, 2, 0.9, 1, total_steps=7, dense_fraction=0.0, recompute_every=3)
    assert [s.kind(t) for t in range(7)] == ["recompute", "reuse", "reuse", "recompute", "reuse", "reuse", "recompute"]
    s = ParkSchedule(8, 2, 0.9, 1, total_steps=7, dense_fraction=0.2)   # floor(1.4) = 1 dense step
    assert s.dense_steps == 1 and s.kind(0) == "dense" and s.kind(1) == "recompute"


def test_bad_arguments():
    with pytest.raises(ValueError):
        ParkSchedule(8, 2, 0.9, 1, total_steps=0)
    with pytest.raises(ValueError):
        ParkSchedule(8, 2, 0.9, 1, recompute_every=0)
    with pytest.raises(ValueError):
        ParkSchedule(8, 2, 0.9, 1, dense_fraction=1.5)
    s = ParkSchedule(8, 2, 0.9, 1, total_steps=5)
    with pytest.raises(ValueError):
        s.attention(5, None, None, None)
