"""The layer-wise prefetch schedule's copy waits (host logic, no GPU): every row copy of layer
l must follow the table resolve of layer l, either by its own wait or by a wait of an earlier
copy on the same stream for the tables of layer l or a later one (the tables run in layer order
on one stream)."""
import pytest

from hierarchical_kv_cache_hs_amd.decode_step import copy_waits


@pytest.mark.parametrize("layers", list(range(1, 70)))
def test_every_copy_follows_its_tables(layers):
    waits = copy_waits(layers)
    assert waits[0] == 0
    covered = -1
    for l in range(layers):
        if l in waits:
            assert 0 <= waits[l] < layers
            covered = max(covered, waits[l])
        assert covered >= l, f"copy {l} of {layers} could start before its tables"


def test_waits_for_eight_layers():
    assert copy_waits(8) == {0: 0, 1: 1, 2: 3, 4: 7}
    assert len(copy_waits(61)) == 7          # copies 0, 1, 2, 4, 8, 16, 32
