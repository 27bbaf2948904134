"""The attention kernel's workgroup protocol, checked on the CPU with the
model in schedule_model.py: no LDS race in the schedule as built (2 K and 4 V
tile buffers, V-operand reads left in flight across the VALU-phase barrier),
in either order of visiting a workgroup's row blocks; the model does find the
races of a schedule with one V buffer fewer, so it sees that hazard; and the
split schedule's piece slots and counters match between the workgroups that
write pieces and the one that merges them."""
import random

import pytest

from schedule_model import check_pieces, random_workgroups


@pytest.mark.parametrize("reverse", [False, True])
def test_protocol_has_no_lds_race(reverse):
    assert random_workgroups(random.Random(1), 200, kbufs=2, vbufs=4, reverse=reverse) == []


def test_model_sees_the_race_of_three_value_buffers():
    # with 3 V buffers the buffer read in flight is rewritten one phase later
    assert len(random_workgroups(random.Random(2), 100, kbufs=2, vbufs=3)) > 0


def test_piece_slots_and_counters():
    rng = random.Random(3)
    for _ in range(400):
        n_qt, H = rng.randint(1, 20), rng.randint(1, 24)
        n_v = rng.randint(1, 64) * rng.randint(1, 25)
        n_wg = rng.randint(1, min(4096, n_qt * H * n_v))
        check_pieces(n_qt, H, n_v, n_wg)
        check_pieces(n_qt, H, n_v, n_wg, reverse=True)
