"""Pins for the oracle's closed forms: the worked example printed on the auturnal.com guide
("Worked calculation", Eq. (2)-(3)), hand-derived tail waste, and brute force."""

import json
import os

import pytest

from oracle import closed_forms as cf


@pytest.fixture(scope="module")
def worked(golden_dir):
    with open(os.path.join(golden_dir, "worked_example.json")) as f:
        return json.load(f)


def test_worked_example_totals(worked):
    lens = worked["lengths"]
    assert sum(lens) == worked["used_slots"] == 968
    fx = worked["fixed_reservation"]
    assert cf.fixed_reservation_slots(lens, fx["max_len"]) == fx["allocated_slots"]
    for row in worked["paged"]:
        assert sum(cf.allocated_slots(n, row["block_size"]) for n in lens) == row["allocated_slots"]


def test_worked_example_percentages(worked):
    lens = worked["lengths"]
    fx = worked["fixed_reservation"]
    assert round(100 * float(cf.fixed_utilisation(lens, fx["max_len"])), 2) == fx["utilisation_pct"]
    for row in worked["paged"]:
        assert round(100 * float(cf.utilisation(lens, row["block_size"])), 2) == row["utilisation_pct"]


def test_tail_waste_by_hand():
    # Worked by hand: next multiple of 16 (resp. 32) minus n.
    lens = [37, 91, 128, 201, 511]
    assert [cf.tail_waste(n, 16) for n in lens] == [11, 5, 0, 7, 1]
    assert [cf.tail_waste(n, 32) for n in lens] == [27, 5, 0, 23, 1]
    assert [cf.blocks_for(n, 16) for n in lens] == [3, 6, 8, 13, 32]
    assert [cf.blocks_for(n, 32) for n in lens] == [2, 3, 4, 7, 16]


@pytest.mark.parametrize("B", [1, 4, 16, 32])
def test_allocation_brute_force(B):
    # A_B(n) is the least multiple of B that holds n; waste never exceeds B - 1 (guide section 2).
    for n in range(0, 200):
        a = 0
        while a < n:
            a += B
        assert cf.allocated_slots(n, B) == a
        assert 0 <= cf.tail_waste(n, B) <= B - 1


def test_kv_bytes_eq1():
    # One layer of the 8 x 32768-token, 8-KV-head, d=128 bf16 batch is exactly 2^30 bytes.
    assert cf.kv_bytes(1, 8 * 32768, 8, 128, 2) == 2 ** 30
    # Factor 2 (K and V) and linearity in every factor.
    assert cf.kv_bytes(3, 5, 7, 11, 2) == 2 * 3 * 5 * 7 * 11 * 2


def test_fixed_reservation_rejects_overflow():
    with pytest.raises(ValueError):
        cf.fixed_reservation_slots([600], 512)
