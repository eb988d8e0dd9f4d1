"""The float64 oracle against its pins (CPU only)."""
import json
import os

import pytest

import oracle
from tests import oracle_pins as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


@pytest.mark.parametrize("pin", P.DENSE_PINS + P.ROPE_PINS + P.SPARSE_PINS + P.TOPK_PINS + P.PROJ_PINS + P.FP8_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


def test_pieces_against_printed_figures():
    with open(GOLDEN) as f:
        P.pin_pieces(oracle, json.load(f))
