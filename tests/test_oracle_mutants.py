"""Each planted oracle mistake must be caught by at least one pin.

The mutants are the injected bugs the indexer-CP page lists (sglang PR 42614,
Accuracy Tests: the group's block count in place of the row's, the group sized
by its shortest row, the forced local window dropped, a wrong score-row index,
the fp8-to-bf16 cast dropped, K addressed by group index instead of through
the slot table) plus ones of this build's own (ties to the higher id, the
partial-block mask dropped, the sign of zero codes dropped, e2m1 ties away
from zero, the scale rounded toward zero, nibble order swapped, the init block
not forced, the lse computed without the softmax scale, a bad page scored -inf) and, for the
sparse attention over the selected blocks, the scale dropped, the length mask dropped, the
selection ignored, another head's selection, no normalization, V read untransposed, query heads
out of order and the fp8 K/V cast dropped.  Each is compiled into its own copy of the oracle (ORACLE_MUTANT).
"""
import pytest

import pins
from oracle import build as obuild
from oracle.binding import Oracle

MUTANTS = {
    1: "group block count in place of the row's",
    2: "group sized by its shortest row",
    3: "forced local window dropped",
    4: "wrong score-row index",
    5: "fp8-to-bf16 cast dropped",
    6: "K addressed by group index",
    7: "ties to the higher block id",
    8: "partial-block mask dropped",
    9: "sign of zero codes dropped",
    10: "e2m1 ties away from zero",
    11: "scale rounded toward zero",
    12: "nibble order swapped",
    13: "init block not forced",
    14: "lse without the softmax scale",
    15: "a visible block on a bad page scored -inf, not NaN",
    16: "attention: softmax scale dropped",
    17: "attention: length mask dropped",
    18: "attention: selection ignored (every block attended)",
    19: "attention: another KV head's selection",
    20: "attention: output not normalized",
    21: "attention: V read untransposed",
    22: "attention: query heads in the wrong order",
    23: "attention: fp8 K/V cast dropped",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: f"m{m}")
def test_mutant_is_caught(mutant, tmp_path_factory):
    path = obuild.build(tmp_path_factory.mktemp(f"m{mutant}") / "liboracle.so", mutant=mutant)
    o = Oracle(path)
    caught = []
    for pin in pins.PINS:
        try:
            pin(o)
        except AssertionError:
            caught.append(pin.__name__)
            break
    assert caught, f"mutant {mutant} ({MUTANTS[mutant]}) passes every pin"
