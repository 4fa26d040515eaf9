"""The grouped expert products pick one code path per 128-row expert tile by its count of 16-row
fragments: the BF16-activation tiled kernel has paths for 2 (1-2 fragments), 3, 4, 5, 6 and 8 (7-8),
the A4W4 kernel for 1, 2, 3, 4, 5, 6 and 8. This checks on the CPU that the small GPU parity cases
(the prefill_small and nolat_tiled shapes, and the A4W4 ragged prefixes of prefill_small) route
tokens so that every path meets at least one tile. Routing is taken from the oracle's logits; a
near-tie flipped on the GPU moves one pair, and the margins below are wide."""
import numpy as np

from oracle import oracle as O
from tests.test_gpu_parity import NOLAT_TILED, PREFILL_SMALL
from workload import make_inputs

TILE_ROWS = 128
TILED_MIN_ROWS = 32          # expert tiles from 32 routed rows per expert on average


def _fragment_counts(shape, T):
    inp = make_inputs(shape, ["x", "w_router", "router_bias"])
    ids = O.select(O.logits(inp["x"][:T], inp["w_router"], inp.get("router_bias")), shape.K)
    assert T * shape.K >= TILED_MIN_ROWS * shape.E, "the case must take the tiled expert path"
    counts = np.bincount(ids.ravel(), minlength=shape.E)
    frags = []
    for n in counts[counts > 0]:
        frags += [TILE_ROWS // 16] * (n // TILE_ROWS)
        if n % TILE_ROWS:
            frags.append((n % TILE_ROWS + 15) // 16)
    return frags


def _tiled_path(nmf):
    return 2 if nmf <= 2 else 8 if nmf >= 7 else nmf


def _a4_path(nmf):
    return 8 if nmf >= 7 else nmf


def test_every_tiled_path_meets_a_tile():
    frags = _fragment_counts(PREFILL_SMALL, PREFILL_SMALL.T) + _fragment_counts(NOLAT_TILED, NOLAT_TILED.T)
    # the BF16 parity tests run prefill_small at its full size and at ragged prefixes
    for T in (128, 131, 257):
        frags += _fragment_counts(PREFILL_SMALL, T)
    assert {_tiled_path(f) for f in frags} == {2, 3, 4, 5, 6, 8}


def test_every_a4_path_meets_a_tile():
    frags = _fragment_counts(PREFILL_SMALL, PREFILL_SMALL.T)
    for T in (128, 131, 257):
        frags += _fragment_counts(PREFILL_SMALL, T)
    assert {_a4_path(f) for f in frags} == {1, 2, 3, 4, 5, 6, 8}
