"""Host-side logic of bench.py checked against the oracle's masks (no GPU)."""

import numpy as np
import pytest

import bench
from g4inputs import gen
from oracle import attention as oat


@pytest.mark.parametrize("S,w,images", [(50, 8, [(3, 5), (20, 25)]), (64, 0, [(0, 10), (30, 34)]),
                                        (100, 16, []), (300, 64, [(0, 20), (40, 150), (250, 50)])])
def test_span_pair_count_matches_the_mask(S, w, images):
    lo, hi = gen.image_spans(S, images)
    assert bench.span_pairs(S, w, lo, hi) == int(oat.mask_spans(S, w, lo, hi).sum())


def test_image_spans_layout():
    lo, hi = gen.image_spans(12, [(2, 3), (9, 3)])
    assert lo.tolist() == [0, 1, 2, 2, 2, 5, 6, 7, 8, 9, 9, 9]
    assert hi.tolist() == [0, 1, 4, 4, 4, 5, 6, 7, 8, 11, 11, 11]


@pytest.mark.parametrize("S,w", [(1024, 512), (8192, 0), (16384, 1024), (5, 8), (100, 1), (3000, 700)])
def test_visible_pair_count_matches_the_mask(S, w):
    assert bench.visible_pairs(S, w) == oat.visible_pairs(S, w)
