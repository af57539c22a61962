"""CPU checks of the test helpers themselves: the validity check that the
GPU tests apply to near-tie selection rows must accept every correct kept
list and reject wrong ones."""
import numpy as np
import pytest

from gpu_helpers import valid_near_tie_list
from oracle import sparse as osp


def test_near_tie_validity_accepts_correct_lists_and_rejects_wrong_ones():
    g = np.random.default_rng(0)
    s = g.standard_normal(40)
    s[7] = s[3] * (1 + 1e-9)  # tiles 3 and 7 nearly tie
    k = int(np.sum(s > max(s[3], s[7]))) + 1  # the cut falls between them
    kept, tie, _ = osp.select_one(s, k)
    assert tie
    valid_near_tie_list(kept, s, k)
    # the other member of the tie group is just as valid
    alt = np.sort(np.concatenate([kept[kept != 3], [7]]) if 3 in kept else
                  np.concatenate([kept[kept != 7], [3]]))
    valid_near_tie_list(alt, s, k)
    low = int(np.argmin(s))
    wrong = np.sort(np.concatenate([kept[kept != kept[0]], [low]]))
    with pytest.raises(AssertionError):
        valid_near_tie_list(wrong, s, k)  # a tile far below the band kept
    with pytest.raises(AssertionError):
        valid_near_tie_list(kept[:-1], s, k)  # k - 1 tiles
    with pytest.raises(AssertionError):
        valid_near_tie_list(kept[::-1], s, k)  # not ascending
