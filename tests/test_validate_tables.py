"""Host-side debug check of the block table and lengths (no GPU)."""
import pytest
import torch

from sparse_kv_cache_amd.decode import validate_tables


def test_accepts_consistent_tables():
    bt = torch.tensor([[3, 1, 0, 0], [2, 4, 5, 6]], dtype=torch.int32)
    sl = torch.tensor([17, 64], dtype=torch.int32)
    validate_tables(bt, sl, num_blocks=7, page_size=16)
    # entries past a request's pages are not looked at
    bt[0, 2:] = -9
    validate_tables(bt, sl, num_blocks=7, page_size=16)
    validate_tables(bt, torch.tensor([0, 1], dtype=torch.int32), 7, 16)


@pytest.mark.parametrize("seq, ids, msg", [
    ([65, 1], [[0, 1, 2, 3], [4, 0, 0, 0]], "need 5 pages"),
    ([-1, 1], [[0, 1, 2, 3], [4, 0, 0, 0]], "< 0"),
    ([33, 1], [[0, 7, 2, 3], [4, 0, 0, 0]], "block id 7"),
    ([1, 16], [[0, 1, 2, 3], [-2, 0, 0, 0]], "block id -2"),
])
def test_rejects_bad_tables(seq, ids, msg):
    with pytest.raises(ValueError, match=msg):
        validate_tables(torch.tensor(ids, dtype=torch.int32),
                        torch.tensor(seq, dtype=torch.int32), num_blocks=7, page_size=16)
