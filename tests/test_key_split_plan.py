"""Key split of a visiting block (no GPU): the host-side choice and layout that
RingEmulator.run(key_split=...) and bench.py use when the query block alone
would leave compute units idle.  The keys of each visiting block are cut into
ranges folded into separate partial states and merged once at the end; the
merge of partial online-softmax states makes the grouping of keys irrelevant
(pinned for the oracle in test_oracle.py: merges of random partitions equal the
dense result)."""
import pytest

torch = pytest.importorskip("torch")

from ring_attention_block_amd.ring import key_split_for, split_keys


def test_key_split_choice():
    # causal rings and blocks that fill the chip fold whole blocks
    assert key_split_for(32, 4096, 4096, True) == 1
    assert key_split_for(32, 4096, 4096, False) == 1
    assert key_split_for(8, 16384, 16384, False) == 1
    # the 8-head 2048-row stress ring: 64 query tiles of 256 rows -> halves,
    # 256 workgroups of 128 rows
    assert key_split_for(8, 2048, 2048, False) == 2
    assert key_split_for(4, 2048, 2048, False) == 4
    # only whole 64-key tiles per range
    assert key_split_for(4, 300, 300, False) == 1
    assert key_split_for(1, 128, 128, False) == 2
    assert key_split_for(1, 192, 192, False) == 1


@pytest.mark.parametrize("parts", [1, 2, 4])
def test_split_keys_layout(parts):
    h, n, d = 3, 256, 8
    t = torch.arange(h * n * d, dtype=torch.float32).reshape(1, h, n, d)
    s = split_keys(t, parts)
    assert s.shape == (parts, h, n // parts, d) and s.is_contiguous()
    for p in range(parts):
        assert torch.equal(s[p], t[0, :, p * n // parts:(p + 1) * n // parts])


def test_split_keys_rejects():
    with pytest.raises(ValueError):
        split_keys(torch.zeros(2, 1, 8, 4), 2)
    with pytest.raises(ValueError):
        split_keys(torch.zeros(1, 1, 6, 4), 4)
