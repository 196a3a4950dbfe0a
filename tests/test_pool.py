"""Host logic of the state pool: slot allocator and capacity arithmetic."""
import pytest
import torch

from block_hybrid_attention_amd.pool import StatePool, slot_bytes, slots_for_budget


def test_slot_bytes_and_budget():
    # S [16][256][128] + Z [16][256] fp32 per slot and layer
    assert slot_bytes(16, 128, 128) == 4 * 16 * 256 * 129 == 2_113_536
    # 288 GB of HBM3E, 6 hybrid layers per request
    n = slots_for_budget(288 * 10**9, 16, 128, 128, layers=6)
    assert n == 288 * 10**9 // (6 * 2_113_536) == 22710
    # one 128-request batch of one layer is 270.5 MB: past a 256 MB cache
    assert 128 * slot_bytes(16, 128, 128) == 270_532_608


def test_alloc_free_cycle_host_only():
    p = StatePool(4, 2, 64, 64, device="cpu", allocate=False)
    a = p.alloc(3)
    assert a.dtype == torch.int32 and a.tolist() == [0, 1, 2]
    assert p.free_slots == 1
    with pytest.raises(MemoryError):
        p.alloc(2)
    p.free([1])
    assert p.alloc(2).tolist() == [1, 3]
    with pytest.raises(ValueError):
        p.free([1, 1])


def test_alloc_zeroes_and_save_restore_on_host():
    p = StatePool(3, 1, 64, 64, device="cpu")
    s = p.alloc(2)
    p.S[s.long()] = 1.5
    p.Z[s.long()] = 2.5
    saved = p.save(s)
    p.free(s)
    t = p.alloc(2)                      # recycled slots come back zeroed
    assert float(p.S[t.long()].abs().sum()) == 0.0
    p.restore(torch.tensor([2, 0]), saved)
    assert torch.equal(p.S[2], saved[0][0]) and torch.equal(p.Z[0], saved[1][1])
