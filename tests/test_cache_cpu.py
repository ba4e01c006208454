"""Host-side logic of the KV-cache layer (no GPU): write positions of linear
and ring caches, trimming, and the byte accounting against the cache page's
storage formula (hand-worked values in tests/golden/cache_bytes.txt)."""
import pytest
import torch

from vector_quantized_kv_amd import CacheLayout, VQKVCache
from conftest import read_golden


def test_linear_layout():
    L = CacheLayout(B=2, S_cap=10)
    assert L.append_spans(4) == [(0, 0, 4)]
    L.advance(4)
    assert L.append_spans(6) == [(4, 0, 6)]
    with pytest.raises(ValueError, match="overflows"):
        L.append_spans(7)
    L.advance(6)
    assert L.size() == 10 and L.is_trimmable()
    assert L.trim(3) == 3 and L.offset == 7 and L.size() == 7
    assert L.append_spans(2) == [(7, 0, 2)]      # the trimmed slots are written next
    assert L.trim(100) == 7 and L.size() == 0


def test_ring_layout():
    L = CacheLayout(B=1, S_cap=10, ring=True)
    L.advance(8)
    assert L.trim(2) == 2 and L.offset == 6      # not wrapped yet: trimmable
    L.advance(2)
    assert L.append_spans(5) == [(8, 0, 2), (0, 2, 5)]
    L.advance(5)
    assert L.offset == 13 and L.size() == 10 and L.wrapped()
    assert not L.is_trimmable() and L.trim(1) == 0 and L.offset == 13
    assert L.append_spans(10) == [(3, 0, 7), (0, 7, 10)]
    with pytest.raises(ValueError, match="longer than the ring"):
        L.append_spans(11)


def test_byte_accounting():
    rows = read_golden("cache_bytes.txt")[None].reshape(-1, 6)
    for bits, kb, vb, f16, cbb, avg in rows:
        n_c = 2 ** int(bits)
        c = VQKVCache(2, 8, 128, 256, torch.zeros(n_c, 8), torch.zeros(n_c, 4),
                      code_bits=int(bits), device="cpu")
        assert c.empty() and c.compressed_key_bytes == 0
        c.layout.advance(100)
        assert c.size() == 100
        assert c.compressed_key_bytes == kb and c.compressed_value_bytes == vb
        assert c.fp16_key_bytes == f16 and c.fp16_value_bytes == f16
        assert c.codebook_bytes == cbb and c.assigned_avg_bits == avg
        # index buffers held: 256 slots x (16 + 32) code bytes x rows x heads (8-bit)
        assert c.nbytes == 2 * 8 * 256 * (128 // 8 + 128 // 4) * int(bits) // 8
        c.trim(30)
        assert c.compressed_key_bytes == kb * 70 // 100
    s = VQKVCache(2, 8, 128, 256, torch.zeros(256, 8), torch.zeros(256, 4), mode="standard",
                  device="cpu")
    assert s.nbytes == 2 * 2 * 8 * 256 * 128 * 2   # two fp16 buffers
    with pytest.raises(ValueError):
        VQKVCache(1, 1, 128, 8, torch.zeros(256, 8), torch.zeros(256, 4), mode="standard",
                  ring=True, device="cpu")
