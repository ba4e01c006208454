"""KV-cache management on top of the C ABI ("veloxquant_mlx.cache.vecinfer_cache
module" page, VecInferKVCache): appends, the two storage modes, trimming and
byte accounting.  Every step of the method (smoothing, rotation, product-VQ
encode and decode, attention from codes) runs in libvq's kernels; this module
only keeps buffers and write positions.

Modes (the page's update_and_fetch and state):
  standard  keys and values are quantized and immediately dequantized
            (vq_encode_decode); the fp16 reconstructions are kept in a
            [B, H, S_cap, D] buffer and update_and_fetch returns the
            reconstructions of every stored token, for an ordinary SDPA.
  fused     only the code indices are kept ([B, H, S_cap, row_bytes] index
            buffers, vq_encode_kv); fused_sdpa attends straight from them
            (vq_attend), applying the query's dual transform itself.

Positions.  `offset` counts the tokens appended so far.  A linear cache
stores token p in slot p and holds at most S_cap tokens.  A ring cache
(fused mode) stores token p in slot p mod S_cap and keeps the last S_cap
tokens: a sliding window of S_cap keys for decoding.  Once a ring has
wrapped, its slots are no longer in token order, so attention over it must
be permutation invariant: one query per row (S_q = 1), causal, and no window
shorter than the ring.

trim(n) drops the last n tokens by moving every write position back, so the
next append overwrites them and no stale tail is attended (the failure the
page describes for index buffers advanced separately from the offset).  A
ring that has wrapped is not trimmable: its older tokens are already gone.
"""
from __future__ import annotations

import torch

from . import api

HALF_BYTES = 2


class CacheLayout:
    """Write positions of a linear or ring cache, per batch row (host-only)."""

    def __init__(self, B: int, S_cap: int, ring: bool = False):
        if B <= 0 or S_cap <= 0:
            raise ValueError("B and S_cap must be positive")
        self.B, self.S_cap, self.ring = B, S_cap, ring
        self.offset = 0          # tokens appended (the same for every row)

    def size(self) -> int:
        """Tokens currently stored."""
        return min(self.offset, self.S_cap)

    def wrapped(self) -> bool:
        return self.ring and self.offset > self.S_cap

    def is_trimmable(self) -> bool:
        return not self.wrapped()

    def append_spans(self, S: int):
        """Slot spans [(slot, token_lo, token_hi)] that receive tokens
        [0, S) of an append: one span, or two when a ring wraps."""
        if S < 0:
            raise ValueError("negative append")
        if not self.ring:
            if self.offset + S > self.S_cap:
                raise ValueError(f"append of {S} tokens overflows the linear cache "
                                 f"({self.offset} of {self.S_cap} slots used)")
            return [(self.offset, 0, S)] if S else []
        if S > self.S_cap:
            raise ValueError(f"append of {S} tokens is longer than the ring ({self.S_cap})")
        spans, done = [], 0
        while done < S:
            slot = (self.offset + done) % self.S_cap
            n = min(S - done, self.S_cap - slot)
            spans.append((slot, done, done + n))
            done += n
        return spans

    def advance(self, S: int):
        self.offset += S

    def trim(self, n: int) -> int:
        """Drop the last n tokens (at most the stored count); returns how many
        were dropped.  A wrapped ring drops none."""
        if n < 0:
            raise ValueError("negative trim")
        if not self.is_trimmable():
            return 0
        n = min(n, self.offset)
        self.offset -= n
        return n


def storage_bytes(tokens: int, B: int, H: int, D: int, sub_dim: int, bits: int) -> int:
    """Packed code bytes of `tokens` tokens of every (batch row, head): the
    per-token storage (D / d) * b / 8 of the cache page's formula."""
    return B * H * tokens * (D // sub_dim) * bits // 8


class VQKVCache:
    """Product-VQ KV cache of B rows x H kv heads x up to S_cap tokens of head
    dim D, with key codebook [2^b_k, d_k] and value codebook [2^b_v, d_v]
    (code_bits b = 8 or 4 for both), smooth factors [H, D] or None and the
    Walsh-Hadamard rotation of the keys (transform=True)."""

    def __init__(self, B, H, D, S_cap, k_codebook, v_codebook, *, smooth=None, transform=True,
                 code_bits=8, mode="fused", ring=False, device="cuda"):
        if mode not in ("standard", "fused"):
            raise ValueError("mode must be 'standard' or 'fused'")
        if ring and mode != "fused":
            raise ValueError("a ring buffer holds code indices: fused mode only")
        self.B, self.H, self.D, self.S_cap = B, H, D, S_cap
        self.k_codebook, self.v_codebook = k_codebook, v_codebook
        self.dk, self.dv = k_codebook.shape[1], v_codebook.shape[1]
        self.smooth, self.transform, self.code_bits = smooth, transform, code_bits
        self.mode = mode
        self.layout = CacheLayout(B, S_cap, ring)
        rb = lambda d: (D // d) * code_bits // 8
        if mode == "fused":
            self.k_codes = torch.zeros((B, H, S_cap, rb(self.dk)), dtype=torch.uint8, device=device)
            self.v_codes = torch.zeros((B, H, S_cap, rb(self.dv)), dtype=torch.uint8, device=device)
            self._lens = torch.zeros(B, dtype=torch.int32, device=device)
            self._lens_val = -1
        else:
            self.k_hat = torch.zeros((B, H, S_cap, D), dtype=torch.float16, device=device)
            self.v_hat = torch.zeros((B, H, S_cap, D), dtype=torch.float16, device=device)

    # -- the page's cache protocol ------------------------------------------
    @property
    def offset(self) -> int:
        return self.layout.offset

    def size(self) -> int:
        return self.layout.size()

    def empty(self) -> bool:
        return self.size() == 0

    def is_trimmable(self) -> bool:
        return self.layout.is_trimmable()

    def trim(self, n: int) -> int:
        return self.layout.trim(n)

    def update_and_fetch(self, keys, values):
        """Append fp16 keys and values [B, H, S, D].  Standard mode returns the
        dequantized fp16 (K_hat, V_hat) of every stored token [B, H, size, D];
        fused mode returns None (use fused_sdpa)."""
        B, H, S, D = keys.shape
        if (B, H, D) != (self.B, self.H, self.D) or tuple(values.shape) != tuple(keys.shape):
            raise ValueError("keys/values do not match the cache's [B, H, *, D]")
        for slot, lo, hi in self.layout.append_spans(S):
            k, v = keys[:, :, lo:hi].contiguous(), values[:, :, lo:hi].contiguous()
            if self.mode == "fused":
                api.vq_encode_kv(k, v, self.k_codebook, self.dk, self.v_codebook, self.dv,
                                 smooth=self.smooth, transform=self.transform,
                                 k_codes=self.k_codes, v_codes=self.v_codes, S_off=slot,
                                 code_bits=self.code_bits)
            else:
                # quantize and dequantize; the reconstructions go into the
                # fp16 buffer (the plain cache's concatenation)
                rk, _ = api.vq_encode_decode(k, self.k_codebook, self.dk, smooth=self.smooth,
                                             transform=self.transform, code_bits=self.code_bits)
                rv, _ = api.vq_encode_decode(v, self.v_codebook, self.dv, transform=False,
                                             code_bits=self.code_bits)
                self.k_hat[:, :, slot:slot + hi - lo].copy_(rk)
                self.v_hat[:, :, slot:slot + hi - lo].copy_(rv)
        self.layout.advance(S)
        if self.mode == "fused":
            return None
        n = self.size()
        return self.k_hat[:, :, :n], self.v_hat[:, :, :n]

    @property
    def state(self):
        """Standard mode: the fp16 (K_hat, V_hat) of the stored tokens; fused
        mode: the raw (key, value) index buffers of the stored slots."""
        n = self.size()
        if self.mode == "fused":
            return self.k_codes[:, :, :n], self.v_codes[:, :, :n]
        return self.k_hat[:, :, :n], self.v_hat[:, :, :n]

    def fused_sdpa(self, q, scale, *, causal=True, sliding_window=0):
        """Attention of raw fp16 queries [B, H_q, S_q, D] over the stored codes
        (the dual transform is applied inside)."""
        if self.mode != "fused":
            raise RuntimeError("fused_sdpa needs a fused-mode cache")
        n = self.size()
        if self.layout.wrapped():
            if q.shape[2] != 1 or not causal or (0 < sliding_window < self.S_cap):
                raise ValueError("a wrapped ring holds slots out of token order: one causal "
                                 "query per row and no window shorter than the ring")
        if self._lens_val != n:
            self._lens.fill_(n)
            self._lens_val = n
        return api.vq_attend(q, self.k_codes, self.k_codebook, self.v_codes, self.v_codebook,
                             scale=scale, smooth=self.smooth, transform=self.transform,
                             kv_lens=self._lens, causal=causal, sliding_window=sliding_window,
                             code_bits=self.code_bits)

    def decode_step(self, q, keys, values, scale, *, causal=True, sliding_window=0):
        """One decode step of a fused-mode cache: append one token per row
        (keys, values [B, H, 1, D]) and attend q [B, H_q, 1, D] over the
        updated cache.  When the new token lands in slot size - 1 (a linear
        cache, or a ring that has not wrapped) and the shape runs on the
        streaming kernel, both happen in one vq_decode_step launch; otherwise
        as update_and_fetch followed by fused_sdpa.  Same codes either way."""
        if self.mode != "fused":
            raise RuntimeError("decode_step needs a fused-mode cache")
        B, H, S, D = keys.shape
        if S != 1 or q.shape[2] != 1:
            raise ValueError("decode_step appends one token and attends one query position per row")
        n_after = self.size() + 1
        (slot, _, _), = self.layout.append_spans(1)
        fused = (slot == n_after - 1 and self.dk == 8 and self.dv == 4
                 and api.vq_attend_path(self.B, q.shape[1], 1, self.D, self.dk, self.dv,
                                        self.k_codebook.shape[0], self.H, self.S_cap, sliding_window,
                                        code_bits=self.code_bits, transform=int(bool(self.transform))) == "stream")
        if not fused:
            self.update_and_fetch(keys, values)
            return self.fused_sdpa(q, scale, causal=causal, sliding_window=sliding_window)
        if (B, H, D) != (self.B, self.H, self.D) or tuple(values.shape) != tuple(keys.shape):
            raise ValueError("keys/values do not match the cache's [B, H, *, D]")
        if self._lens_val != n_after:
            self._lens.fill_(n_after)
            self._lens_val = n_after
        out = api.vq_decode_step(q, keys.contiguous(), values.contiguous(), self.k_codes, self.k_codebook,
                                 self.v_codes, self.v_codebook, scale=scale, kv_lens=self._lens,
                                 smooth=self.smooth, transform=self.transform, causal=causal,
                                 sliding_window=sliding_window, code_bits=self.code_bits)
        self.layout.advance(1)
        return out

    # -- byte accounting ------------------------------------------------------
    @property
    def compressed_key_bytes(self) -> int:
        """Packed key-code bytes of the stored tokens (codebook excluded)."""
        return storage_bytes(self.size(), self.B, self.H, self.D, self.dk, self.code_bits)

    @property
    def compressed_value_bytes(self) -> int:
        return storage_bytes(self.size(), self.B, self.H, self.D, self.dv, self.code_bits)

    @property
    def fp16_key_bytes(self) -> int:
        """What the stored keys would take uncompressed (fp16)."""
        return self.B * self.H * self.size() * self.D * HALF_BYTES

    @property
    def fp16_value_bytes(self) -> int:
        return self.fp16_key_bytes

    @property
    def codebook_bytes(self) -> int:
        """Static codebook overhead: 2^b * d entries per codebook, counted in
        fp16 as on the page (this library stores them in fp32)."""
        b = self.code_bits
        return ((2 ** b) * self.dk + (2 ** b) * self.dv) * HALF_BYTES

    @property
    def assigned_avg_bits(self) -> float:
        """Bits per element averaged over keys and values: (b / d_k + b / d_v) / 2."""
        return (self.code_bits / self.dk + self.code_bits / self.dv) / 2

    @property
    def nbytes(self) -> int:
        """Device bytes the cache holds: the index buffers (fused) or the fp16
        reconstruction buffers (standard), as allocated."""
        if self.mode == "fused":
            return self.k_codes.numel() + self.v_codes.numel()
        return (self.k_hat.numel() + self.v_hat.numel()) * HALF_BYTES
