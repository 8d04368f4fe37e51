"""Seeded synthetic workloads shaped like the chunked-prefill pages' examples.

Every random value comes from ``numpy.random.Generator(PCG64(SeedSequence(key)))``
with ``key = (workload index, request index, stream, generator block)``:

* stream 0: queries, stream 1: keys, stream 2: values (fp32 standard normal,
  multiplied by the workload's ``mult`` in fp32, then rounded to the workload's
  dtype with round-to-nearest-even);
* stream 3: the physical block permutation of the paged cache;
* stream 4: decode-row context lengths (uniform integers, inclusive bounds).

Token values are drawn in generator blocks of ``GEN_BLOCK`` tokens, so any token
range can be regenerated alone (sampled parity checks at 128k tokens need that).

The five named workloads follow the shapes the pages use as examples: a
4000-token prompt cut at 512 (token-budget blog, section 2), 32768 tokens with a
0.5 prefix-cache hit rate cut at 8192 (msmodeling chunked-prefill RFC, section
2.2), a 2048-token mixed step with decode rows (token-budget blog, section 5),
and 131072 tokens cut at 1024 (msmodeling latency-table RFC, section 1.2).
Head counts, head size, block size and value distributions are not on the pages;
they are fixed here.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

GEN_BLOCK = 1024  # tokens per independently seeded generator block

STREAM_Q, STREAM_K, STREAM_V, STREAM_PERM, STREAM_DECODE = 0, 1, 2, 3, 4


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def round_to_bf16(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Round fp32 values to bfloat16 with round-to-nearest-even.

    Returns ``(values, bits)``: ``values`` are fp32 numbers exactly equal to the
    bf16 results, ``bits`` the bf16 bit patterns as uint16. Inputs are finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs stay below 0xFF800000, so the sums cannot wrap in uint32
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    t += u
    t >>= np.uint32(16)
    r = t.astype(np.uint16)
    t <<= np.uint32(16)
    return t.view(np.float32), r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def token_values(key: tuple, stream: int, t0: int, t1: int, heads: int, dim: int,
                 mult: float, dtype: str) -> np.ndarray:
    """Values for tokens ``[t0, t1)`` of one stream, shape ``[t1-t0, heads, dim]``.

    The result is fp32 and exactly representable in ``dtype`` ("f32" or "bf16").
    """
    if t1 <= t0:
        return np.zeros((0, heads, dim), np.float32)
    out = np.empty((t1 - t0, heads, dim), np.float32)
    b0, b1 = t0 // GEN_BLOCK, (t1 - 1) // GEN_BLOCK
    for b in range(b0, b1 + 1):
        blk = _rng(*key, stream, b).standard_normal((GEN_BLOCK, heads, dim), dtype=np.float32)
        if mult != 1.0:
            blk *= np.float32(mult)
        lo, hi = max(t0, b * GEN_BLOCK), min(t1, (b + 1) * GEN_BLOCK)
        out[lo - t0:hi - t0] = blk[lo - b * GEN_BLOCK:hi - b * GEN_BLOCK]
    if dtype == "bf16":
        out, _ = round_to_bf16(out)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return out


def block_permutation(key: tuple, num_blocks: int) -> np.ndarray:
    return _rng(*key, STREAM_PERM).permutation(num_blocks).astype(np.int32)


def decode_context_lengths(key: tuple, n: int, lo: int, hi: int) -> np.ndarray:
    """``n`` uniform integers in ``[lo, hi]`` (both ends included)."""
    return _rng(*key, STREAM_DECODE).integers(lo, hi, size=n, endpoint=True).astype(np.int64)


@dataclass
class Request:
    """One sequence in the paged cache.

    ``n_ctx`` is the number of tokens whose K/V the cache must hold for the
    request's last launch; ``blocks`` are its physical block ids in logical order.
    ``launch`` is either ``None`` (the workload is planned with a chunk plan) or an
    explicit ``(prefix_len, extend_len)`` for a single mixed-step launch.
    """

    index: int
    n_ctx: int
    blocks: np.ndarray
    launch: tuple[int, int] | None = None


@dataclass
class Workload:
    name: str
    index: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str            # "f32" or "bf16"
    mult: float           # multiplier on the standard normal draws
    scale: float          # softmax scale passed to the kernel (fp32 value)
    block_size: int
    num_blocks: int
    requests: list[Request]
    plan: tuple[int, int, float] | None = None   # (n_tokens, chunk_size, hit_rate)
    notes: str = ""
    extra: dict = field(default_factory=dict)

    def key(self, req: Request) -> tuple:
        return (self.index, req.index)

    def q(self, req: Request, t0: int, t1: int) -> np.ndarray:
        return token_values(self.key(req), STREAM_Q, t0, t1, self.n_q_heads, self.head_dim, self.mult, self.dtype)

    def k(self, req: Request, t0: int, t1: int) -> np.ndarray:
        return token_values(self.key(req), STREAM_K, t0, t1, self.n_kv_heads, self.head_dim, self.mult, self.dtype)

    def v(self, req: Request, t0: int, t1: int) -> np.ndarray:
        return token_values(self.key(req), STREAM_V, t0, t1, self.n_kv_heads, self.head_dim, self.mult, self.dtype)

    def block_table(self) -> np.ndarray:
        """``[num_requests, max_blocks]`` int32, unused entries ``-1``."""
        mb = max(len(r.blocks) for r in self.requests)
        bt = np.full((len(self.requests), mb), -1, np.int32)
        for i, r in enumerate(self.requests):
            bt[i, :len(r.blocks)] = r.blocks
        return bt


def _assign_blocks(key: tuple, n_ctx: list[int], block_size: int, permute: bool,
                   spare: int = 0) -> tuple[list[np.ndarray], int]:
    need = [-(-n // block_size) for n in n_ctx]
    total = sum(need) + spare
    ids = block_permutation(key, total) if permute else np.arange(total, dtype=np.int32)
    out, pos = [], 0
    for n in need:
        out.append(ids[pos:pos + n].copy())
        pos += n
    return out, total


def _single(name: str, index: int, n_tokens: int, chunk: int, hit: float, hq: int, hkv: int,
            d: int, dtype: str, mult: float, permute: bool, notes: str) -> Workload:
    blocks, nb = _assign_blocks((index, 0), [n_tokens], 16, permute)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    return Workload(name, index, hq, hkv, d, dtype, mult, scale, 16, nb,
                    [Request(0, n_tokens, blocks[0])], plan=(n_tokens, chunk, hit), notes=notes)


def _mixed(index: int = 4) -> Workload:
    lens = decode_context_lengths((index, 0), 64, 512, 8192)
    n_ctx = [int(x) for x in lens] + [6144 + 1984]
    blocks, nb = _assign_blocks((index, 0), n_ctx, 16, True)
    reqs = [Request(i, int(L), blocks[i], launch=(int(L) - 1, 1)) for i, L in enumerate(lens)]
    reqs.append(Request(64, 6144 + 1984, blocks[64], launch=(6144, 1984)))
    scale = float(np.float32(1.0 / math.sqrt(128)))
    return Workload("mixed_budget2048", index, 32, 8, 128, "bf16", 0.5, scale, 16, nb, reqs,
                    notes="64 decode rows (context U{512..8192}) then one 1984-token chunk at prefix 6144")


def make_workload(name: str) -> Workload:
    if name == "tiny_f32":
        return _single(name, 1, 64, 16, 0.0, 1, 1, 64, "f32", 1.0, False,
                       "N=64, C=16, 1/1 heads, D=64, fp32, contiguous blocks")
    if name == "prompt4000":
        return _single(name, 2, 4000, 512, 0.0, 32, 8, 128, "bf16", 0.5, True,
                       "N=4000, C=512, 32/8 heads, D=128, bf16")
    if name == "prefix_cache32k":
        return _single(name, 3, 32768, 8192, 0.5, 32, 8, 128, "bf16", 0.5, True,
                       "N=32768, hit rate 0.5, C=8192, 32/8 heads, D=128, bf16")
    if name == "mixed_budget2048":
        return _mixed()
    if name == "sweep128k":
        return _single(name, 5, 131072, 1024, 0.0, 64, 8, 128, "bf16", 0.5, True,
                       "N=131072, C=1024, 64/8 heads, D=128, bf16")
    raise KeyError(name)


WORKLOADS = ("tiny_f32", "prompt4000", "prefix_cache32k", "mixed_budget2048", "sweep128k")


def custom_workload(seed: int, launches: list[tuple[int, int]], n_q_heads: int, n_kv_heads: int,
                    head_dim: int, dtype: str = "bf16", mult: float = 0.5, permute: bool = True,
                    spare_blocks: int = 0, scale: float | None = None) -> Workload:
    """Edge-case workload: one request per ``(prefix_len, extend_len)`` launch entry."""
    index = 1000 + seed
    n_ctx = [p + e for p, e in launches]
    blocks, nb = _assign_blocks((index, 0), n_ctx, 16, permute, spare=spare_blocks)
    reqs = [Request(i, n_ctx[i], blocks[i], launch=launches[i]) for i in range(len(launches))]
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(head_dim)))
    return Workload(f"custom{seed}", index, n_q_heads, n_kv_heads, head_dim, dtype, mult, scale, 16,
                    nb, reqs)


def device_normal(shape, seed: int, mult: float, dtype, device="cuda"):
    """Seeded standard-normal values drawn on the device (torch Philox), times
    ``mult`` in fp32, rounded to ``dtype``. Used where the bench needs gigabytes
    of inputs quickly; parity tests use the NumPy streams above."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    if mult != 1.0:
        x.mul_(mult)
    return x.to(dtype)
