"""Seeded synthetic inputs for MLA decode over a paged latent KV cache.

This module only builds inputs: query rows, a paged cache (bf16 or the
656-byte FP8 record), a block table and sequence lengths.  It holds none of the
decode arithmetic and is shared by the tests, the smoke check and the
benchmark so that the GPU library and the CPU oracle read identical bytes.

Recipe (fixed draw order, numpy PCG64 seeded per case):
  1. sequence lengths, when drawn (uniform integers);
  2. q ~ N(0, 1) in fp32, rounded to bf16 (round to nearest even);
  3. cache values ~ N(0, 1) for every slot of every logical page, in logical
     (request, token) order, rounded to bf16;
  4. a permutation of the physical page ids (logical pages are scattered).
Optional extras: spare physical pages and NaN-poisoned tail slots (slots at or
beyond a request's length), and -1 in unused block-table entries.

FP8 records (token-major, 656 bytes): 512 OCP E4M3FN codes, four fp32 scales
(one per 128-dim tile, amax / 448), then the 64 RoPE dims as bf16.  Codes come
from torch's float8_e4m3fn cast (round to nearest even) of value / scale after
clamping to +-448; an all-zero tile gets scale 0 and codes 0.
"""
import math

import numpy as np

D_QK = 576
D_V = 512
D_ROPE = 64
PAGE = 64
FP8_RECORD = 656
FP8_TILE = 128
E4M3_MAX = 448.0


def bf16_bits(x):
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_fp8_records(k_bits):
    """bf16 keys [n, 576] (uint16 bits) -> FP8 records [n, 656] (uint8)."""
    import torch

    k = bf16_to_f32(k_bits).reshape(-1, D_QK)
    n = k.shape[0]
    lat = k[:, :D_V].reshape(n, D_V // FP8_TILE, FP8_TILE)
    amax = np.abs(lat).max(axis=2)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    x = (lat / safe[:, :, None]).astype(np.float32)
    x = np.clip(x, -E4M3_MAX, E4M3_MAX)
    codes = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    codes = np.where(scale[:, :, None] > 0, codes, 0).astype(np.uint8)
    rec = np.empty((n, FP8_RECORD), dtype=np.uint8)
    rec[:, :D_V] = codes.reshape(n, D_V)
    rec[:, D_V:D_V + 16] = scale.astype("<f4").view(np.uint8).reshape(n, 16)
    rec[:, D_V + 16:] = np.ascontiguousarray(k_bits.reshape(n, D_QK)[:, D_V:]).astype("<u2").view(
        np.uint8).reshape(n, 2 * D_ROPE)
    return rec


class Case:
    """One decode problem in host memory."""

    def __init__(self, q, cache, kind, block_table, seqlens, s_q, h_q, causal, scale, name=""):
        self.q = q                      # uint16 [batch, s_q, h_q, 576]
        self.cache = cache              # uint16 [pages, 64, 576] or uint8 [pages, 64, 656]
        self.kind = kind                # 0 = bf16 cache, 1 = fp8 cache
        self.block_table = block_table  # int32 [batch, width]
        self.seqlens = seqlens          # int32 [batch]
        self.s_q = s_q
        self.h_q = h_q
        self.causal = causal
        self.scale = scale
        self.name = name

    @property
    def batch(self):
        return int(self.seqlens.shape[0])

    @property
    def num_pages(self):
        return int(self.cache.shape[0])


def make_case(seqlens, s_q, h_q, seed, causal=False, fp8=False, spare_pages=0, poison=False,
              permute=True, scale=None, name="", rng=None, rope_ramp=0.0):
    """Build a Case.  ``seqlens`` is a sequence of ints (already drawn).

    ``rope_ramp`` > 0 multiplies the 64 RoPE dims of the key at position j by
    (1 + rope_ramp * j): scores then grow along the sequence (a running max
    that keeps rising) while the 512 value dims keep unit scale."""
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    seqlens = np.asarray(seqlens, dtype=np.int32)
    batch = seqlens.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(D_QK)
    q = bf16_bits(rng.standard_normal((batch, s_q, h_q, D_QK), dtype=np.float32))
    pages = [(int(L) + PAGE - 1) // PAGE for L in seqlens]
    n_log = sum(pages)
    n_phys = n_log + spare_pages
    width = max(1, max(pages) if pages else 1)
    rec_shape = (FP8_RECORD,) if fp8 else (D_QK,)
    cache = np.empty((n_phys, PAGE) + rec_shape, dtype=np.uint8 if fp8 else np.uint16)
    logical = []
    for b in range(batch):
        n_tok = pages[b] * PAGE
        raw = rng.standard_normal((n_tok, D_QK), dtype=np.float32)
        if rope_ramp:
            raw[:, D_V:] *= (1.0 + rope_ramp * np.arange(n_tok, dtype=np.float32))[:, None]
        vals = bf16_bits(raw)
        if fp8:
            vals = quantize_fp8_records(vals)
        logical.append(vals.reshape(pages[b], PAGE, *rec_shape))
    perm = rng.permutation(n_phys) if permute else np.arange(n_phys)
    block_table = np.full((batch, width), -1, dtype=np.int32)
    k = 0
    for b in range(batch):
        for j in range(pages[b]):
            phys = int(perm[k])
            block_table[b, j] = phys
            cache[phys] = logical[b][j]
            k += 1
        logical[b] = None
    poison_byte = 0xFF  # NaN for bf16, e4m3fn codes, fp32 scales
    for s in range(n_log, n_phys):
        cache[int(perm[s])] = poison_byte if fp8 else 0xFFFF
    if poison:
        for b in range(batch):
            L = int(seqlens[b])
            if pages[b] and L % PAGE:
                phys = block_table[b, pages[b] - 1]
                cache[phys, L % PAGE:] = poison_byte if fp8 else 0xFFFF
    return Case(q, cache, 1 if fp8 else 0, block_table, seqlens, s_q, h_q, causal, scale, name)


# The five workloads: (seqlens or a rule drawing them, s_q, h_q, causal, fp8).
CONFIGS = {
    "tiny": dict(seqlens=[37, 100], s_q=1, h_q=16, causal=False, fp8=False, seed=1,
                 desc="batch 2, seqlens {37,100}, s_q=1, h_q=16, bf16"),
    "membound": dict(seqlens=[4096] * 128, s_q=1, h_q=16, causal=False, fp8=False, seed=2,
                     desc="batch 128 x 4096, s_q=1, h_q=16, bf16"),
    "computebound": dict(seqlens=("uniform", 64, 2048, 8192), s_q=2, h_q=128, causal=True,
                         fp8=False, seed=3,
                         desc="batch 64, seqlens U[2048,8192], s_q=2 causal, h_q=128, bf16"),
    "fp8": dict(seqlens=[16384] * 64, s_q=1, h_q=128, causal=False, fp8=True, seed=4,
                desc="batch 64 x 16384, s_q=1, h_q=128, FP8 656-B records"),
    "longctx": dict(seqlens=[131072] * 8, s_q=1, h_q=128, causal=False, fp8=False, seed=5,
                    desc="batch 8 x 131072, s_q=1, h_q=128, bf16"),
}


def config_seqlens(name, rng):
    spec = CONFIGS[name]["seqlens"]
    if isinstance(spec, tuple) and spec[0] == "uniform":
        _, n, lo, hi = spec
        return rng.integers(lo, hi + 1, size=n).astype(np.int32)
    return np.asarray(spec, dtype=np.int32)


def make_config(name, spare_pages=0, poison=False):
    cfg = CONFIGS[name]
    rng = np.random.Generator(np.random.PCG64(cfg["seed"]))
    seqlens = config_seqlens(name, rng)
    return make_case(seqlens, cfg["s_q"], cfg["h_q"], cfg["seed"], causal=cfg["causal"],
                     fp8=cfg["fp8"], spare_pages=spare_pages, poison=poison, name=name, rng=rng)


def algorithmic_bytes(seqlens, s_q, h_q, fp8):
    """Bytes the method must move: every cached token once, q, out, lse, table, lengths."""
    tok = FP8_RECORD if fp8 else 2 * D_QK
    L = np.asarray(seqlens, dtype=np.int64)
    pages = (L + PAGE - 1) // PAGE
    b = L.shape[0]
    return int(L.sum() * tok + b * s_q * h_q * (2 * D_QK + 2 * D_V + 4) + pages.sum() * 4 + 4 * b)


def algorithmic_flops(seqlens, s_q, h_q, causal):
    """2 * h_q * (576 + 512) multiply-adds per visible (row, key) pair."""
    L = np.asarray(seqlens, dtype=np.int64)
    total = 0
    for i in range(s_q):
        n = L - (s_q - 1 - i) if causal else L
        total += int(np.clip(n, 0, None).sum())
    return 2 * h_q * (D_QK + D_V) * total


def make_config_device(name, device="cuda"):
    """The same workload shapes generated directly in device memory (torch's
    seeded CUDA generator; N(0,1) rounded to bf16; shuffled physical pages).
    For timing runs, where regenerating gigabytes on the host would dominate.
    Returns (q, kcache, block_table, seqlens, s_q, h_q, causal, scale, fp8)."""
    cfg = CONFIGS[name]
    rng = np.random.Generator(np.random.PCG64(cfg["seed"]))
    seqlens = config_seqlens(name, rng)
    q, kc, bt, sl = make_device_inputs(seqlens, cfg["s_q"], cfg["h_q"], cfg["fp8"], cfg["seed"],
                                       device)
    return q, kc, bt, sl, cfg["s_q"], cfg["h_q"], cfg["causal"], 1.0 / math.sqrt(D_QK), cfg["fp8"]


def make_device_inputs(seqlens, s_q, h_q, fp8, seed, device="cuda"):
    """Device-memory inputs of any shape: q, kcache (bf16 or FP8 records),
    block_table (a seeded permutation of the physical pages) and seqlens."""
    import torch

    seqlens = np.asarray(seqlens, dtype=np.int32)
    batch = seqlens.shape[0]
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    q = torch.randn((batch, s_q, h_q, D_QK), generator=g, device=device).to(torch.bfloat16)
    pages = (seqlens.astype(np.int64) + PAGE - 1) // PAGE
    n_pages = int(pages.sum())
    perm = torch.randperm(n_pages, generator=g, device=device).to(torch.int32)
    width = int(pages.max())
    bt = torch.full((batch, width), -1, dtype=torch.int32, device=device)
    starts = np.concatenate([[0], np.cumsum(pages)[:-1]])
    for b in range(batch):
        bt[b, : pages[b]] = perm[starts[b]: starts[b] + pages[b]]
    if not fp8:
        kc = torch.empty((n_pages, PAGE, D_QK), dtype=torch.bfloat16, device=device)
        chunk = 1024
        for p0 in range(0, n_pages, chunk):
            p1 = min(n_pages, p0 + chunk)
            kc[p0:p1] = torch.randn((p1 - p0, PAGE, D_QK), generator=g, device=device).to(torch.bfloat16)
    else:
        kc = torch.empty((n_pages, PAGE, FP8_RECORD), dtype=torch.uint8, device=device)
        chunk = 1024
        for p0 in range(0, n_pages, chunk):
            p1 = min(n_pages, p0 + chunk)
            x = torch.randn((p1 - p0, PAGE, D_QK), generator=g, device=device).to(torch.bfloat16).float()
            lat = x[..., :D_V].reshape(p1 - p0, PAGE, D_V // FP8_TILE, FP8_TILE)
            scale = lat.abs().amax(dim=-1) / E4M3_MAX
            safe = torch.where(scale > 0, scale, torch.ones_like(scale))
            codes = (lat / safe[..., None]).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
            codes = torch.where(scale[..., None] > 0, codes.view(torch.uint8), 0)
            kc[p0:p1, :, :D_V] = codes.reshape(p1 - p0, PAGE, D_V)
            kc[p0:p1, :, D_V:D_V + 16] = scale.contiguous().view(torch.uint8).reshape(p1 - p0, PAGE, 16)
            kc[p0:p1, :, D_V + 16:] = x[..., D_V:].to(torch.bfloat16).contiguous().view(torch.uint8)
    sl = torch.from_numpy(seqlens).to(device)
    return q, kc, bt, sl
