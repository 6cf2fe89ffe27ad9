"""Seeded synthetic inputs for paged-attention decode over a block-paged KV cache.

This module only *draws inputs*: context lengths, block tables, new-token
slots, and Q / K / V values (fp16, or int8 / fp8 codes plus fp32
per-(token, kv-head) scales, laid out [num_blocks, kv_heads, 16]).  It computes none of the attention, quantisation or KV-write
arithmetic, so the CPU oracle side and the GPU side of a test can both take
their inputs from here without sharing any of the method.

Workload shapes follow the pages' own examples:

* block_size = 16 tokens ("Paged KV Cache" section of the adg.csdn.net ATB
  KV-cache article; "二、优化方向" of the discosf.com KV-cache optimisation
  article).
* "llama2_7b" is one layer of the Llama2-7B arithmetic in "KV Cache 的显存需求"
  (32 kv heads, head_dim 128, 4096 tokens, batch 32); its block table keeps
  85 % of entries in their contiguous position, the contiguous-allocation rate
  reported in "显存碎片问题" of the same article.
* "prefix_shared" aliases one 1024-token prefix in every table ("Prefix
  Caching" section).

Recipe (seed = 2380 + config index unless given):
  rng = numpy.random.default_rng(seed); structure first (lengths, tables),
  then values in the order q, k_pool, v_pool, k_new, v_new, each
  rng.standard_normal(dtype=float32).astype(float16).  int8 pools draw codes
  uniformly from [-128, 127] and scales uniformly from [2.3/127, 3.8/127]
  (the range of absmax/127 for 128 N(0,1) values).  fp8 pools (OCP E4M3,
  stored as raw uint8 codes) draw codes uniformly from the 254 finite codes
  (every code but 0x7F and 0xFF) and scales from [2.3/448, 3.8/448].
  Poisoned runs fill every block no table references and every tail slot
  (token >= L in a sequence's last block) with fp16 NaN (int8 / fp8 pools:
  NaN scales), so a stray read shows.
  Source mode (fill_source_numpy / fill_source_torch) draws the long-context
  8-bit workloads as their configuration states them: fp16 N(0,1) K / V for
  every slot of the pool, in the order q, k_src, v_src, k_new, v_new; the
  caller quantises them into codes and scales with a quantiser of its own
  (the library's quantising write, or the oracle's), so this module still
  holds none of that arithmetic.
  The torch backend draws the same kind of values on the device with a seeded
  torch.Generator (used for full-size workloads; values differ from numpy's).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Any

import numpy as np

BLOCK = 16                     # tokens per physical block
FP16_NAN_BITS = 0x7E00

# name -> (index, shape parameters)
SPECS: dict[str, dict[str, Any]] = {
    # tiny GQA decode plus a one-token KV write per sequence
    "tiny_gqa": dict(idx=1, batch=4, q_heads=8, kv_heads=2, head_dim=64,
                     kv_dtype="fp16", scale=1.0 / 8.0),
    # Llama2-7B-shaped single layer: 32 x 4096 tokens, MHA, 85/15 table
    "llama2_7b": dict(idx=2, batch=32, q_heads=32, kv_heads=32, head_dim=128,
                      kv_dtype="fp16", ctx=4096, scatter=0.15),
    # GQA-70B-shaped mixed lengths, log-uniform [128, 8192], 95 % pool occupancy
    "gqa70b_mixed": dict(idx=3, batch=64, q_heads=64, kv_heads=8, head_dim=128,
                         kv_dtype="fp16", lmin=128, lmax=8192, occupancy=0.95),
    # 64 requests sharing one 1024-token prefix, private suffixes U{16..512}
    "prefix_shared": dict(idx=4, batch=64, q_heads=32, kv_heads=32, head_dim=128,
                          kv_dtype="fp16", prefix=1024, smin=16, smax=512),
    # 128K-token split-K decode over an int8 cache with per-token scales
    "long128k_int8": dict(idx=5, batch=4, q_heads=64, kv_heads=8, head_dim=128,
                          kv_dtype="int8", ctx=131072, scatter=0.15,
                          partition_size=512),
    # the same 128K-token decode over an FP8 (E4M3) cache
    "long128k_fp8": dict(idx=6, batch=4, q_heads=64, kv_heads=8, head_dim=128,
                         kv_dtype="fp8", ctx=131072, scatter=0.15,
                         partition_size=512),
}

# Scaled-down twins used for element-by-element parity (same structure,
# several partitions and a ragged tail, small enough for the oracle).
SMALL: dict[str, dict[str, Any]] = {
    "llama2_7b": dict(batch=4, q_heads=4, kv_heads=4, ctx=1037),
    "gqa70b_mixed": dict(batch=8, q_heads=16, kv_heads=2, lmin=1, lmax=1500),
    "prefix_shared": dict(batch=6, q_heads=4, kv_heads=4, prefix=128, smin=1, smax=100),
    "long128k_int8": dict(batch=2, q_heads=16, kv_heads=2, ctx=3000, partition_size=512),
    "long128k_fp8": dict(batch=2, q_heads=16, kv_heads=2, ctx=3000, partition_size=512),
}

ORDER = ["tiny_gqa", "llama2_7b", "gqa70b_mixed", "prefix_shared", "long128k_int8",
         "long128k_fp8"]

# the 254 finite OCP E4M3 codes (0x7F and 0xFF are NaN)
FP8_FINITE_CODES = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


@dataclass
class Workload:
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    num_blocks: int
    max_blocks: int
    kv_dtype: str                     # "fp16", "int8" or "fp8"
    scale: float
    partition_size: int               # 0 = library's choice
    context_lens: np.ndarray          # int32 [B]
    block_table: np.ndarray           # int32 [B, max_blocks]
    new_slots: np.ndarray             # int32 [B]; slot of token L_b - 1
    seed: int
    poison: bool
    used_blocks: np.ndarray           # bool [num_blocks]; referenced within ceil(L/16)
    twin_table: np.ndarray | None = None   # prefix_shared: private-copy table
    twin_src: np.ndarray | None = None     # prefix_shared: twin block -> source block
    values: dict[str, Any] = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.batch else 0


# ----------------------------------------------------------------------------
# structure

def _scatter_table(rng, batch: int, per_seq: int, frac: float) -> np.ndarray:
    """Identity table bt[b][j] = b*per_seq + j with a fraction of entries
    deranged among themselves (shuffle the chosen set, rotate by one), so
    exactly round(frac*n) entries leave their contiguous position."""
    n = batch * per_seq
    flat = np.arange(n, dtype=np.int64)
    k = int(round(frac * n))
    if k >= 2:
        chosen = rng.choice(n, k, replace=False)
        chosen = rng.permutation(chosen)
        flat[chosen] = np.roll(chosen, 1)
    return flat.reshape(batch, per_seq).astype(np.int32)


def make(name: str, seed: int | None = None, *, small: bool = False,
         poison: bool = True, overrides: dict | None = None) -> Workload:
    """Draw the structure of a workload: lengths, block table, new-token slots."""
    spec = dict(SPECS[name])
    if small and name in SMALL:
        spec.update(SMALL[name])
    if overrides:
        spec.update(overrides)
    if seed is None:
        seed = 2380 + spec["idx"] + (100 if small else 0)
    rng = np.random.default_rng(seed)
    B, Hkv = spec["batch"], spec["kv_heads"]
    scale = spec.get("scale", 1.0 / math.sqrt(spec["head_dim"]))
    twin_table = twin_src = None

    if name == "tiny_gqa":
        nb = spec.get("num_blocks", 128)
        maxb = spec.get("max_blocks", 16)
        lens = rng.integers(1, maxb * BLOCK + 1, size=B)
        perm = rng.permutation(nb)
        bt = np.zeros((B, maxb), dtype=np.int64)
        pos = 0
        for b in range(B):
            n = cdiv(int(lens[b]), BLOCK)
            bt[b, :n] = perm[pos:pos + n]
            pos += n
        used_n = pos
        spare = perm[used_n:]
    elif name in ("llama2_7b", "long128k_int8", "long128k_fp8"):
        ctx = spec["ctx"]
        per = cdiv(ctx, BLOCK)
        maxb = spec.get("max_blocks", per)
        nb = spec.get("num_blocks", B * per)
        lens = np.full(B, ctx)
        core = _scatter_table(rng, B, per, spec["scatter"])
        bt = np.zeros((B, maxb), dtype=np.int64)
        bt[:, :per] = core
        spare = np.arange(B * per, nb)
    elif name == "gqa70b_mixed":
        lo, hi = spec["lmin"], spec["lmax"]
        u = rng.uniform(math.log(lo), math.log(hi), size=B)
        lens = np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int64)
        need = [cdiv(int(x), BLOCK) for x in lens]
        used = int(sum(need))
        nb = int(math.ceil(used / spec["occupancy"]))
        maxb = spec.get("max_blocks", cdiv(hi, BLOCK))
        ids = rng.permutation(nb)
        bt = np.zeros((B, maxb), dtype=np.int64)
        pos = 0
        for b in range(B):
            bt[b, :need[b]] = ids[pos:pos + need[b]]
            pos += need[b]
        spare = ids[pos:]
    elif name == "prefix_shared":
        pre = spec["prefix"]
        npre = pre // BLOCK
        suf = rng.integers(spec["smin"], spec["smax"] + 1, size=B)
        nsuf = [cdiv(int(s), BLOCK) for s in suf]
        nb = npre + int(sum(nsuf))
        maxb = spec.get("max_blocks", npre + cdiv(spec["smax"], BLOCK))
        ids = rng.permutation(nb)
        P0 = ids[:npre]
        bt = np.zeros((B, maxb), dtype=np.int64)
        pos = npre
        for b in range(B):
            bt[b, :npre] = P0
            bt[b, npre:npre + nsuf[b]] = ids[pos:pos + nsuf[b]]
            pos += nsuf[b]
        lens = pre + suf
        spare = ids[pos:]
        # private-copy twin: every row gets its own copy of the prefix blocks,
        # appended after the shared pool
        twin_table = bt.copy()
        src = list(range(nb))
        for b in range(B):
            for j in range(npre):
                twin_table[b, j] = len(src)
                src.append(int(P0[j]))
        twin_src = np.asarray(src, dtype=np.int64)
    else:
        raise KeyError(name)

    lens = np.asarray(lens, dtype=np.int64)
    # table entries past ceil(L/16) are never read: point them at a spare
    # (poisoned) block when one exists, else block 0
    fill = int(spare[0]) if len(spare) else 0
    for b in range(B):
        n = cdiv(int(lens[b]), BLOCK)
        bt[b, n:] = fill
        if twin_table is not None:
            twin_table[b, n:] = fill
    used_mask = np.zeros(nb, dtype=bool)
    for b in range(B):
        used_mask[bt[b, :cdiv(int(lens[b]), BLOCK)]] = True
    last = np.maximum(lens - 1, 0)
    new_slots = np.array([bt[b, last[b] // BLOCK] * BLOCK + last[b] % BLOCK
                          for b in range(B)], dtype=np.int64)
    new_slots[lens == 0] = -1

    return Workload(
        name=name, batch=B, q_heads=spec["q_heads"], kv_heads=Hkv,
        head_dim=spec["head_dim"], num_blocks=nb, max_blocks=maxb,
        kv_dtype=spec["kv_dtype"], scale=float(scale),
        partition_size=int(spec.get("partition_size", 0)),
        context_lens=lens.astype(np.int32), block_table=bt.astype(np.int32),
        new_slots=new_slots.astype(np.int32), seed=seed, poison=poison,
        used_blocks=used_mask,
        twin_table=None if twin_table is None else twin_table.astype(np.int32),
        twin_src=twin_src)


def poison_mask(wl: Workload) -> np.ndarray:
    """bool [num_blocks, 16]: slots holding no valid token of any sequence."""
    valid = np.zeros((wl.num_blocks, BLOCK), dtype=bool)
    for b in range(wl.batch):
        L = int(wl.context_lens[b])
        for j in range(cdiv(L, BLOCK)):
            n = min(BLOCK, L - j * BLOCK)
            valid[wl.block_table[b, j], :n] = True
    return ~valid


# ----------------------------------------------------------------------------
# values

def _normal16(rng, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


def fill_numpy(wl: Workload, *, new_slot_poison: bool = True) -> dict[str, np.ndarray]:
    """Draw all values on the host with numpy (small workloads)."""
    rng = np.random.default_rng(wl.seed + 7919)
    B, Hq, Hkv, D, NB = wl.batch, wl.q_heads, wl.kv_heads, wl.head_dim, wl.num_blocks
    v: dict[str, np.ndarray] = {}
    v["q"] = _normal16(rng, (B, Hq, D))
    if wl.kv_dtype == "fp16":
        v["k_pool"] = _normal16(rng, (NB, BLOCK, Hkv, D))
        v["v_pool"] = _normal16(rng, (NB, BLOCK, Hkv, D))
    elif wl.kv_dtype == "fp8":
        v["k_pool"] = rng.choice(FP8_FINITE_CODES, size=(NB, BLOCK, Hkv, D))
        v["v_pool"] = rng.choice(FP8_FINITE_CODES, size=(NB, BLOCK, Hkv, D))
        v["k_scale"] = rng.uniform(2.3 / 448, 3.8 / 448, size=(NB, Hkv, BLOCK)).astype(np.float32)
        v["v_scale"] = rng.uniform(2.3 / 448, 3.8 / 448, size=(NB, Hkv, BLOCK)).astype(np.float32)
    else:
        v["k_pool"] = rng.integers(-128, 128, size=(NB, BLOCK, Hkv, D), dtype=np.int8)
        v["v_pool"] = rng.integers(-128, 128, size=(NB, BLOCK, Hkv, D), dtype=np.int8)
        v["k_scale"] = rng.uniform(2.3 / 127, 3.8 / 127, size=(NB, Hkv, BLOCK)).astype(np.float32)
        v["v_scale"] = rng.uniform(2.3 / 127, 3.8 / 127, size=(NB, Hkv, BLOCK)).astype(np.float32)
    v["k_new"] = _normal16(rng, (B, Hkv, D))
    v["v_new"] = _normal16(rng, (B, Hkv, D))
    if wl.poison:
        bad = poison_mask(wl)
        if new_slot_poison:
            for s in wl.new_slots:
                if s >= 0:
                    bad[s // BLOCK, s % BLOCK] = True
        nan16 = np.array([FP16_NAN_BITS], dtype=np.uint16).view(np.float16)[0]
        if wl.kv_dtype == "fp16":
            v["k_pool"][bad] = nan16
            v["v_pool"][bad] = nan16
        else:
            v["k_scale"].transpose(0, 2, 1)[bad] = np.nan    # scales are [NB, Hkv, 16]
            v["v_scale"].transpose(0, 2, 1)[bad] = np.nan
    wl.values = v
    return v


def fill_torch(wl: Workload, device, *, chunk_rows: int = 1 << 12) -> dict[str, Any]:
    """Draw all values on `device` with a seeded torch.Generator (large
    workloads).  Poisoning, if requested, NaN-fills the same slots as
    fill_numpy."""
    import torch
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed + 7919)
    B, Hq, Hkv, D, NB = wl.batch, wl.q_heads, wl.kv_heads, wl.head_dim, wl.num_blocks

    def normal16(shape):
        out = torch.empty(shape, dtype=torch.float16, device=dev)
        flat = out.view(shape[0], -1)
        for i in range(0, shape[0], chunk_rows):
            j = min(shape[0], i + chunk_rows)
            flat[i:j] = torch.randn((j - i, flat.shape[1]), generator=gen,
                                    device=dev, dtype=torch.float32).to(torch.float16)
        return out

    v: dict[str, Any] = {}
    v["q"] = normal16((B, Hq, D))
    if wl.kv_dtype == "fp16":
        v["k_pool"] = normal16((NB, BLOCK, Hkv, D))
        v["v_pool"] = normal16((NB, BLOCK, Hkv, D))
    elif wl.kv_dtype == "fp8":
        for nm in ("k_pool", "v_pool"):
            idx = torch.randint(0, 254, (NB, BLOCK, Hkv, D), generator=gen, device=dev,
                                dtype=torch.int32)
            # index -> code, skipping the NaN codes 0x7F and 0xFF
            v[nm] = (idx + (idx >= 0x7F).to(torch.int32)).to(torch.uint8)
        for nm in ("k_scale", "v_scale"):
            t = torch.rand((NB, Hkv, BLOCK), generator=gen, device=dev, dtype=torch.float32)
            v[nm] = t * (1.5 / 448) + (2.3 / 448)
    else:
        for nm in ("k_pool", "v_pool"):
            v[nm] = torch.randint(-128, 128, (NB, BLOCK, Hkv, D), generator=gen,
                                  device=dev, dtype=torch.int8)
        for nm in ("k_scale", "v_scale"):
            t = torch.rand((NB, Hkv, BLOCK), generator=gen, device=dev, dtype=torch.float32)
            v[nm] = t * (1.5 / 127) + (2.3 / 127)
    v["k_new"] = normal16((B, Hkv, D))
    v["v_new"] = normal16((B, Hkv, D))
    if wl.poison:
        bad = torch.from_numpy(poison_mask(wl)).to(dev)
        if wl.kv_dtype == "fp16":
            v["k_pool"][bad] = float("nan")
            v["v_pool"][bad] = float("nan")
        else:
            v["k_scale"].permute(0, 2, 1)[bad] = float("nan")
            v["v_scale"].permute(0, 2, 1)[bad] = float("nan")
    wl.values = v
    return v


def fill_source_numpy(wl: Workload) -> dict[str, np.ndarray]:
    """Source mode, on the host: fp16 N(0,1) q, k_src, v_src ([num_blocks,
    16, kv_heads, head_dim], every slot), k_new, v_new.  No codes or scales:
    the caller quantises k_src / v_src."""
    rng = np.random.default_rng(wl.seed + 7919)
    B, Hq, Hkv, D, NB = wl.batch, wl.q_heads, wl.kv_heads, wl.head_dim, wl.num_blocks
    v = {"q": _normal16(rng, (B, Hq, D)),
         "k_src": _normal16(rng, (NB, BLOCK, Hkv, D)),
         "v_src": _normal16(rng, (NB, BLOCK, Hkv, D)),
         "k_new": _normal16(rng, (B, Hkv, D)),
         "v_new": _normal16(rng, (B, Hkv, D))}
    wl.values = v
    return v


def fill_source_torch(wl: Workload, device, *, chunk_rows: int = 1 << 12) -> dict[str, Any]:
    """Source mode on `device` with a seeded torch.Generator: the tensors of
    fill_source_numpy (values differ from numpy's)."""
    import torch
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed + 7919)
    B, Hq, Hkv, D, NB = wl.batch, wl.q_heads, wl.kv_heads, wl.head_dim, wl.num_blocks

    def normal16(shape):
        out = torch.empty(shape, dtype=torch.float16, device=dev)
        flat = out.view(shape[0], -1)
        for i in range(0, shape[0], chunk_rows):
            j = min(shape[0], i + chunk_rows)
            flat[i:j] = torch.randn((j - i, flat.shape[1]), generator=gen,
                                    device=dev, dtype=torch.float32).to(torch.float16)
        return out

    v = {"q": normal16((B, Hq, D)),
         "k_src": normal16((NB, BLOCK, Hkv, D)),
         "v_src": normal16((NB, BLOCK, Hkv, D)),
         "k_new": normal16((B, Hkv, D)),
         "v_new": normal16((B, Hkv, D))}
    wl.values = v
    return v


# ----------------------------------------------------------------------------
# byte accounting (measurement, not method arithmetic)

def kv_bytes_per_token_head(head_dim: int, kv_dtype: str) -> int:
    """K+V bytes one token of one kv head occupies in the cache (int8 pools
    add one fp32 scale each for K and V)."""
    if kv_dtype == "fp16":
        return 2 * head_dim * 2
    return 2 * head_dim * 1 + 2 * 4


def kv_ideal_bytes(wl: Workload, unique: bool = True) -> int:
    """Algorithmic KV bytes one decode must read: every valid (block, slot)
    once (unique) or once per referencing sequence (logical)."""
    per = wl.kv_heads * kv_bytes_per_token_head(wl.head_dim, wl.kv_dtype)
    if not unique:
        return int(wl.context_lens.astype(np.int64).sum()) * per
    slots = []
    for b in range(wl.batch):
        t = np.arange(int(wl.context_lens[b]), dtype=np.int64)
        slots.append(wl.block_table[b, t // BLOCK].astype(np.int64) * BLOCK + t % BLOCK)
    n = len(np.unique(np.concatenate(slots))) if slots else 0
    return n * per


def permute_blocks(wl: Workload, pi: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Physical relabelling: block i moves to pi[i].  Returns (new table,
    inverse map inv with new_pool[j] = pool[inv[j]])."""
    inv = np.empty_like(pi)
    inv[pi] = np.arange(len(pi))
    return pi[wl.block_table].astype(np.int32), inv
