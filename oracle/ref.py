"""CPU fp64 oracle for paged-attention decode over a block-paged KV cache.

TEST INFRASTRUCTURE ONLY.  This module is imported by the tests, by the smoke
check (__graft_entry__.smoke) and by the benchmark's CPU-baseline leg, and by
nothing else: the HIP library and its Python binding never import, call or
link it, and it shares no code, constants or helpers with them.

What it computes is the plain definition the paged method reorganises.  The
paging, the split into partitions, the online softmax and the sharing of one
K/V head by a group of query heads are all exact reorganisations of this
result, so the oracle gathers each sequence's tokens into a dense fp64 array
and runs textbook two-pass softmax attention on it:

  K_b[t] = k_pool[block_table[b][t // 16], t % 16, g, :]     t = 0 .. L_b - 1
  s_t    = scale * sum_d q[b, h, d] * K_b[t][d]              g = h // (Hq / Hkv)
  out[b, h, :] = sum_t softmax(s)_t * V_b[t]                 lse = log sum_t exp(s_t)

Sources (the three web pages on KV-cache paging):
  * zskr.cn article on ATB's PagedAttention, section "PagedAttention 的
    Attention 计算修改": the standard attention loop (dot of Q with every K,
    exp of the score) and the per-page kernel; and PagedAttentionMemory's
    logical-to-physical translation (page index = offset / page size,
    in-page offset = offset % page size, physical id from the page table).
  * adg.csdn.net article on ATB's KV Cache management, section "Paged KV
    Cache": 16-token blocks, block count ceil(tokens / 16).
  * discosf.com article "KV Cache 优化与显存管理": section "二、优化方向"
    (query heads grouped to share one K/V head; FP16 -> INT8 cache) and
    section "三、实现示例" (PhysicalPagePool.write_page, KVCacheQuantizer with
    its per_channel branch and dequantize).

Readings where the pages are silent or garbled (each is listed with its
reason in the design notes):
  * scale is an argument (the page's kernel has none; 1/sqrt(d) in practice);
  * kv head of query head h is h // G (contiguous groups);
  * the max starts at -inf, not the fp16 lowest value;
  * only tokens 0 .. L-1 count; slots past L in the last block never
    influence the result, whatever they hold;
  * the output is indexed [b, h, :] (the page's kernel drops the head index);
  * L = 0 gives a zero output row and lse = -inf;
  * the int8 dequantised value is code * scale evaluated exactly (fp64),
    not rounded to fp16 as the page's dequantize does;
  * FP8, which "二、优化方向" of the discosf.com article names beside INT8
    without giving a format or scale rule, is the OCP FP8 E4M3 format
    (largest finite value 448, no infinities); pools hold its raw codes
    (uint8), dequantised exactly as code value * scale, and the quantiser is
    the per_channel int8 rule with 448 in place of 127 and rounding to the
    nearest E4M3 value (ties to the even code), saturating at +-448.
"""
from __future__ import annotations

import numpy as np

TOKENS_PER_BLOCK = 16
FP8_E4M3_MAX = 448.0


def fp8_e4m3_value(code: int) -> float:
    """Value of one OCP FP8 E4M3 code, from the format's definition (OCP
    8-bit floating point specification): bit 7 sign, bits 6-3 exponent with
    bias 7, bits 2-0 mantissa; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111
    is NaN; there are no infinities, so 0x7E = 1.75 * 2^8 = 448 is the
    largest finite value."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


FP8_E4M3_VALUES = np.array([fp8_e4m3_value(c) for c in range(256)], dtype=np.float64)


def fp8_e4m3_to_float(codes) -> np.ndarray:
    """fp64 values of an array of E4M3 codes (uint8)."""
    return FP8_E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def _element_values(rows: np.ndarray) -> np.ndarray:
    """fp64 values of pool elements: fp16 or int8 as they are, uint8 as
    E4M3 codes."""
    if rows.dtype == np.uint8:
        return fp8_e4m3_to_float(rows)
    return rows.astype(np.float64)


def blocks_needed(num_tokens: int) -> int:
    """Blocks a sequence of num_tokens occupies: ceil(n / 16) (adg.csdn.net
    ATB article, "BlockManager 的调度": num_blocks = ceil(num_tokens /
    block_size); "Paged KV Cache": token 48 needs 3 blocks)."""
    return (int(num_tokens) + TOKENS_PER_BLOCK - 1) // TOKENS_PER_BLOCK


def gather_sequence(pool: np.ndarray, table_row: np.ndarray, length: int,
                    kv_head: int, scale_pool: np.ndarray | None = None) -> np.ndarray:
    """Dense fp64 [L, D] K (or V) of one sequence and one kv head.

    Walks the logical blocks in order and copies each physical block's slots
    (zskr.cn article, PagedAttentionMemory logical-to-physical translation,
    in token units).  For an int8 or fp8 pool every code's value is
    multiplied by its per-(token, kv head) scale in fp64 (discosf.com
    article, "三、实现示例", KVCacheQuantizer.dequantize: code times scale
    broadcast over the last axis)."""
    L = int(length)
    D = pool.shape[-1]
    dense = np.empty((L, D), dtype=np.float64)
    for j in range(blocks_needed(L)):
        phys = int(table_row[j])
        if not 0 <= phys < pool.shape[0]:
            raise IndexError(f"block id {phys} out of range [0, {pool.shape[0]})")
        n = min(TOKENS_PER_BLOCK, L - j * TOKENS_PER_BLOCK)
        rows = _element_values(pool[phys, :n, kv_head, :])
        if scale_pool is not None:
            rows = rows * scale_pool[phys, kv_head, :n].astype(np.float64)[:, None]
        dense[j * TOKENS_PER_BLOCK:j * TOKENS_PER_BLOCK + n] = rows
    return dense


def attend(qv: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Two-pass softmax attention of one query vector over dense K/V (fp64).
    Returns (out [D], lse).  Textbook form of the zskr.cn article's standard
    loop, with the max subtracted before exp."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64), -np.inf
    s = float(scale) * (K @ qv.astype(np.float64))
    m = s.max()
    p = np.exp(s - m)
    l = p.sum()
    return (p @ V) / l, m + np.log(l)


def _check(q, k_pool, v_pool, block_table, context_lens):
    B, Hq, D = q.shape
    NB, bs, Hkv, D2 = k_pool.shape
    if bs != TOKENS_PER_BLOCK:
        raise ValueError("block size must be 16 tokens")
    if D2 != D or v_pool.shape != k_pool.shape:
        raise ValueError("pool shapes disagree with q")
    if Hq % Hkv:
        raise ValueError("q_heads must be a multiple of kv_heads")
    if block_table.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("batch mismatch")
    for b in range(B):
        if context_lens[b] < 0 or blocks_needed(context_lens[b]) > block_table.shape[1]:
            raise ValueError(f"context length {context_lens[b]} does not fit the table")
    return B, Hq, Hkv, D


def ref_decode(q, k_pool, v_pool, block_table, context_lens, scale,
               k_scale=None, v_scale=None, rows=None):
    """Decode attention for one query token per sequence.

    q [B, Hq, D] fp16; k_pool / v_pool [NB, 16, Hkv, D] fp16 or int8;
    k_scale / v_scale [NB, Hkv, 16] fp32 for int8 pools (one scale per token
    and kv head, the 16 slots of a (block, kv head) adjacent); block_table
    [B, max_blocks]; context_lens [B] (including the newest token).
    rows: optional iterable of (b, h) to evaluate; the others stay NaN.
    Returns out fp64 [B, Hq, D] and lse fp64 [B, Hq] (natural log)."""
    q = np.asarray(q)
    block_table = np.asarray(block_table)
    context_lens = np.asarray(context_lens)
    B, Hq, Hkv, D = _check(q, k_pool, v_pool, block_table, context_lens)
    G = Hq // Hkv
    out = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    want = None if rows is None else {}
    if rows is not None:
        for b, h in rows:
            want.setdefault(int(b), set()).add(int(h))
    for b in range(B):
        if want is not None and b not in want:
            continue
        L = int(context_lens[b])
        for g in range(Hkv):
            heads = [h for h in range(g * G, (g + 1) * G)
                     if want is None or h in want[b]]
            if not heads:
                continue
            K = gather_sequence(k_pool, block_table[b], L, g, k_scale)
            V = gather_sequence(v_pool, block_table[b], L, g, v_scale)
            for h in heads:
                out[b, h], lse[b, h] = attend(q[b, h], K, V, scale)
    return out, lse


def ref_partials(q, k_pool, v_pool, block_table, context_lens, scale,
                 partition_size, k_scale=None, v_scale=None):
    """Per-partition softmax statistics for token ranges [pP, min((p+1)P, L)):
    running max m_p, sum l_p = sum exp(s - m_p) and unnormalised
    O_p = sum exp(s - m_p) V (natural-log domain).  Test-only: used to check
    that merging partitions by log-sum-exp reproduces ref_decode.
    Returns lists indexed [b][h] of (m [n], l [n], O [n, D])."""
    B, Hq, Hkv, D = _check(np.asarray(q), k_pool, v_pool, block_table, context_lens)
    G = Hq // Hkv
    P = int(partition_size)
    res = [[None] * Hq for _ in range(B)]
    for b in range(B):
        L = int(context_lens[b])
        n = (L + P - 1) // P
        for g in range(Hkv):
            K = gather_sequence(k_pool, block_table[b], L, g, k_scale)
            V = gather_sequence(v_pool, block_table[b], L, g, v_scale)
            for h in range(g * G, (g + 1) * G):
                m = np.empty(n)
                l = np.empty(n)
                O = np.empty((n, D))
                for p in range(n):
                    s = float(scale) * (K[p * P:(p + 1) * P] @ q[b, h].astype(np.float64))
                    m[p] = s.max()
                    e = np.exp(s - m[p])
                    l[p] = e.sum()
                    O[p] = e @ V[p * P:(p + 1) * P]
                res[b][h] = (m, l, O)
    return res


def ref_merge(m, l, O):
    """Log-sum-exp merge of partition statistics: M = max m_p,
    w_p = exp(m_p - M), out = sum w_p O_p / sum w_p l_p,
    lse = M + log sum w_p l_p.  An empty list gives zeros and -inf."""
    m = np.asarray(m, dtype=np.float64)
    if m.size == 0:
        return np.zeros(np.asarray(O).shape[-1] if np.asarray(O).ndim == 2 else 0), -np.inf
    M = m.max()
    w = np.exp(m - M)
    den = (w * np.asarray(l)).sum()
    return (w[:, None] * np.asarray(O)).sum(0) / den, M + np.log(den)


def ref_write_kv(k_pool, v_pool, k_new, v_new, slot_mapping):
    """KV write of new tokens into their slots (reshape-and-cache).

    Token i's K/V rows [Hkv, D] go to pool[slot // 16, slot % 16]; a negative
    slot is skipped.  Byte copy only (discosf.com article, "三、实现示例",
    PhysicalPagePool.write_page: storage[page, kv, layer, offset] = data;
    zskr.cn article, "踩坑三", WriteKV appends the new K, V into a page).
    Returns new pools; the inputs are left untouched.  Duplicate or
    out-of-range slots raise ValueError."""
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    cap = k_pool.shape[0] * TOKENS_PER_BLOCK
    seen = set()
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        if slot >= cap:
            raise ValueError(f"slot {slot} out of range")
        if slot in seen:
            raise ValueError(f"duplicate slot {slot}")
        seen.add(slot)
        blk, off = divmod(slot, TOKENS_PER_BLOCK)
        k_out[blk, off] = k_new[i]
        v_out[blk, off] = v_new[i]
    return k_out, v_out


def ref_quantize_int8(x):
    """Per-(token, kv head) int8 quantisation over the last axis (head_dim).

    Follows the per_channel branch of KVCacheQuantizer.quantize (discosf.com
    article, "三、实现示例"), in fp32 as printed there: absmax of |x| over the
    last axis, scale = absmax / 127, a zero scale replaced by 1.0, codes =
    clip(round-half-to-even(x / scale), -128, 127) as int8.
    Returns (codes int8 x.shape, scales fp32 x.shape[:-1])."""
    x32 = np.asarray(x).astype(np.float32)
    amax = np.max(np.abs(x32), axis=-1, keepdims=True)
    s = amax / np.float32(127.0)
    s = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    codes = np.clip(np.round(x32 / s), -128, 127).astype(np.int8)
    return codes, s[..., 0]


def _nearest_e4m3(y) -> np.ndarray:
    """E4M3 codes of fp32 values: the nearest finite E4M3 value, a tie going
    to the code with an even mantissa (round half to even), magnitudes at or
    beyond 448 saturating to 448; the sign bit is the sign of y (so -0.0
    gives 0x80)."""
    y = np.asarray(y, dtype=np.float32)
    pos = FP8_E4M3_VALUES[:0x7F]                   # codes 0 .. 126, increasing
    a = np.abs(y.astype(np.float64))
    hi = np.clip(np.searchsorted(pos, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - pos[lo]
    d_hi = pos[hi] - a
    pick = np.where(d_hi < d_lo, hi, lo)
    tie = d_hi == d_lo
    pick = np.where(tie, np.where(hi % 2 == 0, hi, lo), pick)
    pick = np.where(a >= FP8_E4M3_MAX, 0x7E, pick)
    return (pick | (np.signbit(y).astype(np.int64) << 7)).astype(np.uint8)


def ref_quantize_fp8(x):
    """Per-(token, kv head) FP8 E4M3 quantisation over the last axis.

    The per_channel rule of KVCacheQuantizer.quantize (discosf.com article,
    "三、实现示例") with E4M3's largest finite value in place of 127 (the
    same article's "二、优化方向" names FP8 next to INT8 and gives no rule of
    its own): in fp32, absmax of |x| over the last axis, scale = absmax /
    448, a zero scale replaced by 1.0, codes = the E4M3 value nearest to
    x / scale (ties to even, saturating at +-448).
    Returns (codes uint8 x.shape, scales fp32 x.shape[:-1])."""
    x32 = np.asarray(x).astype(np.float32)
    amax = np.max(np.abs(x32), axis=-1, keepdims=True)
    s = amax / np.float32(FP8_E4M3_MAX)
    s = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    codes = _nearest_e4m3(x32 / s)
    return codes, s[..., 0]



def ref_copy_blocks(k_pool, v_pool, pairs, k_scale=None, v_scale=None):
    """Copy-on-write block copy: for each (src, dst) pair, every slot of
    block src (K, V and, for 8-bit pools, the scales) is copied to block
    dst.  The zskr.cn article on ATB's PagedAttention ("踩坑三") takes a
    fresh page for a shared page that is about to be written, copies the old
    page into it and then writes.  Returns new arrays (scales None when not
    given).  Out-of-range ids, a repeated dst, or a dst that is also a src
    raise ValueError (the result would depend on the order of the copies)."""
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    ks_out = None if k_scale is None else np.array(k_scale, copy=True)
    vs_out = None if v_scale is None else np.array(v_scale, copy=True)
    pairs = [(int(a), int(b)) for a, b in np.asarray(pairs).reshape(-1, 2).tolist()]
    nb = k_pool.shape[0]
    dsts = [d for _, d in pairs]
    if len(set(dsts)) != len(dsts) or set(dsts) & {s for s, _ in pairs}:
        raise ValueError("copy pairs: dst blocks must be distinct and not sources")
    for src, dst in pairs:
        if not (0 <= src < nb and 0 <= dst < nb):
            raise ValueError(f"block pair ({src}, {dst}) out of range")
        k_out[dst] = k_pool[src]
        v_out[dst] = v_pool[src]
        if ks_out is not None:
            ks_out[dst] = k_scale[src]
            vs_out[dst] = v_scale[src]
    return k_out, v_out, ks_out, vs_out
