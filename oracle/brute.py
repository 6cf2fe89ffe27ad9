"""Brute-force paged decode attention in pure Python (tiny inputs only).

TEST INFRASTRUCTURE ONLY (imported by the tests and nothing else).  It shares
no code with the numpy oracle: every token is found through its own
logical-to-physical lookup (page index and in-page offset from the page
table, as PagedAttentionMemory translates addresses in the zskr.cn ATB
PagedAttention article), every score is a Python loop over head_dim, and the
softmax uses math.exp over a list.  It exists to pin the oracle's gather,
head grouping and softmax against an independent spelling of the definition.
"""
from __future__ import annotations

import math

PAGE_TOKENS = 16


def logical_to_physical(table_row, token: int):
    """(physical block, slot) of logical token `token` of one sequence."""
    page_index = token // PAGE_TOKENS
    offset_in_page = token % PAGE_TOKENS
    return int(table_row[page_index]), offset_in_page


def e4m3_brute(code: int) -> float:
    """Value of an OCP FP8 E4M3 code spelled out with math.ldexp: sign bit,
    4 exponent bits (bias 7, 0 = subnormal), 3 mantissa bits, all-ones = NaN."""
    neg = (code >> 7) & 1
    exp_bits = (code >> 3) & 15
    man = code & 7
    if exp_bits == 15 and man == 7:
        return math.nan
    if exp_bits == 0:
        mag = math.ldexp(man, -9)                 # man/8 * 2^-6
    else:
        mag = math.ldexp(8 + man, exp_bits - 10)  # (1 + man/8) * 2^(e-7)
    return -mag if neg else mag


def brute_decode(q, k_pool, v_pool, block_table, context_lens, scale,
                 k_scale=None, v_scale=None, element=float):
    """Nested lists out[b][h][d] and lse[b][h].  `element` maps a pool
    element to its value (float for fp16 / int8, e4m3_brute for fp8 codes)."""
    B = len(q)
    Hq = len(q[0])
    D = len(q[0][0])
    Hkv = len(k_pool[0][0])
    G = Hq // Hkv
    out, lse = [], []
    for b in range(B):
        L = int(context_lens[b])
        ob, lb = [], []
        for h in range(Hq):
            g = h // G
            scores, vals = [], []
            for t in range(L):
                blk, off = logical_to_physical(block_table[b], t)
                ks = float(k_scale[blk][g][off]) if k_scale is not None else 1.0
                vs = float(v_scale[blk][g][off]) if v_scale is not None else 1.0
                acc = 0.0
                for d in range(D):
                    acc += float(q[b][h][d]) * (element(k_pool[blk][off][g][d]) * ks)
                scores.append(float(scale) * acc)
                vals.append([element(v_pool[blk][off][g][d]) * vs for d in range(D)])
            if L == 0:
                ob.append([0.0] * D)
                lb.append(-math.inf)
                continue
            top = max(scores)
            w = [math.exp(s - top) for s in scores]
            tot = math.fsum(w)
            ob.append([math.fsum(w[t] * vals[t][d] for t in range(L)) / tot for d in range(D)])
            lb.append(top + math.log(tot))
        out.append(ob)
        lse.append(lb)
    return out, lse


def brute_write(k_pool, v_pool, k_new, v_new, slots):
    """Element-by-element write of new tokens, as nested lists (tiny pools)."""
    kp = [[[list(r) for r in tok] for tok in blk] for blk in k_pool]
    vp = [[[list(r) for r in tok] for tok in blk] for blk in v_pool]
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        blk, off = slot // PAGE_TOKENS, slot % PAGE_TOKENS
        for g in range(len(k_new[i])):
            for d in range(len(k_new[i][g])):
                kp[blk][off][g][d] = k_new[i][g][d]
                vp[blk][off][g][d] = v_new[i][g][d]
    return kp, vp
