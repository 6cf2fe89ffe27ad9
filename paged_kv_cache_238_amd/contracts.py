"""Host-side check of the caller contracts the kernels rely on but do not
verify (verifying them on the device would need a synchronisation).

The zskr.cn article on ATB's PagedAttention keeps a reference count per page
and checks it before a page is freed or written (section "踩坑二",
ValidateRefCount), and copies a shared page before writing into it (section
"踩坑三").  validate() is that check for this library's arguments: it reads
the block table, the lengths and (optionally) the write slots, the shared
prefix and the copy pairs on the host, and reports every broken contract.

Contracts (include/pa.h):
  * 0 <= context_lens[b] <= max_context_len, ceil(L_b / 16) <= max_blocks;
  * 0 <= block_table[b][j] < num_blocks for j < ceil(L_b / 16);
  * write slots: unique (negative ones are skipped), inside the pool, and in
    blocks that no two sequences share (copy-on-write is the caller's job);
  * new_tokens (the append step): the slot of position L_b - 1 lies in a
    block no other sequence uses;
  * shared prefix: prefix_len a positive multiple of 16, every row holds
    row 0's first prefix_len / 16 ids, and L_b >= prefix_len;
  * block copies: ids inside the pool, destinations distinct and none of
    them also a source.

Pure numpy; torch tensors are copied to the host first.
"""
from __future__ import annotations

import numpy as np

BLOCK = 16


def _host(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x)


def _ref_counts(bt, lens, num_blocks):
    """Sequences referencing each block within their live range."""
    refs = np.zeros(num_blocks, dtype=np.int64)
    for b in range(bt.shape[0]):
        n = -(-int(lens[b]) // BLOCK)
        ids = bt[b, :n]
        ids = ids[(ids >= 0) & (ids < num_blocks)]
        refs[np.unique(ids)] += 1
    return refs


def validate(block_table, context_lens, num_blocks, *, max_context_len=None,
             slot_mapping=None, new_tokens=False, prefix_len=0, copy_pairs=None,
             raise_on_error=True) -> list[str]:
    """Check the caller contracts of a decode / write / copy call.  Returns
    the list of problems found (empty when every contract holds); raises
    ValueError listing them when raise_on_error."""
    bt = _host(block_table).astype(np.int64)
    lens = _host(context_lens).astype(np.int64)
    problems: list[str] = []
    if bt.ndim != 2 or lens.ndim != 1 or bt.shape[0] != lens.shape[0]:
        problems.append("block_table must be [batch, max_blocks] and context_lens [batch]")
        if raise_on_error:
            raise ValueError("; ".join(problems))
        return problems
    B, max_blocks = bt.shape
    bound = max_blocks * BLOCK if max_context_len is None else int(max_context_len)
    if bound > max_blocks * BLOCK:
        problems.append(f"max_context_len {bound} exceeds the table ({max_blocks} blocks)")
    for b in range(B):
        L = int(lens[b])
        if L < 0 or L > bound:
            problems.append(f"sequence {b}: length {L} outside [0, {bound}]")
            continue
        n = -(-L // BLOCK)
        if n > max_blocks:
            problems.append(f"sequence {b}: {n} blocks exceed the table width {max_blocks}")
            continue
        ids = bt[b, :n]
        bad = np.nonzero((ids < 0) | (ids >= num_blocks))[0]
        for j in bad[:4]:
            problems.append(f"sequence {b}: block_table[{b}][{int(j)}] = {int(ids[j])} "
                            f"outside [0, {num_blocks})")
        if len(bad) > 4:
            problems.append(f"sequence {b}: {len(bad) - 4} more ids outside the pool")
    refs = _ref_counts(bt, np.clip(lens, 0, max_blocks * BLOCK), num_blocks)

    def check_slots(slots, what):
        live = slots[slots >= 0]
        out = live[live >= num_blocks * BLOCK]
        if len(out):
            problems.append(f"{what}: slot {int(out[0])} outside the pool "
                            f"({num_blocks * BLOCK} slots)")
        live = live[live < num_blocks * BLOCK]
        uniq, cnt = np.unique(live, return_counts=True)
        for s in uniq[cnt > 1][:4]:
            problems.append(f"{what}: slot {int(s)} written more than once")
        shared = uniq[refs[uniq // BLOCK] > 1]
        for s in shared[:4]:
            problems.append(f"{what}: slot {int(s)} lies in block {int(s) // BLOCK}, shared by "
                            f"{int(refs[int(s) // BLOCK])} sequences (copy it first)")

    if slot_mapping is not None:
        check_slots(_host(slot_mapping).astype(np.int64).ravel(), "slot_mapping")
    if new_tokens:
        slots = []
        for b in range(B):
            L = int(lens[b])
            if 0 < L <= max_blocks * BLOCK:
                blk = int(bt[b, (L - 1) // BLOCK])
                if 0 <= blk < num_blocks:
                    slots.append(blk * BLOCK + (L - 1) % BLOCK)
        check_slots(np.asarray(slots, dtype=np.int64), "new-token slots")
    if prefix_len:
        P = int(prefix_len)
        if P <= 0 or P % BLOCK or P > max_blocks * BLOCK:
            problems.append(f"prefix_len {P} must be a positive multiple of 16 within the table")
        else:
            n = P // BLOCK
            rows = np.nonzero((bt[:, :n] != bt[0, :n]).any(axis=1))[0]
            for b in rows[:4]:
                problems.append(f"sequence {int(b)}: prefix ids differ from row 0's")
            short = np.nonzero(lens < P)[0]
            for b in short[:4]:
                problems.append(f"sequence {int(b)}: length {int(lens[b])} below prefix_len {P}")
    if copy_pairs is not None:
        pairs = _host(copy_pairs).astype(np.int64).reshape(-1, 2)
        bad = np.nonzero(((pairs < 0) | (pairs >= num_blocks)).any(axis=1))[0]
        for i in bad[:4]:
            problems.append(f"copy pair {int(i)} ({int(pairs[i, 0])}, {int(pairs[i, 1])}) "
                            f"outside [0, {num_blocks})")
        dst = pairs[:, 1]
        uniq, cnt = np.unique(dst, return_counts=True)
        for d in uniq[cnt > 1][:4]:
            problems.append(f"copy pairs: destination block {int(d)} repeated")
        both = np.intersect1d(dst, pairs[:, 0])
        for d in both[:4]:
            problems.append(f"copy pairs: block {int(d)} is both a source and a destination")
    if problems and raise_on_error:
        raise ValueError("caller contract broken: " + "; ".join(problems))
    return problems
