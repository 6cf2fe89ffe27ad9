"""Pins of the CPU oracle against things other than itself: brute force on
tiny inputs, a library attention routine, closed forms, invariants of the
paged layout, and the byte counts the pages print."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute, ref
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny_case(rng, B, Hq, Hkv, D, lens, nb=None, int8=False):
    need = sum(ref.blocks_needed(L) for L in lens)
    nb = nb or need + 3
    maxb = max(1, max(ref.blocks_needed(L) for L in lens))
    perm = rng.permutation(nb)
    bt = np.zeros((B, maxb), dtype=np.int32)
    pos = 0
    for b, L in enumerate(lens):
        n = ref.blocks_needed(L)
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    q = rng.standard_normal((B, Hq, D), dtype=np.float32).astype(np.float16)
    if int8:
        k = rng.integers(-127, 128, (nb, 16, Hkv, D), dtype=np.int8)
        v = rng.integers(-127, 128, (nb, 16, Hkv, D), dtype=np.int8)
        ks = rng.uniform(0.01, 0.03, (nb, Hkv, 16)).astype(np.float32)
        vs = rng.uniform(0.01, 0.03, (nb, Hkv, 16)).astype(np.float32)
    else:
        k = rng.standard_normal((nb, 16, Hkv, D), dtype=np.float32).astype(np.float16)
        v = rng.standard_normal((nb, 16, Hkv, D), dtype=np.float32).astype(np.float16)
        ks = vs = None
    return q, k, v, bt, np.asarray(lens, dtype=np.int32), ks, vs


CASES = [
    (1, 1, 1, 4, [1]),
    (2, 2, 2, 8, [17, 40]),
    (3, 4, 2, 8, [0, 16, 33]),
    (2, 4, 1, 5, [15, 32]),
    (3, 8, 2, 6, [2, 31, 40]),
]


@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize("case", CASES)
def test_oracle_matches_brute_force(case, int8):
    B, Hq, Hkv, D, lens = case
    rng = np.random.default_rng(11 + len(lens) + D)
    q, k, v, bt, cl, ks, vs = tiny_case(rng, B, Hq, Hkv, D, lens, int8=int8)
    scale = 1 / math.sqrt(D)
    out, lse = ref.ref_decode(q, k, v, bt, cl, scale, ks, vs)
    bo, bl = brute.brute_decode(q.tolist(), k.tolist(), v.tolist(), bt.tolist(), cl.tolist(),
                                scale, None if ks is None else ks.tolist(),
                                None if vs is None else vs.tolist())
    np.testing.assert_allclose(out, np.array(bo), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, np.array(bl), rtol=1e-12, atol=1e-13)


def dense_gather(pool, row, L, g):
    t = np.arange(L)
    return pool[row[t // 16], t % 16, g].astype(np.float64)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_oracle_matches_library_sdpa(G):
    """Gathered K/V with kv heads repeat-interleaved, run through torch's
    scaled_dot_product_attention in fp64 on the CPU."""
    rng = np.random.default_rng(100 + G)
    Hkv, D = 2, 16
    Hq = G * Hkv
    lens = [1, 37, 64, 129]
    q, k, v, bt, cl, _, _ = tiny_case(rng, len(lens), Hq, Hkv, D, lens)
    scale = 0.3
    out, lse = ref.ref_decode(q, k, v, bt, cl, scale)
    for b, L in enumerate(lens):
        K = np.stack([dense_gather(k, bt[b], L, g) for g in range(Hkv)])   # [Hkv, L, D]
        V = np.stack([dense_gather(v, bt[b], L, g) for g in range(Hkv)])
        Kt = torch.from_numpy(K).repeat_interleave(G, dim=0)[None]
        Vt = torch.from_numpy(V).repeat_interleave(G, dim=0)[None]
        Q = torch.from_numpy(q[b].astype(np.float64))[None, :, None, :]
        o = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, scale=scale)
        np.testing.assert_allclose(out[b], o[0, :, 0].numpy(), rtol=1e-12, atol=1e-14)
        s = scale * np.einsum("hld,hd->hl", Kt[0].numpy(), q[b].astype(np.float64))
        np.testing.assert_allclose(lse[b], np.logaddexp.reduce(s, axis=1), rtol=1e-12)
        # softmax weights recovered from lse sum to one
        np.testing.assert_allclose(np.exp(s - lse[b][:, None]).sum(1), 1.0, rtol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, D = 3, 4, 2, 8
    lens = [1, 2, 37]
    q, k, v, bt, cl, _, _ = tiny_case(rng, B, Hq, Hkv, D, lens)
    # L = 1 returns V[0] exactly
    out, _ = ref.ref_decode(q, k, v, bt, cl, 0.7)
    for h in range(Hq):
        assert np.array_equal(out[0, h], v[bt[0, 0], 0, h // 2].astype(np.float64))
    # L = 2: sigmoid weights
    for h in range(Hq):
        g = h // 2
        k0, k1 = (k[bt[1, 0], i, g].astype(np.float64) for i in (0, 1))
        v0, v1 = (v[bt[1, 0], i, g].astype(np.float64) for i in (0, 1))
        d = 0.7 * (q[1, h].astype(np.float64) @ (k1 - k0))
        sig = 1 / (1 + math.exp(-d))
        np.testing.assert_allclose(out[1, h], sig * v1 + (1 - sig) * v0, rtol=1e-12, atol=1e-14)
    # K = 0 (or scale = 0): mean of V over the L tokens
    out0, lse0 = ref.ref_decode(q, np.zeros_like(k), v, bt, cl, 0.7)
    out1, _ = ref.ref_decode(q, k, v, bt, cl, 0.0)
    for b, L in enumerate(lens):
        for h in range(Hq):
            mean = np.mean([v[bt[b, t // 16], t % 16, h // 2].astype(np.float64) for t in range(L)], 0)
            np.testing.assert_allclose(out0[b, h], mean, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(out1[b, h], mean, rtol=1e-12, atol=1e-14)
            assert math.isclose(lse0[b, h], math.log(L), rel_tol=1e-12)
    # V = c: output c
    vc = np.full_like(v, 1.5)
    outc, _ = ref.ref_decode(q, k, vc, bt, cl, 0.7)
    np.testing.assert_allclose(outc, 1.5, rtol=1e-12)
    # one dominant score selects its V row
    k2 = (k * np.float16(0.01)).astype(np.float16)
    b, h, t = 2, 3, 20
    g = h // 2
    qn = q[b, h].astype(np.float64)
    k2[bt[b, t // 16], t % 16, g] = (60 * qn / np.linalg.norm(qn)).astype(np.float16)
    outd, _ = ref.ref_decode(q, k2, v, bt, cl, 1.0)
    np.testing.assert_allclose(outd[b, h], v[bt[b, t // 16], t % 16, g].astype(np.float64),
                               rtol=1e-12, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, D = 2, 8, 2, 8
    q, k, v, bt, cl, _, _ = tiny_case(rng, B, Hq, Hkv, D, [19, 48])
    G = Hq // Hkv
    out, lse = ref.ref_decode(q, k, v, bt, cl, 0.4)
    km = np.repeat(k, G, axis=2)
    vm = np.repeat(v, G, axis=2)
    out2, lse2 = ref.ref_decode(q, km, vm, bt, cl, 0.4)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("name", ["tiny_gqa", "gqa70b_mixed", "long128k_int8"])
def test_block_permutation_invariance(name):
    wl = gen.make(name, small=True)
    vals = gen.fill_numpy(wl, new_slot_poison=False)
    pi = np.random.default_rng(3).permutation(wl.num_blocks)
    bt2, inv = gen.permute_blocks(wl, pi)
    args = [vals.get("k_scale"), vals.get("v_scale")]
    out, lse = ref.ref_decode(vals["q"], vals["k_pool"], vals["v_pool"], wl.block_table,
                              wl.context_lens, wl.scale, *args)
    perm = [None if a is None else a[inv] for a in args]
    out2, lse2 = ref.ref_decode(vals["q"], vals["k_pool"][inv], vals["v_pool"][inv], bt2,
                                wl.context_lens, wl.scale, *perm)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    assert np.isfinite(out).all()          # poisoned blocks and tails never read


def test_prefix_aliasing_equals_private_copies():
    wl = gen.make("prefix_shared", small=True)
    vals = gen.fill_numpy(wl, new_slot_poison=False)
    src = wl.twin_src
    out, lse = ref.ref_decode(vals["q"], vals["k_pool"], vals["v_pool"], wl.block_table,
                              wl.context_lens, wl.scale)
    out2, lse2 = ref.ref_decode(vals["q"], vals["k_pool"][src], vals["v_pool"][src],
                                wl.twin_table, wl.context_lens, wl.scale)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    assert np.isfinite(out).all()


@pytest.mark.parametrize("P", [16, 64, 512, 4096])
def test_partition_merge_reproduces_decode(P):
    wl = gen.make("gqa70b_mixed", small=True)
    vals = gen.fill_numpy(wl, new_slot_poison=False)
    out, lse = ref.ref_decode(vals["q"], vals["k_pool"], vals["v_pool"], wl.block_table,
                              wl.context_lens, wl.scale)
    parts = ref.ref_partials(vals["q"], vals["k_pool"], vals["v_pool"], wl.block_table,
                             wl.context_lens, wl.scale, P)
    for b in range(wl.batch):
        for h in range(wl.q_heads):
            o, lz = ref.ref_merge(*parts[b][h])
            np.testing.assert_allclose(o, out[b, h], rtol=1e-12, atol=1e-14)
            assert math.isclose(lz, lse[b, h], rel_tol=1e-12, abs_tol=1e-13)


def test_empty_sequence():
    rng = np.random.default_rng(1)
    q, k, v, bt, cl, _, _ = tiny_case(rng, 2, 2, 1, 4, [0, 3])
    out, lse = ref.ref_decode(q, k, v, bt, cl, 1.0)
    assert np.array_equal(out[0], np.zeros((2, 4))) and np.all(lse[0] == -np.inf)


def test_write_matches_brute_and_leaves_other_bytes():
    rng = np.random.default_rng(2)
    nb, Hkv, D = 6, 2, 4
    kp = np.full((nb, 16, Hkv, D), 7.0, dtype=np.float16)
    vp = np.full((nb, 16, Hkv, D), -3.0, dtype=np.float16)
    kn = rng.standard_normal((5, Hkv, D), dtype=np.float32).astype(np.float16)
    vn = rng.standard_normal((5, Hkv, D), dtype=np.float32).astype(np.float16)
    slots = [3, -1, 95, 16, 40]
    k2, v2 = ref.ref_write_kv(kp, vp, kn, vn, slots)
    bk, bv = brute.brute_write(kp.tolist(), vp.tolist(), kn.tolist(), vn.tolist(), slots)
    assert np.array_equal(k2, np.array(bk, dtype=np.float16))
    assert np.array_equal(v2, np.array(bv, dtype=np.float16))
    touched = np.zeros((nb, 16), bool)
    for s in slots:
        if s >= 0:
            touched[s // 16, s % 16] = True
    assert np.all(k2[~touched] == 7.0) and np.all(v2[~touched] == -3.0)
    assert np.array_equal(k2[1, 0], kn[3]) and np.array_equal(v2[5, 15], vn[2])
    with pytest.raises(ValueError):
        ref.ref_write_kv(kp, vp, kn[:2], vn[:2], [4, 4])


def test_byte_accounting_matches_page_numbers():
    g = json.load(open(os.path.join(GOLDEN, "byte_accounting.json")))
    c = g["llama2_7b"]
    per = gen.kv_bytes_per_token_head(c["head_dim"], "fp16") * c["num_kv_heads"] * c["seq_len"]
    assert per == g["per_layer_per_sequence_bytes"]
    assert per * c["layers"] == g["all_layers_per_sequence_bytes"]
    assert per * c["layers"] * g["batch"] == g["all_layers_batch_bytes"]
    assert gen.kv_bytes_per_token_head(128, "fp16") * 32 * 16 == g["block_bytes"]
    assert ref.blocks_needed(48) == g["blocks_for_48_tokens"]
    assert ref.blocks_needed(49) == 4 and ref.blocks_needed(0) == 0
    wl = gen.make("llama2_7b", poison=False)
    assert gen.kv_ideal_bytes(wl) == g["batch"] * g["per_layer_per_sequence_bytes"]


def test_quantiser_worked_rows():
    g = json.load(open(os.path.join(GOLDEN, "quant_rule.json")))
    for row in g["rows"]:
        codes, s = ref.ref_quantize_int8(np.array([row["x"]], dtype=np.float32))
        assert s[0] == np.float32(row["scale"])
        assert codes[0].tolist() == row["codes"]


def _brute_round_code(x: float, s: float) -> int:
    """Nearest integer to the fp32 quotient x / s, halves to even, clipped."""
    qt = float(np.float32(x) / np.float32(s))      # IEEE fp32 division
    lo = math.floor(qt)
    frac = qt - lo
    if frac > 0.5 or (frac == 0.5 and lo % 2 == 1):
        lo += 1
    return max(-128, min(127, lo))


def test_quantiser_properties_and_brute_rounding():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 3, 16), dtype=np.float32).astype(np.float16)
    x[5, 1] = 0
    codes, s = ref.ref_quantize_int8(x)
    assert codes.dtype == np.int8 and s.dtype == np.float32 and s.shape == (64, 3)
    assert s[5, 1] == 1.0 and not codes[5, 1].any()
    nz = np.abs(x.astype(np.float32)).max(-1) > 0
    assert np.all(np.abs(codes.astype(int)).max(-1)[nz] == 127)
    err = np.abs(x.astype(np.float64) - codes * s[..., None].astype(np.float64))
    # half a step, plus the fp32 rounding of the quotient x / s (|x / s| <= 127)
    assert np.all(err <= s[..., None] * (0.5 + 127 * 2.0 ** -23))
    for i in range(0, 64, 7):
        for h in range(3):
            for d in range(16):
                assert codes[i, h, d] == _brute_round_code(float(x[i, h, d]), float(s[i, h]))


# --- mutation checks: a plausible slip planted in the oracle must fail a pin

def _brute_pin_fails(monkeypatch, attr, fake):
    monkeypatch.setattr(ref, attr, fake)
    try:
        test_oracle_matches_brute_force((3, 4, 2, 8, [0, 16, 33]), False)
    except AssertionError:
        return True
    return False


def test_pins_catch_planted_mistakes(monkeypatch):
    orig_gather = ref.gather_sequence

    def wrong_head(pool, row, L, g, sp=None):          # kv head off by one
        return orig_gather(pool, row, L, (g + 1) % pool.shape[2], sp)

    def wrong_slot(pool, row, L, g, sp=None):          # in-block offset off by one
        dense = np.empty((L, pool.shape[-1]))
        for t in range(L):
            blk, off = int(row[t // 16]), (t + 1) % 16
            val = pool[blk, off, g].astype(np.float64)
            dense[t] = val if sp is None else val * float(sp[blk, off, g])
        return dense

    def one_more(pool, row, L, g, sp=None):            # a tail token leaks in
        if L % 16 and L > 0:
            extra = orig_gather(pool, row, L + 1, g, sp)
            return extra
        return orig_gather(pool, row, L, g, sp)

    orig_attend = ref.attend

    def no_scale(qv, K, V, scale):                     # dropped scale
        return orig_attend(qv, K, V, 1.0)

    for attr, fake in [("gather_sequence", wrong_head), ("gather_sequence", wrong_slot),
                       ("gather_sequence", one_more), ("attend", no_scale)]:
        assert _brute_pin_fails(monkeypatch, attr, fake), attr
        monkeypatch.undo()


# ----------------------------------------------------------------- FP8 E4M3

def test_fp8_code_values_from_format_definition():
    g = json.load(open(os.path.join(GOLDEN, "fp8_e4m3.json")))
    for c in g["codes"]:
        got = ref.fp8_e4m3_value(c["code"])
        if c["value"] == "nan":
            assert math.isnan(got)
        else:
            assert got == c["value"] and math.copysign(1, got) == math.copysign(1, c["value"])


def test_fp8_table_matches_bitwise_spelling_and_is_ordered():
    for code in range(256):
        a, b = ref.fp8_e4m3_value(code), brute.e4m3_brute(code)
        assert (math.isnan(a) and math.isnan(b)) or a == b
    pos = ref.FP8_E4M3_VALUES[:0x7F]
    assert np.all(np.diff(pos) > 0)                        # codes 0..126 increase
    assert np.array_equal(ref.FP8_E4M3_VALUES[0x80:0xFF], -pos)
    finite = ref.FP8_E4M3_VALUES[np.isfinite(ref.FP8_E4M3_VALUES)]
    assert len(finite) == 254 and len(np.unique(finite)) == 253   # +-0 share a value
    assert finite.max() == 448.0


def test_fp8_quantiser_worked_rows():
    g = json.load(open(os.path.join(GOLDEN, "fp8_e4m3.json")))
    for row in g["rows"]:
        codes, s = ref.ref_quantize_fp8(np.array([row["x"]], dtype=np.float32))
        assert s[0] == np.float32(row["scale"])
        assert codes[0].tolist() == row["codes"]


def _brute_nearest_code(y: float) -> int:
    """Scan every finite E4M3 code for the nearest value; ties to the even
    code; beyond 448 saturate."""
    mag = abs(y)
    best, best_d = None, None
    for c in range(0x7F):
        d = abs(brute.e4m3_brute(c) - mag)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    if mag >= 448.0:
        best = 0x7E
    return best | (0x80 if math.copysign(1.0, y) < 0 else 0)


def test_fp8_quantiser_properties_and_brute_rounding():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((48, 2, 32), dtype=np.float32).astype(np.float16)
    x[3, 1] = 0
    codes, s = ref.ref_quantize_fp8(x)
    assert codes.dtype == np.uint8 and s.dtype == np.float32 and s.shape == (48, 2)
    assert s[3, 1] == 1.0 and not codes[3, 1].any()
    vals = ref.fp8_e4m3_to_float(codes)
    assert np.all(np.isfinite(vals)) and np.abs(vals).max() <= 448.0
    nz = np.abs(x.astype(np.float32)).max(-1) > 0
    assert np.all(np.abs(vals).max(-1)[nz] == 448.0)       # the absmax element maps to 448
    # error: half the E4M3 spacing at the value (2^-3 relative, 2^-10 absolute
    # in the subnormal range), plus the fp32 rounding of x / s
    y = x.astype(np.float64) / s[..., None]
    half_gap = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10)
    assert np.all(np.abs(y - vals) <= half_gap * (1 + 1e-6) + np.abs(y) * 2.0 ** -23)
    for i in range(0, 48, 5):
        for j in range(32):
            q = float(np.float32(x[i, 0, j]) / np.float32(s[i, 0]))
            assert codes[i, 0, j] == _brute_nearest_code(q)
    # every tie between neighbouring codes, both signs
    pos = ref.FP8_E4M3_VALUES[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    for sign in (1.0, -1.0):
        got = ref._nearest_e4m3(sign * mids)
        want = [_brute_nearest_code(sign * float(m)) for m in mids]
        assert got.tolist() == want
    assert ref._nearest_e4m3(np.float32([500.0, -1e30]))[0] == 0x7E


def test_fp8_decode_against_brute_force():
    rng = np.random.default_rng(21)
    B, Hq, Hkv, D, NB = 2, 4, 2, 8, 6
    q = rng.standard_normal((B, Hq, D), dtype=np.float32).astype(np.float16)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    kp = rng.choice(finite, size=(NB, 16, Hkv, D))
    vp = rng.choice(finite, size=(NB, 16, Hkv, D))
    ks = rng.uniform(1e-3, 2e-2, size=(NB, Hkv, 16)).astype(np.float32)
    vs = rng.uniform(1e-3, 2e-2, size=(NB, Hkv, 16)).astype(np.float32)
    bt = np.array([[4, 1, 0], [2, 5, 3]], dtype=np.int32)
    cl = np.array([37, 20], dtype=np.int32)
    out, lse = ref.ref_decode(q, kp, vp, bt, cl, 0.3, ks, vs)
    bo, bl = brute.brute_decode(q.tolist(), kp.tolist(), vp.tolist(), bt.tolist(), cl.tolist(),
                                0.3, ks.tolist(), vs.tolist(), element=brute.e4m3_brute)
    np.testing.assert_allclose(out, np.array(bo), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(bl), rtol=1e-12, atol=1e-12)
