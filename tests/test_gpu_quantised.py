"""8-bit caches quantised from fp16 sources, the way the long-context
configuration states its int8 cache: fp16 N(0,1) K / V, one absmax/127 fp32
scale per (token, kv head) (discosf.com article "KV Cache 优化与显存管理",
section "三、实现示例", KVCacheQuantizer.quantize, per_channel branch; FP8
E4M3 with 448 in place of 127).

Each side quantises the same fp16 source with its own quantiser: the GPU pool
comes from the library's quantising write over every slot of the pool
(pa_write_kv_int8 / pa_write_kv_fp8), the oracle's from ref_quantize_int8 /
ref_quantize_fp8.  The two pools must be bit-identical (codes and scales)
before anything is decoded; the oracle never reads the GPU's pool.  Decode
outputs are then compared with the oracle on its own pool (the gate), and
the error against the oracle on the fp16 source itself (the quantisation
error, which the gate does not cover) is printed as a report.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import ref
from workloads import gen

from test_gpu_parity import DEV, check_close, say, t

pytestmark = pytest.mark.gpu

QUANTISERS = {"int8": (ref.ref_quantize_int8, np.int8, torch.int8),
              "fp8": (ref.ref_quantize_fp8, np.uint8, torch.uint8)}


@pytest.fixture(scope="module")
def pa():
    import paged_kv_cache_238_amd as m
    return m


def oracle_pool(src, kind, chunk=1024, workers=8):
    """Oracle quantiser over a fp16 pool [NB, 16, Hkv, D]: codes of the same
    shape and scales in the cache layout [NB, Hkv, 16]."""
    quantise, np_dtype, _ = QUANTISERS[kind]
    NB, _, Hkv, _ = src.shape
    codes = np.empty(src.shape, np_dtype)
    scales = np.empty((NB, Hkv, 16), np.float32)

    def one(i):
        c, s = quantise(src[i:i + chunk])
        codes[i:i + chunk] = c
        scales[i:i + chunk] = s.transpose(0, 2, 1)

    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(one, range(0, NB, chunk)))
    return codes, scales


def gpu_pools(pa, k_src, v_src, kind):
    """The library's quantising write over every slot of the pool."""
    NB, _, Hkv, D = k_src.shape
    _, _, th_dtype = QUANTISERS[kind]
    kc = torch.empty(k_src.shape, dtype=th_dtype, device=DEV)
    vc = torch.empty_like(kc)
    ks = torch.empty((NB, Hkv, 16), dtype=torch.float32, device=DEV)
    vs = torch.empty_like(ks)
    slots = torch.arange(NB * 16, dtype=torch.int32, device=DEV)
    write = pa.write_kv_int8 if kind == "int8" else pa.write_kv_fp8
    write(k_src.view(NB * 16, Hkv, D), v_src.view(NB * 16, Hkv, D), slots, kc, vc, ks, vs)
    return kc, vc, ks, vs


def assert_pools_identical(got, want, what):
    kc, vc, ks, vs = (x.cpu().numpy() for x in got)
    for name, g, w in (("k codes", kc, want[0]), ("v codes", vc, want[1])):
        bad = np.count_nonzero(g.view(np.uint8) != w.view(np.uint8))
        assert bad == 0, f"{what}: {bad} {name} differ"
    for name, g, w in (("k scales", ks, want[2]), ("v scales", vs, want[3])):
        bad = np.count_nonzero(g.view(np.uint32) != w.view(np.uint32))
        assert bad == 0, f"{what}: {bad} {name} differ"


def poison_scales(wl, host, dev):
    """NaN scales at every slot no sequence uses (both sides, same places)."""
    bad = gen.poison_mask(wl)
    if not bad.any():
        return
    for arr in host[2:]:
        arr.transpose(0, 2, 1)[bad] = np.nan
    mask = torch.from_numpy(bad).to(DEV)
    for ten in dev[2:]:
        ten.permute(0, 2, 1)[mask] = float("nan")


def decode(pa, wl, q, pools, bt, cl, P):
    kc, vc, ks, vs = pools
    fn = pa.decode_int8 if wl.kv_dtype == "int8" else pa.decode_fp8
    return fn(q, kc, vc, ks, vs, bt, cl, scale=wl.scale, partition_size=P,
              max_context_len=wl.max_context_len, return_lse=True)


def report(got, want, what):
    err = np.asarray(got, np.float64) - want
    rel = float(np.linalg.norm(err) / np.linalg.norm(want))
    say(f"  REPORT {what}: max_abs={np.abs(err).max():.3e} rel_rms={rel:.3e} (not gated)")
    return rel


# --------------------------------------------------------------------------- full size

class Built:
    pass


@pytest.fixture(scope="module", params=["int8", "fp8"])
def long128k(pa, request):
    """The 128K-token workload at full size, its cache quantised from fp16
    N(0,1) sources on both sides."""
    kind = request.param
    name = "long128k_int8" if kind == "int8" else "long128k_fp8"
    wl = gen.make(name, poison=True)
    say(f"long128k {kind}: B={wl.batch} NB={wl.num_blocks} L={wl.max_context_len} "
        f"P={wl.partition_size}")
    src = gen.fill_source_torch(wl, DEV)
    dev = gpu_pools(pa, src["k_src"], src["v_src"], kind)
    b = Built()
    b.wl, b.kind = wl, kind
    b.q = src["q"]
    b.q_host = src["q"].cpu().numpy()
    b.k_src = src["k_src"].cpu().numpy()
    b.v_src = src["v_src"].cpu().numpy()
    del src
    torch.cuda.empty_cache()
    kc, ks = oracle_pool(b.k_src, kind)
    vc, vs = oracle_pool(b.v_src, kind)
    b.host = [kc, vc, ks, vs]
    b.dev = list(dev)
    b.identical = None
    try:
        assert_pools_identical(b.dev, b.host, f"long128k {kind}")
        b.identical = True
    except AssertionError as e:
        b.identical = str(e)
    poison_scales(wl, b.host, b.dev)
    b.bt = t(wl.block_table)
    b.cl = t(wl.context_lens)
    yield b
    del b.dev
    torch.cuda.empty_cache()


def test_long128k_pools_bit_identical(long128k):
    """The library's quantising write and the oracle's quantiser agree on
    every code and scale of the 1 GiB cache."""
    assert long128k.identical is True, long128k.identical


def test_long128k_every_row_vs_oracle(pa, long128k):
    """Every (sequence, query head) row of the full-size 128K decode, in the
    benchmark's launch configuration (partition_size 512: balanced chunks of
    at least 512 tokens), against the oracle on its own quantised cache."""
    b = long128k
    assert b.identical is True, b.identical
    wl = b.wl
    out, lse = decode(pa, wl, b.q, b.dev, b.bt, b.cl, wl.partition_size)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    want, want_lse = ref.ref_decode(b.q_host, b.host[0], b.host[1], wl.block_table,
                                    wl.context_lens, wl.scale, b.host[2], b.host[3])
    b.out = out
    check_close(out, want, f"long128k {b.kind}: all {wl.batch * wl.q_heads} rows")
    np.testing.assert_allclose(lse, want_lse, rtol=0, atol=1e-4)


def test_long128k_quantisation_error_report(pa, long128k):
    """Reported, not gated: the decode of the quantised cache against the
    oracle on the fp16 source it was quantised from (every row)."""
    b = long128k
    wl = b.wl
    out = getattr(b, "out", None)
    if out is None:
        out = decode(pa, wl, b.q, b.dev, b.bt, b.cl, wl.partition_size)[0].cpu().numpy()
    src_ref, _ = ref.ref_decode(b.q_host, b.k_src, b.v_src, wl.block_table, wl.context_lens,
                                wl.scale)
    assert np.isfinite(out).all()
    rel = report(out, src_ref, f"long128k {b.kind} GPU vs oracle on the fp16 source")
    assert rel < 0.1


def test_long128k_record_rounding_budget(pa, long128k):
    """The error the fp16 split-K records add on the 128K workload: the
    benchmark's launch (512-token minimum chunks, 64 fp16 records per row,
    merged) against direct mode (one wave per (sequence, kv head) over the
    whole 131072 tokens, no records), both against the oracle on every row.
    The matrix-core kernel's fp16 probabilities are in both."""
    b = long128k
    assert b.identical is True, b.identical
    wl = b.wl
    want, _ = ref.ref_decode(b.q_host, b.host[0], b.host[1], wl.block_table, wl.context_lens,
                             wl.scale, b.host[2], b.host[3])
    errs = {}
    for what, P in (("split, fp16 records", wl.partition_size), ("direct, no records", 131072)):
        out = decode(pa, wl, b.q, b.dev, b.bt, b.cl, P)[0].cpu().numpy()
        check_close(out, want, f"long128k {b.kind} {what}")
        err = out.astype(np.float64) - want
        errs[what] = float(np.linalg.norm(err) / np.linalg.norm(want))
    say(f"  REPORT long128k {b.kind} relative RMS: {errs}")


# --------------------------------------------------------------------------- small shapes

def small_case(pa, kind, G, seed, q_mul=1.0, v_sigma=1.0, k_sigma=1.0, D=128, ctx=3000):
    over = dict(batch=2, q_heads=2 * G, kv_heads=2, head_dim=D, ctx=ctx,
                kv_dtype=kind, partition_size=512)
    wl = gen.make("long128k_int8", seed=seed, overrides=over)
    src = gen.fill_source_numpy(wl)
    q = src["q"].astype(np.float32) * np.float32(q_mul)
    src["q"] = q.astype(np.float16)
    src["k_src"] = (src["k_src"].astype(np.float32) * np.float32(k_sigma)).astype(np.float16)
    src["v_src"] = (src["v_src"].astype(np.float32) * np.float32(v_sigma)).astype(np.float16)
    dev = gpu_pools(pa, t(src["k_src"]), t(src["v_src"]), kind)
    kc, ks = oracle_pool(src["k_src"], kind)
    vc, vs = oracle_pool(src["v_src"], kind)
    host = [kc, vc, ks, vs]
    assert_pools_identical(dev, host, f"{kind} G={G}")
    return wl, src, host, dev


@pytest.mark.parametrize("kind", ["int8", "fp8"])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_small_source_quantised(pa, kind, G):
    """Both kernels on a source-quantised cache (ragged 3000-token contexts,
    several partitions)."""
    wl, src, host, dev = small_case(pa, kind, G, seed=700 + G)
    say(f"source-quantised {kind} G={G}")
    for P in (0, 512):
        out, lse = decode(pa, wl, t(src["q"]), dev, t(wl.block_table), t(wl.context_lens), P)
        want, want_lse = ref.ref_decode(src["q"], host[0], host[1], wl.block_table,
                                        wl.context_lens, wl.scale, host[2], host[3])
        check_close(out.cpu().numpy(), want, f"{kind} G={G} P={P}")
        np.testing.assert_allclose(lse.cpu().numpy(), want_lse, rtol=0, atol=1e-4)


@pytest.mark.parametrize("kind", ["int8", "fp8"])
@pytest.mark.parametrize("G", [4, 8, 16])
def test_same_sign_large_query(pa, kind, G):
    """q = 16 |N(0,1)|: every element positive, so sum(q) is about 1600 and
    the scores spread over tens of units; the int8 K path must not lose
    precision to the size of sum(q)."""
    wl, src, host, dev = small_case(pa, kind, G, seed=800 + G)
    src["q"] = (np.abs(src["q"].astype(np.float32)) * 16).astype(np.float16)
    say(f"same-sign q x16 {kind} G={G}: sum q = {src['q'].astype(np.float64).sum(-1).mean():.0f}")
    want, want_lse = ref.ref_decode(src["q"], host[0], host[1], wl.block_table,
                                    wl.context_lens, wl.scale, host[2], host[3])
    for P in (0, 512):
        out, lse = decode(pa, wl, t(src["q"]), dev, t(wl.block_table), t(wl.context_lens), P)
        check_close(out.cpu().numpy(), want, f"same-sign q {kind} G={G} P={P}")
        np.testing.assert_allclose(lse.cpu().numpy(), want_lse, rtol=0, atol=1e-3)


@pytest.mark.parametrize("kind", ["int8", "fp8"])
@pytest.mark.parametrize("G", [4, 8, 16])
@pytest.mark.parametrize("sigma", [1e-3, 1e-2])
def test_small_value_scale(pa, kind, G, sigma):
    """V drawn from N(0, sigma^2): its per-token scales are about
    2.7 sigma / 127 (int8) or / 448 (FP8), so a product of a probability and
    a scale can fall below fp16's normal range; the output must still meet
    the relative tolerance."""
    wl, src, host, dev = small_case(pa, kind, G, seed=900 + G, v_sigma=sigma)
    say(f"small V sigma={sigma} {kind} G={G}")
    want, _ = ref.ref_decode(src["q"], host[0], host[1], wl.block_table, wl.context_lens,
                             wl.scale, host[2], host[3])
    for P in (0, 512):
        out, _ = decode(pa, wl, t(src["q"]), dev, t(wl.block_table), t(wl.context_lens), P)
        check_close(out.cpu().numpy(), want, f"V sigma={sigma} {kind} G={G} P={P}")
