"""The binding launches on the caller's current stream: work queued before
the call on a side stream (a spin, then the write of q) must finish before
the decode reads q.  Were the kernels sent to another stream, they would read
the NaN-poisoned q left in place while the side stream still spins."""
import numpy as np
import pytest
import torch

from workloads import gen

from test_gpu_parity import DEV, check_close, device_inputs, oracle_decode, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    import paged_kv_cache_238_amd as m
    return m


@pytest.mark.parametrize("P", [0, 16])
def test_decode_on_a_side_stream(pa, P):
    wl = gen.make("tiny_gqa", small=True)
    vals = gen.fill_numpy(wl, new_slot_poison=False)
    d = device_inputs(wl, vals)
    q_real = d["q"].clone()
    d["q"].fill_(float("nan"))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        torch.cuda._sleep(50_000_000)           # tens of milliseconds of spinning on s
        d["q"].copy_(q_real)
        out = pa.decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["context_lens"],
                        scale=wl.scale, partition_size=P, max_context_len=wl.max_context_len)
    s.synchronize()
    want, _ = oracle_decode(wl, vals)
    say(f"side stream P={P}")
    check_close(out.cpu().numpy(), want, f"decode on a side stream P={P}")
