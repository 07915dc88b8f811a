"""iq_append_decode_attention_noalloc (records in the library's scratch array)
against iq_append_decode_attention (records in a caller's workspace).

Both run the same kernels with the same plan, so the outputs and the cache
contents they leave must be identical bit for bit; each is also checked
against the oracle at the attention tolerance. Two calls in a row, the second
on a smaller input, show that nothing depends on what the first call left in
the scratch array.
"""
import math

import numpy as np
import pytest
import torch

import iqinputs
import quantized_kv_cache_wht_amd as iq
from oracle import iqref as R
from parity_util import C32, SCALE, _t, _np, _assert_attention_close

pytestmark = pytest.mark.gpu


def _step_inputs(seed, hq, hkv, lens, k_bits):
    lens = np.array(lens, np.int32)
    starts = (np.concatenate([[0], np.cumsum(lens + 1)[:-1]]) + 3).astype(np.int32)
    cap = -(-(int(starts[-1] + lens[-1]) + 1) // 32) * 32
    rot = iqinputs.rotation_params(seed, 0, hkv)
    k = iqinputs.kv(seed, 0, "k", cap, hkv, "student_t6", "f16")
    v = iqinputs.kv(seed, 0, "v", cap, hkv, "student_t6", "f16")
    q = iqinputs.queries(seed, 1, len(lens), hq)
    caches = []
    for _ in range(2):
        c = iq.PackedKVCache.allocate(hkv, cap, _t(rot), k_bits=k_bits)
        iq.iq_rotate_quantize_append(c, _t(k), _t(v), first_slot=0)
        caches.append(c)
    new = starts + lens
    return caches, rot, _t(k[new]), _t(v[new]), q, starts, lens


@pytest.mark.parametrize("k_bits", [3, 4])
def test_noalloc_step_equals_workspace_step_on_two_calls(k_bits):
    print(f"[noalloc] k_bits={k_bits}", flush=True)
    # call 1: 3 ragged sequences up to 9000 tokens, 32 / 8 heads; call 2: one sequence of 700, 16 / 1 heads
    for seed, hq, hkv, lens in ((31, 32, 8, [9000, 13, 4000]), (32, 16, 1, [700])):
        caches, rot, kn, vn, q, starts, lens = _step_inputs(seed + k_bits, hq, hkv, lens, k_bits)
        ml = int(lens.max())
        need = iq.iq_decode_workspace_bytes(len(lens), hq, hkv, ml)
        assert need <= iq.NOALLOC_SCRATCH_BYTES
        ref = iq.iq_append_decode_attention(caches[0], kn, vn, _t(q), _t(starts), _t(lens), ml)
        out = torch.full_like(ref, float("nan"))
        got = iq.iq_append_decode_attention_noalloc(caches[1], kn, vn, _t(q), _t(starts), _t(lens), ml, out=out)
        torch.cuda.synchronize()
        assert got is out
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), (seed, hq, hkv, list(lens))
        for name in ("k_codes", "v_codes", "k_norms", "v_norms"):
            assert torch.equal(getattr(caches[0], name), getattr(caches[1], name)), name
        c_k, _, _ = R.codebook(levels=16 if k_bits == 4 else 8)
        oracle = R.decode_attention(q, _np(caches[1].k_codes), _np(caches[1].k_norms), _np(caches[1].v_codes),
                                    _np(caches[1].v_norms), rot, starts, lens + 1, SCALE, C32, k_centroids32=c_k)
        _assert_attention_close(_np(got), oracle, f"noalloc step hq={hq} hkv={hkv} lens={list(lens)}")


def test_noalloc_step_refuses_records_past_the_scratch():
    hq, hkv, n = 32, 4, 64
    assert iq.iq_decode_workspace_bytes(n, hq, hkv, 32768) > iq.NOALLOC_SCRATCH_BYTES
    rot = torch.zeros((hkv, 32, 8), device="cuda")
    cache = iq.PackedKVCache.allocate(hkv, 64, rot)
    kn = torch.zeros((n, hkv, 128), dtype=torch.float16, device="cuda")
    q = torch.zeros((n, hq, 128), device="cuda")
    st = torch.zeros(n, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(iq.IqError):
        iq.iq_append_decode_attention_noalloc(cache, kn, kn, q, st, st, 32768, out=out)
