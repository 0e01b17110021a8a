"""The allocation-free decode entry point (static device scratch) against the
workspace entry point, through the C ABI: the same kernels and launch plan,
so the outputs agree bit for bit; two calls in a row, the second smaller
(the scratch keeps the first call's partials, which the second must not
read), and a third call back at the first shape."""
import numpy as np
import pytest
import torch

from kv_cache_bit_amd import nsnq, synth

from helpers import DEV, capacity, cb_tensor, check_attention, gpu_encode, gpu_records

import oracle

pytestmark = pytest.mark.gpu

D = 128


def _case(oracle_codebooks, bits, B, Hq, Hkv, L, R=128, seed=0):
    cb = oracle_codebooks[bits]
    k, v = synth.kv_layer(1300 + seed, 0, B, Hkv, L, D)
    q = synth.queries(1300 + seed, 0, B, Hq, D)
    p, cbt, cache = gpu_encode(k, v, bits, R, cb)
    return p, cbt, cache, q.to(DEV), cb


@pytest.mark.parametrize("bits,Hq,Hkv", [(2, 4, 4), (2, 8, 2), (1, 2, 2)])
def test_noalloc_matches_workspace_call(oracle_codebooks, bits, Hq, Hkv):
    first = _case(oracle_codebooks, bits, 3, Hq, Hkv, 2100, seed=bits + Hq)
    second = _case(oracle_codebooks, bits, 1, Hq, Hkv, 300, seed=bits + Hq + 1)  # smaller: fewer rows, splits
    outs = []
    for p, cbt, cache, q, cb in (first, second, first):
        for ns in (0, 2):
            ref = nsnq.nsnq_decode_attention(p, cbt, q, cache, num_splits=ns)
            out = torch.full_like(q, float("nan"))
            nsnq.nsnq_decode_attention_noalloc(p, cbt, q, cache, out, num_splits=ns)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (bits, Hq, Hkv, ns)
            outs.append(out.float().cpu().numpy())
        # and the oracle's attention over the same records
        R = 128
        o_ref = oracle.reference_decode(q.cpu(), gpu_records(cache, 0), gpu_records(cache, 1), cache.n_quant,
                                        cache.n_resid, R, cb)
        check_attention(outs[-1], o_ref)


def test_noalloc_rejects_oversize_without_launching(oracle_codebooks):
    p, cbt, cache, q, _ = _case(oracle_codebooks, 2, 1, 2, 2, 300, seed=9)
    need = nsnq.nsnq_decode_workspace_bytes(p, cache, q.shape[1])
    assert need <= nsnq.NSNQ_SCRATCH_BYTES
    big = nsnq.KVCache(p, 512, 32, 4096, DEV)
    big.n_quant, big.n_resid = 3968, 128
    qb = torch.zeros(512, 32, D, dtype=torch.float16, device=DEV)
    assert nsnq.nsnq_decode_workspace_bytes(p, big, 32) > nsnq.NSNQ_SCRATCH_BYTES
    with pytest.raises(nsnq.NsnqError) as ei:
        nsnq.nsnq_decode_attention_noalloc(p, cbt, qb, big, torch.empty_like(qb))
    assert ei.value.status == nsnq.NSNQ_ESCRATCH
