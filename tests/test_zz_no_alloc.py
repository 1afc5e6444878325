"""GPU test of fa_decode_noalloc, the decode entry point that allocates
nothing: through the C ABI, two calls in a row (the second on a smaller
input) are each compared bitwise with fa_decode on the same inputs, and with
the float64 oracle within |err| <= 1e-2 + 1e-2 |ref|.
"""
import ctypes
import math

import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import bits_of, parity, to_dev

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, D, cap, lens, seed):
    """Caches with a NaN-poisoned tail past each valid length, a query, the
    device valid lengths and an output buffer."""
    import torch
    kb = np.full((B, cap, Hkv, D), wl.BF16_QNAN, dtype=np.uint16)
    vb = kb.copy()
    for b, L in enumerate(lens):
        kb[b, :L] = wl.normal_bits((L, Hkv, D), seed + 2 * b, "bf16")
        vb[b, :L] = wl.normal_bits((L, Hkv, D), seed + 2 * b + 1, "bf16")
    qb = wl.normal_bits((B, Hq, D), seed + 100, "bf16")
    vl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    return kb, vb, qb, vl


def _noalloc(lib, q, kc, vc, vl, out, cap, B, Hq, Hkv, D, scale):
    import torch
    st = lib.fa_decode_noalloc(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), vl.data_ptr(), cap,
                               out.data_ptr(), B, Hq, Hkv, D, 0, scale, 0,
                               torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.fa_status_string(st)


def test_noalloc_matches_decode_on_two_calls():
    import torch

    import flash_attention_forward_fwd_amd as fa
    lib = fa.lib()
    # first call: a long cache split over many runs; second: a smaller batch
    # and cache with fewer runs, so the built-in workspace is reused with
    # another layout
    cases = [(1, 8, 2, 128, 65536, [65536], 900), (2, 8, 2, 128, 4096, [3000, 17], 920)]
    outs = []
    for B, Hq, Hkv, D, cap, lens, seed in cases:
        print(f"\n[noalloc] B={B} Hq={Hq} Hkv={Hkv} D={D} cap={cap} lens={lens}", flush=True)
        kb, vb, qb, vl = _case(B, Hq, Hkv, D, cap, lens, seed)
        q, kc, vc = to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16")
        scale = 1 / math.sqrt(D)
        out = torch.empty_like(q)
        _noalloc(lib, q, kc, vc, vl, out, cap, B, Hq, Hkv, D, scale)
        torch.cuda.synchronize()
        outs.append((bits_of(out), kb, vb, qb, lens, D, scale, q, kc, vc, vl))
    for got, kb, vb, qb, lens, D, scale, q, kc, vc, vl in outs:
        ref_bits = bits_of(fa.decode(q, kc, vc, vl, scale=scale))
        torch.cuda.synchronize()
        assert np.array_equal(got, ref_bits)
        ref = oracle.decode_ref(oracle.widen(qb, "bf16"), oracle.widen(kb, "bf16"),
                                oracle.widen(vb, "bf16"), lens, scale)
        parity(oracle.widen(got, "bf16"), ref, f"noalloc lens={lens}")
