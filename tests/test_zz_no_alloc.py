"""bsattn_decode_fwd_noalloc (the decode without a workspace argument, for
callers that cannot allocate) against bsattn_decode_fwd on the same inputs,
through the C ABI: two calls in a row on the library's per-device scratch,
the second with a smaller input (and another split count), then a third at
lambda = 0.  Outputs to the bf16 bar (max-abs 1e-2, mean-abs 1e-3), skip
states and counters bit-exact."""

import ctypes as C
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_flash_amd as bsa
from workloads import gen_decode_inputs
from workloads.configs import DecodeWorkload

from _parity import compare_out

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(f"[gpu-noalloc] {msg}", file=sys.stderr, flush=True)


def _outputs(B, Hkv, Tc):
    return (torch.zeros((B, Hkv, Tc), dtype=torch.uint8, device=DEV),
            torch.full((B, Hkv, 2), -1, dtype=torch.int32, device=DEV))


def test_decode_noalloc_matches_workspace_call():
    lib = bsa.library()
    cases = [(4, 32, 8, 20000, 128, None), (2, 8, 2, 3000, 64, None), (2, 8, 2, 2900, 128, 0.0)]
    for i, (B, Hq, Hkv, L, d, lam) in enumerate(cases):
        cfg = DecodeWorkload(name="noalloc", description="", B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, Bc=64,
                             lam=40.0 / L if lam is None else lam, seed=60 + i)
        _say(f"call {i}: B{B} Hq{Hq} Hkv{Hkv} L{L} d{d} lambda {cfg.lam:.3g}")
        q, kc, vc = (x.to(DEV) for x in gen_decode_inputs(cfg))
        Tc = -(-L // 64)
        st_ref, cnt_ref = _outputs(B, Hkv, Tc)
        ref = bsa.decode_fwd(q, kc, vc, L=L, scale=cfg.scale, lam=cfg.lam, counters=cnt_ref, block_state=st_ref)
        st, cnt = _outputs(B, Hkv, Tc)
        out = torch.full((B, Hq, d), 5.0, dtype=torch.bfloat16, device=DEV)
        # the argument struct as the binding marshals it, the call straight through the C ABI
        plan = bsa.decode_plan(q, kc, vc, L=L, scale=cfg.scale, lam=cfg.lam, out=out, counters=cnt, block_state=st,
                               noalloc=True)
        status = lib.bsattn_decode_fwd_noalloc(C.byref(plan._args),
                                               C.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert status == 0, lib.bsattn_last_error().decode()
        torch.cuda.synchronize()
        assert bsa.decode_check(None) == 0
        compare_out(out.cpu().double().numpy(), ref.cpu().double().numpy(), False, f"noalloc call {i}")
        assert np.array_equal(st.cpu().numpy(), st_ref.cpu().numpy())
        assert np.array_equal(cnt.cpu().numpy(), cnt_ref.cpu().numpy())
        _say(f"  skipped {int(cnt[..., 1].sum())} of {int(cnt[..., 0].sum())} blocks; "
             f"bit-identical output: {bool(torch.equal(out, ref))}")
