"""cb_attention_step_noalloc: the attention step for callers that cannot
allocate, on the library's fixed per-device scratch array, against
cb_attention_step with a caller workspace (same kernels) and the oracle."""
import numpy as np
import pytest
import torch

import chunked_prefill_attention_amd as cb
from chunked_prefill_attention_amd import _lib
from gpu_util import Step, compare, i32, say, to_dev
from oracle import attention as ora
import workloads as wl


def test_scratch_size_and_refusal_before_any_device_work():
    """A step whose workspace exceeds the array is refused on the host."""
    lib = _lib.load()
    cap = lib.cb_attention_noalloc_scratch_bytes()
    assert cap == 256 << 20
    fake = _lib.C.c_void_p(0x1000)   # never dereferenced: the size check comes first
    need = cb.attention_workspace_bytes(129, 128, 2048, 64, 8, 128, 1 << 20, cb.CB_BF16)
    assert need > cap
    st = lib.cb_attention_step_noalloc(fake, fake, fake, fake, 1 << 16, fake, fake, fake, 129, 128, 2048, 1 << 20,
                                       64, 8, 128, 16, 1 << 20, 0.088, 0, cb.CB_BF16, fake, _lib.C.c_void_p(0))
    assert st == _lib.CB_ERR_WORKSPACE
    assert b"allocation-free" in lib.cb_last_error()


def _both(st: Step, kc, vc):
    """The step through cb_attention_step (own workspace) and through the
    allocation-free entry point; outputs on the host."""
    q = to_dev(np.concatenate(st.q), st.dtype)
    args = (q, kc, vc, i32(st.bt), i32(st.qsl), i32(st.ctx), i32(st.off), st.num_decodes, st.max_ctx, st.scale)
    a = cb.attention_step(*args)
    b = cb.attention_step_noalloc(*args)
    torch.cuda.synchronize()
    return a.float().cpu().numpy(), b.float().cpu().numpy(), a, b


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 32, 8, 128), ("bf16", 16, 4, 64)])
def test_noalloc_matches_workspace_entry_point_on_two_calls(dtype, hq, hkv, d):
    """Two calls in a row, the second smaller: bitwise equal to the
    workspace entry point's output, and within the oracle tolerance."""
    cases = [
        [(3000, 1), (700, 1), (5200, 1), (1500, 300), (900, 257)],   # decodes with splits + two chunks
        [(300, 1), (120, 40)],                                      # smaller: one decode, one chunk
    ]
    for n, seqs in enumerate(cases):
        say(f"noalloc call {n}: {dtype} {hq}q/{hkv}kv D{d}, seqs {seqs}")
        st = Step(seqs, hq, hkv, d, dtype, seed=60 + n, table_seed=61 + n)
        kc, vc = st.upload()
        ga, gb, ta, tb = _both(st, kc, vc)
        assert torch.equal(ta.view(torch.int16), tb.view(torch.int16)), "outputs differ bitwise"
        for s in range(len(seqs)):
            a, e = st.qsl[s], st.qsl[s + 1]
            ref = ora.attend(st.q[s], st.k_hist[s], st.v_hist[s], st.scale)
            am = ora.attend(st.q[s], st.k_hist[s], np.abs(st.v_hist[s]), st.scale)
            compare(gb[a:e], ref, dtype, f"noalloc call {n} seq {s}", am)
