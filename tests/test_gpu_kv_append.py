"""cb_kv_append on the GPU, bit for bit against the host page model."""
import numpy as np
import pytest
import torch

from gpu_util import dev, i32, say
from oracle import paging
import chunked_prefill_attention_amd as cb

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.view(torch.int32).cpu().numpy()


@pytest.mark.parametrize("dtype,d,hkv,T", [("bf16", 128, 8, 2048), ("bf16", 64, 3, 37), ("f32", 64, 8, 1000),
                                         ("f32", 128, 2, 17), ("bf16", 128, 8, 1)])
def test_append_bit_exact(dtype, d, hkv, T):
    say(f"kv_append {dtype} D={d} Hkv={hkv} T={T}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    rng = np.random.default_rng(T + d)
    pages = (T * 3) // 16 + 4
    # sentinel: a NaN payload pattern that a float conversion would not preserve
    sentinel = 0x7FA5 if dtype == "bf16" else 0x7FC0ABCD
    ibits = torch.int16 if dtype == "bf16" else torch.int32
    kc = torch.full((pages, hkv, 16, d), sentinel, dtype=ibits, device=dev()).view(tdt)
    vc = torch.full((pages, hkv, d, 16), sentinel, dtype=ibits, device=dev()).view(tdt)
    # new rows: random bit patterns (including NaN/Inf payloads) as raw integers
    kn_bits = rng.integers(-2**15, 2**15, size=(T, hkv, d)) if dtype == "bf16" else rng.integers(-2**31, 2**31, size=(T, hkv, d))
    vn_bits = rng.integers(-2**15, 2**15, size=(T, hkv, d)) if dtype == "bf16" else rng.integers(-2**31, 2**31, size=(T, hkv, d))
    npdt = np.int16 if dtype == "bf16" else np.int32
    kn_bits, vn_bits = kn_bits.astype(npdt), vn_bits.astype(npdt)
    slots = rng.permutation(pages * 16)[:T].astype(np.int32)
    slots[rng.random(T) < 0.1] = -1
    kn = torch.from_numpy(kn_bits).to(dev()).view(tdt)
    vn = torch.from_numpy(vn_bits).to(dev()).view(tdt)
    cb.kv_append(kn, vn, kc, vc, i32(slots))
    torch.cuda.synchronize()
    mk = np.full((pages, hkv, 16, d), sentinel, npdt)
    mv = np.full((pages, hkv, d, 16), sentinel, npdt)
    paging.append(mk, mv, kn_bits, vn_bits, slots)
    assert np.array_equal(_bits(kc), mk)
    assert np.array_equal(_bits(vc), mv)


def test_append_out_of_range_slot_is_skipped():
    kc = torch.zeros((2, 1, 16, 64), dtype=torch.bfloat16, device=dev())
    vc = torch.zeros((2, 1, 64, 16), dtype=torch.bfloat16, device=dev())
    kn = torch.ones((3, 1, 64), dtype=torch.bfloat16, device=dev())
    cb.kv_append(kn, kn, kc, vc, i32([5, 32, 1 << 20]))
    torch.cuda.synchronize()
    assert kc.float().sum().item() == 64 and vc.float().sum().item() == 64
    assert kc[0, 0, 5].float().min().item() == 1
