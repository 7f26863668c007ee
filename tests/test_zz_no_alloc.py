"""GPU: the allocation-free decode (paged_attn_decode_noalloc) against the
decode with a caller workspace, through the C ABI.

Both run the same kernels and the same split plan, so the outputs must be
identical bit for bit; each is also checked against the oracle.  Two calls
in a row share the library's static scratch, the second on a smaller batch
(the buffer then holds the first call's partials, which the second must not
read).  Collected last: it must pass alone in a fresh process and after the
other tests.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (TOL, np_to_gpu, oracle_cache, poisoned_gpu_cache, q_tensor, say, to_f64,
                         used_slot_mask)
from workloads import custom_workload, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_attention_10_amd as lib
    return lib


def _case(w):
    cache = oracle_cache(w)
    gc = poisoned_gpu_cache(cache, used_slot_mask(w))
    return cache, gc


def _both(pkv, w, gc, window=0):
    q = q_tensor(w)
    bt, cl = np_to_gpu(w.block_tables), np_to_gpu(w.context_lens)
    ref = pkv.paged_attn_decode(q, gc["k"], gc["v"], bt, cl, w.max_context_len, w.scale,
                                k_scales=gc["ks"], v_scales=gc["vs"], window=window)
    out = torch.full_like(ref, float("nan"))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    pkv.paged_attn_decode_noalloc(q, gc["k"], gc["v"], bt, cl, w.max_context_len, w.scale, out,
                                  k_scales=gc["ks"], v_scales=gc["vs"], window=window)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return ref, out


def test_noalloc_equals_decode_two_calls(pkv):
    """The C2 decode batch (64 sequences, contexts 512-4096, two splits each
    at most), then a smaller batch (6 sequences up to 4096 tokens: more
    splits per sequence, fewer partial rows in all): both bit-identical to
    paged_attn_decode and within tolerance of the oracle."""
    w1 = make_workload("C2")
    w2 = custom_workload(context_lens=[4096, 1, 0, 2049, 77, 3000],
                         num_q_heads=12, num_kv_heads=2, head_dim=128, kv_dtype="bf16", seed=91)
    n1 = pkv.paged_attn_decode_workspace_bytes(64, 12, 2, 128, w1.max_context_len)
    n2 = pkv.paged_attn_decode_workspace_bytes(6, 12, 2, 128, w2.max_context_len)
    assert 0 < n2 < n1      # both use the scratch, the second less of it
    for w in (w1, w2):
        say(f"noalloc decode B={w.batch} max ctx {w.max_context_len}")
        cache, gc = _case(w)
        ref, out = _both(pkv, w, gc)
        assert torch.equal(ref.view(torch.int32), out.view(torch.int32))
        gold = oracle.ref_decode(w.q.astype(np.float64), cache, w.block_tables, w.context_lens,
                                 w.scale, w.num_q_heads)
        assert oracle.max_abs_err(to_f64(out), gold) <= TOL[w.kv_dtype]


@pytest.mark.parametrize("kv", ["f32", "i8", "fp8"])
def test_noalloc_other_kv_dtypes_and_window(pkv, kv):
    w = custom_workload(context_lens=[3000, 45, 700, 6000], num_q_heads=8, num_kv_heads=2,
                        head_dim=64, kv_dtype=kv, seed=92)
    say(f"noalloc decode kv={kv}")
    cache, gc = _case(w)
    for window in (0, 1000):
        ref, out = _both(pkv, w, gc, window=window)
        assert torch.equal(ref.view(torch.int32), out.view(torch.int32))


def test_noalloc_refuses_beyond_the_scratch(pkv):
    """A shape whose split partials exceed the static scratch is refused
    with PKV_ERR_SCRATCH_TOO_SMALL before anything is launched (the output
    keeps its contents)."""
    w = custom_workload(context_lens=[20, 30], num_q_heads=4, num_kv_heads=1, head_dim=64,
                        kv_dtype="bf16", seed=93)
    _, gc = _case(w)
    need = pkv.paged_attn_decode_workspace_bytes(4096, 4, 1, 64, 262144)
    assert need > pkv._lib.NOALLOC_SCRATCH_BYTES
    # claim a batch of 4096 over a 262144-token maximum; the host refuses it
    # from the sizes alone, so the small tensors are never read
    q = torch.zeros((4096, 4, 64), dtype=torch.float32, device="cuda")
    out = torch.full((4096, 4, 64), 7.0, device="cuda")
    bt = torch.zeros((4096, 16384), dtype=torch.int32, device="cuda")
    cl = torch.zeros(4096, dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attn_decode_noalloc(q, gc["k"], gc["v"], bt, cl, 262144, w.scale, out)
    assert e.value.status == 6
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))
