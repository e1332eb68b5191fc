"""moe_forward_noalloc (the entry point for callers that cannot allocate: its workspace is the library's
static device scratch) against moe_forward with a caller-owned workspace: bitwise equal outputs and
routing copies, on two calls in a row whose second input is smaller, for the register-staged 16-row
tiles, the 256-row bf16 tiles and fp8; and the decode configuration at full size."""
import pytest
import torch

from gpu_util import say
from sparse_mixture_experts_08_amd import binding as B
from sparse_mixture_experts_08_amd import workloads as W

pytestmark = pytest.mark.gpu
BF16, FP8 = W.BF16, W.FP8_E4M3


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _check(wl, seed):
    say(f"[noalloc] {wl.name} T={wl.T}")
    inp = W.generate(wl, seed=seed, device="cuda")
    y_ref, r_ref = B.forward_inputs(inp, wl.k, routing=True)
    y = torch.full_like(inp["x"], float("nan"))
    y, r = B.forward_inputs_noalloc(inp, wl.k, y=y, routing=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(y_ref))
    for k in r_ref:
        assert torch.equal(r[k], r_ref[k]), k


@pytest.mark.parametrize("big,small", [
    (W.Workload("na-bf16-16row", 200, 1024, 64, 6, 384, 256, BF16, BF16),
     W.Workload("na-bf16-16row-small", 37, 512, 32, 4, 256, 128, BF16, BF16)),
    (W.Workload("na-bf16-256row", 320, 512, 8, 4, 256, 384, BF16, BF16),
     W.Workload("na-bf16-256row-small", 90, 512, 8, 2, 256, 256, BF16, BF16)),
    (W.Workload("na-fp8", 300, 512, 16, 4, 256, 256, BF16, FP8),
     W.Workload("na-fp8-small", 41, 256, 16, 4, 128, 128, BF16, FP8)),
    (W.Workload("na-fp8-256row", 1100, 512, 8, 2, 256, 384, BF16, FP8),
     W.Workload("na-fp8-256row-small", 700, 512, 8, 2, 256, 256, BF16, FP8)),
], ids=lambda w: w.name)
def test_noalloc_matches_moe_forward_twice(big, small):
    _check(big, seed=31)
    _check(small, seed=32)


def test_noalloc_decode_full_size_then_smaller():
    _check(W.DECODE_BF16, seed=0)
    torch.cuda.empty_cache()
    _check(W.DECODE_BF16.with_T(17), seed=1)


def test_noalloc_refuses_a_shape_beyond_its_scratch():
    wl = W.Workload("na-too-big", 5000, 512, 16, 8, 512, 512, BF16, BF16)
    shape = B.make_shape(wl.T, wl.d, wl.E, wl.k, wl.inter, wl.inter_shared, wl.act_dtype, wl.w_dtype)
    assert B.moe_workspace_size(shape) > B.NOALLOC_SCRATCH_BYTES
    inp = W.generate(wl, seed=33, device="cuda")
    with pytest.raises(B.MoeError) as e:
        B.forward_inputs_noalloc(inp, wl.k)
    assert e.value.status == 5
