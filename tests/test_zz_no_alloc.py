"""The allocation-free backward (ss_bwd_noalloc) against ss_bwd.

ss_bwd_noalloc runs ss_bwd's kernels with its workspace in the library's
device-resident scratch array, so on the same inputs its gradients must be
the same bits as ss_bwd's.  Two calls in a row, the second on a smaller
input, check that the array's leftover contents from the first call do not
leak into the second; a shape that needs more scratch than the array holds
is refused before anything is launched.
"""
import pytest
import torch

from selective_state_space_scan_amd import binding
from selective_state_space_scan_amd import inputs as ssin

from gpu_util import dev_inputs, require_gpu, say

pytestmark = pytest.mark.gpu


def _args(d):
    return (d["u"], d["delta"], d["A"], d["B"], d["C"], d.get("D"), d.get("z"),
            d.get("delta_bias"), True)


def _equal(a, b, name):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    assert torch.equal(a, b), f"{name} differs from ss_bwd"


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_noalloc_matches_ss_bwd_twice_second_smaller(io):
    require_gpu()
    cases = [  # (batch, dim, dstate, L, with the forward's saved record): large first, then smaller
        (4, 200, 16, 300, True),
        (2, 72, 16, 130, False),
        # several 16-state slices, chained through the scratch array
        (2, 40, 40, 96, False),
        (1, 24, 33, 70, True),
    ]
    for batch, dim, N, L, with_ckpt in cases:
        say(f"noalloc {io} batch {batch} dim {dim} dstate {N} L {L} ckpt {with_ckpt}")
        w = ssin.custom("bwd", batch, dim, N, L, io, seed=batch * 100 + dim + L + N)
        d = dev_inputs(ssin.make(w))
        ck = None
        if with_ckpt:
            ck = binding.ss_ckpt_empty(d["u"], dstate=N)
            binding.ss_fwd(*_args(d), ckpt=ck)
        dl = torch.randn(batch, dim, N, device=d["u"].device)
        ref = binding.ss_bwd(*_args(d), d["dout"], dlast=dl, want_dh0=True, ckpt=ck)
        got = binding.ss_bwd_noalloc(*_args(d), d["dout"], dlast=dl, want_dh0=True, ckpt=ck)
        torch.cuda.synchronize()
        assert set(got) == set(ref)
        for k in ref:
            _equal(got[k], ref[k], k)


def test_noalloc_refuses_shapes_beyond_its_scratch():
    require_gpu()
    cap = binding.ss_bwd_noalloc_max_scratch()
    assert cap == 96 << 20
    # without the forward's record the block states of 8 x 1536 x 2048 alone
    # take 100 MB: refused before any launch
    w = ssin.custom("bwd", 8, 1536, 16, 16, "f32", seed=1)
    d = dev_inputs(ssin.make(w))
    u = torch.empty(8, 1536, 2048, device=d["u"].device)
    B = torch.empty(8, 16, 2048, device=d["u"].device)
    with pytest.raises(binding.SSError) as e:
        binding.ss_bwd_noalloc(u, u, d["A"], B, B, None, None, None, True, u)
    assert "scratch" in str(e.value)
