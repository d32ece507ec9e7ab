"""The truncation entry point that allocates nothing (its partial lists live in a fixed device
array) against spec_truncate with a caller workspace: identical lists, counts and flags on two
calls in a row, the second smaller than the first, so that what the first call left in the
array must not show through; and a request above the array's size is refused."""
import numpy as np
import pytest
import torch

from speculative_decoding_token_amd import binding as B

pytestmark = pytest.mark.gpu


def truncate_both(x: torch.Tensor, samp):
    rows, V = x.shape
    dt = B.DTYPE_BF16 if x.dtype == torch.bfloat16 else B.DTYPE_F32
    s = B.sampler(*samp)
    cap = samp[1] if samp[0] > 0 else 1
    ref, got = B.Probs(rows, cap), B.Probs(rows, cap)
    fr = torch.full((rows,), 0xAA, dtype=torch.uint8, device="cuda")
    fg = torch.full((rows,), 0x55, dtype=torch.uint8, device="cuda")
    nbytes = B.spec_truncate_scratch_size(rows, V)
    assert nbytes <= B.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    B.spec_truncate(x, dt, rows, V, x.stride(0), s, ref, fr, ws, nbytes)
    B.spec_truncate_noalloc(x, dt, rows, V, x.stride(0), s, got, fg)
    torch.cuda.synchronize()
    return ref, got, fr.cpu().numpy(), fg.cpu().numpy()


def assert_same(ref, got, fr, fg):
    assert np.array_equal(fr, fg)
    lr, lg = ref.to_lists(), got.to_lists()
    assert len(lr) == len(lg)
    compared = 0
    for (ir, pr), (ig, pg) in zip(lr, lg):
        assert np.array_equal(ir, ig)
        assert np.array_equal(np.asarray(pr).view(np.uint32), np.asarray(pg).view(np.uint32))
        compared += len(ir)
    return compared


def test_noalloc_truncate_matches_workspace_entry_point_twice():
    g = torch.Generator().manual_seed(5)
    # first call: the accept workload's shape, 64 sequences x 9 target rows of bf16 logits
    big = (torch.randn(576, 151936, generator=g) * 3.0).to(torch.bfloat16).cuda()
    n1 = assert_same(*truncate_both(big, (1.0, 20, 0.95)))
    # second call, smaller (fewer rows, fewer segments, another sampler and dtype)
    small = (torch.randn(7, 40000, generator=g) * 3.0).cuda()
    small[3, 123] = float("nan")  # a bad row: count 0 and the flag, on both entry points
    ref, got, fr, fg = truncate_both(small, (0.7, 64, 0.5))
    n2 = assert_same(ref, got, fr, fg)
    assert fg[3] & B.FLAG_BAD_ROW
    # and greedy on a third, smaller still
    tiny = (torch.randn(3, 1000, generator=g) * 3.0).to(torch.bfloat16).cuda()
    n3 = assert_same(*truncate_both(tiny, (0.0, 20, 0.95)))
    print(f"no-alloc truncation: {n1}, {n2}, {n3} list entries identical to the workspace entry point")
    assert n1 > 0 and n2 > 0 and n3 == 3


def test_noalloc_truncate_refuses_more_than_its_array():
    V = 151936
    rows = 2000  # 2000 x 10 segments x 64 keys x 8 bytes = 10.2 MB > 8 MiB
    assert B.spec_truncate_scratch_size(rows, V) > B.NOALLOC_SCRATCH_BYTES
    # inputs of the full size, so that nothing could read out of bounds were the call accepted
    x = torch.zeros((rows, V), dtype=torch.bfloat16, device="cuda")
    out = B.Probs(rows, 20)
    with pytest.raises(B.SpecError) as e:
        B.spec_truncate_noalloc(x, B.DTYPE_BF16, rows, V, V, B.sampler(1.0, 20, 0.95), out, None)
    assert e.value.code == B.SPEC_E_RANGE
