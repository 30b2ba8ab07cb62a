"""atopk_bucketed_noalloc (the library's own device scratch array as the
workspace) against atopk_bucketed (a caller-allocated workspace): bit-equal
values and indices on two calls in a row, the second with a smaller input
whose workspace is smaller too, for every stage-1 route that uses a
workspace; and shapes whose workspace exceeds the array are refused."""

import pytest
import torch

import top_sparse_attention_exact_amd as atk
from top_sparse_attention_exact_amd import _lib

pytestmark = pytest.mark.gpu


def _rows(m, n, dtype, seed, gpu):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randn((m, n), generator=g).to(dtype).to(gpu)


# (dtype, m, n, k, b, kb, final_exact): the one-pass wide kernel with its
# final, the split-row stage 1 with its finish (with and without the final
# stage), the exact route through the certified pass, bf16 rows
PAIRS = [
    ((torch.float32, 16, 1 << 20, 8192, 512, 16, True), (torch.float32, 3, 70001, 4096, 256, 16, True)),
    ((torch.float32, 8, 300007, 64, 1024, 2, True), (torch.float32, 2, 100003, 64, 512, 2, True)),
    ((torch.float32, 3, 300007, 64, 1024, 2, False), (torch.float32, 1, 70001, 64, 256, 1, False)),
    ((torch.bfloat16, 4, 777777, 200, 256, 1, True), (torch.bfloat16, 2, 50000, 100, 128, 1, True)),
    ((torch.float32, 2, 40000, 5000, 1, 5000, True), (torch.float32, 1, 9000, 300, 1, 300, True)),
]


@pytest.mark.parametrize("big,small", PAIRS)
def test_noalloc_matches_bucketed_twice(gpu, big, small):
    for i, (dt, m, n, k, b, kb, fin) in enumerate((big, small)):
        x = _rows(m, n, dt, 100 * i + n, gpu)
        need = atk.bucketed_workspace_bytes(dt, m, n, k, b, kb, fin)
        assert 0 < need <= atk.NOALLOC_SCRATCH_BYTES
        print("case", i, dt, m, n, k, b, kb, fin, need, flush=True)
        rv, ri = atk.bucketed(x, k, b, kb, fin)
        nv, ni = atk.bucketed_noalloc(x, k, b, kb, fin)
        torch.cuda.synchronize()
        assert torch.equal(ri, ni)
        assert torch.equal(rv.view(torch.int16) if dt == torch.bfloat16 else rv.view(torch.int32),
                           nv.view(torch.int16) if dt == torch.bfloat16 else nv.view(torch.int32))


def test_noalloc_refuses_oversized(gpu):
    # 128 x 2^20 fp32 with (8192, 1) and the final stage needs 8 MiB of lists:
    # inside the array; 8 x 2^24 with (4096, 16) needs far more: refused
    # before anything is enqueued
    dt, m, n, k, b, kb = torch.float32, 8, 1 << 24, 64, 4096, 16
    need = atk.bucketed_workspace_bytes(dt, m, n, k, b, kb, True)
    assert need > atk.NOALLOC_SCRATCH_BYTES
    x = torch.empty((m, n), dtype=dt, device=gpu)
    with pytest.raises(_lib.AtopkError) as e:
        atk.bucketed_noalloc(x, k, b, kb, True)
    assert e.value.status == 5  # ATOPK_ERR_WORKSPACE
