"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Selection on given buffers must match bit for bit (indices and value bits).
Decode: scores within 1e-3 * max(1, |s|) of the float64 oracle; the selected
index set equal to the oracle's selection run on the GPU's own fp32 scores
(bit-exact), and equal to the float64 selection wherever every boundary the
selection crosses has a score gap above 1e-3; the bf16 output within 2e-2
(max-abs) of the float64 softmax over the GPU's index set.
"""

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import top_sparse_attention_exact_amd as atk
from top_sparse_attention_exact_amd import workloads

pytestmark = pytest.mark.gpu


def bits16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host(x):
    """(numpy array as the oracle wants it, dtype tag)."""
    if x.dtype == torch.bfloat16:
        return bits16(x), "bf16"
    return x.detach().cpu().numpy(), "f32"


def out_bits(v):
    if v.dtype == torch.bfloat16:
        return bits16(v)
    return v.detach().cpu().numpy().view(np.uint32)


def ref_bits(vals, tag):
    return vals if tag == "bf16" else vals.view(np.uint32)


def check_exact(x, k):
    vals, idx = atk.exact(x, k)
    hx, tag = host(x)
    ridx, rvals = oracle.exact_topk(hx, k, tag)
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_array_equal(out_bits(vals), ref_bits(rvals, tag))


def check_bucketed(x, k, b, kb, final, assignment="interleaved"):
    vals, idx = atk.bucketed(x, k, b, kb, final, assignment=assignment)
    hx, tag = host(x)
    ridx, rvals = oracle.bucketed_topk(hx, k, b, kb, final, tag, assignment=assignment)
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_array_equal(out_bits(vals), ref_bits(rvals, tag))


def host_pool():
    """Threads for the oracle side of the full-size checks (numpy releases
    the GIL in its sorts and products)."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 4
    return ThreadPoolExecutor(max(1, min(16, cores)))


def check_rows_all(x, k, runs):
    """Every row of a large batch against the oracle, rows spread over host
    threads.  runs: list of (name, gpu (vals, idx), oracle function of one
    host row block -> (idx, vals))."""
    hx, tag = host(x)
    got = [(name, idx.cpu().numpy(), out_bits(vals), fn) for name, (vals, idx), fn in runs]
    chunk = 4

    def one(r0):
        rows = slice(r0, min(r0 + chunk, hx.shape[0]))
        for name, gi, gv, fn in got:
            ridx, rvals = fn(hx[rows], tag)
            np.testing.assert_array_equal(gi[rows], ridx, err_msg="%s rows %s" % (name, rows))
            np.testing.assert_array_equal(gv[rows], ref_bits(rvals, tag), err_msg="%s rows %s" % (name, rows))

    with host_pool() as pool:
        list(pool.map(one, range(0, hx.shape[0], chunk)))


def rand_rows(m, n, dtype, seed, gpu):
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn((m, n), generator=g, dtype=torch.float32)
    return x.to(dtype).to(gpu)


# ------------------------------------------------------------ selection ----

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n", [1, 7, 100, 2048 + 37, 5000, 16384 + 123, 70001])
def test_exact_shapes(gpu, dtype, n):
    x = rand_rows(3, n, dtype, n, gpu)
    for k in sorted({1, min(n, 5), min(n, 64), min(n, 300)}):
        check_exact(x, k)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n", [64, 520, 1024, 1536, 3000, 4096, 8192 - 8])
def test_exact_short_aligned_rows(gpu, dtype, n):
    # 16-byte aligned rows with k <= 64 take the one-workgroup row kernel; a
    # row shorter than one pass of its 16 waves (4096 fp32 / 8192 bf16
    # elements) leaves the last waves without elements, and the first-tile
    # bound is pooled over the waves that hold some.  k > 64 takes the kernel
    # that ranks a row of at most 8192 elements whole in LDS.
    x = rand_rows(5, n, dtype, 40 + n, gpu)
    for k in sorted({1, 2, 17, min(n, 63), min(n, 64), min(n, 65), min(n, 300), min(n, 1025), n}):
        check_exact(x, k)
    xt = workloads.rows_ties_bf16(3, n, 4, seed=n, device="cpu").to(dtype).to(gpu)
    for k in sorted({1, 33, min(n, 64), min(n, 200), n}):
        check_exact(xt, k)
    # odd row strides (not 16-byte aligned): every k takes the whole-row kernel
    xs = rand_rows(4, n + 3, dtype, 7 + n, gpu)[:, 1:n + 1]
    for k in sorted({1, min(n, 64), min(n, 500)}):
        check_exact(xs, k)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_exact_large_k(gpu, dtype):
    x = rand_rows(2, 40000, dtype, 5, gpu)
    for k in (2047, 2049, 5000, 8192):
        check_exact(x, k)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n,b,kb", [(4096, 64, 1), (4096, 32, 2), (5000, 16, 4), (3001, 4, 3), (2048 + 37, 128, 2),
                                    (70001, 512, 16), (70001, 256, 8), (999, 3, 5), (11, 3, 2), (64, 64, 1),
                                    (20000, 2048, 1), (20000, 1000, 2), (70001, 4096, 4)])
def test_bucketed_shapes(gpu, dtype, n, b, kb):
    x = rand_rows(3, n, dtype, n + b + kb, gpu)
    k = max(1, min(b * kb, 64))
    check_bucketed(x, k, b, kb, False)
    check_bucketed(x, k, b, kb, True)
    if b * kb <= n and b * kb <= 8192:
        check_bucketed(x, b * kb, b, kb, True)


def test_fig2_toy(gpu):
    x = torch.tensor([[5, 9, 1, 7, 3, 2, 0, 8, 4, 6, 10]], dtype=torch.float32, device=gpu)
    vals, idx = atk.bucketed(x, 4, 3, 2, False)
    assert idx.cpu().tolist() == [[3, 9, 10, 1, 8, 5]]
    vals, idx = atk.bucketed(x, 4, 3, 2, True)
    assert idx.cpu().tolist() == [[10, 1, 3, 9]]


def test_ties_and_special_values(gpu):
    x = workloads.rows_ties_bf16(6, 9000, 8, seed=1, device="cpu").to(gpu)
    for k in (1, 64, 1000):
        check_exact(x, k)
    for b, kb in [(64, 1), (16, 4), (128, 2), (5, 3)]:
        check_bucketed(x, min(64, b * kb), b, kb, True)
        check_bucketed(x, min(64, b * kb), b, kb, False)
    xf = x.float()  # fp32 copy: -0.0 / +0.0 ties, infinities
    check_exact(xf, 100)
    check_bucketed(xf, 64, 64, 2, True)


def test_all_equal_rows(gpu):
    for dtype in (torch.float32, torch.bfloat16):
        x = torch.full((2, 5000), 1.5, dtype=dtype, device=gpu)
        check_exact(x, 700)
        # k <= 64: every wave keeps a full region of ties, the final ranks 16 x 64 keys by index
        check_exact(x, 64)
        check_exact(x, 1)
        check_bucketed(x, 64, 32, 2, True)
        check_bucketed(x, 64, 32, 2, False)


def test_strided_and_misaligned_rows(gpu):
    base = rand_rows(4, 3000, torch.float32, 7, gpu)
    x = base[:, 1:2900]  # rows start at odd offsets: 16-byte loads impossible
    check_exact(x, 50)
    check_bucketed(x, 50, 32, 2, True)
    xb = rand_rows(4, 3000, torch.bfloat16, 8, gpu)[:, :2048]  # ldx != n, aligned
    check_exact(xb, 64)
    check_bucketed(xb, 64, 64, 1, False)
    check_bucketed(xb, 64, 128, 2, True)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("off", [1, 2, 3, 5, 7])
def test_bucketed_row_offsets(gpu, dtype, off):
    """Rows starting at every element offset from a 16-byte boundary (and an
    odd row stride, so each row's offset differs): the vectorised stage 1
    takes the leading elements in a scalar head sweep.  Several (b, k_b),
    splits of long rows, a row shorter than the head, and b above the
    vectorised limit (the per-bucket walk)."""
    base = rand_rows(5, 40011, dtype, 20 + off, gpu)
    x = base[:, off:off + 39001]
    for b, kb, fin in [(2, 4, True), (4, 3, True), (64, 1, False), (256, 2, True), (1024, 1, True), (512, 4, False),
                       (2048, 1, True), (8192, 2, True)]:
        print("case", dtype, off, b, kb, fin, flush=True)
        k = min(b * kb, 64)
        check_bucketed(x, k, b, kb, fin)
    tiny = base[:, off:off + 3]
    check_bucketed(tiny, 2, 2, 1, True)


@pytest.mark.parametrize("m,n", [(1, 1 << 20), (3, 777777)])
def test_bucketed_few_rows_many_splits(gpu, m, n):
    """Few long rows: stage 1 splits every row over many workgroups (the
    finish merges up to 1024 lists per bucket through its LDS tree), and
    the per-bucket walk (b above the vectorised limit, or not a power of
    two) splits rows too."""
    x = rand_rows(m, n, torch.float32, 30 + m, gpu)
    for b, kb, fin, k in [(32, 2, True, 64), (32, 2, False, 64), (4, 4, True, 16), (256, 1, True, 200),
                          (2048, 1, True, 1000), (3000, 2, True, 64), (4096, 2, False, 64), (1000, 3, True, 300)]:
        print("case", m, n, b, kb, fin, k, flush=True)
        check_bucketed(x, k, b, kb, fin)


@pytest.mark.parametrize("dtype,m,n", [(torch.float32, 3, 50000), (torch.float32, 1, 16384 + 5),
                                      (torch.bfloat16, 2, 70001)])
def test_bucketed_final_large_k(gpu, dtype, m, n):
    """Split-row finish sorting many survivors (64 < k <= 8192): runs of 64
    sorted in registers, then bitonic merges in LDS and by shuffles (k = b *
    k_b keeps every candidate, without the select)."""
    x = rand_rows(m, n, dtype, 60 + m + n, gpu)
    for b, kb, k in [(2048, 1, 2000), (4096, 2, 5000), (8192, 1, 8192), (4096, 2, 1024), (1024, 1, 1000),
                     (2048, 4, 1025)]:
        if b * kb > n:
            continue
        print("case", dtype, m, n, b, kb, k, flush=True)
        check_bucketed(x, k, b, kb, True)


def test_single_row_and_empty(gpu):
    x = rand_rows(1, 4096, torch.float32, 9, gpu)
    check_exact(x, 64)
    check_bucketed(x, 64, 64, 1, False)
    check_bucketed(x, 64, 32, 2, True)
    e = torch.empty((0, 100), dtype=torch.float32, device=gpu)
    v, i = atk.exact(e, 5)
    assert v.shape == (0, 5)


def test_repeatable(gpu):
    x = rand_rows(8, 50000, torch.bfloat16, 10, gpu)
    a = atk.bucketed(x, 64, 128, 2, True)
    b = atk.bucketed(x, 64, 128, 2, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ------------------------------------------- workload sizes, sampled rows ----

def test_sel4k_recall_vs_model(gpu):
    """4096 iid rows of the 1 x 4096 fp32 workload: outputs equal the oracle
    on a sample, and the mean recall matches the finite-n expectation and
    sits above Eq. (1)."""
    x = workloads.rows_uniform(4096, 4096, seed=0, device="cpu").to(gpu)
    ev, ei = atk.exact(x, 64)
    sample = slice(0, 64)
    hx = x[sample].cpu().numpy()
    ridx, _ = oracle.exact_topk(hx, 64, "f32")
    np.testing.assert_array_equal(ei[sample].cpu().numpy(), ridx)
    for b, kb, final in [(64, 1, False), (32, 2, True)]:
        bv, bi = atk.bucketed(x, 64, b, kb, final)
        ridx, _ = oracle.bucketed_topk(hx, 64, b, kb, final, "f32")
        np.testing.assert_array_equal(bi[sample].cpu().numpy(), ridx)
        r = oracle.recall(bi.cpu().numpy(), ei.cpu().numpy())
        se = r.std() / math.sqrt(len(r))
        assert abs(r.mean() - oracle.eq1_finite(4096, 64, b, kb)) < 5 * se
        assert r.mean() > oracle.eq1(64, b, kb) - 5 * se


def test_vocab128k_full(gpu):
    x = workloads.rows_normal_bf16(256, 131072, 2.0, seed=0, device="cpu").to(gpu)
    hx = bits16(x)
    ev, ei = atk.exact(x, 64)
    ridx, rv = oracle.exact_topk(hx, 64, "bf16")
    np.testing.assert_array_equal(ei.cpu().numpy(), ridx)
    np.testing.assert_array_equal(bits16(ev), rv)
    for b, kb, final in [(64, 1, False), (128, 2, True)]:
        bv, bi = atk.bucketed(x, 64, b, kb, final)
        oidx, ov = oracle.bucketed_topk(hx, 64, b, kb, final, "bf16")
        np.testing.assert_array_equal(bi.cpu().numpy(), oidx)
        np.testing.assert_array_equal(bits16(bv), ov)


@pytest.mark.timeout(600)
def test_wide1m_all_rows_and_worst_case(gpu):
    """The 64 x 2^20 fp32 batch with k = 8192 in the launches the benchmark
    times: exact, (512, 16) + final and (512, 16) stage 1 alone, every row
    bit for bit against the oracle; the adversarial rows' recall is exactly
    the Eq. (2) worst case."""
    m, n, b, kb, k = 64, 1 << 20, 512, 16, 8192
    x = workloads.rows_planted_residues(m, n, b, k, seed=0, device=gpu)
    bv, bi = atk.bucketed(x, k, b, kb, True)
    ev, ei = atk.exact(x, k)
    sv, si = atk.bucketed(x, k, b, kb, False)
    check_rows_all(x, k, [
        ("exact", (ev, ei), lambda h, tag: oracle.exact_topk(h, k, tag)),
        ("b512k16_final", (bv, bi), lambda h, tag: oracle.bucketed_topk(h, k, b, kb, True, tag)),
        ("b512k16", (sv, si), lambda h, tag: oracle.bucketed_topk(h, k, b, kb, False, tag)),
    ])
    r = oracle.recall(bi.cpu().numpy(), ei.cpu().numpy())
    worst = oracle.eq2(n, k, b, kb)
    assert worst == 64 / 8192
    np.testing.assert_array_equal(r[1::2], worst)  # planted rows: exactly the worst case
    assert abs(r[0::2].mean() - oracle.eq1_finite(n, k, b, kb)) < 0.01


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["vocab-sampling", "kg-2.65m"])
def test_tradeoff_shapes_all_rows(gpu, name):
    """The runtime/accuracy trade-off shapes at full size, in the launches the
    sweep times: exact top-k and three (b, k_b) of the sweep, final exact, bit
    for bit against the oracle on every row; for every (b, k_b) the mean
    recall over all rows within 0.02 of Eq.(1)'s finite-n expectation (iid
    rows)."""
    c = workloads.TRADEOFF[name]
    m, n, k = c["m"], c["n"], c["k"]
    x = workloads.rows_normal(m, n, c["std"], seed=0, device=gpu, workload=name)
    ev, ei = atk.exact(x, k)
    runs = [("exact", (ev, ei), lambda h, tag: oracle.exact_topk(h, k, tag))]
    ex = ei.cpu().numpy()
    for b, kb in workloads.tradeoff_modes(k):
        print("case", name, b, kb, flush=True)
        bv, bi = atk.bucketed(x, k, b, kb, True)
        if (b, kb) in ((1024, 1), (512, 2), (8192, 1)):
            runs.append(("b%dk%d" % (b, kb), (bv, bi),
                         lambda h, tag, b=b, kb=kb: oracle.bucketed_topk(h, k, b, kb, True, tag)))
        r = oracle.recall(bi.cpu().numpy(), ex).mean()
        assert abs(r - oracle.eq1_finite(n, k, b, kb)) < 0.02, (b, kb, r)
    check_rows_all(x, k, runs)


@pytest.mark.parametrize("name,dtype", [("vocab-sampling", torch.float32), ("vocab-sampling", torch.bfloat16)])
def test_choose(gpu, name, dtype):
    """The measured chooser: its pick meets the recall target by the model,
    its outputs equal a plain call of the picked (b, k_b) and the oracle on
    every row, and the measured recall agrees with the model."""
    c = workloads.TRADEOFF[name]
    m, n, k = c["m"], c["n"], c["k"]
    x = workloads.rows_normal(m, n, c["std"], seed=3, device=gpu, workload=name).to(dtype)
    _, ex = atk.exact(x, k)
    for target in (0.9, 0.99, 1.0):
        res = atk.choose(x, k, target)
        b, kb = res["b"], res["kb"]
        print("case", name, dtype, target, b, kb, res["us"], flush=True)
        assert res["recall"] >= target and res["us"] > 0
        if b == 1:
            assert kb == k and res["recall"] == 1.0
        else:
            assert b * kb <= 8192 and res["recall"] == atk.expected_recall(n, k, b, kb)
        v, i = atk.bucketed(x, k, b, kb, True)
        assert torch.equal(v, res["values"]) and torch.equal(i, res["indices"])
        check_rows_all(x, k, [("chosen", (v, i), lambda h, tag, b=b, kb=kb: oracle.bucketed_topk(h, k, b, kb, True,
                                                                                               tag))])
        if dtype == torch.float32:
            r = oracle.recall(i.cpu().numpy(), ex.cpu().numpy()).mean()
            assert abs(r - res["recall"]) < 0.02


# ------------------------------- certified exact (bucketed pass + rescan) ----

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("m,n,k", [(1, 1 << 20, 100), (2, 300007, 256), (64, 128256, 256), (3, 70001, 16),
                                   (1, 4_000_003, 64), (5, 9000, 300)])
def test_certified_exact_shapes(gpu, dtype, m, n, k):
    """Shapes whose exact top-k runs as a bucketed pass plus the finish's
    certification (k above the one-row kernel's limit, or few long rows);
    fp32 rows of 2^14 or more elements with k > 64 take the sampled wide
    route instead, which these shapes then cover."""
    x = rand_rows(m, n, dtype, m + n + k, gpu)
    rows = sorted({0, m - 1})
    vals, idx = atk.exact(x, k)
    hx, tag = host(x[rows])
    ridx, rvals = oracle.exact_topk(hx, k, tag)
    np.testing.assert_array_equal(idx[rows].cpu().numpy(), ridx)
    np.testing.assert_array_equal(out_bits(vals[rows]), ref_bits(rvals, tag))


def test_certified_exact_rescan_and_fallback(gpu):
    """Rows that defeat the bucket candidates: row 0 holds 20 large values at
    multiples of 4096 (one bucket for every power-of-two b <= 4096, so the
    rescan must bring back all but k_b of them); row 1 lifts every 16th
    element (with k = 16 the certified plan uses 16 buckets, so one bucket
    holds 8192 values above the threshold and the pool overflows into the
    full-row fallback); row 2 has two levels (heavy ties); row 3 is plain."""
    m, n, k = 4, 131072 + 5, 16
    g = torch.Generator(device="cpu").manual_seed(77)
    x = torch.rand((m, n), generator=g)
    x[0, 0:20 * 4096:4096] = 10.0 + torch.rand(20, generator=g)
    x[1, 0::16] = 10.0 + torch.rand(x[1, 0::16].shape[0], generator=g)
    x[2] = torch.floor(torch.rand(n, generator=g) * 2) / 2
    for kk in (16, 100, 256):
        xx = x.to(gpu)
        vals, idx = atk.exact(xx, kk)
        ridx, rvals = oracle.exact_topk(x.numpy(), kk, "f32")
        np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
        np.testing.assert_array_equal(vals.cpu().numpy().view(np.uint32), rvals.view(np.uint32))
        xb = x.to(torch.bfloat16)
        vals, idx = atk.exact(xb.to(gpu), kk)
        ridx, rvals = oracle.exact_topk(bits16(xb), kk, "bf16")
        np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
        np.testing.assert_array_equal(bits16(vals), rvals)


# -------------------------------------- wide fp32 rows (two-pass route) ----

def quantized_rows(m, n, levels, seed, gpu):
    """fp32 rows holding only `levels` distinct values (heavy ties)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.floor(torch.rand((m, n), generator=g) * levels) / levels).to(gpu)


@pytest.mark.parametrize("m,n", [(1, 16384), (3, 65536 + 77), (5, 100000)])
def test_wide_exact(gpu, m, n):
    x = rand_rows(m, n, torch.float32, m * n, gpu)
    for k in (65, 1000, 8192):
        check_exact(x, k)


def test_wide_exact_ties(gpu):
    # three levels: the collection holds every tie at the threshold
    check_exact(quantized_rows(2, 65536, 3, 1, gpu), 5000)
    # two levels: more elements reach the threshold than the collection
    # holds, so each row runs the full radix select with index-ordered ties
    check_exact(quantized_rows(2, 131072, 2, 2, gpu), 8192)
    x = torch.full((1, 40000), -0.0, device=gpu)
    x[0, ::7] = 0.0
    check_exact(x, 3000)  # -0.0 and +0.0 are one value: lowest indices win


def _sampled_positions(row, n):
    """Element positions the wide exact route samples in `row` (n / 1024
    strata, one 16-element chunk at a hashed offset in each), written from
    the kernel's sampling rule so that a test can plant values exactly there."""
    def mix32(v):
        v &= 0xFFFFFFFF
        v ^= v >> 16
        v = (v * 0x7FEB352D) & 0xFFFFFFFF
        v ^= v >> 15
        v = (v * 0x846CA68B) & 0xFFFFFFFF
        v ^= v >> 16
        return v

    st = n // 1024
    slots = st // 16
    pos = []
    for t in range(1024):
        off = (mix32(row * 1024 + t + 0x9E3779B9) % slots) * 16
        pos.extend(range(t * st + off, t * st + off + 16))
    return np.array(pos)


def test_wide_exact_sample_fallback(gpu):
    """The largest values of the row sit exactly on the sampled positions, so
    the sampled threshold lands above the row's k-th largest and fewer than k
    elements reach it: the final must fall back to the full-row select and
    still return the exact top-k."""
    m, n, k = 2, 131072, 4096
    g = torch.Generator(device="cpu").manual_seed(17)
    x = torch.rand((m, n), generator=g)
    for row in range(m):
        pos = torch.from_numpy(_sampled_positions(row, n))
        x[row, pos] = 1000.0 + torch.rand(len(pos), generator=g)
    check_exact(x.to(gpu), k)


def test_wide_exact_special_values(gpu):
    x = workloads.rows_ties_bf16(3, 70000, 8, seed=3, device="cpu").float().to(gpu)
    for k in (100, 4000):
        check_exact(x, k)


@pytest.mark.parametrize("b,kb", [(512, 16), (256, 8), (64, 5), (1024, 12), (4096, 16), (192, 7)])
def test_wide_bucketed(gpu, b, kb):
    n = 70001
    x = rand_rows(3, n, torch.float32, b * 100 + kb, gpu)
    check_bucketed(x, min(64, b * kb), b, kb, False)
    if b * kb <= 8192:
        check_bucketed(x, b * kb, b, kb, True)
        check_bucketed(x, b * kb // 3, b, kb, True)


@pytest.mark.parametrize("m", [100, 300])
def test_wide_final_parts(gpu, m):
    # 100 rows: each row's final sort split over two workgroups; 300 rows:
    # one workgroup per row
    x = rand_rows(m, 12000, torch.float32, m, gpu)
    check_bucketed(x, 8192, 512, 16, True)
    check_bucketed(x, 1000, 512, 16, True)
    check_exact(x, 2000)


@pytest.mark.parametrize("levels", [2, 64, 1024])
def test_wide_bucketed_ties(gpu, levels):
    # 2 levels: hundreds of ties per bucket (index-ordered walk); 64 and 1024
    # levels: a few ties at T_r (the recorded tie list)
    x = quantized_rows(2, 65536 + 33, levels, levels, gpu)
    for b, kb in [(256, 8), (512, 16)]:
        check_bucketed(x, 64, b, kb, False)
        check_bucketed(x, b * kb, b, kb, True)
        check_bucketed(x, 1000, b, kb, True)


def test_wide_strided_and_misaligned(gpu):
    n = 50000
    big = rand_rows(3, n + 9, torch.float32, 77, gpu)
    x = big[:, 1:n + 1]  # row stride n + 9, start one element in
    check_exact(x, 1000)
    check_bucketed(x, 64, 512, 16, False)
    check_bucketed(x, 4096, 512, 8, True)


# ----------------------------------------- contiguous bucket assignment ----

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n,b,kb", [(4096, 64, 1), (4096, 32, 2), (131072, 64, 1), (131072, 128, 2), (5000, 7, 3),
                                    (11, 3, 2), (1000, 1000, 1), (70001, 512, 16), (20000, 100, 8), (3000, 16, 5)])
def test_contiguous_shapes(gpu, dtype, n, b, kb):
    x = rand_rows(3, n, dtype, n * 7 + b + kb, gpu)
    k = max(1, min(b * kb, 64))
    check_bucketed(x, k, b, kb, False, "contiguous")
    check_bucketed(x, k, b, kb, True, "contiguous")
    if b * kb <= 8192:
        check_bucketed(x, b * kb, b, kb, True, "contiguous")


def test_contiguous_ties_strided_and_exact_route(gpu):
    x = workloads.rows_ties_bf16(4, 9000, 8, seed=5, device="cpu").to(gpu)
    for b, kb in [(64, 1), (16, 4), (9, 3)]:
        check_bucketed(x, min(64, b * kb), b, kb, True, "contiguous")
        check_bucketed(x, min(64, b * kb), b, kb, False, "contiguous")
    check_bucketed(x.float(), 64, 64, 2, True, "contiguous")
    big = rand_rows(3, 8192 + 3, torch.bfloat16, 91, gpu)
    xs = big[:, 1:8193]  # misaligned rows: element loads
    check_bucketed(xs, 64, 64, 1, False, "contiguous")
    check_bucketed(xs, 64, 32, 4, True, "contiguous")
    check_bucketed(xs, 50, 1, 50, True, "contiguous")  # (1, k): the exact route


def test_contiguous_recall_under_correlation(gpu):
    """The interleaved / contiguous comparison on AR(1) rows, run on the GPU:
    recall per row equals the oracle's bucket-count identity, and contiguous
    buckets lose recall where interleaved ones keep Eq.(1)'s."""
    n, k, b, kb = 131072, 64, 64, 1
    x = workloads.rows_ar1(32, n, 0.99, seed=2, device=gpu)
    _, ex = atk.exact(x, k)
    ex = ex.cpu().numpy()
    rec = {}
    for assign in ("interleaved", "contiguous"):
        _, idx = atk.bucketed(x, k, b, kb, False, assignment=assign)
        r = oracle.recall(idx.cpu().numpy(), ex)
        np.testing.assert_array_equal(r, oracle.recall_by_bucket_counts(ex, n, b, kb, assign))
        rec[assign] = r.mean()
    assert rec["interleaved"] > oracle.eq1_finite(n, k, b, kb) - 0.03
    assert rec["contiguous"] < 0.2


# --------------------------------------------------------------- decode ----

def _decode_check(q, K, V, k_sel, b, kb, rows=None):
    """The decode in three forms: the call as the benchmark times it (output
    only), with the selection, and with the selection and the score dump.
    All three must agree bit for bit (the dump and the selection output do
    not change what is computed).  Then, for every (batch, query head) -- or
    the given pairs -- against the float64 oracle: scores within
    1e-3 * max(1, |s|); the selection bit-exact against the oracle's
    selection on the GPU's own fp32 scores, and equal as a set to the float64
    selection where every crossed boundary has a clear gap; the output within
    2e-2 of the float64 softmax over the GPU's set."""
    out_t = atk.sparse_attn_decode(q, K, V, k_sel, b, kb)
    out_s, sel_s = atk.sparse_attn_decode(q, K, V, k_sel, b, kb, return_sel=True)
    out, sel, sc = atk.sparse_attn_decode(q, K, V, k_sel, b, kb, return_sel=True, return_scores=True)
    assert torch.equal(out_t, out), "the output-only call differs from the dumping call"
    assert torch.equal(out_s, out) and torch.equal(sel_s, sel), "the selection call differs from the dumping call"
    bsz, hq, d = q.shape
    hkv = K.shape[1]
    g = hq // hkv
    scale32 = float(np.float32(1.0 / math.sqrt(d)))
    pairs = rows if rows is not None else [(i, h) for i in range(bsz) for h in range(hq)]
    groups = {}
    for (i, h) in pairs:
        groups.setdefault((i, h // g), []).append(h)
    q_h = bits16(q)
    sel_h = sel.cpu().numpy()
    out_h = out.float().cpu().numpy()

    def one(item):
        (i, kvh), heads = item
        kb_bits = bits16(K[i:i + 1, kvh:kvh + 1])
        vv = oracle.bf16_bits_to_f64(bits16(V[i, kvh]))
        ref = oracle.decode_scores(q_h[i:i + 1, heads[0]:heads[-1] + 1], kb_bits, scale32)[0]
        gpu = sc[i, heads[0]:heads[-1] + 1].cpu().numpy()
        for h in heads:
            ref_s = ref[h - heads[0]]
            gpu_s = gpu[h - heads[0]]
            assert np.all(np.abs(gpu_s - ref_s) <= 1e-3 * np.maximum(1.0, np.abs(ref_s))), (i, h)
            gsel = sel_h[i, h]
            # selection on the GPU's own scores: bit-exact
            ssel = oracle.attention.select(gpu_s[None, :].astype(np.float64), k_sel, b, kb)[0]
            np.testing.assert_array_equal(gsel, ssel, err_msg="head %d,%d" % (i, h))
            # against the float64 selection where every crossed boundary has a
            # clear gap: the selected set is then fixed (the order inside it is
            # not, where two selected scores sit within fp32 rounding)
            if _clear_gaps(ref_s, k_sel, b, kb):
                fsel = oracle.attention.select(ref_s[None, :], k_sel, b, kb)[0]
                np.testing.assert_array_equal(np.sort(gsel), np.sort(fsel), err_msg="head %d,%d" % (i, h))
            ref_o = oracle.softmax_v_subset(ref_s, gsel, vv)
            assert np.max(np.abs(out_h[i, h] - ref_o)) <= 2e-2, (i, h)
        return len(heads)

    with host_pool() as pool:
        done = sum(pool.map(one, sorted(groups.items())))
    assert done == len(pairs)
    return out, sel, sc


def _clear_gaps(s, k_sel, b, kb, gap=1e-3):
    n = s.shape[0]
    if not (b == 1 and kb == k_sel):
        cand = []
        for r in range(b):
            v = np.sort(s[r::b])[::-1]
            if len(v) > kb and v[kb - 1] - v[kb] <= gap:
                return False
            cand.extend(v[:kb].tolist())
        s = np.array(cand)
    v = np.sort(s)[::-1]
    return len(v) <= k_sel or v[k_sel - 1] - v[k_sel] > gap


@pytest.mark.parametrize("hq,hkv,ctx,k_sel,planted", [
    (2, 2, 3000, 64, "stride256"),    # one query head per KV head: a flagged bucket is rescored
    (8, 2, 3000, 64, "stride256"),    # query-head groups: a flagged bucket is rescored on the matrix cores
    (1, 1, 131072, 16, "mod8"),       # one bucket far above the rest: the rescan overflows, full-row fallback
    (4, 2, 131072, 64, "mod64lt5"),   # the same for query-head groups (5 buckets of 2048 keys)
])
def test_decode_exact_certified_planted(gpu, hq, hkv, ctx, k_sel, planted):
    """Exact Top-K decode on caches that defeat the bucket candidates: keys
    aligned with a query head planted in positions that share a bucket for
    every power-of-two b the certified plans use, so buckets are flagged and
    rescanned (or overflow into the full-row fallback)."""
    g = torch.Generator(device="cpu").manual_seed(ctx + hq)
    q = torch.randn((1, hq, 128), generator=g)
    K = torch.randn((1, hkv, ctx, 128), generator=g) * 0.5
    V = torch.randn((1, hkv, ctx, 128), generator=g)
    j = torch.arange(ctx)
    if planted == "stride256":
        mask = (j % 256 == 0) & (j < 12 * 256)
    elif planted == "mod8":
        mask = j % 8 == 0
    else:
        mask = j % 64 < 5
    G = hq // hkv
    for h in range(hkv):
        K[0, h, mask] = 2.0 * q[0, h * G] + 0.05 * torch.randn((int(mask.sum()), 128), generator=g)
    q, K, V = (t.to(torch.bfloat16).to(gpu) for t in (q, K, V))
    print("case", hq, hkv, ctx, k_sel, planted, flush=True)
    _decode_check(q, K, V, k_sel, 1, k_sel)


def test_decode_scores_position_invariant(gpu):
    """The matrix-core scores of query-head groups do not depend on where a key
    sits among the 16 columns of an MFMA tile, or in which step or chunk it is
    scored: copies of a key row at other positions get bit-identical scores.
    The certified exact decode relies on it when it rescores flagged buckets
    with their keys in other columns; the copies here are the top keys, so
    their exact ties decide the Top-K and are rescanned."""
    g = torch.Generator(device="cpu").manual_seed(11)
    hq, hkv, ctx, k_sel = 8, 2, 6000, 64
    G = hq // hkv
    q = torch.randn((1, hq, 128), generator=g)
    K = torch.randn((1, hkv, ctx, 128), generator=g) * 0.5
    V = torch.randn((1, hkv, ctx, 128), generator=g)
    src = torch.arange(40) * 37 + 5
    offs = [1, 3, 6, 16, 529, 4103]
    for h in range(hkv):
        K[0, h, src] = 2.0 * q[0, h * G + 1] + 0.3 * torch.randn((len(src), 128), generator=g)
        for o in offs:
            K[0, h, src + o] = K[0, h, src]
    q, K, V = (t.to(torch.bfloat16).to(gpu) for t in (q, K, V))
    for b, kb in [(1, k_sel), (16, 8)]:
        _, _, sc = _decode_check(q, K, V, k_sel, b, kb)
        s = sc[0].cpu().numpy().view(np.uint32)
        for o in offs:
            np.testing.assert_array_equal(s[:, src.numpy() + o], s[:, src.numpy()])


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 2), (6, 2)])
@pytest.mark.parametrize("ctx,k_sel,b,kb", [(3000, 64, 16, 8), (3000, 64, 64, 1), (3000, 64, 1, 64),
                                            (4096, 256, 128, 2), (5000, 100, 7, 16)])
def test_decode_small(gpu, hq, hkv, ctx, k_sel, b, kb):
    g = torch.Generator(device="cpu").manual_seed(ctx + hq + b)
    q = torch.randn((2, hq, 128), generator=g).to(torch.bfloat16).to(gpu)
    K = torch.randn((2, hkv, ctx, 128), generator=g).to(torch.bfloat16).to(gpu)
    V = torch.randn((2, hkv, ctx, 128), generator=g).to(torch.bfloat16).to(gpu)
    _decode_check(q, K, V, k_sel, b, kb)


@pytest.mark.parametrize("hq,hkv,ctx,k_sel,b,kb", [
    (8, 1, 3007, 100, 1, 100),    # the largest query-head group (G = 8), exact Top-K (certified)
    (16, 2, 2049, 64, 32, 4),     # G = 8, bucketed with the final stage, ragged context
    (8, 1, 777, 77, 11, 7),       # G = 8, non-power-of-two b and k_b
    (2, 2, 65, 64, 1, 64),        # context barely above K
    (4, 4, 5000, 1, 1, 1),        # K = 1: the arg-max key
])
def test_decode_groups_and_edges(gpu, hq, hkv, ctx, k_sel, b, kb):
    g = torch.Generator(device="cpu").manual_seed(ctx + hq + k_sel)
    q = torch.randn((2, hq, 128), generator=g).to(torch.bfloat16).to(gpu)
    K = torch.randn((2, hkv, ctx, 128), generator=g).to(torch.bfloat16).to(gpu)
    V = torch.randn((2, hkv, ctx, 128), generator=g).to(torch.bfloat16).to(gpu)
    print("case", hq, hkv, ctx, k_sel, b, kb, flush=True)
    _decode_check(q, K, V, k_sel, b, kb)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2)])
def test_decode_exact_large_k(gpu, hq, hkv):
    """Exact Top-K with K = ctx / 2: no certified plan fits, so the decode runs
    as separate passes (all scores, exact selection, softmax-V)."""
    g = torch.Generator(device="cpu").manual_seed(hq * 7 + hkv)
    q = torch.randn((1, hq, 128), generator=g).to(torch.bfloat16).to(gpu)
    K = torch.randn((1, hkv, 4096, 128), generator=g).to(torch.bfloat16).to(gpu)
    V = torch.randn((1, hkv, 4096, 128), generator=g).to(torch.bfloat16).to(gpu)
    _decode_check(q, K, V, 2048, 1, 2048)


@pytest.mark.parametrize("hq,hkv,planted", [(8, 2, "mod64lt5"), (8, 2, "none"), (2, 2, "mod64lt5")])
def test_decode_exact_without_scores_matches(gpu, hq, hkv, planted):
    """The certified exact decode without a score output (its rescans and any
    fallback row use the workspace alone) selects and outputs exactly what it
    does with one."""
    g = torch.Generator(device="cpu").manual_seed(hq * 31 + hkv)
    ctx = 40000
    q = torch.randn((2, hq, 128), generator=g)
    K = torch.randn((2, hkv, ctx, 128), generator=g) * 0.5
    V = torch.randn((2, hkv, ctx, 128), generator=g)
    if planted == "mod64lt5":  # five buckets far above the rest: flagged and rescanned
        mask = torch.arange(ctx) % 64 < 5
        G = hq // hkv
        for b in range(2):
            for h in range(hkv):
                K[b, h, mask] = 2.0 * q[b, h * G] + 0.05 * torch.randn((int(mask.sum()), 128), generator=g)
    q, K, V = (t.to(torch.bfloat16).to(gpu) for t in (q, K, V))
    out1, sel1, _ = atk.sparse_attn_decode(q, K, V, 64, return_sel=True, return_scores=True)
    out2, sel2 = atk.sparse_attn_decode(q, K, V, 64, return_sel=True)
    assert torch.equal(sel1, sel2)
    assert torch.equal(out1, out2)


def test_decode_in_place_finish_matches_finish_kernel(gpu):
    """With one query head per KV head, one context chunk per head and
    b * k_b = K, the scoring workgroup finishes its head itself (512 heads:
    one workgroup each).  The first half of the same batch alone has 256
    heads and is planned in bucket ranges, whose lists go to the separate
    finish kernel: the same candidates, so sel_idx and the output must agree
    bit for bit, with and without the selection output."""
    g = torch.Generator(device=gpu).manual_seed(5)
    bsz, h, ctx, k_sel, b, kb = 16, 32, 8192, 512, 256, 2
    q = torch.randn((bsz, h, 128), generator=g, device=gpu).to(torch.bfloat16)
    K = torch.randn((bsz, h, ctx, 128), generator=g, device=gpu).to(torch.bfloat16)
    V = torch.randn((bsz, h, ctx, 128), generator=g, device=gpu).to(torch.bfloat16)
    out, sel = atk.sparse_attn_decode(q, K, V, k_sel, b, kb, return_sel=True)
    out_only = atk.sparse_attn_decode(q, K, V, k_sel, b, kb)
    half = bsz // 2
    ref, rsel = atk.sparse_attn_decode(q[:half].contiguous(), K[:half].contiguous(), V[:half].contiguous(), k_sel, b,
                                       kb, return_sel=True)
    assert torch.equal(sel[:half], rsel)
    assert torch.equal(out[:half], ref)
    assert torch.equal(out_only, out)
    # and the selection is the oracle's on the kernel's own scores for a few heads
    _, _, sc = atk.sparse_attn_decode(q[:1].contiguous(), K[:1].contiguous(), V[:1].contiguous(), k_sel, b, kb,
                                      return_sel=True, return_scores=True)
    got = sc.cpu().numpy()
    for hh in (0, 17, 31):
        own = oracle.attention.select(got[0, hh][None].astype(np.float64), k_sel, b, kb)[0]
        assert np.array_equal(sel[0, hh].cpu().numpy(), own)


def test_decode_ctx_stride(gpu):
    g = torch.Generator(device="cpu").manual_seed(3)
    q = torch.randn((1, 4, 128), generator=g).to(torch.bfloat16).to(gpu)
    K = torch.randn((1, 4, 4000, 128), generator=g).to(torch.bfloat16).to(gpu)
    V = torch.randn((1, 4, 4000, 128), generator=g).to(torch.bfloat16).to(gpu)
    out, sel, sc = atk.sparse_attn_decode(q, K, V, 32, 32, 1, ctx=2500, return_sel=True, return_scores=True)
    assert int(sel.max()) < 2500
    ref, rsel = atk.sparse_attn_decode(q, K[:, :, :2500].contiguous(), V[:, :, :2500].contiguous(), 32, 32, 1,
                                       return_sel=True)
    assert torch.equal(sel, rsel)
    assert torch.equal(out, ref)


@pytest.mark.timeout(900)
def test_decode_mha32k_all_heads(gpu):
    """B16 H32 L32768, Top-512 via (256, 2): all 512 heads, in the call the
    benchmark times and with the dumps (see _decode_check); then the exact
    Top-512 (certified route) on all heads as well."""
    c = workloads.DECODE["mha-32k"]
    q, K, V, planted = workloads.decode_mha(c["bsz"], c["hq"], c["ctx"], c["d"], 64, 0.8, seed=0, device=gpu)
    out, sel, sc = _decode_check(q, K, V, c["k_sel"], c["b"], c["kb"])
    # Planted keys outscore every other key, so stage 1 keeps exactly
    # min(k_b, t_r) of the t_r planted keys that fall in bucket r.
    s = sel.cpu().numpy()
    p = planted.cpu().numpy()
    for i in range(c["bsz"]):
        for h in range(c["hq"]):
            kept = len(set(p[i, h].tolist()) & set(s[i, h].tolist()))
            t = np.bincount(p[i, h] % c["b"], minlength=c["b"])
            assert kept == np.minimum(t, c["kb"]).sum()
    del out, sel, sc
    _decode_check(q, K, V, c["k_sel"], 1, c["k_sel"])
    # The certified route is one function of the inputs: repeated calls, with
    # and without the selection output, give the same bits.  (Its select once
    # returned a threshold that the finish then overwrote in LDS before every
    # thread had read it; that showed in about one call in eight.)
    out0, sel0 = atk.sparse_attn_decode(q, K, V, c["k_sel"], 1, c["k_sel"], return_sel=True)
    for _ in range(6):
        out1, sel1 = atk.sparse_attn_decode(q, K, V, c["k_sel"], 1, c["k_sel"], return_sel=True)
        assert torch.equal(sel1, sel0) and torch.equal(out1, out0)
        assert torch.equal(atk.sparse_attn_decode(q, K, V, c["k_sel"], 1, c["k_sel"]), out0)


@pytest.mark.timeout(900)
def test_decode_gqa128k_all_heads(gpu):
    """B4 Hq32 Hkv8 L131072, Top-512 via (512, 4) + final and exact: all 128
    query heads in both modes, in the calls the benchmark times and with the
    dumps (see _decode_check)."""
    c = workloads.DECODE["gqa-128k"]
    q, K, V, _ = workloads.decode_gqa(c["bsz"], c["hq"], c["hkv"], c["ctx"], c["d"], 0.01, 3.0, seed=0, device=gpu)
    _decode_check(q, K, V, c["k_sel"], c["b"], c["kb"])
    _decode_check(q, K, V, c["k_sel"], 1, c["k_sel"])


# ------------------------------------------------------ candidate rerank ----

def _rerank_check(q, K, V, cand, window, k_sel, heads=None):
    """GPU rerank against the float64 oracle.  The call without dumps must
    equal the dumping call bit for bit.  Per head: the dumped fp32 scores of
    the candidates within 1e-3 * max(1, |s|) of float64; the selection
    bit-exact (order included) against the oracle's Top-K of the candidate
    set on the GPU's own scores; equal as a set to the float64 selection where
    the K-th / (K+1)-th float64 scores differ by more than 1e-3; the output
    within 2e-2 of the float64 softmax over the GPU's selection."""
    out_t = atk.sparse_attn_rerank(q, K, V, cand, window, k_sel)
    out, sel, scd = atk.sparse_attn_rerank(q, K, V, cand, window, k_sel, return_sel=True, return_scores=True)
    assert torch.equal(out_t, out), "the output-only call differs from the dumping call"
    bsz, hq, d = q.shape
    g = hq // K.shape[1]
    length = K.shape[2]
    scale = float(np.float32(1.0 / math.sqrt(d)))
    cand_h = cand.cpu().numpy()
    sel_h = sel.cpu().numpy()
    out_h = out.float().cpu().numpy()
    q_h = bits16(q)
    todo = heads or [(i, h) for i in range(bsz) for h in range(hq)]

    def one(ih):
        i, h = ih
        kb = bits16(K[i:i + 1, h // g:h // g + 1])
        vb = bits16(V[i, h // g])
        c = oracle.rerank_candidates(cand_h[i, h], window, length)
        sc = oracle.decode_scores(q_h[i:i + 1, h:h + 1], kb, scale)[0, 0]
        gs = scd[i, h].cpu().numpy()
        assert not np.isnan(gs[c]).any(), (i, h)
        assert np.all(np.abs(gs[c] - sc[c]) <= 1e-3 * np.maximum(1.0, np.abs(sc[c]))), (i, h)
        kk = min(k_sel, len(c))
        got = sel_h[i, h]
        assert (got[kk:] == -1).all()
        got = got[:kk]
        # the oracle's Top-K of the set on the GPU's own scores: bit-exact
        own = np.full(len(gs), -np.inf)
        own[c] = gs[c]
        _, ref_own, _ = oracle.rerank_decode(None, None, vb[None, None], scale, cand_h[i:i + 1, h:h + 1], window,
                                             k_sel, scores=own[None, None])
        np.testing.assert_array_equal(got, ref_own[0, 0, :kk], err_msg="head %d,%d" % (i, h))
        cs = np.sort(sc[c])[::-1]
        if kk < len(c) and cs[kk - 1] - cs[kk] > 1e-3:
            _, ref_sel, _ = oracle.rerank_decode(None, None, vb[None, None], scale, cand_h[i:i + 1, h:h + 1], window,
                                                 k_sel, scores=sc[None, None])
            assert set(got.tolist()) == set(ref_sel[0, 0, :kk].tolist()), (i, h)
        ref = oracle.softmax_v_subset(sc, got, oracle.bf16_bits_to_f64(vb))
        assert np.abs(out_h[i, h] - ref).max() <= 2e-2, (i, h)

    with host_pool() as pool:
        list(pool.map(one, todo))


def _rerank_inputs(bsz, hq, hkv, length, ncand, seed, gpu):
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn((bsz, hq, 128), generator=g).to(torch.bfloat16).to(gpu)
    K = torch.randn((bsz, hkv, length, 128), generator=g).to(torch.bfloat16).to(gpu)
    V = torch.randn((bsz, hkv, length, 128), generator=g).to(torch.bfloat16).to(gpu)
    cand = torch.randint(-5, length + 5, (bsz, hq, ncand), generator=g, dtype=torch.int32)
    cand[:, :, ncand // 2:ncand // 2 + ncand // 8] = cand[:, :, :ncand // 8]  # repeats
    return q, K, V, cand.to(gpu)


@pytest.mark.parametrize("hq,hkv,length,ncand,window,k_sel", [(8, 2, 3000, 600, 37, 64), (4, 4, 5000, 1000, 128, 200),
                                                              (6, 3, 777, 40, 5, 64), (4, 1, 20000, 8000, 192, 512),
                                                              (2, 2, 300, 1, 300, 17)])
def test_rerank_small(gpu, hq, hkv, length, ncand, window, k_sel):
    q, K, V, cand = _rerank_inputs(2, hq, hkv, length, ncand, length + ncand, gpu)
    _rerank_check(q, K, V, cand, window, k_sel)


def test_rerank_whole_cache_matches_exact_decode(gpu):
    q, K, V, cand = _rerank_inputs(1, 4, 2, 2000, 8, 3, gpu)
    empty = cand[:, :, :0].contiguous()
    out, sel = atk.sparse_attn_rerank(q, K, V, empty, 2000, 64, return_sel=True)
    out2, sel2 = atk.sparse_attn_decode(q, K, V, 64, 1, 64, return_sel=True)
    np.testing.assert_array_equal(np.sort(sel.cpu().numpy(), axis=2), np.sort(sel2.cpu().numpy(), axis=2))
    assert (out.float() - out2.float()).abs().max().item() <= 1e-2


@pytest.mark.timeout(900)
def test_rerank_gqa128k_shape_all_heads(gpu):
    """The long-context shape: 4 retrieved supports of 512 keys per head plus
    a 512-key window, Top-512, at B4 Hq32 Hkv8 L131072, every query head."""
    c = workloads.DECODE["gqa-128k"]
    q, K, V, _ = workloads.decode_gqa(c["bsz"], c["hq"], c["hkv"], c["ctx"], c["d"], 0.01, 3.0, seed=0, device=gpu)
    g = torch.Generator(device="cpu").manual_seed(7)
    cand = torch.randint(0, c["ctx"], (c["bsz"], c["hq"], 4 * 512), generator=g, dtype=torch.int32).to(gpu)
    _rerank_check(q, K, V, cand, 512, 512)


# ------------------------------------------------------ HIP graph replay ----

def test_graph_replay_matches_eager(gpu):
    """Library calls captured in one HIP graph (exact, bucketed with and
    without the final stage, fp32 and bf16, and a decode) replayed three
    times; between replays the inputs are rewritten eagerly, and every replay
    must equal an eager call on the same inputs."""
    g = torch.Generator(device="cpu").manual_seed(5)
    xf = torch.randn((3, 70001), generator=g).to(gpu)
    xb = torch.randn((200, 4096), generator=g).to(torch.bfloat16).to(gpu)
    q = torch.randn((2, 8, 128), generator=g).to(torch.bfloat16).to(gpu)
    K = torch.randn((2, 2, 3000, 128), generator=g).to(torch.bfloat16).to(gpu)
    V = torch.randn((2, 2, 3000, 128), generator=g).to(torch.bfloat16).to(gpu)

    def step():
        return [atk.exact(xf, 100), atk.bucketed(xf, 100, 512, 1, True), atk.exact(xb, 64),
                atk.bucketed(xb, 64, 64, 1, False), atk.bucketed(xb, 64, 128, 2, True),
                atk.sparse_attn_decode(q, K, V, 64, 16, 8, return_sel=True)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = step()
    for rep in range(3):
        for t in (xf, xb, q, K, V):
            t.copy_(torch.randn(t.shape, generator=g).to(t.dtype))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = step()
        for i, (a, b) in enumerate(zip(captured, eager)):
            for ta, tb in zip(a, b):
                assert torch.equal(ta, tb), (rep, i)
