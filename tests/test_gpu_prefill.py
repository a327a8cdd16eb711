"""GPU parity of the prefill page fill paged_kv_prefill.

Bar: bit-exact.  Every row is the append of one token, so the pool and the
rotated q must equal the oracle's prefill (token-by-token appends) and the
GPU's own paged_kv_append called once per token, bit for bit.  Cases: fresh
prompts and chunked prompts that start mid-page, several sequences in one
call, no q, positions outside the RoPE table, bad page ids, and 64 prompts
of 2,048 tokens (the decode benchmark's geometry) at full size.
"""
import numpy as np
import pytest

import oracle
from oracle import PoolView
import paged_kv_cache_172_amd as pkv
from paged_kv_cache_172_amd import workload as wl
from paged_kv_cache_172_amd.runner import HALF_PAGE, PAGE_ELEMS

from tests.gpu_util import say, to_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU (run with -m 'not gpu' on CPU)"
    pkv.load()
    return torch


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.fixture(scope="module")
def rope(orc):
    return orc.rope_table(500000.0, 2048)


def make_case(seed, starts, counts, extra_pages=5):
    """Seeded tables (a shuffled pool), packed rows and a NaN-poisoned pool."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B = len(starts)
    need = [-(-(a + c) // 16) for a, c in zip(starts, counts)]
    num_pages = sum(need) + extra_pages
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.full((B, 128), -1, np.int32)
    cur = 0
    for s, c in enumerate(need):
        bt[s, :c] = perm[cur:cur + c]
        cur += c
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(counts)
    T = int(cu[-1])
    q = wl.f32_to_bf16_bits(rng.standard_normal((T, 2048), dtype=np.float32))
    k = wl.f32_to_bf16_bits(rng.standard_normal((T, 512), dtype=np.float32))
    v = wl.f32_to_bf16_bits(rng.standard_normal((T, 512), dtype=np.float32))
    pages = np.full((num_pages, 2, 8, 16, 64), wl.BF16_NAN, np.uint16)
    return dict(bt=bt, start=np.asarray(starts, np.int32), cu=cu, q=q, k=k, v=v, pages=pages)


class Dev:
    """Device copies of one case and the calls on them."""

    def __init__(self, torch, c, rope):
        d = torch.device("cuda")
        u = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(d)
        i = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(d)
        self.torch = torch
        self.pages = u(c["pages"])
        self.P = c["pages"].shape[0]
        self.bt, self.start, self.cu = i(c["bt"]), i(c["start"]), i(c["cu"])
        self.q, self.k, self.v = u(c["q"]), u(c["k"]), u(c["v"])
        self.cos = torch.from_numpy(rope[0]).to(d)
        self.sin = torch.from_numpy(rope[1]).to(d)
        self.max_pos = rope[0].shape[0]
        base = self.pages.data_ptr()
        self.pool = pkv.make_pool(base, base + HALF_PAGE * 2, self.P, PAGE_ELEMS, 1024, 64)
        self.B = c["bt"].shape[0]
        self.T = int(c["cu"][-1])

    def prefill(self, with_q=True):
        pkv.paged_kv_prefill(self.pool, self.bt, 128, self.start, self.cu, self.B, self.T,
                             self.q if with_q else None, 2048, self.k, 512, self.v, 512,
                             self.cos, self.sin, self.max_pos)
        self.torch.cuda.synchronize()

    def appends(self, c):
        """paged_kv_append once per row, in row order (one sequence each)."""
        torch = self.torch
        for s in range(self.B):
            for row in range(int(c["cu"][s]), int(c["cu"][s + 1])):
                n = torch.tensor([int(c["start"][s]) + row - int(c["cu"][s]) + 1],
                                 dtype=torch.int32, device=self.pages.device)
                pkv.paged_kv_append(self.pool, self.bt[s:s + 1], 128, n, 1, self.q[row:row + 1],
                                    2048, self.k[row:row + 1], 512, self.v[row:row + 1], 512,
                                    self.cos, self.sin, self.max_pos)
        torch.cuda.synchronize()


def oracle_prefill(orc, c, rope, with_q=True):
    pages = c["pages"].copy()
    q = c["q"].copy() if with_q else None
    orc.prefill(PoolView.from_pages(pages), c["bt"], c["start"], c["cu"], q, c["k"], c["v"],
                rope[0], rope[1])
    return pages, q


CASES = {
    "fresh_prompts": ([0, 0, 0], [37, 16, 1]),
    "chunked_mid_page": ([5, 17, 2040, 100], [30, 15, 8, 64]),
    "many_seqs": (list(range(0, 400, 7))[:48], [int(x) for x in
                                                np.random.default_rng(700).integers(1, 80, 48)]),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("with_q", [True, False], ids=["q", "no_q"])
def test_prefill_matches_oracle(torch_gpu, orc, rope, name, with_q):
    starts, counts = CASES[name]
    c = make_case(710, starts, counts)
    dev = Dev(torch_gpu, c, rope)
    dev.prefill(with_q)
    ref_pages, ref_q = oracle_prefill(orc, c, rope, with_q)
    assert np.array_equal(to_u16(dev.pages).reshape(ref_pages.shape), ref_pages)
    if with_q:
        assert np.array_equal(to_u16(dev.q).reshape(ref_q.shape), ref_q)
    else:
        assert np.array_equal(to_u16(dev.q).reshape(c["q"].shape), c["q"])


def test_prefill_equals_gpu_appends(torch_gpu, rope):
    c = make_case(711, [0, 9, 31], [40, 23, 2])
    a, b = Dev(torch_gpu, c, rope), Dev(torch_gpu, c, rope)
    a.prefill()
    b.appends(c)
    assert torch_gpu.equal(a.pages, b.pages) and torch_gpu.equal(a.q, b.q)


def _rows(c, picks):
    """A case with only the rows picks[s] (a count from the start) of each
    sequence, same data, same tables."""
    cu = c["cu"]
    sel = np.concatenate([np.arange(cu[s], cu[s] + n) for s, n in enumerate(picks)])
    out = dict(c)
    out["cu"] = np.concatenate([[0], np.cumsum(picks)]).astype(np.int32)
    for key in ("q", "k", "v"):
        out[key] = np.ascontiguousarray(c[key][sel])
    return out


def test_prefill_guards(torch_gpu, orc, rope):
    """A row past the RoPE table is skipped (q not rotated, nothing written);
    a bad table entry skips only its K/V write (q is still rotated); other
    rows are unaffected."""
    c = make_case(712, [0, 0, 60], [20, 20, 10])
    spare = int(np.setdiff1d(np.arange(c["pages"].shape[0]), c["bt"])[0])   # an unused page
    c["bt"][1, 1] = c["pages"].shape[0] + 9         # rows 16..19 of sequence 1: bad page
    short = (rope[0][:64].copy(), rope[1][:64].copy())   # sequence 2 rows 4..9 (pos 64..69)
    dev = Dev(torch_gpu, c, short)
    dev.prefill()
    got_pages = to_u16(dev.pages).reshape(c["pages"].shape)
    got_q = to_u16(dev.q).reshape(c["q"].shape)
    cu = c["cu"]
    # pool: the oracle over the rows that write (all of sequence 0, rows
    # 0..15 of sequence 1, rows 0..3 of sequence 2)
    ref_pages, ref_q = oracle_prefill(orc, _rows(c, [20, 16, 4]), short)
    assert np.array_equal(got_pages, ref_pages)
    # q: rows with a position inside the table are rotated, bad page or not
    # (the oracle with the bad entry pointed at an unused page)
    fixed = dict(c)
    fixed["bt"] = c["bt"].copy()
    fixed["bt"][1, 1] = spare
    _, q_rot = oracle_prefill(orc, _rows(fixed, [20, 20, 4]), short)
    want = c["q"].copy()
    want[cu[0]:cu[0] + 20] = q_rot[0:20]
    want[cu[1]:cu[1] + 20] = q_rot[20:40]
    want[cu[2]:cu[2] + 4] = q_rot[40:44]
    assert np.array_equal(got_q, want)


def test_prefill_full_size(torch_gpu, orc, rope):
    """64 prompts of 2,048 tokens (rows drawn on the GPU, seeded) into a
    shuffled 8,256-page pool, with q, in one launch: all 64 prompts, every
    row's pages and q, against the oracle's prefill bit for bit (the whole
    pool, so the 64 pages no table names stay untouched too)."""
    torch = torch_gpu
    B, n = 64, 2048
    rng = np.random.Generator(np.random.PCG64(713))
    num_pages = B * n // 16 + 64
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.full((B, 128), -1, np.int32)
    bt[:, :] = perm[:B * 128].reshape(B, 128)
    cu = (np.arange(B + 1) * n).astype(np.int32)
    start = np.zeros(B, np.int32)
    g = torch.Generator(device="cuda").manual_seed(713)
    draw = lambda cols: torch.randn((B * n, cols), generator=g, device="cuda").to(
        torch.bfloat16).view(torch.int16)
    c = dict(bt=bt, start=start, cu=cu, q=np.zeros((1, 2048), np.uint16),
             k=np.zeros((1, 512), np.uint16), v=np.zeros((1, 512), np.uint16),
             pages=np.zeros((1, 2, 8, 16, 64), np.uint16))
    dev = Dev(torch, c, rope)
    dev.q, dev.k, dev.v = draw(2048), draw(512), draw(512)
    dev.pages = torch.full((num_pages, 2, 8, 16, 64), wl.BF16_NAN, dtype=torch.int16,
                           device="cuda")
    base = dev.pages.data_ptr()
    dev.P = num_pages
    dev.pool = pkv.make_pool(base, base + HALF_PAGE * 2, num_pages, PAGE_ELEMS, 1024, 64)
    dev.B, dev.T = B, B * n
    whole = dict(bt=bt, start=start, cu=cu, q=to_u16(dev.q).reshape(B * n, 2048),
                 k=to_u16(dev.k).reshape(B * n, 512), v=to_u16(dev.v).reshape(B * n, 512),
                 pages=np.full((num_pages, 2, 8, 16, 64), wl.BF16_NAN, np.uint16))
    say(f"[prefill] full size: {B * n} rows, {num_pages} pages")
    dev.prefill()
    got_pages = to_u16(dev.pages).reshape(num_pages, 2, 8, 16, 64)
    got_q = to_u16(dev.q).reshape(B * n, 2048)
    ref_pages, ref_q = oracle_prefill(orc, whole, rope)
    if not np.array_equal(got_q, ref_q):
        rows = np.nonzero((got_q != ref_q).any(axis=1))[0]
        raise AssertionError(f"rotated q differs on {rows.size} rows, e.g. {rows[:8].tolist()}")
    if not np.array_equal(got_pages, ref_pages):
        bad = np.nonzero((got_pages != ref_pages).reshape(num_pages, -1).any(axis=1))[0]
        raise AssertionError(f"pool differs on {bad.size} pages, e.g. {bad[:8].tolist()}")
    unused = np.setdiff1d(np.arange(num_pages), bt.ravel())
    assert unused.size == 64 and (got_pages[unused] == wl.BF16_NAN).all()
    say(f"[prefill] full size: all {B} prompts ({B * n} rows) bit-exact, pool and q")


def _edge_bf16(rng, shape):
    """BF16 bit patterns aimed at the rounding of the rotation: mostly short
    mantissas (so that products land on or near BF16 half-way points), some
    Gaussian values, and the edges: values near the top of the range,
    subnormals, zeros, infinities and NaN."""
    n = int(np.prod(shape))
    kind = rng.choice(7, size=n, p=[0.62, 0.14, 0.07, 0.06, 0.04, 0.04, 0.03])
    sign = rng.integers(0, 2, n).astype(np.uint16) << 15
    short_m = rng.choice(np.array([0, 1, 2, 3, 64, 65, 127], np.uint16), n)
    mid_e = rng.integers(127 - 20, 127 + 21, n).astype(np.uint16)
    top_e = rng.integers(250, 255, n).astype(np.uint16)
    rand_m = rng.integers(0, 128, n).astype(np.uint16)
    gauss = wl.f32_to_bf16_bits(rng.standard_normal(n, dtype=np.float32))
    out = np.where(kind == 0, sign | (mid_e << 7) | short_m, 0).astype(np.uint16)
    out = np.where(kind == 1, gauss, out)
    out = np.where(kind == 2, sign | (top_e << 7) | rand_m, out)                      # near overflow
    out = np.where(kind == 3, sign | rng.integers(1, 128, n).astype(np.uint16), out)  # subnormal
    out = np.where(kind == 4, sign | (rng.integers(1, 4, n).astype(np.uint16) << 7) | rand_m, out)
    out = np.where(kind == 5, sign, out)                                              # +-0
    special = rng.choice(np.array([0x7F80, 0xFF80, 0x7FC0, 0x7F7F, 0xFF7F], np.uint16), n)
    out = np.where(kind == 6, special, out)
    return out.reshape(shape)


def _edge_table(rng, rows):
    """FP32 cos/sin rows whose products with short BF16 values fall on
    half-way points, just beside them (an s of 2^-30 moves a half-way point
    by far less than an FP32 ulp), or outside the FP32 range."""
    c_set = np.array([1.0, 1.0 + 2.0**-8, 1.0 - 2.0**-9, 0.75, 0.5 + 2.0**-9, 2.0**-20, 0.0,
                      -1.0, 1.0 + 2.0**-7 + 2.0**-30, 2.0**-126, 2.0**100, -(1.0 + 2.0**-8)],
                     np.float64).astype(np.float32)
    s_set = np.array([0.0, 2.0**-30, -2.0**-30, 2.0**-8, -2.0**-8, 2.0**-24, 0.5, 2.0**-100,
                      1e-40, 2.0**-9 * (1 + 2.0**-23), 2.0**90], np.float64).astype(np.float32)
    c = rng.choice(c_set, (rows, 32))
    s = rng.choice(s_set, (rows, 32))
    mix = rng.random((rows, 32)) < 0.15             # some ordinary entries
    c = np.where(mix, rng.uniform(-1, 1, (rows, 32)).astype(np.float32), c)
    s = np.where(mix, rng.uniform(-1, 1, (rows, 32)).astype(np.float32), s)
    return np.ascontiguousarray(c, np.float32), np.ascontiguousarray(s, np.float32)


def _is_nan16(b):
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)


def test_rotation_rounding_edges(torch_gpu, orc, rope):
    """The rotation's single rounding to BF16 at its edges: exact half-way
    points (ties to even), values beside a half-way point by less than an
    FP32 ulp (where rounding first to FP32 would go wrong), overflow to
    infinity, subnormal results, signed zeros, infinities and NaN, through
    paged_kv_prefill and paged_kv_append.  Bar: the oracle's bits wherever
    the oracle's result is a number; NaN where it is NaN (the sign of a NaN
    made by arithmetic is not portable).  Rows mix these with ordinary rows
    and table entries, so that every rounding path of the kernels runs."""
    rng = np.random.Generator(np.random.PCG64(714))
    edge_c, edge_s = _edge_table(rng, 32)
    real = orc.rope_table(500000.0, 1032)
    table = (np.concatenate([edge_c, real[0][1000:1032]]),
             np.concatenate([edge_s, real[1][1000:1032]]))
    starts = [0, 0, 0, 0, 32, 32, 32, 0]          # rows at positions 0..31 use the edge table
    counts = [32] * 8
    c = make_case(715, starts, counts)
    T = int(c["cu"][-1])
    edge_rows = np.concatenate([np.arange(32 * s, 32 * s + 32) for s in (0, 1, 2, 3, 6)])
    c["q"][edge_rows] = _edge_bf16(rng, (len(edge_rows), 2048))
    c["k"][edge_rows] = _edge_bf16(rng, (len(edge_rows), 512))
    c["v"][edge_rows] = _edge_bf16(rng, (len(edge_rows), 512))

    # The inputs hold what the test is about (the oracle and numpy only):
    # exact ties, and values that a rounding through FP32 would get wrong.
    ys = []
    for row in range(T):
        s = int(np.searchsorted(c["cu"], row, side="right") - 1)
        pos = int(c["start"][s]) + row - int(c["cu"][s])
        heads = np.concatenate([c["q"][row].reshape(32, 64), c["k"][row].reshape(8, 64)])
        for h in heads:
            ys.append(orc.rope_rotate_f64(oracle.bf16_to_f64(h), table[0][pos], table[1][pos]))
    y = np.concatenate(ys)
    with np.errstate(all="ignore"):
        exact = orc.bf16_round_array(y)
        y32 = y.astype(np.float32)
        via_f32 = wl.f32_to_bf16_bits(y32)
        num = ~np.isnan(y)
        ties = num & (y32.astype(np.float64) == y) & ((y32.view(np.uint32) & 0xFFFF) == 0x8000)
    hazards = num & (via_f32 != exact)
    say(f"[edges] {y.size} rotated values: {int(ties.sum())} exact ties, "
        f"{int(hazards.sum())} that rounding through FP32 gets wrong, "
        f"{int((~num).sum())} NaN, {int(np.isinf(y).sum())} infinite")
    assert ties.sum() >= 100 and hazards.sum() >= 100

    dev = Dev(torch_gpu, c, table)
    dev.prefill()
    ref_pages, ref_q = oracle_prefill(orc, c, table)
    for name, got, ref in (("pages", to_u16(dev.pages).reshape(ref_pages.shape), ref_pages),
                           ("q", to_u16(dev.q).reshape(ref_q.shape), ref_q)):
        nan = _is_nan16(ref)
        assert np.array_equal(_is_nan16(got), nan), name
        bad = (got != ref) & ~nan
        assert not bad.any(), f"{name}: {int(bad.sum())} values differ, first at {np.argwhere(bad)[0]}"
    one = Dev(torch_gpu, c, table)
    one.appends(c)
    assert torch_gpu.equal(one.pages, dev.pages) and torch_gpu.equal(one.q, dev.q)


def test_prefill_strided_layouts(torch_gpu, orc, rope):
    """Packed QKV rows ([T][3072]: q, then k, then v) and a [slot][head][dim]
    page layout: the fill rotates q in place inside the packed rows, leaves
    k and v as given, and writes the oracle's pool bits through the strides."""
    torch = torch_gpu
    c = make_case(716, [0, 5, 2000], [40, 27, 48])
    ref_pages, ref_q = oracle_prefill(orc, c, rope)
    d = torch.device("cuda")
    T = int(c["cu"][-1])
    P = c["pages"].shape[0]
    # [page][K|V][slot 16][head 8][dim 64], NaN-poisoned like the default case
    inter = torch.from_numpy(np.ascontiguousarray(c["pages"].transpose(0, 1, 3, 2, 4)).view(np.int16)).to(d)
    half = 16 * 8 * 64
    pool = pkv.make_pool(inter.data_ptr(), inter.data_ptr() + 2 * half, P, 2 * half, 64, 512)
    qkv = torch.zeros((T, 3072), dtype=torch.int16, device=d)
    qkv[:, :2048] = torch.from_numpy(c["q"].view(np.int16)).to(d)
    qkv[:, 2048:2560] = torch.from_numpy(c["k"].view(np.int16)).to(d)
    qkv[:, 2560:] = torch.from_numpy(c["v"].view(np.int16)).to(d)
    kv_before = qkv[:, 2048:].clone()
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(d)
    cos, sin = torch.from_numpy(rope[0]).to(d), torch.from_numpy(rope[1]).to(d)
    pkv.paged_kv_prefill(pool, i32(c["bt"]), 128, i32(c["start"]), i32(c["cu"]), len(c["start"]), T,
                         qkv, 3072, qkv[:, 2048:], 3072, qkv[:, 2560:], 3072, cos, sin,
                         rope[0].shape[0])
    torch.cuda.synchronize()
    back = to_u16(inter).reshape(P, 2, 16, 8, 64).transpose(0, 1, 3, 2, 4)
    assert np.array_equal(back, ref_pages), "pool differs from the oracle"
    assert np.array_equal(to_u16(qkv[:, :2048].contiguous()), ref_q), "q differs from the oracle"
    assert torch.equal(qkv[:, 2048:], kv_before), "k and v must be left as given"
