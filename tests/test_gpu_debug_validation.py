"""Device-side contract validation (PKV_DEBUG=1), through the C ABI.

With PKV_DEBUG=1 every call first validates what the host cannot see -- page ids the
call addresses in [0, num_pages), lengths within their bounds, consistent prefix sums,
no two appended rows in one slot, valid copy pairs -- and a call that breaks the
contract leaves the pool and its outputs untouched and raises bits that
paged_kv_debug_status() reports.  Every bad case here stays inside allocated memory
even if a check were missed: out-of-range page ids still lie inside the pool tensor
(num_pages is passed smaller than the tensor), and table rows are wide enough for
every length used."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

HKV, HQ, D, P = 2, 8, 64, 16
N_ALLOC, N_PAGES, WIDTH = 40, 32, 8     # ids 32..39 are "outside" the pool yet allocated
NAN16 = 0x7FC1


@pytest.fixture
def debug(gpu_lib, monkeypatch):
    monkeypatch.setenv("PKV_DEBUG", "1")
    gpu_lib.paged_kv_debug_status(True)   # start clean
    yield gpu_lib
    gpu_lib.paged_kv_debug_status(True)


class Batch:
    def __init__(self, B, lens, tables, seed=0):
        g = torch.Generator().manual_seed(seed)
        self.B = B
        self.dev = "cuda"
        self.pool = (torch.randn((N_ALLOC, 2, HKV, P, D), generator=g) * 0.5).to(torch.bfloat16).to(self.dev)
        self.lens = torch.tensor(lens, dtype=torch.int32, device=self.dev)
        t = np.full((len(lens), WIDTH), -1, np.int32)
        for s, row in enumerate(tables):
            t[s, :len(row)] = row
        self.bt = torch.from_numpy(t).to(self.dev)
        self.cache = B.PkvCache(self.pool.data_ptr(), N_PAGES, P, HKV, D, B.PKV_BF16, None, None, None, None)
        self.q = torch.randn((len(lens), HQ, D), generator=g).to(torch.bfloat16).to(self.dev)

    def seqs(self, max_len=None, window=0):
        return self.B.make_seqs(self.bt, self.lens, int(self.lens.max()) if max_len is None else max_len, window)

    def decode(self, seqs, out):
        B = self.B
        ws = B.paged_attn_decode_workspace_size(self.cache, seqs, B.PKV_BF16, HQ, 0)
        w = torch.empty(max(ws, 1), dtype=torch.uint8, device=self.dev)
        B.paged_attn_decode(self.cache, seqs, self.q, B.PKV_BF16, HQ, 0.125, 0, out, None, w, ws)

    def pool_bytes(self):
        torch.cuda.synchronize()
        return self.pool.view(torch.int16).clone()


LENS = [20, 33, 5]
TABLES = [[3, 7], [11, 0, 25], [30]]


def _out():
    return torch.full((len(LENS), HQ, D), NAN16, dtype=torch.int16, device="cuda")


def test_clean_calls_raise_nothing_and_compute(debug, monkeypatch):
    b = Batch(debug, LENS, TABLES)
    out_dbg = _out()
    b.decode(b.seqs(), out_dbg.view(torch.bfloat16))
    assert debug.paged_kv_debug_status(True) == 0
    monkeypatch.delenv("PKV_DEBUG")
    out = _out()
    b.decode(b.seqs(), out.view(torch.bfloat16))
    torch.cuda.synchronize()
    assert torch.equal(out, out_dbg)
    assert torch.isfinite(out.view(torch.bfloat16).float()).all()


def test_page_id_outside_the_pool_leaves_outputs_untouched(debug):
    b = Batch(debug, LENS, [[3, 7], [11, 35, 25], [30]])   # 35 >= num_pages, inside the tensor
    out = _out()
    b.decode(b.seqs(), out.view(torch.bfloat16))
    assert debug.paged_kv_debug_status(True) == debug.PKV_DEBUG_PAGE_RANGE
    assert (out == NAN16).all()


def test_append_to_a_page_outside_the_pool_leaves_the_pool_untouched(debug):
    b = Batch(debug, LENS, [[3, 37], [11, 0, 25], [30]])   # seq 0 appends position 19: page 37
    before = b.pool_bytes()
    k = torch.ones((3, HKV, D), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 1, 2, 3], dtype=torch.int32, device="cuda")
    debug.kv_append(b.cache, b.seqs(), k, k, cu, 3)
    assert debug.paged_kv_debug_status(True) == debug.PKV_DEBUG_PAGE_RANGE
    assert torch.equal(b.pool_bytes(), before)


def test_length_past_max_context_len(debug):
    b = Batch(debug, [20, 60, 5], [[3, 7], [11, 0, 25, 4], [30]])
    out = _out()
    b.decode(b.seqs(max_len=40), out.view(torch.bfloat16))
    assert debug.paged_kv_debug_status(True) == debug.PKV_DEBUG_LENGTH
    assert (out == NAN16).all()


def test_two_rows_appending_to_one_slot(debug):
    # both sequences hold 20 tokens and share their second page: both append slot 3 of page 7
    b = Batch(debug, [20, 20], [[3, 7], [11, 7]])
    before = b.pool_bytes()
    k = torch.ones((2, HKV, D), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda")
    debug.kv_append(b.cache, b.seqs(), k, k, cu, 2)
    assert debug.paged_kv_debug_status(True) == debug.PKV_DEBUG_DUP_SLOT
    assert torch.equal(b.pool_bytes(), before)
    # the same pages, different slots: allowed (a shared page, as a common prefix is)
    b2 = Batch(debug, [20, 21], [[3, 7], [11, 7]])
    debug.kv_append(b2.cache, b2.seqs(), k, k, cu, 2)
    assert debug.paged_kv_debug_status(True) == 0


def test_decreasing_prefix_sums(debug):
    b = Batch(debug, LENS, TABLES)
    before = b.pool_bytes()
    k = torch.ones((3, HKV, D), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 2, 1, 3], dtype=torch.int32, device="cuda")
    debug.kv_append(b.cache, b.seqs(), k, k, cu, 3)
    assert debug.paged_kv_debug_status(True) & debug.PKV_DEBUG_CU
    assert torch.equal(b.pool_bytes(), before)


def test_prefill_chunk_longer_than_max_q_len(debug):
    b = Batch(debug, LENS, TABLES)
    B = debug
    cu = torch.tensor([0, 4, 6, 7], dtype=torch.int32, device="cuda")   # chunk of 4 > max_q_len 2
    q = torch.randn((7, HQ, D), device="cuda").to(torch.bfloat16)
    out = torch.full((7, HQ, D), NAN16, dtype=torch.int16, device="cuda")
    seqs = b.seqs()
    ws = B.paged_attn_prefill_workspace_size(b.cache, seqs, B.PKV_BF16, HQ, 7, 2)
    w = torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda")
    B.paged_attn_prefill_chunk(b.cache, seqs, q, B.PKV_BF16, cu, 7, 2, HQ, 0.125, out.view(torch.bfloat16),
                               None, w, ws)
    assert B.paged_kv_debug_status(True) == B.PKV_DEBUG_LENGTH
    assert (out == NAN16).all()


def test_copy_pairs(debug):
    b = Batch(debug, LENS, TABLES)
    before = b.pool_bytes()
    t = lambda x: torch.tensor(x, dtype=torch.int32, device="cuda")
    debug.kv_copy_pages(b.cache, t([1, 2]), t([2, 5]), 2)        # page 2 is a source and a destination
    assert debug.paged_kv_debug_status(True) == debug.PKV_DEBUG_COPY_PAIRS
    debug.kv_copy_pages(b.cache, t([1]), t([36]), 1)             # 36 >= num_pages
    assert debug.paged_kv_debug_status(True) == debug.PKV_DEBUG_PAGE_RANGE
    assert torch.equal(b.pool_bytes(), before)
    debug.kv_copy_pages(b.cache, t([1]), t([5]), 1)              # a valid copy goes through
    assert debug.paged_kv_debug_status(True) == 0
    torch.cuda.synchronize()
    assert torch.equal(b.pool[5].view(torch.int16), b.pool[1].view(torch.int16))


def test_released_pages_before_a_window_are_not_flagged(debug):
    """Under a limited attention window the entries of pages before the window may be
    released (-1): the kernels never read them and validation does not flag them."""
    lens = [90, 100]
    tables = [[-1, -1, -1, 4, 5, 6], [-1, -1, -1, 8, 9, 10, 12]]
    b = Batch(debug, lens, tables)
    out = _out()[:2]
    b.decode(b.seqs(window=20), out.view(torch.bfloat16))      # first key 70 / 80: block 64 -> page 4
    assert debug.paged_kv_debug_status(True) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(out.view(torch.bfloat16).float()).all()


def test_status_is_sticky_until_cleared_and_calls_recover(debug):
    bad = Batch(debug, LENS, [[3, 7], [11, 35, 25], [30]])
    good = Batch(debug, LENS, TABLES)
    out = _out()
    bad.decode(bad.seqs(), out.view(torch.bfloat16))
    good.decode(good.seqs(), out.view(torch.bfloat16))        # a later valid call runs normally
    assert debug.paged_kv_debug_status(False) == debug.PKV_DEBUG_PAGE_RANGE
    assert debug.paged_kv_debug_status(True) == debug.PKV_DEBUG_PAGE_RANGE
    assert debug.paged_kv_debug_status(True) == 0
    assert torch.isfinite(out.view(torch.bfloat16).float()).all()
