"""Host emulation of the KV-cache kernels' page arithmetic (no GPU).

The KV-cache forward and decode kernels find the cache row of token j of a
sequence of length L through a block table (page bt[j >> shift], slot
j & (2^shift - 1)).  These tests replay, on random block tables and
lengths, the index arithmetic each kernel path uses to fetch a tile, and
check the invariant that makes the kernels safe: every row fetched is a
token j < L of the right page and slot, or reads as zero through a buffer
bound; no path touches a slot that holds no token (the GPU tests fill those
with NaN, so a stray read would show there too).  The arithmetic follows
the kernels' source; the page sizes are those the host check admits
(powers of two >= 16).
"""
import numpy as np
import pytest

BN_FWD = 64          # keys per forward tile
BNK_DEC = 32         # keys per decode block
WINDOW = 64          # block-table entries one wave holds (one per lane)


class Window:
    """The wave's window of block-table entries: entry `base + lane`."""

    def __init__(self, bt, last_page_no):
        self.bt, self.last, self.base, self.pages = bt, last_page_no, -1, None

    def cover(self, first, last):
        if self.base < 0 or first < self.base or last >= self.base + WINDOW:
            self.base = first
            lanes = np.arange(WINDOW)
            self.pages = self.bt[np.minimum(first + lanes, self.last)]
        assert last - self.base < WINDOW and first >= self.base

    def page(self, page_no):
        k = np.asarray(page_no) - self.base
        assert np.all((k >= 0) & (k < WINDOW))
        return self.pages[k]


def case(seed, page, L):
    rng = np.random.default_rng(seed)
    npages = (L + page - 1) // page
    bt = rng.permutation(npages + 7)[:max(npages, 1)]
    return bt, (L - 1) // page if L > 0 else 0


def check_rows(tokens, pages, slots, valid, bt, page, L):
    """Each fetched row: a token < L of its page and slot (valid), or a row
    past the buffer bound, which reads as zero and stands for a key >= L
    (masked by the kernel)."""
    tokens, pages, slots, valid = map(np.asarray, (tokens, pages, slots, valid))
    assert np.all(tokens[valid] < L)
    assert np.all(pages[valid] == bt[tokens[valid] // page])
    assert np.all(slots[valid] == tokens[valid] % page)
    assert np.all((slots[valid] >= 0) & (slots[valid] < page))
    assert np.all(tokens[~valid] >= L)


@pytest.mark.parametrize("page", [16, 32])
def test_forward_small_pages(page):
    """Pages below 64 tokens (register staging): thread row lrow + 32 u of
    the tile at j0 reads token min(j0 + row, L - 1) through the window."""
    shift = page.bit_length() - 1
    for seed in range(40):
        L = int(np.random.default_rng(seed).integers(1, 5000))
        bt, last = case(seed, page, L)
        win = Window(bt, last)
        for j0 in range(0, L, BN_FWD):
            win.cover(j0 >> shift, min(j0 + BN_FWD - 1, L - 1) >> shift)
            rows = np.arange(BN_FWD)
            j = np.minimum(j0 + rows, L - 1)
            check_rows(j, win.page(j >> shift), j & (page - 1), np.ones_like(j, bool), bt, page, L)


@pytest.mark.parametrize("page", [64, 128, 256, 1024])
def test_forward_large_pages(page):
    """Pages of >= 64 tokens (LDS DMA): the tile at j0 lies in page
    j0 >> shift; row r reads slot j0 - first + r through a buffer over the
    page's min(L - first, page) rows holding tokens (else zero)."""
    shift = page.bit_length() - 1
    for seed in range(40):
        L = int(np.random.default_rng(100 + seed).integers(1, 20000))
        bt, last = case(seed, page, L)
        win = Window(bt, last)
        for j0 in range(0, L, BN_FWD):
            pn = j0 >> shift
            assert (j0 + BN_FWD - 1) >> shift == pn        # one page per tile
            win.cover(pn, pn)
            first = pn << shift
            nrows = min(L - first, page)
            slot = j0 - first + np.arange(BN_FWD)
            valid = slot < nrows
            check_rows(first + slot, np.full(BN_FWD, win.page(pn)), slot, valid, bt, page, L)


@pytest.mark.parametrize("page", [16, 64, 256])
@pytest.mark.parametrize("rpi", [4, 8])          # rows per 1 KB DMA block: d = 128, 64
def test_decode_blocks(page, rpi):
    """Decode: split s covers keys [s c, (s+1) c) with c a multiple of 32;
    block j0 = kbeg + 32 t issues one DMA per rpi rows, each through the
    page of its first (clamped) row over that page's rows holding tokens."""
    shift = page.bit_length() - 1
    for seed in range(30):
        rng = np.random.default_rng(200 + seed)
        L = int(rng.integers(1, 20000))
        nsplit = int(rng.integers(1, 9))
        chunk = ((L + nsplit - 1) // nsplit + 31) // 32 * 32
        bt, last = case(seed, page, L)
        for kbeg in range(0, L, chunk):
            kend = min(L, kbeg + chunk)
            win = Window(bt, last)
            for j0 in range(kbeg, kend, BNK_DEC):
                win.cover(j0 >> shift, min(j0 + BNK_DEC - 1, L - 1) >> shift)
                for u in range(BNK_DEC // rpi):
                    pn = min(j0 + rpi * u, L - 1) >> shift
                    first = pn << shift
                    nrows = max(0, min(L - first, page))
                    slot = j0 - first + rpi * u + np.arange(rpi)
                    valid = slot < nrows
                    check_rows(first + slot, np.full(rpi, win.page(pn)), slot, valid, bt, page, L)
