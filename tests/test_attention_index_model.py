"""Host-side models of the attention kernels' index arithmetic (no GPU).

1. The dS scratch of the backward: a model of the dK/dV kernel's dS stores
   and of the dQ kernel's dS DMA and reads, over sequence lengths 1..2048, all
   work splits (OWN 1, 2, 4; tile pairs on and off), causal and full.  Every
   store and DMA source must stay inside the [s_pad, s_pad] matrix of one
   (sequence, head), and every dS entry the dQ kernel uses must have been
   written by the dK/dV kernel.
2. The LDS addressing of the staged blocks: with the chunk swizzle, a lane's
   row-fragment addresses are one base XOR (kk << 5), and its transposed
   fragment addresses one base XOR a lane-independent mask plus row offsets;
   checked for every lane against the plain swizzled address.
3. The workgroup permutation: a bijection of the launch grid, and with a
   multiple of 8 (sequence, head) pairs each XCD (workgroup index mod 8)
   serves whole heads."""
import itertools

import numpy as np
import pytest

RB, NW = 32, 4


def acc_row(r, hl):
    return (r >> 2) * 8 + hl * 4 + (r & 3)


def s_pad_of(s):
    return (s + 63) // 64 * 64


def ds_model(s, own_n, pair, causal):
    sp_ = s_pad_of(s)
    split = NW // own_n
    ntile = (s + 32 * own_n - 1) // (32 * own_n)
    wgs = (ntile + 1) // 2 if pair else ntile
    written = np.zeros((sp_, sp_), bool)
    lanes = np.arange(64)
    l32, hl, odd = lanes & 31, lanes >> 5, lanes & 1
    # dK/dV kernel: a lane stores, per even r, the word of row
    # acc_row(r, hl) + odd at the even key column kj & ~1
    for bx in range(wgs):
        for rep in range(1 + pair):
            tile = bx if rep == 0 else ntile - 1 - bx
            if rep == 1 and tile <= bx:
                break
            k0 = tile * 32 * own_n
            nqb = (s + RB - 1) // RB
            qb0 = k0 // RB if causal else 0
            nst = (nqb - qb0 + split - 1) // split
            for wave in range(NW):
                own, sp = wave % own_n, wave // own_n
                kw0 = k0 + own * 32
                if not kw0 < s:
                    continue
                kj = kw0 + l32
                for st in range(nst):
                    qb = qb0 + st * split + sp
                    qs0 = qb * RB
                    if qb >= nqb or (causal and qs0 + 31 < kw0):
                        continue
                    for r in range(0, 16, 2):
                        rows = qs0 + acc_row(r, hl) + odd
                        cols = kj & ~1
                        assert rows.min() >= 0 and rows.max() < sp_ and cols.max() + 1 < sp_
                        written[rows, cols] = True
                        written[rows, cols + 1] = True
    # dQ kernel: DMA of 16-row halves of each staged 32 x 32 dS block, then
    # the reads of the blocks of each wave's causal range
    for bx in range(wgs):
        for rep in range(1 + pair):
            tile = ntile - 1 - bx if rep == 0 else bx
            if rep == 1 and tile >= ntile - 1 - bx:
                break
            q0 = tile * 32 * own_n
            kend = min(s, q0 + 32 * own_n) if causal else s
            nkb = (kend + RB - 1) // RB
            nst = (nkb + split - 1) // split
            for st in range(nst):
                for bi in range(own_n * split):
                    o, spb = bi // split, bi % split
                    for u in range(2):
                        row = u * 16 + (lanes >> 2)
                        q = np.minimum(q0 + o * 32 + row, s - 1)
                        kb = min(st * split + spb, nkb - 1)
                        col = kb * RB + ((lanes & 3) ^ ((row >> 2) & 3)) * 8
                        assert q.min() >= 0 and q.max() < sp_ and col.min() >= 0 and col.max() + 8 <= sp_
                for wave in range(NW):
                    own, sp = wave % own_n, wave // own_n
                    qw0 = q0 + own * 32
                    kb = st * split + sp
                    k0 = kb * RB
                    if kb >= nkb or (causal and k0 > qw0 + 31):
                        continue
                    rows = np.arange(qw0, min(qw0 + 32, s))  # rows past s are never stored
                    assert written[np.ix_(rows, np.arange(k0, k0 + 32))].all(), (s, own_n, pair, causal, k0)


SEQS = list(range(1, 70)) + [95, 96, 97, 127, 128, 129, 255, 256, 257, 511, 512, 1000, 1024, 1030]


@pytest.mark.parametrize("own_n,pair,causal", list(itertools.product((1, 2, 4), (0, 1), (0, 1))))
def test_ds_scratch_indexing(own_n, pair, causal):
    for s in SEQS:
        ds_model(s, own_n, pair, causal)


def test_ds_scratch_indexing_longest_sequence():
    for own_n, pair in ((1, 1), (1, 0), (2, 0)):
        ds_model(2048, own_n, pair, 1)


def swz(d, k):
    if d == 64:
        a = (k >> 1) & 7
        return a ^ ((a & 1) << 2)
    return ((k & 3) << 2) | ((k >> 2) & 3)


def frag_addr(d, row, kk, hl):
    return row * d * 2 + (((kk * 2 + hl) ^ swz(d, row)) << 4)


def frag_t_addr(d, lane, col, k_lo, hl, r):
    i = lane & 15
    n = (col - i) + 4 * (i & 3)
    k = k_lo + r * 8 + hl * 4 + (i >> 2)
    return k * d * 2 + ((((n >> 3) ^ swz(d, k)) << 3) + (n & 7)) * 2


def tmask(d, t, r):
    return ((t << 6) ^ (r << 5)) if d == 128 else (((t ^ r) & 1) << 6)


@pytest.mark.parametrize("d", [64, 128])
def test_lds_fragment_address_identities(d):
    for lane in range(64):
        l32, hl = lane & 31, lane >> 5
        base = frag_addr(d, l32, 0, hl)
        for kk in range(d // 16):
            assert frag_addr(d, l32, kk, hl) == base ^ (kk << 5)
        base_t = frag_t_addr(d, lane, l32, 0, hl, 0)
        for t in range(d // 32):
            for hh in range(2):
                for r in range(2):
                    want = frag_t_addr(d, lane, t * 32 + l32, hh * 16, hl, r)
                    assert want == (base_t ^ tmask(d, t, r)) + (hh * 16 + r * 8) * d * 2


@pytest.mark.parametrize("tiles,nbh", [(32, 8), (16, 16), (64, 8), (37, 3), (1, 1), (5, 24)])
def test_workgroup_permutation(tiles, nbh):
    seen = set()
    xcd_heads = {}
    for by in range(nbh):
        for bx in range(tiles):
            lin = by * tiles + bx
            bh, x = lin % nbh, lin // nbh
            assert 0 <= bh < nbh and 0 <= x < tiles
            seen.add((x, bh))
            xcd_heads.setdefault(lin % 8, set()).add(bh)
    assert len(seen) == tiles * nbh
    if nbh % 8 == 0:
        for xcd, heads in xcd_heads.items():
            assert all(h % 8 == xcd for h in heads)
