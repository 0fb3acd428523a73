"""Host-side models of the bf16 GEMM kernel's LDS addressing and k loop (no GPU).

1. KC fragment addresses: a k-contiguous operand tile is stored as [rows][BK]
   with 16-byte chunk c of row r at c ^ key(r).  The kernel reads a lane's
   fragments from one base address per operand: substep ks is the base XOR
   (ks << 5), the fragment 32 i rows further down additionally flips address
   bit 6 for odd i when BK = 64, and the slot and row offsets are added as
   immediates.  Checked for every lane, wave, fragment and substep against the
   plain swizzled address.
2. The software-pipelined k loop: the prologue puts every ring slot's tile in
   flight; in the last substep of tile kt each wave waits for its DMA of tile
   kt+1, passes the workgroup barrier, reads tile kt+1's first fragments and
   refills tile kt's slot with tile kt+STAGES.  A model of one wave's program
   (all waves run the same one) checks, for every k-tile count, ring depth and
   full-tile count: each fragment read finds its tile in the slot with the
   DMA completed before an earlier barrier; no DMA overwrites a slot whose old
   tile is still read after the last barrier; every tile is loaded once and
   read once per substep, in order; a tile issued as full is a full k tile."""
import pytest


def kc_key(bk, r):
    return ((r ^ (r >> 3)) & 7) if bk == 64 else ((r >> 2) & 3)


@pytest.mark.parametrize("bk", [32, 64])
@pytest.mark.parametrize("rows,waves", [(64, 1), (64, 2), (128, 2), (128, 4), (256, 2), (256, 4)])
def test_kc_fragment_address_identity(bk, rows, waves):
    wt = rows // waves
    for stage in range(3):
        slot = stage * rows * bk * 2
        for w in range(waves):
            for lane in range(64):
                l32, hl = lane & 31, lane >> 5
                wrow = w * wt + l32
                base = wrow * bk * 2 + ((hl ^ kc_key(bk, wrow)) << 4)
                for i in range(wt // 32):
                    row = w * wt + i * 32 + l32
                    for ks in range(bk // 16):
                        plain = slot + (row * bk + (((ks * 2 + hl) ^ kc_key(bk, row)) << 3)) * 2
                        mask = (ks << 5) ^ (((i & 1) << 6) if bk == 64 else 0)
                        assert (base ^ mask) + slot + i * 32 * bk * 2 == plain, (bk, rows, w, lane, i, ks)


def pipelined_program(nk, nkf, stages, nks):
    """One wave's k-loop events, in program order, as the kernel issues them."""
    ev = []
    for s in range(stages):
        if s < nk:
            ev.append(("dma", s, s, False))
    ev.append(("wait", min(stages - 1, nk - 1)))
    ev.append(("barrier",))
    ev.append(("read", 0, 0, 0))

    def step(slot, kt, full):
        for ks in range(nks):
            if ks + 1 < nks:
                ev.append(("read", kt, slot, ks + 1))
            elif full:
                ev.append(("wait", stages - 2))
                ev.append(("barrier",))
                ev.append(("read", kt + 1, (slot + 1) % stages, 0))
                ev.append(("dma", kt + stages, slot, True))
            elif kt + 1 < nk:
                ev.append(("wait", min(stages - 2, nk - 2 - kt)))
                ev.append(("barrier",))
                if kt + stages < nk:
                    ev.append(("dma", kt + stages, slot, False))
                ev.append(("read", kt + 1, (slot + 1) % stages, 0))

    kt = 0
    while kt + 2 * stages <= nkf:
        for s in range(stages):
            step(s, kt + s, True)
        kt += stages
    while kt + stages <= nk:
        for s in range(stages):
            step(s, kt + s, False)
        kt += stages
    for s in range(stages - 1):
        if kt + s < nk:
            step(s, kt + s, False)
    return ev


def check_program(ev, nk, nkf, stages, nks):
    outstanding = []         # DMA'd tiles not yet known complete, oldest first
    done_at = {}             # tile -> index of the barrier its completion precedes
    content = {}             # slot -> tile last DMA'd into it
    barriers = 0
    reads_since_barrier = set()  # slots read since the last barrier
    loaded, reads = [], []
    for e in ev:
        kind = e[0]
        if kind == "dma":
            _, tile, slot, full = e
            assert 0 <= tile < nk
            assert not full or tile < nkf
            assert slot == tile % stages
            assert slot not in reads_since_barrier, "slot refilled while its old tile is still read"
            content[slot] = tile
            outstanding.append(tile)
            loaded.append(tile)
        elif kind == "wait":
            n = e[1]
            assert 0 <= n <= stages - 1
            while len(outstanding) > n:
                done_at[outstanding.pop(0)] = barriers + 1  # visible after the next barrier
        elif kind == "barrier":
            barriers += 1
            reads_since_barrier.clear()
        else:
            _, tile, slot, ks = e
            assert content.get(slot) == tile, "fragment read from a slot holding another tile"
            assert done_at.get(tile, 1 << 30) <= barriers, "fragment read before its DMA is visible"
            reads_since_barrier.add(slot)
            reads.append((tile, ks))
    assert loaded == list(range(nk))
    assert reads == [(t, ks) for t in range(nk) for ks in range(nks)]


@pytest.mark.parametrize("stages", [2, 3, 4, 5, 6])
@pytest.mark.parametrize("nks", [2, 4])
def test_pipelined_k_loop(stages, nks):
    for nk in range(1, 41):
        # all tiles full, the last one partial, and a k group whose full tiles end early
        for nkf in sorted({nk, nk - 1, max(0, nk - 3)}):
            check_program(pipelined_program(nk, nkf, stages, nks), nk, nkf, stages, nks)
