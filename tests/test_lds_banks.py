"""CPU model of the LDS bank rules, applied to the LDS access patterns of the bf16 MFMA
prefill kernels (csrc/prefill_mfma.hip: the chunk-64 output pass, the chunk-128 output
pass and the segment-map pass).

Bank rules (measured on gfx950 with a conflict-counting probe): 64 banks of four bytes;
8-byte reads (including the transposing ds_read_b64_tr_b16) are served 32 lanes per
cycle, 16-byte reads 16 lanes per cycle, and writes at 128 bytes per cycle (8 lanes of
16 bytes, 16 lanes of 8 bytes).  Within the lanes served in one cycle, two different
four-byte words in one bank conflict; lanes reading the same word do not.

Where the model stops: a later probe (SQ_LDS_BANK_CONFLICT per instruction) confirmed it
for the 8-byte and transposing reads and the 16-byte row stores of the staged tiles (no
conflicts at 272-byte rows) and for contiguous or 16-granule-swizzled 16-byte reads, but
the 16-byte score operand reads, 16 rows of 272 bytes with lane group g taking granule g,
cost about 4 extra cycles per read on the device (none at 288-byte rows, where the 8-byte
reads conflict instead).  Those reads are therefore not claimed conflict-free here
(`score_reads` below is left out of the check); reading them as two 8-byte halves removes
the conflicts but measured slower in every output pass, so the kernels keep them.

The index formulas below restate the kernels' own: a staged tile holds one token row of
128 bf16 per token, padded to 136 elements (272 bytes); lane = (lg4, lr) with lane =
16 lg4 + lr; the transposing load takes, in each 16-lane group, 4 adjacent columns
4 (lr & 3) .. of token row e = lr >> 2 of the group's set.  A change of layout in the
kernels has to be mirrored here.  Tile base addresses are multiples of 16 bytes and only
permute the banks, so they are left out.
"""
from __future__ import annotations

import collections

ROW = 136  # padded row, in bf16 elements
LANES = range(64)


def sigma(m: int) -> int:
    """Token order of the K~ rows in the score tiles: even tokens of the tile first."""
    return 2 * (m & 7) + (m >> 3)


def pr_off(row: int, col: int, row_len: int = ROW) -> int:
    return row * row_len + col


def ys_off(row: int, col: int) -> int:
    """y tile of the chunk-64 pass: granule g of row j at granule g ^ (j & 15)."""
    return row * 128 + ((((col >> 3) ^ (row & 15)) << 3) | (col & 7))


def lane_parts(lane: int):
    lr, lg4 = lane & 15, lane >> 4
    return lr, lg4, lr >> 2, 4 * (lr & 3)  # lr, lg4, te, tc


def extra_cycles(byte_addrs, width: int, lanes_per_cycle: int) -> int:
    """Cycles beyond one per lane group, for one wave-wide access of `width` bytes per lane."""
    extra = 0
    for g in range(0, 64, lanes_per_cycle):
        banks = collections.defaultdict(set)
        for a in byte_addrs[g:g + lanes_per_cycle]:
            assert a % width == 0 or width == 8 and a % 8 == 0, "misaligned access"
            for w in range(width // 4):
                word = a // 4 + w
                banks[word % 64].add(word)
        extra += max(len(s) for s in banks.values()) - 1
    return extra


READ8, READ16, TR8, WRITE16, WRITE8 = (8, 32), (16, 16), (8, 32), (16, 8), (8, 16)


def elem_access(fn):
    """Byte addresses of one wave-wide access given an element-offset function of the lane."""
    return [2 * fn(lane) for lane in LANES]


# ------------------------------------------------------------------ access patterns
def producer_stores(tpt: int, n_producer_waves: int):
    """Row stores of the staged tiles: thread (fg, tg) writes granule fg of tokens tpt tg + p."""
    for pw in range(n_producer_waves):
        for p in range(tpt):
            def f(lane, pw=pw, p=p):
                pt = pw * 64 + lane
                fg, tg = pt & 15, pt >> 4
                return pr_off(tg * tpt + p, fg * 8)
            yield ("stage p=%d wave=%d" % (p, pw), elem_access(f), WRITE16)


def inter_chunk_reads(ntj: int):
    """(2) and phi(q).z_prev: two 8-byte halves of the permuted k order per 32-feature step."""
    for tj in range(ntj):
        for kf in range(4):
            for half in (0, 16):
                def f(lane, tj=tj, kf=kf, half=half):
                    lr, lg4, _, _ = lane_parts(lane)
                    return pr_off(tj * 16 + lr, kf * 32 + half + lg4 * 4)
                yield ("(2) tj=%d kf=%d half=%d" % (tj, kf, half), elem_access(f), READ8)


def score_reads(ntj: int, order=sigma):
    """(1): K~ rows in the order sigma, Q~ rows in natural order, 16 bytes per lane."""
    for t in range(ntj):
        for kf in range(4):
            def fk(lane, t=t, kf=kf):
                lr, lg4, _, _ = lane_parts(lane)
                return pr_off(t * 16 + order(lr), kf * 32 + lg4 * 8)

            def fq(lane, t=t, kf=kf):
                lr, lg4, _, _ = lane_parts(lane)
                return pr_off(t * 16 + lr, kf * 32 + lg4 * 8)
            yield ("(1) K tile=%d kf=%d" % (t, kf), elem_access(fk), READ16)
            yield ("(1) Q tile=%d kf=%d" % (t, kf), elem_access(fq), READ16)


def intra_value_reads(nki: int, order=sigma, row_len: int = ROW):
    """(3): V^T in the score tiles' k order, two transposing loads per 32-token step."""
    for ki in range(nki):
        for wave in range(8):
            for second in (0, 16):
                def f(lane, ki=ki, wave=wave, second=second):
                    _, lg4, te, tc = lane_parts(lane)
                    return pr_off(ki * 32 + order(lg4 * 4 + te) + second, wave * 16 + tc, row_len)
                yield ("(3) ki=%d wave=%d +%d" % (ki, wave, second), elem_access(f), TR8)


def state_update_reads(nki: int):
    """(4): V and the write weights, tokens 8 lg4 + 2 e and 8 lg4 + 2 e + 1 of each step."""
    for ki in range(nki):
        for col_tile in range(8):  # wave (V, z) or feature tile tf (write weights)
            for second in (0, 1):
                def f(lane, ki=ki, ct=col_tile, second=second):
                    _, lg4, te, tc = lane_parts(lane)
                    return pr_off(ki * 32 + lg4 * 8 + 2 * te + second, ct * 16 + tc)
                yield ("(4) ki=%d tile=%d +%d" % (ki, col_tile, second), elem_access(f), TR8)


def score_tile_accesses(n_slots: int):
    """Score tiles in accumulator layout: 8 bytes per lane, or a pair of tiles as 16 bytes."""
    for slot in range(n_slots):
        for half in (0, 1):
            yield ("P write slot=%d half=%d" % (slot, half), [(slot * 64 + lane) * 16 + 8 * half for lane in LANES], WRITE8)
        yield ("P pair read slot=%d" % slot, [(slot * 64 + lane) * 16 for lane in LANES], READ16)
        yield ("P single read slot=%d" % slot, [(slot * 64 + lane) * 8 for lane in LANES], READ8)


def y_tile_accesses(tpt: int):
    """Chunk-64 pass: consumers write y as 8-byte pieces, producers read whole rows."""
    for wave in range(8):
        for tj in range(4):
            def f(lane, wave=wave, tj=tj):
                lr, lg4, _, _ = lane_parts(lane)
                return ys_off(tj * 16 + lr, wave * 16 + lg4 * 4)
            yield ("y write wave=%d tj=%d" % (wave, tj), elem_access(f), WRITE8)
    for pw in range(4):
        for u in range(tpt):
            def g(lane, pw=pw, u=u):
                row = pw * 4 * tpt + u * 4 + (lane >> 4)
                return row * 128 + (lane & 15) * 8
            yield ("y row read wave=%d u=%d" % (pw, u), elem_access(g), READ16)


def kernel_patterns():
    # chunk-64 output pass: 4 producer waves, 4 tokens per thread and tile
    for name, addrs, (w, lpc) in producer_stores(4, 4):
        yield "pc " + name, addrs, w, lpc
    for gen in (inter_chunk_reads(4), intra_value_reads(2), state_update_reads(2),
                score_tile_accesses(6), y_tile_accesses(4)):
        for name, addrs, (w, lpc) in gen:
            yield "pc " + name, addrs, w, lpc
    # chunk-128 output pass: 4 producer waves, 8 tokens per thread and tile
    for name, addrs, (w, lpc) in producer_stores(8, 4):
        yield "p8 " + name, addrs, w, lpc
    for gen in (inter_chunk_reads(8), intra_value_reads(4), state_update_reads(4)):
        for name, addrs, (w, lpc) in gen:
            yield "p8 " + name, addrs, w, lpc
    # segment-map pass (chunk 64): stores of the write weights and V, then (4)
    for name, addrs, (w, lpc) in producer_stores(4, 4):
        yield "sum " + name, addrs, w, lpc
    for name, addrs, (w, lpc) in state_update_reads(2):
        yield "sum " + name, addrs, w, lpc


def test_every_kernel_access_is_conflict_free():
    checked = 0
    bad = []
    for name, addrs, width, lpc in kernel_patterns():
        e = extra_cycles(addrs, width, lpc)
        checked += 1
        if e:
            bad.append((name, e))
    assert checked > 200
    assert not bad, bad[:10]


def test_model_sees_conflicts_without_the_padding():
    """Unpadded 256-byte rows put the 16 rows of an MFMA operand in the same banks."""
    def f(lane):
        lr, lg4, _, _ = lane_parts(lane)
        return pr_off(lr, lg4 * 4, row_len=128)
    assert extra_cycles(elem_access(f), 8, 32) > 0


def test_model_sees_conflicts_without_the_sigma_order():
    """With K~ rows in natural order, the transposing loads of (3) mix even and odd rows."""
    total = sum(extra_cycles(a, w, lpc) for _, a, (w, lpc) in intra_value_reads(4, order=lambda m: m))
    assert total > 0
    assert sum(extra_cycles(a, w, lpc) for _, a, (w, lpc) in intra_value_reads(4)) == 0


def test_sigma_is_a_permutation_of_the_tile():
    assert sorted(sigma(m) for m in range(16)) == list(range(16))
    assert [sigma(m) % 2 for m in range(8)] == [0] * 8
    assert [sigma(m) % 2 for m in range(8, 16)] == [1] * 8


def test_bank_rules_on_plain_cases():
    # 64 lanes reading consecutive 4-byte words of one row: no conflict at any width
    assert extra_cycles([lane * 8 for lane in LANES], 8, 32) == 0
    assert extra_cycles([lane * 16 for lane in LANES], 16, 16) == 0
    # every lane of a group reading the same word is a broadcast
    assert extra_cycles([0] * 64, 8, 32) == 0
    # two words 256 bytes apart share a bank
    assert extra_cycles([0, 256] + [512 * 4] * 62, 8, 32) == 2
