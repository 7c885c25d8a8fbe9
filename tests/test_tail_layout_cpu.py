"""CPU model of the fused block-tail kernel's data placement (tail.hip).

The kernel moves tiles between global memory, LDS and MFMA fragments with
hand-computed offsets.  This test restates those offsets in Python, with the
kernel's own names, and checks for every thread of a workgroup that

* every LDS access lies inside its buffer (the A tile: 128 rows x 512 bf16,
  the hidden chunk: 128 x 128 bf16, the partial sums: 8 x 128 floats);
* the direct loads fill every A-tile slot exactly once, and each fragment
  read then finds the logical row and columns its lane needs;
* the bf16(x1) stores and the hidden-chunk stores cover their tiles exactly
  once, in the layout the following fragment reads expect;
* every code-fragment load lies inside its fragment-order buffer, and each
  wave reads every code of its columns exactly once per tile;
* the fragment order of the codes (the layout the shuffle kernel writes)
  pairs each weight code with the activation element it multiplies.
"""
import numpy as np
import pytest

TM, DM, HC, NTH = 128, 512, 128, 512
ABYTES, HBYTES = TM * DM * 2, TM * HC * 2
KSTEP = 4 * 2 * 64 * 16


def perm16(u):
    return ((u & 12) << 2) | ((u >> 4) & 3) << 2 | (u & 3)


def phys_row(r):
    return (r & ~63) | perm16(r & 63)


def pair_logical32(p):
    return (p & 3) | (((p >> 4) & 1) << 2) | (((p >> 2) & 3) << 3)


def a_off(p, c):
    return p * (DM * 2) + ((c ^ (2 * (p & 15))) << 4)


def h_off(p, c):
    return p * (HC * 2) + ((c ^ (p & 15)) << 4)


def lanes():
    for tid in range(NTH):
        w, lane = tid >> 6, tid & 63
        yield tid, w, lane, lane & 15, lane >> 4


def arow(i, lr):
    return 64 * (i >> 2) + 16 * (lr >> 2) + (lr & 3) + 4 * (i & 3)


def colj(j, w, lg):
    return 64 * w + 32 * (j >> 1) + 8 * lg + 4 * (j & 1)


def shuffle_source(N, K, c):
    """(row, k0) of the 16-byte fragment chunk c written by the shuffle
    kernel: codes k0 .. k0+7 and k0+32 .. k0+39 of weight row `row`."""
    nk = K // 64
    lane, j, wv = c & 63, (c >> 6) & 1, (c >> 7) & 3
    q = c >> 9
    kt, tn = q % nk, q // nk
    row = tn * 128 + 32 * wv + pair_logical32(16 * j + (lane & 15))
    return row, kt * 64 + 8 * (lane >> 4)


def test_placement_helpers_are_permutations():
    assert sorted(perm16(u) for u in range(64)) == list(range(64))
    assert all(perm16(perm16(u)) == u for u in range(64))
    assert sorted(phys_row(r) for r in range(TM)) == list(range(TM))
    assert sorted(pair_logical32(p) for p in range(32)) == list(range(32))


def test_direct_tile_loads_fill_the_a_tile_once():
    seen = np.zeros(ABYTES // 16, dtype=np.int64)
    content = {}
    for tid, w, lane, lr, lg in lanes():
        for u in range(TM // 8):
            p = w + 8 * u
            assert 0 <= p < TM
            src_row, src_chunk = phys_row(p), lane ^ (2 * (p & 15))
            assert 0 <= src_chunk < DM // 8
            dst = p * (DM * 2) + 16 * lane            # the hardware places lane s at base + 16 s
            assert 0 <= dst and dst + 16 <= ABYTES
            seen[dst // 16] += 1
            content[dst] = (src_row, src_chunk)
    assert np.all(seen == 1)
    # a fragment read (block i, k-chunk kc) finds logical row arow(i), chunk kc
    for tid, w, lane, lr, lg in lanes():
        for i in range(8):
            for kc in range(64):
                off = a_off(16 * i + lr, kc)
                assert content[off] == (arow(i, lr), kc)


def test_x1_stores_cover_the_a_tile_in_fragment_layout():
    seen = {}
    for tid, w, lane, lr, lg in lanes():
        for i in range(8):
            for h in range(2):
                off = a_off(16 * i + lr, 8 * w + 4 * h + lg)
                assert 0 <= off and off + 16 <= ABYTES
                assert off not in seen
                # columns held: colj(2h) .. colj(2h) + 3, colj(2h+1) .. + 3
                cols = [colj(2 * h, w, lg) + e for e in range(4)] + [colj(2 * h + 1, w, lg) + e for e in range(4)]
                assert cols == list(range(cols[0], cols[0] + 8)) and cols[0] % 8 == 0
                seen[off] = (arow(i, lr), cols[0] // 8)
    assert len(seen) == ABYTES // 16
    # the up projection's fragment reads (wave rows 64 wm .. +63) find row, chunk
    for tid, w, lane, lr, lg in lanes():
        wm = w >> 2
        for i in range(4):
            for kc in range(64):
                assert seen[a_off(64 * wm + 16 * i + lr, kc)] == (64 * wm + arow(i, lr), kc)


def test_hidden_chunk_stores_and_reads():
    seen = {}
    for tid, w, lane, lr, lg in lanes():
        wm, wn = w >> 2, w & 3
        for i in range(4):
            off = h_off(64 * wm + 16 * i + lr, 4 * wn + lg)
            assert 0 <= off and off + 16 <= HBYTES
            assert off not in seen
            # hidden columns of fa[i][jj][e]: weight row 16 jj + 4 lg + e of slice wn
            cols = [32 * wn + pair_logical32(16 * jj + 4 * lg + e) for jj in range(2) for e in range(4)]
            assert cols == list(range(32 * wn + 8 * lg, 32 * wn + 8 * lg + 8))
            seen[off] = (64 * wm + arow(i, lr), cols[0] // 8)
    assert len(seen) == HBYTES // 16
    for tid, w, lane, lr, lg in lanes():
        for i in range(8):
            for kc in range(16):
                assert seen[h_off(16 * i + lr, kc)] == (arow(i, lr), kc)


def _lds_pass_slots(offsets):
    """16-byte slots (of the 512 bytes that 128 four-byte banks cover) hit
    by the lanes of one LDS pass."""
    return sorted((off % 512) // 16 for off in offsets)


def test_fragment_reads_and_stores_are_free_of_bank_conflicts():
    """A ds_read_b128 / ds_write_b128 is served 32 lanes at a time; each
    pass must touch 32 distinct 16-byte slots."""
    for half in range(2):          # lanes 0-31 and 32-63 of a wave
        for i in range(8):
            for c0 in range(0, 64, 4):
                offs = [a_off(16 * i + lr, c0 + 2 * half + lg) for lg in range(2) for lr in range(16)]
                assert _lds_pass_slots(offs) == list(range(32)), (i, c0)
            for c0 in range(0, 16, 4):
                offs = [h_off(16 * i + lr, c0 + 2 * half + lg) for lg in range(2) for lr in range(16)]
                assert len(set(off % 512 // 16 for off in offs)) == 32, (i, c0)
    # the normalised MLP input written by the output-projection epilogue
    for w in range(8):
        for i in range(8):
            for h in range(2):
                for half in range(2):
                    offs = [a_off(16 * i + lr, 8 * w + 4 * h + 2 * half + lg) for lg in range(2) for lr in range(16)]
                    assert _lds_pass_slots(offs) == list(range(32))


def test_partial_sums_stay_in_the_hidden_buffer():
    for tid, w, lane, lr, lg in lanes():
        for i in range(8):
            assert 0 <= 4 * (w * TM + arow(i, lr)) < HBYTES
    for tid in range(NTH):
        r, tn = tid & (TM - 1), tid >> 7
        assert tn < 4 and 4 * ((2 * tn + 1) * TM + r) < HBYTES


@pytest.mark.parametrize("F", [1024, 1536, 2048])
def test_code_loads_and_pairing(F):
    nk_proj = F // 64
    o_bytes, fc_bytes, p_bytes = DM * DM, F * DM, DM * F
    for w in range(8):
        wn = w & 3
        o_base = ((w >> 1) * 8 * 4 + 2 * (w & 1)) * 2 * 64 * 16
        p_base = ((w >> 1) * nk_proj * 4 + 2 * (w & 1)) * 2 * 64 * 16
        f_base = wn * 2 * 64 * 16
        o_read, p_read, f_read = set(), set(), set()
        for lane in range(64):
            lr, lg = lane & 15, lane >> 4
            loff = 16 * lane
            for kt in range(8):
                for j in range(4):
                    off = o_base + kt * KSTEP + loff + 1024 * j
                    assert 0 <= off and off + 16 <= o_bytes
                    row, k0 = shuffle_source(DM, DM, off // 16)
                    # fragment j holds weight row = output column of lane group lg
                    assert row == 64 * w + 32 * (j >> 1) + pair_logical32(16 * (j & 1) + lr)
                    # its codes multiply A chunk kc = 8 kt + 4 ks + lg, i.e. k0 and k0 + 32
                    assert k0 == 64 * kt + 8 * lg
                    o_read.add(off // 16)
            for c in range(F // HC):
                for kt in range(8):
                    for jj in range(2):
                        off = f_base + (c * 8 + kt) * KSTEP + loff + 1024 * jj
                        assert 0 <= off and off + 16 <= fc_bytes
                        row, k0 = shuffle_source(F, DM, off // 16)
                        assert row == HC * c + 32 * wn + pair_logical32(16 * jj + lr)
                        assert k0 == 64 * kt + 8 * lg
                        f_read.add(off // 16)
                for kk in range(2):
                    for j in range(4):
                        off = p_base + (2 * c + kk) * KSTEP + loff + 1024 * j
                        assert 0 <= off and off + 16 <= p_bytes
                        row, k0 = shuffle_source(DM, F, off // 16)
                        assert row == 64 * w + 32 * (j >> 1) + pair_logical32(16 * (j & 1) + lr)
                        # hidden columns of h chunk c, k-chunk 8 kk + 4 ks + lg
                        assert k0 == HC * c + 64 * kk + 8 * lg
                        p_read.add(off // 16)
        # each wave reads the codes of its 64 (o, proj) or, per row half, its
        # 32 (fc) columns exactly once
        assert len(o_read) == 64 * DM // 16 and len(p_read) == 64 * F // 16
        assert len(f_read) == (F // 4) * DM // 16     # a quarter of the hidden columns
