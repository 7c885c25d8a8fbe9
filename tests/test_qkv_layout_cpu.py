"""CPU model of the one-tile q/k/v kernel's data placement (qkv.hip).

The kernel and the load-time rearrangement of the codes (shuffle_qkv_kernel)
use hand-computed indices.  This test restates them in Python, with the
kernel's names, and checks that

* the rearranged codes hold every code of every weight row exactly once;
* for q and k heads (C^T accumulation) the MFMA output that a lane holds in
  accumulator block j, element e is the weight row of the dim the epilogue
  treats it as: the first dim of rotation pair c1b + t for t < 8 and its
  second dim for t >= 8, for every partial-RoPE width the library accepts;
* for v heads (C accumulation) a lane holds 16 consecutive rows of one
  column;
* the A-tile direct loads fill every LDS slot once, and every Q, K and V^T
  element of a batch is written exactly once, inside its buffer, when
  windows straddle tiles and the last tile is half full.
"""
import numpy as np
import pytest

TM, DM, HD, NW = 128, 512, 64, 8
NK = DM // 64


def perm16(u):
    return ((u & 12) << 2) | ((u >> 4) & 3) << 2 | (u & 3)


def phys_row(r):
    return (r & ~63) | perm16(r & 63)


def pair_first(p, R):
    return p if p < R // 2 else R + (p - R // 2)


def pair_second(p, R):
    return p + R // 2 if p < R // 2 else R + (HD - R) // 2 + (p - R // 2)


def rope_phys(u, R):
    q8 = HD // 8
    h2, rest2 = R // 2, (HD - R) // 2
    if u < h2:
        p, second = u, 0
    elif u < R:
        p, second = u - h2, 1
    elif u < R + rest2:
        p, second = h2 + (u - R), 0
    else:
        p, second = h2 + (u - R - rest2), 1
    t = p % q8 + second * q8
    return 16 * (t >> 2) + 4 * (p // q8) + (t & 3)


def shuffle_source(c, n_qk, R):
    """(weight row, k0) of 16-byte chunk c of the rearranged codes: codes
    k0 .. k0+7 and k0+32 .. k0+39 of that row."""
    lane, j = c & 63, (c >> 6) & 3
    q = c >> 8
    kt, h = q % NK, q // NK
    pr = 16 * j + (lane & 15)
    u = pr
    if h < n_qk:
        u = [v for v in range(HD) if rope_phys(v, R) == pr][0]
    return h * HD + u, kt * 64 + 8 * (lane >> 4)


@pytest.mark.parametrize("R", [16, 32, 48, 64])
def test_rope_placement_is_a_permutation(R):
    assert sorted(rope_phys(u, R) for u in range(HD)) == list(range(HD))


@pytest.mark.parametrize("R", [16, 64])
def test_rearranged_codes_cover_every_code_once(R):
    n_heads, n_kv = 8, 4
    n_qk, n_all = n_heads + n_kv, n_heads + 2 * n_kv
    seen = np.zeros((n_all * HD, DM // 8), dtype=np.int64)
    for c in range(n_all * NK * 256):
        row, k0 = shuffle_source(c, n_qk, R)
        assert 0 <= row < n_all * HD and k0 % 8 == 0 and k0 + 40 <= DM
        seen[row, k0 // 8] += 1
        seen[row, k0 // 8 + 4] += 1
    assert np.all(seen == 1)


@pytest.mark.parametrize("R", [16, 32, 48, 64])
def test_qk_accumulators_hold_whole_rotation_pairs(R):
    """C^T: the output row of fragment j at lane group lg, element e is
    fragment row 4 lg + e, whose weight row is the dim rope_phys put there."""
    inv = {rope_phys(u, R): u for u in range(HD)}
    for lg in range(4):
        c1b = 8 * lg
        f0, s0 = pair_first(c1b, R), pair_second(c1b, R)
        for t in range(8):
            first = inv[16 * (t >> 2) + 4 * lg + (t & 3)]
            second = inv[16 * ((t + 8) >> 2) + 4 * lg + ((t + 8) & 3)]
            assert first == f0 + t and second == s0 + t
            # and they are rotation pair c1b + t
            assert pair_first(c1b + t, R) == f0 + t and pair_second(c1b + t, R) == s0 + t


def test_v_accumulators_hold_consecutive_rows():
    """C: the output of fragment j for A row-block i at lane (lr, lg),
    element e is A physical row 16 i + 4 lg + e, i.e. logical row
    64 (i >> 2) + 16 lg + 4 (i & 3) + e, and weight row 16 j + lr."""
    for lg in range(4):
        for s in range(2):
            # accumulator block i = 4 s + (t >> 2), element e = t & 3: A
            # physical row 16 i + 4 lg + e; phys_row is its own inverse
            rows = [phys_row(16 * (4 * s + (t >> 2)) + 4 * lg + (t & 3)) for t in range(16)]
            assert rows == list(range(64 * s + 16 * lg, 64 * s + 16 * lg + 16))


def _arow(i, lr):
    return 64 * (i >> 2) + 16 * (lr >> 2) + (lr & 3) + 4 * (i & 3)


def test_direct_loads_fill_the_a_tile_once():
    seen = np.zeros(TM * DM * 2 // 16, dtype=np.int64)
    content = {}
    for w in range(NW):
        for lane in range(64):
            for u in range(TM // NW):
                p = w + NW * u
                dst = p * DM * 2 + 16 * lane
                seen[dst // 16] += 1
                content[dst] = (phys_row(p), lane ^ (2 * (p & 15)))
    assert np.all(seen == 1)
    for lr in range(16):
        for lg in range(4):
            for i in range(8):
                for kc in range(0, 64, 4):
                    off = (16 * i + lr) * DM * 2 + (((kc + lg) ^ (2 * ((16 * i + lr) & 15))) << 4)
                    assert content[off] == (_arow(i, lr), kc + lg)


@pytest.mark.parametrize("R", [16, 64])
@pytest.mark.parametrize("W,Lp", [(3, 192), (2, 128), (1, 320)])
def test_stores_cover_q_k_vt_once(R, W, Lp):
    n_heads, n_kv = 8, 4
    n_qk, n_all = n_heads + n_kv, n_heads + 2 * n_kv
    M = W * Lp
    assert Lp >= TM and Lp % 64 == 0 and M % 64 == 0
    q = np.zeros(W * n_heads * Lp * HD, dtype=np.int64)
    k = np.zeros(W * n_kv * Lp * HD, dtype=np.int64)
    vt = np.zeros(W * n_kv * HD * Lp, dtype=np.int64)
    tiles = (M + TM - 1) // TM
    for tile in range(tiles):
        m0 = tile * TM
        win0, pos0 = m0 // Lp, m0 % Lp
        for w in range(NW):
            for h in range(w, n_all, NW):
                for lane in range(64):
                    lr, lg = lane & 15, lane >> 4
                    if h < n_qk:
                        is_q = h < n_heads
                        head = h if is_q else h - n_heads
                        nh = n_heads if is_q else n_kv
                        buf = q if is_q else k
                        c1b = 8 * lg
                        f0, s0 = pair_first(c1b, R), pair_second(c1b, R)
                        for i in range(8):
                            ml = _arow(i, lr)
                            if m0 + ml >= M:
                                continue
                            pos, win = pos0 + ml, win0
                            if pos >= Lp:
                                pos, win = pos - Lp, win + 1
                            # the row really is batch row m0 + ml
                            assert win * Lp + pos == m0 + ml
                            base = ((win * nh + head) * Lp + pos) * HD
                            for d0 in (f0, s0):
                                assert 0 <= base + d0 and base + d0 + 8 <= buf.size
                                buf[base + d0:base + d0 + 8] += 1
                    else:
                        head = h - n_qk
                        for s in range(2):
                            ml = 64 * s + 16 * lg
                            if m0 + ml >= M:
                                continue
                            pos, win = pos0 + ml, win0
                            if pos >= Lp:
                                pos, win = pos - Lp, win + 1
                            assert win * Lp + pos == m0 + ml and pos + 16 <= Lp
                            for j in range(4):
                                dd = 16 * j + lr
                                base = ((win * n_kv + head) * HD + dd) * Lp + pos
                                assert base + 16 <= vt.size
                                vt[base:base + 16] += 1
    assert np.all(q == 1) and np.all(k == 1) and np.all(vt == 1)
