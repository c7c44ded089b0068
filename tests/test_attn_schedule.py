"""The MLA attention's work schedule, written out in Python: the arithmetic of
mla_attn_schedule_kernel (csrc/attn_mla.hip) for its two forms, and the
invariants the attention and merge kernels rely on.

  balanced     workgroup w owns tiles [w T / nb, (w + 1) T / nb) of the T tiles;
  row-aligned  (extend token rows, B <= nb / 2) row b owns
               n_b = 1 + floor(t_b (nb - B) / T) workgroups (t_b its tiles),
               consecutive from W_b = n_0 + ... + n_{b-1}, and cuts its tiles
               into that many equal chunks; the workgroups past the last row
               get empty ranges.  Rows with equal tile counts get equal
               chunks, so a sequence's new tokens read the same keys side by
               side.

Invariants: the ranges partition [0, T); a workgroup's first row holds its
first tile; a row's first / last workgroup hold its first / last tile, and
they are equal exactly when one workgroup's range covers the whole row (the
attention then writes the row directly and the merge skips it); the later
segments of a row start at or after the row."""
import random

import pytest


def cdiv(a, b):
    return (a + b - 1) // b


def schedule(tiles, nb, aligned):
    B = len(tiles)
    P = [0]
    for t in tiles:
        P.append(P[-1] + t)
    T = P[-1]
    starts, first_row, wlo, whi = [None] * (nb + 1), [None] * nb, [None] * B, [None] * B
    if not aligned:
        for w in range(nb + 1):
            starts[w] = w * T // nb
        for b in range(B):
            pb, pe = P[b], P[b + 1]
            for w in range(cdiv(pb * nb, T), cdiv(pe * nb, T)):
                first_row[w] = b
            wlo[b] = cdiv((pb + 1) * nb, T) - 1
            whi[b] = cdiv(pe * nb, T) - 1
    else:
        w0 = 0
        for b in range(B):
            pb, v = P[b], tiles[b]
            n = 1 + v * (nb - B) // T
            for c in range(n):
                starts[w0 + c] = pb + c * v // n
                first_row[w0 + c] = b
            wlo[b] = w0 + cdiv(n, v) - 1
            whi[b] = w0 + n - 1
            w0 += n
        assert w0 <= nb
        for w in range(w0, nb + 1):
            starts[w] = T
            if w < nb:
                first_row[w] = B - 1
    return P, starts, first_row, wlo, whi


def check(tiles, nb, aligned):
    P, starts, first_row, wlo, whi = schedule(tiles, nb, aligned)
    B, T = len(tiles), P[-1]
    assert starts[0] == 0 and starts[nb] == T
    assert all(starts[w] <= starts[w + 1] for w in range(nb))
    row_of = [b for b in range(B) for _ in range(tiles[b])]
    whole = set()
    for w in range(nb):
        s, e = starts[w], starts[w + 1]
        if s >= e:
            continue
        assert first_row[w] == row_of[s]
        b, cur = first_row[w], s          # the attention's walk over its range
        while cur < e:
            pb, pe = P[b], P[b + 1]
            t0, t1 = cur - pb, min(e, pe) - pb
            assert 0 <= t0 < t1 <= pe - pb
            if t0 == 0 and t1 == pe - pb:
                whole.add(b)
            cur, b = pb + t1, b + 1
    for b in range(B):
        pb, pe = P[b], P[b + 1]
        assert starts[wlo[b]] <= pb < starts[wlo[b] + 1]
        assert starts[whi[b]] <= pe - 1 < starts[whi[b] + 1]
        assert (wlo[b] == whi[b]) == (b in whole)
        assert all(starts[w] >= pb for w in range(wlo[b] + 1, whi[b] + 1))
        assert whi[b] - wlo[b] + 1 <= 256          # the merge kernels' segment bound


@pytest.mark.parametrize("aligned", [False, True])
def test_schedule_invariants(aligned):
    rng = random.Random(7)
    cases = 0
    while cases < 1500:
        nb = rng.choice([8, 16, 64, 256])
        B = rng.randint(1, nb // 2 if aligned else 2 * nb)
        tiles = [rng.randint(1, rng.choice([1, 3, 40, 200])) for _ in range(B)]
        check(tiles, nb, aligned)
        cases += 1


def test_row_aligned_extend_shape():
    """16 sequences of 4096 cached keys with 1..4 new tokens: consecutive tokens of
    a sequence get the same number of workgroups and chunk starts that differ by
    at most one tile, i.e. they read the same keys side by side."""
    rng = random.Random(3)
    for _ in range(100):
        q = [rng.randint(1, 4) for _ in range(16)]
        tiles = [cdiv(4096 + j + 1, 32) for n in q for j in range(n)]
        check(tiles, 256, True)
        P, starts, _, wlo, whi = schedule(tiles, 256, True)
        r = 0
        for n in q:
            for j in range(1, n):
                a, b = r + j - 1, r + j
                assert whi[a] - wlo[a] == whi[b] - wlo[b]
                for c in range(whi[a] - wlo[a] + 1):
                    assert abs((starts[wlo[b] + c] - P[b]) - (starts[wlo[a] + c] - P[a])) <= 1
            r += n
