"""The record-slot layout the split prefill uses for packed sequences (host-side check of the
integer formulas in csrc/chunk_split.hip, restated here): head hv owns floor(T/C) + N slots;
sequence s, starting at row a_s (offsets clamped into [0, T] as on the device), takes slots
floor(a_s/C) + s onwards, one per chunk; the prep wavefront of slot p serves the last sequence
whose first slot is <= p.  Valid offsets: every chunk gets exactly one slot.  Any offsets:
every slot a chain reads stays below the bound."""
import random


def clamp(x, lo, hi):
    return min(max(x, lo), hi)


def seq_range(cu, T, s):
    a = clamp(cu[s], 0, T)
    return a, min(max(cu[s + 1], a), T) - a


def slots(cu, T, C):
    N = len(cu) - 1
    nrec = T // C + N
    served = {}
    for p in range(nrec):
        s = max([i for i in range(N) if clamp(cu[i], 0, T) // C + i <= p], default=-1)
        if s < 0:
            continue
        c = p - (clamp(cu[s], 0, T) // C + s)
        if c < -(-seq_range(cu, T, s)[1] // C):
            served.setdefault(p, []).append((s, c))
    return nrec, served


def test_packed_slots_cover_every_chunk_once():
    rng = random.Random(0)
    for _ in range(500):
        C = rng.choice([32, 64])
        lens = [rng.choice([0, 1, C - 1, C, C + 1, 2 * C, rng.randint(0, 3 * C)])
                for _ in range(rng.randint(1, 140))]
        cu = [0]
        for n in lens:
            cu.append(cu[-1] + n)
        T = cu[-1]
        nrec, served = slots(cu, T, C)
        for s in range(len(lens)):
            a, n = seq_range(cu, T, s)
            for c in range(-(-n // C)):
                assert served.get(a // C + s + c) == [(s, c)]
        assert sum(map(len, served.values())) == sum(-(-n // C) for n in lens)


def test_packed_slots_stay_in_bounds_for_any_offsets():
    rng = random.Random(1)
    for _ in range(500):
        C, N, T = rng.choice([32, 64]), rng.randint(1, 90), rng.randint(1, 2000)
        cu = [rng.randint(-50, T + 50) for _ in range(N + 1)]
        nrec, served = slots(cu, T, C)
        assert all(0 <= p < nrec for p in served)
        for s in range(N):
            a, n = seq_range(cu, T, s)
            if n:
                assert a // C + s + -(-n // C) <= nrec
