"""CPU: the balanced stream's partition arithmetic, with the set cost.

The vector engine's stream kernel cuts the stream of sets into equal ranges and writes partials into
slots; the merge kernel recomputes, for each output row, which slots hold its set's partials.  The
two sides share no code, so this test restates both computations in Python: the kernel's walk (the
range's first position located through the sequences' prefix, a set taking the set cost C and then
one position per token, a set that ends inside the range written per wave, the range's last set
with tokens combined into one slot) and the merge's reading (first and last range holding the
set's tokens, one combined slot per range before the last, and the last one combined unless the
next set's first token lies inside it).  It checks, over random batches with empty and ragged
sequences, side-by-side lanes and set costs up to 4096, that no slot is written twice, that every
slot the merge reads was written for that set and lane, that every written slot is read, and that
the partials a set's merge reads cover each of its tokens exactly once.  The cost is dropped where
every range would hold as many set changes anyway (equal lengths, sets and ranges dividing one
another), on both sides alike."""
import random

NW = 8  # waves per range: slots per (set, range, lane)


def span(lens, HS, num_ranges, min_tokens, C):
    nz = [n for n in lens if n > 0]
    T0, S = sum(nz) * HS, len(nz) * HS
    R0 = min(num_ranges, (T0 + min_tokens - 1) // min_tokens)
    if S > 0 and R0 > 0 and min(nz) == max(nz) and (R0 % S == 0 or S % R0 == 0):
        C = 0
    T = T0 + S * C
    return T, min(num_ranges, (T + min_tokens - 1) // min_tokens), C


def kernel_writes(lens, HS, L, num_ranges, min_tokens, C):
    """slot -> (sequence, set, lane, first token, end token) for every partial the kernel writes"""
    T, R, C = span(lens, HS, num_ranges, min_tokens, C)
    B, writes = len(lens), {}
    for g in range(R):
        x0, x1 = (g * T + R - 1) // R, ((g + 1) * T + R - 1) // R
        if x0 >= x1:
            continue
        base, b, pb = 0, -1, 0
        for bb in range(B):
            lv = lens[bb] + C if lens[bb] > 0 else 0
            if (base + lv) * HS > x0 and lv > 0:
                b, pb = bb, base
                break
            base += lv
        assert b >= 0
        n, lp = lens[b], lens[b] + C
        uu = (x0 - pb * HS) // lp
        start = pb * HS + uu * lp
        t_lo, t_hi = max(0, x0 - start - C), min(n, x1 - start - C)
        if t_hi <= t_lo:                       # the range lies within one set's charged positions
            assert x1 <= start + C
            continue
        while True:
            assert t_hi > t_lo
            nxt = start + lp
            last = not (nxt + C < x1)
            for lane in range(L):
                slot = ((b * HS + uu + g) * L + lane) * NW
                for s in ([slot] if last else [slot + w for w in range(NW)]):
                    assert s not in writes, f"slot {s} written twice"
                    writes[s] = (b, uu, lane, t_lo, t_hi)
            if last:
                break
            uu += 1
            if uu == HS:
                uu, b = 0, b + 1
                while b < B and lens[b] == 0:
                    b += 1
                assert b < B
                n, lp = lens[b], lens[b] + C
            start, t_lo, t_hi = nxt, 0, min(n, x1 - nxt - C)
    return writes


def merge_reads(lens, HS, L, num_ranges, min_tokens, C, writes):
    T, weff, C = span(lens, HS, num_ranges, min_tokens, C)
    read = set()
    for b, n in enumerate(lens):
        if n == 0:
            continue
        pre = sum((m + C if m > 0 else 0) for m in lens[:b])
        for sq in range(HS):
            first = pre * HS + sq * (n + C) + C
            end = first + n
            wf, wl = first * weff // T, (end - 1) * weff // T
            x1l = ((wl + 1) * T + weff - 1) // weff
            nr = wl - wf
            nparts = nr + (1 if x1l <= end + C else NW)
            u = b * HS + sq
            for lane in range(L):
                s0, sl = ((u + wf) * L + lane) * NW, ((u + wl) * L + lane) * NW
                cover = set()
                for p in range(nparts):
                    q = s0 + p * L * NW if p < nr else sl + (p - nr)
                    assert q in writes, f"slot {q} read but not written"
                    wb, wsq, wln, t_lo, t_hi = writes[q]
                    assert (wb, wsq, wln) == (b, sq, lane), f"slot {q} holds another set"
                    cover.add((t_lo, t_hi))
                    read.add(q)
                pos = 0
                for t_lo, t_hi in sorted(cover):
                    assert t_lo == pos, f"sequence {b} set {sq}: tokens {pos}..{t_lo} covered {cover}"
                    pos = t_hi
                assert pos == n
    assert read == set(writes), f"{len(set(writes) - read)} written slots never read"


def test_stream_slots_with_set_cost():
    rng = random.Random(7)
    cases = dropped = 0
    while cases < 3000:
        B, HS, L = rng.randint(1, 9), rng.randint(1, 6), rng.choice([1, 1, 2, 4])
        lens = [rng.choice([0, rng.randint(1, 40), rng.randint(1, 3000)]) for _ in range(B)]
        if rng.random() < 0.3:
            n0 = rng.choice([1, 64, 100, 2048, 4096])
            lens = [rng.choice([0, n0, n0]) for _ in range(B)]
        if sum(lens) == 0:
            continue
        num_ranges = max(1, rng.choice([1, 3, 8, 64, 256]) // L)
        min_tokens = rng.choice([1, 64, 512])
        C = rng.choice([0, 1, 63, 64, 192, 512, 1000, 4096])
        merge_reads(lens, HS, L, num_ranges, min_tokens, C, kernel_writes(lens, HS, L, num_ranges, min_tokens, C))
        dropped += C > 0 and span(lens, HS, num_ranges, min_tokens, C)[2] == 0
        cases += 1
    assert dropped > 100          # the equal-length rule was exercised


def test_set_cost_moves_tokens_off_ranges_with_a_set_change():
    # two sequences of one set each over 3 ranges: the middle range holds the set change and, with
    # a set cost, fewer tokens
    lens, HS, R = [1000, 1000], 1, 3
    tokens = {}
    for C in (0, 300):
        w = kernel_writes(lens, HS, 1, R, 1, C)
        per_range = {}
        for slot, (b, sq, lane, t_lo, t_hi) in w.items():
            per_range.setdefault(slot // NW - (b * HS + sq), set()).add((b, t_lo, t_hi))
        tokens[C] = {g: sum(h - lo for _, lo, h in v) for g, v in per_range.items()}
    assert tokens[0] == {0: 667, 1: 667, 2: 666}
    assert tokens[300][1] < tokens[0][1] and sum(tokens[300].values()) == 2000
