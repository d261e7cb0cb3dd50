"""Second, independent statements of the two planners, in plain Python, used only as pins of
the C oracle (tests/test_oracle_pins.py).  They are written from the pages' text and the
readings the oracle documents, not from oracle.c, and share nothing with it: lists and
``min``/``max`` with explicit tie keys instead of index loops.

Rank r owns the local experts r*G .. r*G + G - 1 (G = E_loc / P).  Both functions return
(q, moves, blocks) in the oracle's conventions: q[l][r] = rows of expert l on rank r; blocks
(rank, expert, first row, rows) rank by rank, then expert by expert; expert segments start
at multiples of beta.
"""
from __future__ import annotations


def _segment_starts(n, beta):
    starts, at = [], 0
    for c in n:
        starts.append(at)
        at += -(-c // beta) * beta
    return starts


def moonep_plan(n, P, beta):
    """The greedy balance of "MoonEP routing flow -- live" (section "The greedy balance, step
    by step", with its per-rank surplus against S*K entries).  While some rank is below its
    capacity, the rank furthest below it is refilled in a single move from the rank furthest
    above it (lower rank id on ties, both ways); the donor may drop below capacity and be
    refilled later.  A move is cut into slices of the donor's own experts, always from the one
    with the most entries still at home (lower id on ties).  Capacity of rank r:
    floor(N/P) + (r < N mod P), i.e. S*K when P divides N."""
    E = len(n)
    G = E // P
    N = sum(n)
    cap = [N // P + (1 if r < N % P else 0) for r in range(P)]
    surplus = [sum(n[r * G:(r + 1) * G]) - cap[r] for r in range(P)]
    at_home = list(n)
    q = [[0] * P for _ in range(E)]
    moves = []
    while min(surplus) < 0:
        hungriest = min(range(P), key=lambda r: (surplus[r], r))
        donor = max(range(P), key=lambda r: (surplus[r], -r))
        need = -surplus[hungriest]
        surplus[hungriest] += need
        surplus[donor] -= need
        while need > 0:
            candidates = [l for l in range(donor * G, (donor + 1) * G) if at_home[l] > 0]
            if not candidates:
                raise AssertionError("a donor ran out of entries")
            biggest = max(candidates, key=lambda l: (at_home[l], -l))
            take = min(at_home[biggest], need)
            at_home[biggest] -= take
            need -= take
            q[biggest][hungriest] += take
            moves.append([donor, hungriest, biggest, take])
    for l in range(E):
        q[l][l // G] += at_home[l]
    # each rank takes the next consecutive range of the expert's stable order, in rank order
    starts = _segment_starts(n, beta)
    blocks = []
    for r in range(P):
        for l in range(E):
            rows = q[l][r]
            first = starts[l] + sum(q[l][:r])
            done = 0
            while done < rows:
                m = min(beta, rows - done)
                blocks.append([r, l, first + done, m])
                done += m
    return q, moves, blocks


def megaflux_plan(n, P, beta, s):
    """The block-granular planner of "MegaFlux: Skew-Resilient MoE Megakernels via Pipelined
    Expert Replication" (section 3.1 "Bounded greedy search"; appendix A.1 "Candidate
    construction" and "Refinement"), under the oracle's readings: blocks of beta rows; loads
    in blocks; tau = ceil(total blocks / P); four searches (donor order by overload or by the
    largest home-expert block count at home, times one new copy per expert per round or any
    number), each from the no-replica start, rounds visiting every rank over tau at the
    round's start once, a visit scanning its home experts by blocks at home (most first),
    single blocks going to the least-loaded rank under tau already holding a copy, else to the
    least-loaded rank under tau with fewer than s foreign copies (a new copy); a search stops
    after s + 2 rounds or a round without movement.  Winner: least maximum load, then fewest
    replicas, then the first in the order above.  Refinement: replicas by increasing
    allocation (then expert, then rank) go whole to the owner, else to the least-loaded other
    holder, when that stays within the winner's maximum; then single blocks move from the
    most- to the least-loaded rank while their loads differ by more than one and the latter
    holds (or owns) an expert that has blocks on the former (the lowest such expert)."""
    E = len(n)
    G = E // P
    owner = [l // G for l in range(E)]
    b = [-(-c // beta) for c in n]
    tau = -(-sum(b) // P)

    def search(by_overload, many):
        q = [[b[l] if r == owner[l] else 0 for r in range(P)] for l in range(E)]
        load = [sum(b[r * G:(r + 1) * G]) for r in range(P)]
        foreign = [0] * P
        for _ in range(s + 2):
            moved = False
            opened = set()
            prio = {}
            for r in range(P):
                if load[r] > tau:
                    prio[r] = (load[r] - tau if by_overload
                               else max(q[l][r] for l in range(r * G, (r + 1) * G)))
            for d in sorted(prio, key=lambda r: (-prio[r], r)):
                if load[d] <= tau:
                    continue
                scan = sorted((l for l in range(d * G, (d + 1) * G) if q[l][d] > 0),
                              key=lambda l: (-q[l][d], l))
                for l in scan:
                    if load[d] <= tau:
                        break
                    while q[l][d] > 0 and load[d] > tau:
                        holders = [r for r in range(P) if r != d and q[l][r] > 0 and load[r] < tau]
                        if holders:
                            to = min(holders, key=lambda r: (load[r], r))
                        else:
                            if not many and l in opened:
                                break
                            fresh = [r for r in range(P) if r != d and q[l][r] == 0
                                     and foreign[r] < s and load[r] < tau]
                            if not fresh:
                                break
                            to = min(fresh, key=lambda r: (load[r], r))
                            foreign[to] += 1
                            opened.add(l)
                        q[l][d] -= 1
                        q[l][to] += 1
                        load[d] -= 1
                        load[to] += 1
                        moved = True
            if not moved:
                break
        return q, load

    cands = []
    for idx, (by_overload, many) in enumerate(((True, False), (True, True),
                                               (False, False), (False, True))):
        q, load = search(by_overload, many)
        reps = sum(1 for l in range(E) for r in range(P) if r != owner[l] and q[l][r] > 0)
        cands.append((max(load), reps, idx, q, load))
    top, _, _, q, load = min(cands, key=lambda c: c[:3])

    reps = sorted((q[l][r], l, r) for l in range(E) for r in range(P)
                  if r != owner[l] and q[l][r] > 0)
    for _, l, r in reps:
        a = q[l][r]
        if a == 0:
            continue
        h = owner[l]
        if load[h] + a <= top:
            to = h
        else:
            others = [x for x in range(P) if x not in (r, h) and q[l][x] > 0 and load[x] + a <= top]
            to = min(others, key=lambda x: (load[x], x)) if others else None
        if to is not None:
            q[l][to] += a
            load[to] += a
            q[l][r] = 0
            load[r] -= a
    for _ in range(sum(b)):
        hi = max(range(P), key=lambda r: (load[r], -r))
        lo = min(range(P), key=lambda r: (load[r], r))
        if load[hi] - load[lo] <= 1:
            break
        shared = [l for l in range(E) if q[l][hi] > 0 and (owner[l] == lo or q[l][lo] > 0)]
        if not shared:
            break
        l = shared[0]
        q[l][hi] -= 1
        q[l][lo] += 1
        load[hi] -= 1
        load[lo] += 1

    # blocks -> rows: the ranks holding an expert take consecutive runs of its blocks in rank
    # order, so only its last block can be partial
    starts = _segment_starts(n, beta)
    q_rows = [[0] * P for _ in range(E)]
    moves = []
    for l in range(E):
        before = 0
        for r in range(P):
            lo_row = min(before * beta, n[l])
            hi_row = min((before + q[l][r]) * beta, n[l])
            q_rows[l][r] = hi_row - lo_row
            if q[l][r] > 0 and r != owner[l]:
                moves.append([owner[l], r, l, hi_row - lo_row])
            before += q[l][r]
    blocks = []
    for r in range(P):
        for l in range(E):
            before = sum(q[l][:r])
            for j in range(before, before + q[l][r]):
                blocks.append([r, l, starts[l] + j * beta, min(beta, n[l] - j * beta)])
    return q_rows, moves, blocks
