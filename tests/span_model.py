"""The placement model behind the library's choice of segment length, restated
in plain Python for the tests (it is scheduling, not the method: every length
gives the same results, so the oracle does not need it).

A (segment, head) unit is one workgroup of the first-pass kernel, one per CU.
Units are dispatched in table order (every full-length segment in segment
order, then the shorter ones in segment order or longest first; the H heads of
a segment consecutive).
Workgroup b goes to XCD b % 8 and, inside it, to shader engine (b // 8) % 4,
which has 8 CUs; it starts once a CU of that engine is free and not before
the previous workgroup of its XCD started.  A unit costs the chunks it runs
plus a fixed start cost: a full segment runs its chunks plus K more into the
next segment when that one is longer than K; a later segment of K chunks or
fewer ends at once; a sequence shorter than the segment is one unit."""

XCDS, ENGINES, CUS_PER_ENGINE = 8, 4, 8
START_COST = 4
K = 4


def unit_costs(s, chunks, desc=False):
    full, rest = [], []
    for n in chunks:
        nseg = max(1, -(-n // s))
        for j in range(nseg):
            here = min(s, n - j * s) if n else 0
            after = min(s, n - (j + 1) * s) if j + 1 < nseg else 0
            cost = here + (K if after > K else 0)
            if j > 0 and j == nseg - 1 and here <= K:
                cost = 0
            (full if here == s else rest).append(cost)
    if desc:
        rest = sorted(rest, reverse=True)  # stable: ties stay in segment order
    return full + rest


def first_pass_span(s, chunks, H, desc=False):
    free = [[[0] * CUS_PER_ENGINE for _ in range(ENGINES)] for _ in range(XCDS)]
    prev_start = [0] * XCDS
    span, b = 0, 0
    for cost in unit_costs(s, chunks, desc):
        for _ in range(H):
            x, e = b % XCDS, (b // XCDS) % ENGINES
            b += 1
            cus = free[x][e]
            k = min(range(CUS_PER_ENGINE), key=lambda q: cus[q])
            start = max(cus[k], prev_start[x])
            prev_start[x] = start
            cus[k] = start + cost + START_COST
            span = max(span, cus[k])
    return span


def chosen_plan(planned, lengths, H, varlen=False):
    """(length, longest first) a call with this planned length uses when the
    library chooses.  A varlen call chooses on the device, for planned lengths
    of 128 chunks or more only, between both orders of the shorter segments; a
    fixed-length call on the host, in segment order (its shorter segments are
    all equal)."""
    N = len(lengths)
    if not (planned > 0 and 1 <= N <= 16 and H % 8 == 0 and N * H <= 256):
        return planned, False
    if varlen and planned < 128:
        return planned, False
    chunks = [-(-L // 16) for L in lengths]
    cands = range(planned, planned + min(planned // 4, 63) + 1)
    orders = (False, True) if varlen else (False,)
    best = min((first_pass_span(s, chunks, H, d), s, int(d)) for s in cands for d in orders)
    return best[1], bool(best[2])


def chosen_seg(planned, lengths, H, varlen=False):
    return chosen_plan(planned, lengths, H, varlen)[0]


def rest_cost(n, s):
    """First-pass cost of the shorter segment of a sequence of n chunks, or -1 when it has none."""
    f, rem = divmod(n, s)
    if f == 0:
        return n
    if rem == 0:
        return -1
    return rem if rem > K else 0
