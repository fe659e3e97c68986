"""Host model of the decode streaming loop for 64-head column groups
(stream_batch in csrc/pa_device.h): two groups of four waves deal the same
sub-tile stream, each wave computing positions r, r + 4, ... (two in
flight), and meet at workgroup barriers of two kinds: the finish of each
piece (at the position where the next piece starts) and a sync barrier
every kSyncSub positions.  Every wave must meet the same barriers in the
same order, or the workgroup would pair one wave's finish with another's
sync.  The model follows the loop's control flow (the enter() calls and
their positions) step for step; it checks the order rule, not the
kernel's arithmetic."""
import random

K_STRIDE = 4       # waves per column group
K_SYNC = 8 * K_STRIDE


def _wave_events(r, nsub):
    npl, total = len(nsub), sum(nsub)
    start = [0]
    for n in nsub:
        start.append(start[-1] + n)

    def piece(x):
        if x >= total:
            return npl
        return next(p for p in range(npl) if start[p] <= x < start[p + 1])

    ev = []
    st = {"cur": 0, "cur_end": nsub[0] if npl else 0, "next_sync": K_SYNC}

    def enter(p, pos):
        while True:
            fin = st["cur"] < p
            if st["next_sync"] <= pos and (not fin or st["next_sync"] < st["cur_end"]):
                ev.append(("sync", st["next_sync"]))
                st["next_sync"] += K_SYNC
                continue
            if not fin:
                break
            ev.append(("finish", st["cur"]))
            st["cur"] += 1
            if st["cur"] < npl:
                st["cur_end"] += nsub[st["cur"]]

    computed = []
    if r < total:
        p0, s0 = piece(r), r
        p1, s1 = piece(r + K_STRIDE), r + K_STRIDE
        snext = r + 2 * K_STRIDE
        enter(p0, s0)
        while True:
            computed.append((s0, p0, st["cur"]))
            n0, m0 = piece(snext), snext
            snext += K_STRIDE
            more = p1 < npl
            if more:
                enter(p1, s1)
                computed.append((s1, p1, st["cur"]))
            n1, m1 = piece(snext), snext
            snext += K_STRIDE
            p0, s0, p1, s1 = n0, m0, n1, m1
            if not more or p0 >= npl:
                break
            enter(p0, s0)
    enter(npl, total - 1)
    return ev, computed, total


def test_every_wave_meets_the_same_barriers_in_the_same_order():
    rng = random.Random(1)
    for _ in range(3000):
        npl = rng.randint(0, 12)
        nsub = [rng.choice([1, 2, 3, 5, 8, 13, 16, 17, 31, 32, 33, 40, 64, 100]) for _ in range(npl)]
        runs = [_wave_events(w % K_STRIDE, nsub) for w in range(2 * K_STRIDE)]
        ev0, _, total = runs[0]
        for ev, computed, _ in runs:
            assert ev == ev0, nsub
        # every piece finished once, in order; one sync per K_SYNC positions
        # before the end of the stream
        assert [x for k, x in ev0 if k == "finish"] == list(range(npl))
        assert [x for k, x in ev0 if k == "sync"] == list(range(K_SYNC, total, K_SYNC))
        for r in range(K_STRIDE):
            _, computed, _ = runs[r]
            # each wave computes exactly its positions, each in the piece
            # whose state it holds at that moment
            assert [s for s, _, _ in computed] == list(range(r, total, K_STRIDE))
            assert all(p == cur for _, p, cur in computed)
