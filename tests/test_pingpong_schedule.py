"""Model check of the LDS buffer schedule of the ping-pong forward block
(fwd_block_pingpong in exact_attention_26_amd/csrc/fa_fwd_block.h), on the
CPU.  Iteration k: after a barrier every wave issues the loads of K_{k+1}
(into K buffer (k+1) % 2) and V_k (into V buffer k % 2); group A then runs
M(k) and group B the softmax of tile k-1; after a second barrier A runs the
softmax of tile k and B runs M(k); every wave then waits for its loads.  M(k)
reads K_k (scores of tile k, when k < n) and V_{k-1} (PV of tile k-1, when
k >= 1).  The check: every read finds the tile it wants, loaded in an earlier
iteration (so landed and made visible by the barrier), and no load goes into a
buffer that is read in the same iteration (its reads may still be in flight
while the load writes)."""
import pytest


def schedule(n):
    """Events per iteration: loads [(buffer, tile)], reads [(half, group, buffer, tile)]."""
    it = []
    for k in range(n + 1):
        loads = []
        if k + 1 < n:
            loads.append((("K", (k + 1) % 2), ("K", k + 1)))
        if k < n:
            loads.append((("V", k % 2), ("V", k)))
        reads = []
        for half, group in ((0, "A"), (1, "B")):       # M(k) of A, then M(k) of B
            if k < n:
                reads.append((half, group, ("K", k % 2), ("K", k)))
            if k >= 1:
                reads.append((half, group, ("V", (k - 1) % 2), ("V", k - 1)))
        it.append((loads, reads))
    return it


def check(n, sched=schedule):
    content = {("K", 0): (("K", 0), -1)}               # K_0 before the loop, waited for
    for k, (loads, reads) in enumerate(sched(n)):
        read_bufs = {r[2] for r in reads}
        for b, t in loads:
            assert b not in read_bufs, f"n={n} k={k}: load of {t} into {b} while it is read"
        pending = {b: (t, k) for b, t in loads}
        for _, _, b, t in reads:
            have = content.get(b)
            assert have is not None and have[0] == t, f"n={n} k={k}: {b} holds {have}, needs {t}"
            assert have[1] < k, f"n={n} k={k}: {t} was loaded in this iteration"
        content.update(pending)
    # every tile of K and V was read
    seen = {r[3] for _, reads in sched(n) for r in reads}
    assert seen == {("K", t) for t in range(n)} | {("V", t) for t in range(n)}


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 32, 33])
def test_pingpong_buffer_schedule_is_race_free(n):
    check(n)


def test_a_buffer_mistake_is_caught():
    # planted mistake: V_k loaded into buffer (k + 1) % 2 overwrites V_{k-1}
    # while M(k) of both groups reads it
    def bad(n):
        return [([(("V", (t[1] + 1) % 2), t) if b[0] == "V" else (b, t) for b, t in loads],
                 reads) for loads, reads in schedule(n)]
    with pytest.raises(AssertionError):
        check(4, bad)
    # and loading K_{k+1} one iteration later than needed is caught too
    def late(n):
        return [([(b, (t[0], t[1] + 1)) if b[0] == "K" else (b, t) for b, t in loads], reads)
                for loads, reads in schedule(n)]
    with pytest.raises(AssertionError):
        check(4, late)
