"""Host-side check of the decode kernel's load schedule (no GPU).

The decode GEMM issues all of its loads as LDS DMAs in a fixed order per wave
and waits on the wave's vector-memory counter with compile-time counts.  This
replays that order -- chunk 0, the W blocks of the first D positions, then per
chunk: wait for the chunk, barrier, issue the next chunk, and per position:
issue the W block D positions ahead, wait for this position's block -- and
checks, under in-order completion, that every wait count guarantees the loads
the following reads depend on, and that a W ring of D+1 slots is never
overwritten before its block has been read.
"""
import pytest

def replay(KB, D, NPW, KBC=4):
    """KBC: K blocks per X chunk."""
    NC = (KB + KBC - 1) // KBC
    issued = []
    ring_owner = {}

    def issue_chunk(c):
        issued.extend([("x", c)] * NPW)

    def issue_w(q):
        slot = q % (D + 1)
        # the slot's previous block (q - D - 1) must already have been read
        prev = ring_owner.get(slot)
        assert prev is None or prev == q - D - 1
        ring_owner[slot] = q
        issued.extend([("w", q)] * 2)

    def wait(n, need):
        done = issued[: len(issued) - n] if n else issued
        for item in need:
            assert issued.count(item) > 0 and done.count(item) == issued.count(item), (KB, D, NPW, item, n)

    issue_chunk(0)
    for j in range(D):
        issue_w(j)
    for c in range(NC):
        wait(2 * D if c == 0 else 2 * KBC, [("x", c)])   # counts written in the kernel
        issue_chunk(c + 1)
        for pos in range(KBC):
            q = c * KBC + pos
            issue_w(q + D)
            wait(2 * D + (NPW if pos < D else 0), [("w", q), ("x", c)])


@pytest.mark.parametrize("KBC", [4, 8])
@pytest.mark.parametrize("D", [1, 2, 3, 4])
@pytest.mark.parametrize("NPW", [1, 2, 3, 6, 8, 12])
def test_decode_wait_counts(D, NPW, KBC):
    for KB in range(1, 40):
        replay(KB, D, NPW, KBC)


def test_decode_wait_counts_catch_a_short_count():
    """A count one too large (waiting for one load too few) must be caught."""
    with pytest.raises(AssertionError):
        KB, D, NPW = 8, 4, 2
        issued = [("x", 0)] * NPW + [("w", j) for j in range(D) for _ in range(2)]
        n = 2 * D + 1
        done = issued[: len(issued) - n]
        assert done.count(("x", 0)) == NPW
