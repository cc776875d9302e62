"""Host-side check of the main GEMM kernel's load schedule (no GPU).

Per tile, each wave issues its share of every K block's stage as NPIECE
direct-to-LDS loads in a fixed order and waits on its own vector-memory
counter with compile-time counts; one workgroup barrier per block publishes a
stage and frees the buffer of the block before.  This replays that order --
blocks 0 .. S-2 in full, a wait for block 0 and a barrier, the first two
window positions of block S-1; then per block kb and streamed row r: at row
R-2 a wait for block kb+1 and the barrier, and the window position of the
loads of block kb+S-1 (before it) or kb+S (from it on) -- and checks, under
in-order completion of loads:
  * every read of a block's buffer comes after a wait that covers all of that
    block's loads, followed by a barrier (so every wave's share has landed);
  * no load refills a buffer before the barrier after which no wave reads
    the block it held.
Blocks past the last one are issued through an empty range and counted like
the others.  The tile starts with no wait on the counter (it also counts the
previous tile's stores), so a second tile is replayed after the first with
the first tile's last loads still outstanding.
"""
import pytest


def replay(S, NPIECE, R, KB, tiles=2):
    WIN = (3 * R) // 4 if R >= 4 else R
    RB = R - 2
    issued = []              # (tile, block) per load, in issue order
    done_upto = [0]          # loads known complete (a prefix, in-order completion)
    owner = {}               # buffer -> (tile, block) it holds
    freed = set()            # (tile, block) whose reads are over for every wave
    published = set()        # (tile, block) landed for every wave (wait + barrier)
    landed = set()           # (tile, block) landed for this wave

    def issue(t, b, pieces):
        buf = b % S
        if (t, b) not in [owner.get(buf)] and owner.get(buf) is not None:
            prev = owner[buf]
            assert prev in freed, f"refill of buffer {buf} with {(t, b)} before {prev} was freed"
        owner[buf] = (t, b)
        issued.extend([(t, b)] * pieces)

    def window(t, b, pos):
        n = sum(1 for p in range(NPIECE) if p * WIN // NPIECE == pos)
        if n:
            issue(t, b, n)

    def wait(n):
        done_upto[0] = max(done_upto[0], len(issued) - n)
        done = issued[:done_upto[0]]
        for key in set(issued):
            if done.count(key) == issued.count(key):
                landed.add(key)

    def barrier(reads_over):
        published.update(landed)
        freed.update(reads_over)

    def read(t, b):
        if b < KB:
            assert (t, b) in published, f"tile {t} block {b} read before it was published"

    for t in range(tiles):
        # the previous tile's reads are over; no wait on the counter here
        barrier([(t - 1, b) for b in range(KB + S)] if t else [])
        for b in range(S - 1):
            issue(t, b, NPIECE)
        wait((S - 2) * NPIECE)
        barrier([])
        window(t, S - 1, 0)
        window(t, S - 1, 1)
        read(t, 0)                               # resident fragments and first rows of block 0
        for kb in range(KB):
            for r in range(R):
                if r == RB:
                    wait((S - 2) * NPIECE)
                    barrier([(t, kb)])           # every read of block kb is done before it
                    read(t, kb + 1)              # the rows read ahead now come from block kb+1
                if r < RB:
                    window(t, kb + S - 1, r + 2)
                else:
                    window(t, kb + S, r - RB)
            # all pieces of blocks kb+S-1 and kb+S went out over the windows
    wait(0)
    return len(issued)


# (stages, loads per wave and stage, streamed rows per block) of the instances
INSTANCES = [(2, 9, 7), (2, 8, 4), (3, 5, 2), (3, 7, 4), (3, 6, 3), (4, 5, 2), (4, 4, 4)]


@pytest.mark.parametrize("S,NPIECE,R", INSTANCES)
@pytest.mark.parametrize("KB", [1, 2, 3, 5, 12, 16, 56])
def test_gemm_schedule(S, NPIECE, R, KB):
    n = replay(S, NPIECE, R, KB)
    # per tile: blocks 0 .. KB+S-2 in full (the last S-1 past the end, through
    # an empty range) and the first two window positions of block KB+S-1
    WIN = (3 * R) // 4 if R >= 4 else R
    head = sum(1 for p in range(NPIECE) if p * WIN // NPIECE < 2)
    assert n == 2 * ((KB + S - 1) * NPIECE + head)


def test_window_covers_every_piece():
    """Every piece of a stage falls on a window position that is issued:
    positions 0 and 1 after the barrier that frees the buffer, 2 .. R-1 in
    the rows before the next one."""
    for S, NPIECE, R in INSTANCES:
        WIN = (3 * R) // 4 if R >= 4 else R
        pos = {p * WIN // NPIECE for p in range(NPIECE)}
        assert pos <= set(range(R)), (S, NPIECE, R)
