"""Host model of the tiled product's K-loop schedule (gemm_tiled_kernel in csrc/gemm.hip), checked
for every number of 64-element sub-chunks a tile can have.

The kernel stages K chunks of 256 (four sub-chunks) in two LDS stages and runs a chunk as four
pipelined sub-chunks: sub-chunks 0-2 each read the next sub-chunk of the same stage, sub-chunks 0
and 1 also copy parts 1 and 2 of chunk kc+1 into the other stage, and sub-chunk 3 waits for its own
copies, meets the other wavefronts at a barrier, reads chunk kc+1's first sub-chunk and copies part
0 of chunk kc+2 into chunk kc's stage.  The loop runs two chunks per pass; the 0-7 sub-chunks left
after it run after one wait and barrier.  A tile's first chunk is copied whole, part 0 of its second
before the loop.  The model replays that schedule and checks that

* every sub-chunk is contracted exactly once, in order (so the accumulation order of an output
  element is K order, whatever the tile shape or the number of tiles);
* every read of a sub-chunk finds all three parts of its chunk landed in the stage it reads (copies
  land only at a wait followed by a barrier);
* no copy lands in a stage before every sub-chunk of the chunk it held has been read, and that
  read was completed before the last barrier (so no wavefront still reads what a copy overwrites).

It is a model of the schedule, kept in step with the kernel by hand; the GPU parity tests check the
kernel itself (tests/test_gpu_gemm.py and tests/test_gpu_gemm_edges.py cover every remainder of
sub-chunks after the loop)."""

import pytest

SUB = 4    # sub-chunks per chunk
PARTS = 3  # copy parts per chunk


def replay(nsub):
    last = (nsub + SUB - 1) // SUB - 1
    stage = {"s0": [None] * PARTS, "s1": [None] * PARTS}  # per part: [chunk, landed]
    read_log = set()
    state = {"barrier_reads": set()}
    consumed = []
    regs = {}

    def issue(st, chunk, parts):
        for held in {x[0] for x in stage[st] if x is not None}:
            if held == chunk:
                continue
            need = set(range(held * SUB, min(nsub, held * SUB + SUB)))
            assert need <= state["barrier_reads"], (nsub, st, held, chunk)
        for p in parts:
            stage[st][p] = [chunk, False]

    def barrier():  # each wavefront waited for its own copies, then all met
        for st in stage.values():
            for x in st:
                if x is not None:
                    x[1] = True
        state["barrier_reads"] = set(read_log)

    def read(st, c):
        if c is None or c >= nsub:
            return -1  # a clamped, redundant read
        for x in stage[st]:
            assert x is not None and x[0] == c // SUB and x[1], (nsub, st, c, stage[st])
        read_log.add(c)
        return c

    def body(cur, nxt, st, c, has_next, sync, copy):
        consumed.append(regs[cur])
        if has_next:
            if sync:
                barrier()
            regs[nxt] = read(st, c)
            if copy:
                copy()

    def run_chunk(st, nst, kc):
        k1, k2 = min(kc + 1, last), min(kc + 2, last)
        body("f0", "f1", st, kc * SUB + 1, True, False, lambda: issue(nst, k1, [1]))
        body("f1", "f0", st, kc * SUB + 2, True, False, lambda: issue(nst, k1, [2]))
        body("f0", "f1", st, kc * SUB + 3, True, False, None)
        body("f1", "f0", nst, (kc + 1) * SUB, True, True, lambda: issue(st, k2, [0]))

    issue("s0", 0, range(PARTS))
    issue("s1", min(1, last), [0])
    barrier()
    regs["f0"] = read("s0", 0)
    kc = 0
    while 4 * kc + 7 < nsub:
        run_chunk("s0", "s1", kc)
        run_chunk("s1", "s0", kc + 1)
        kc += 2
    sc = SUB * kc
    if sc < nsub:
        issue("s1", min(kc + 1, last), [1, 2])
        barrier()

        def stage_of(c):
            return "s1" if c // SUB > kc else "s0"

        while sc + 1 < nsub:
            body("f0", "f1", stage_of(sc + 1), sc + 1, True, False, None)
            nx = min(sc + 2, nsub - 1)
            body("f1", "f0", stage_of(nx), nx, True, False, None)
            sc += 2
        if sc < nsub:
            body("f0", "f1", "s0", None, False, False, None)
    return consumed


@pytest.mark.parametrize("nsub", list(range(1, 41)) + [80, 272, 1023])
def test_every_sub_chunk_once_in_order(nsub):
    assert replay(nsub) == list(range(nsub))
