"""The wide forward's cross-XCD claim protocol, as a host model run under random interleavings.

Workgroups 0 .. n-1 own item n (XCD = id % 8, position id // 8 in that XCD's order). The
workgroups after them ("takers", dispatched after all of their own XCD's items) each take the
last unclaimed item of another XCD. The device code (attn_fwd_wide.hip, wide_take and the
owner's claim in the item prologue) works on a per-stream block of 64-bit words that is never
cleared between launches:
  * words 16 * x (x < 8): this launch's claims from the back of XCD x, with the launch
    (mark / 2) in the upper 32 bits; a claim that finds an earlier launch there restarts it;
  * word 16 * 8: the launch mark once a taker found nothing left anywhere;
  * words 144 + id: the item marks. An owner raises its item's mark to the launch mark, a taker
    to the launch mark + 1, both with an atomic maximum; a mark below the launch mark is
    unclaimed.
The model runs each step of each workgroup as one atomic operation on that block, in random
orders, over launches of different item counts on one block, and checks that every item runs
exactly once (each workgroup's result is written by whichever runs the item; two runs would
write the same bits, a missed item none). No GPU is needed."""
import random

import pytest

HEAD = 9 * 16
MASK32 = 0xFFFFFFFF


class Block:
    def __init__(self, words):
        self.w = [0] * words

    def add(self, i, v):
        old = self.w[i]
        self.w[i] = (old + v) & 0xFFFFFFFFFFFFFFFF
        return old

    def cas(self, i, expect, new):
        old = self.w[i]
        if old == expect:
            self.w[i] = new
        return old

    def umax(self, i, v):
        old = self.w[i]
        self.w[i] = max(old, v)
        return old

    def xchg(self, i, v):
        old = self.w[i]
        self.w[i] = v
        return old


def owner(blk, epoch, item, ran):
    """Generator of one owner workgroup's atomic steps; records a run unless taken."""
    took = blk.umax(HEAD + item, epoch)
    yield
    if took != (epoch | 1):
        ran[item] += 1


def taker(blk, epoch, xs, nitems, ran):
    """One taker workgroup: the device's wide_take, one atomic per step."""
    launch = (epoch >> 1) & MASK32
    nothing = blk.w[16 * 8]          # (an atomic load)
    yield
    if nothing == epoch:
        return
    for j in range(1, 8):
        x = (xs + j) & 7
        cnt = (nitems - x + 7) >> 3
        w = blk.add(16 * x, 1)
        yield
        if (w >> 32) == launch:
            b = w & MASK32
        else:
            fresh = (launch << 32) | 1
            prev = blk.cas(16 * x, (w + 1) & 0xFFFFFFFFFFFFFFFF, fresh)
            yield
            if prev == (w + 1) & 0xFFFFFFFFFFFFFFFF:
                b = 0
            else:
                w = blk.add(16 * x, 1)
                yield
                if (w >> 32) != launch:
                    continue
                b = w & MASK32
        if b >= cnt:
            continue
        item = x + 8 * (cnt - 1 - b)
        old = blk.umax(HEAD + item, epoch | 1)
        yield
        if old < epoch:
            ran[item] += 1
            return
    blk.xchg(16 * 8, epoch)
    yield


def run_launch(blk, epoch, nitems, ntakers, rng):
    """Interleave owners and takers: each XCD's owners start in order, its takers only after
    all of its owners started (hardware dispatch order); across XCDs and between started
    workgroups the order is random."""
    ran = [0] * nitems
    pending = {x: [("o", i) for i in range(x, nitems, 8)] + [("t", x)] * ntakers
               for x in range(8)}
    live = []
    while any(pending.values()) or live:
        choices = [x for x in range(8) if pending[x]]
        if choices and (not live or rng.random() < 0.5):
            x = rng.choice(choices)
            kind, v = pending[x].pop(0)
            live.append(owner(blk, epoch, v, ran) if kind == "o"
                        else taker(blk, epoch, v, nitems, ran))
            continue
        g = rng.choice(live)
        try:
            next(g)
        except StopIteration:
            live.remove(g)
    return ran


@pytest.mark.parametrize("seed", range(6))
def test_every_item_runs_exactly_once_across_launches(seed):
    rng = random.Random(seed)
    sizes = [rng.choice([257, 288, 300, 384, 512, 700]) for _ in range(8)]
    blk = Block(HEAD + max(sizes))
    epoch = 0
    for nitems in sizes:
        epoch += 2
        ran = run_launch(blk, epoch, nitems, ntakers=rng.choice([1, 4, 16]), rng=rng)
        assert all(r == 1 for r in ran), (nitems, [i for i, r in enumerate(ran) if r != 1][:10])


def test_exchange_instead_of_maximum_can_lose_an_item():
    """The failure the maximum prevents (a pin of the model itself): with an exchange, a taker
    that meets a word left by an earlier, smaller launch (a counter word, far above any mark)
    moves on but leaves its own mark, and the owner then takes that mark for a theft."""
    blk = Block(HEAD + 16)
    epoch = 10
    blk.w[HEAD + 3] = (7 << 32) | 5          # stale counter word where item 3's mark now is
    old = blk.xchg(HEAD + 3, epoch | 1)      # taker: not unclaimed (old >= epoch): moves on
    assert old >= epoch
    took = blk.umax(HEAD + 3, epoch)         # owner arrives afterwards
    assert took == (epoch | 1)               # ... and stops: nobody runs item 3
    # with the maximum the stale word stays, and the owner runs the item
    blk.w[HEAD + 3] = (7 << 32) | 5
    assert blk.umax(HEAD + 3, epoch | 1) >= epoch
    assert blk.umax(HEAD + 3, epoch) != (epoch | 1)
