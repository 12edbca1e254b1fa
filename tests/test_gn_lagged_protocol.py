"""A step-by-step model of the lagged group-norm schedule, run on the CPU
under adversarial scheduling.

The kernel (gn_lagged_kernel in csrc/group_norm_silu.hip) is a small
lock-free protocol.  Workgroup b:
  1. loads its output chunk j = b - lag;
  2. reduces chunk b and publishes its word by compare-and-swap from
     "empty" (the first word published stands);
  3. polls the words of j's group, up to `polls` times each;
  4. reduces each word still empty itself, lowest first, and publishes it the
     same way;
  5. combines the group's words and writes chunk j (in place: over x).

This model keeps those steps and their order.  Every read of x, every
compare-and-swap and every poll is one step.  A scheduler advances one
resident workgroup per step, chosen at random:
  - workgroups start in a given dispatch order (index order, or shuffled,
    which the hardware need not do but other work sharing the dies can
    resemble);
  - at most `slots` workgroups are resident at once;
  - random workgroups are frozen for long stretches.

The checks:
  * every workgroup finishes;
  * the output equals the sequential definition, out of place and in place;
  * without step 4 (polls unbounded), a shuffled dispatch order with few
    slots can leave every resident workgroup waiting for one that cannot
    start: the reason the kernel has step 4.

The data are integers, and the "reduction" and "output" are exact functions
of them.  A reduction that read a chunk its output had already replaced
would publish a different word, and the output check would see it.
"""
import random

import pytest


def run_model(n_groups, chunks, lag, *, in_place, polls, slots, order, seed, freeze=0.02,
              max_steps=2_000_000, cas=True):
    """Simulate one call.  Returns (finished, output exact, steps taken).
    cas=False publishes with a plain store (the last word written stands)."""
    rng = random.Random(seed)
    total = n_groups * chunks
    x0 = [rng.randrange(1, 1 << 20) for _ in range(total)]
    x = list(x0)                       # the input buffer (overwritten in place)
    y = x if in_place else [None] * total
    word = [None] * total              # None: not yet published
    def reduce_(v):                    # chunk statistics; also of a replaced chunk
        key = v if isinstance(v, int) else (v[1] * 31 + v[2]) ^ 0x5A5A5A
        return (key * 2654435761) % (1 << 32)
    combine = lambda ws: sum(ws) % (1 << 32)                  # the group's statistics
    output = lambda v, s: ("y", v, s)                         # never equal to an input

    def workgroup(b):
        """The steps of workgroup b, as a generator (yield = one step)."""
        j = b - lag
        out = 0 <= j < total
        if out:
            w = x[j]                               # the output chunk's loads
            yield
        if b < total:
            v = x[b]                               # own reduction reads its chunk
            yield
            if word[b] is None or not cas:         # compare-and-swap from empty
                word[b] = reduce_(v)
            yield
        if not out:
            return
        q = j // chunks
        grp = range(q * chunks, (q + 1) * chunks)
        seen = {k: word[k] for k in grp}
        yield
        spins = 0
        while any(seen[k] is None for k in grp) and (polls is None or spins < polls):
            spins += 1
            for k in grp:
                if seen[k] is None:
                    seen[k] = word[k]
            yield
        for k in grp:                              # step 4: reduce the missing ones here
            if seen[k] is None:
                v = x[k]
                yield
                if word[k] is None or not cas:
                    word[k] = reduce_(v)
                seen[k] = word[k] if cas else reduce_(v)   # the word that stands
                yield
        y[j] = output(w, combine(seen[k] for k in grp))
        yield

    queue = list(order)
    resident = {}
    frozen = set()
    finished = 0
    steps = 0
    while finished < total + lag:
        while queue and len(resident) < slots:
            b = queue.pop(0)
            resident[b] = workgroup(b)
        live = [b for b in resident if b not in frozen]
        if not live:
            frozen.clear()
            continue
        b = rng.choice(live)
        try:
            next(resident[b])
        except StopIteration:
            del resident[b]
            finished += 1
        steps += 1
        if freeze and rng.random() < freeze and resident:
            frozen.add(rng.choice(list(resident)))
        if rng.random() < 0.01:
            frozen.clear()
        if steps >= max_steps:
            return False, None, steps
    words = [reduce_(v) for v in x0]
    want = [output(x0[j], combine(words[(j // chunks) * chunks:(j // chunks + 1) * chunks]))
            for j in range(total)]
    return True, (y if not in_place else x) == want, steps


def dispatch_order(n, kind, rng):
    if kind == "index":
        return list(range(n))
    if kind == "dies":
        # dealt to 8 dies in turn, each die running ahead or behind: a random
        # interleaving of the 8 index-ordered streams
        streams = [list(range(d, n, 8)) for d in range(8)]
        order = []
        while any(streams):
            d = rng.choice([i for i, s in enumerate(streams) if s])
            order.append(streams[d].pop(0))
        return order
    order = list(range(n))
    rng.shuffle(order)
    return order


@pytest.mark.parametrize("kind", ["index", "dies", "shuffled"])
@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("polls", [0, 3, 50])
def test_every_workgroup_finishes_and_the_output_is_exact(kind, in_place, polls):
    groups, chunks = 6, 4
    lag = chunks + 5
    for seed in range(6):
        rng = random.Random(1000 * seed + polls)
        order = dispatch_order(groups * chunks + lag, kind, rng)
        ok, exact, steps = run_model(groups, chunks, lag, in_place=in_place, polls=polls,
                                     slots=rng.choice([2, 3, 5, 16]), order=order, seed=seed)
        assert ok, "did not finish (seed %d, %s order)" % (seed, kind)
        assert exact, "output differs from the definition (seed %d, %s order)" % (seed, kind)


def test_without_the_helper_a_shuffled_order_can_deadlock():
    """Unbounded polling and no step 4: with few slots and workgroups started
    out of index order, the resident ones can all wait on a chunk whose
    workgroup cannot start.  In index order the same schedule finishes."""
    groups, chunks = 6, 4
    lag = chunks + 5
    stuck = 0
    for seed in range(20):
        rng = random.Random(seed)
        order = dispatch_order(groups * chunks + lag, "shuffled", rng)
        ok, _, _ = run_model(groups, chunks, lag, in_place=False, polls=None, slots=2,
                             order=order, seed=seed, max_steps=20_000)
        stuck += not ok
        ok_index, exact, _ = run_model(groups, chunks, lag, in_place=False, polls=None, slots=2,
                                       order=dispatch_order(groups * chunks + lag, "index", rng),
                                       seed=seed, max_steps=200_000)
        assert ok_index and exact
    assert stuck > 0


def test_a_helper_that_read_an_overwritten_chunk_never_stands():
    """In place, with no polling, helpers race the chunks' own workgroups and
    some read chunks already overwritten by their outputs; the
    compare-and-swap drops those reductions, so the output stays exact.  The
    same model with a plain store in place of the compare-and-swap shows the
    race is real."""
    groups, chunks = 8, 4
    lag = chunks
    exact_runs = 0
    for seed in range(30):
        rng = random.Random(seed)
        order = dispatch_order(groups * chunks + lag, "shuffled", rng)
        ok, exact, _ = run_model(groups, chunks, lag, in_place=True, polls=0,
                                 slots=rng.choice([2, 4, 8]), order=order, seed=seed)
        assert ok and exact
        exact_runs += exact
    assert exact_runs == 30
    wrong = 0
    for seed in range(30):
        rng = random.Random(seed)
        order = dispatch_order(groups * chunks + lag, "shuffled", rng)
        ok, exact, _ = run_model(groups, chunks, lag, in_place=True, polls=0,
                                 slots=rng.choice([2, 4, 8]), order=order, seed=seed, cas=False)
        wrong += ok and not exact
    assert wrong > 0
