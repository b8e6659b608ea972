"""CPU model of the chained forward launch's tile protocol.

``gmm_chain_kernel`` runs both forward products of the grouped GEMM in one
persistent launch: positions [0, total1) are gate/up tiles, [total1, total)
down tiles; a down tile of row tile m may start only once every gate/up tile
of m has finished.  The workgroups of each XCD take positions from their
XCD's counter in blocks of ``wpx``, and once that sequence is used up they
go on with the next XCD's counter; a workgroup owns a gate/up tile only
after exchanging its start word from 0 to 1, and a waiting down tile first
runs every unstarted gate/up tile of its row tile itself.

This model replays that protocol (thread 0's decisions, with one step of
each tile's work per tick) with random tile durations and workgroups that
start late or never until the rest is done, and checks what the kernel
relies on: every tile runs exactly once, a down tile starts only after its
row tile's gate/up tiles, and no waiter waits on a tile nobody runs (the run
ends).  It is a model of the protocol, not of the kernel's code.
"""
import random

import pytest

GM = 8   # row tiles per band


def mtile_of(t, nb, mt):
    band = GM * nb
    first = (t // band) * GM
    return first + (t % band) % min(GM, mt - first)


def tile_at(mi, nbi, nb, mt):
    first = mi // GM * GM
    return first * nb + (mi - first) + nbi * min(GM, mt - first)


def run(mt, nb1, nb2, nwg, seed, late=None):
    rnd = random.Random(seed)
    total1, total = mt * nb1, mt * nb1 + mt * nb2
    nx = 8 if nwg % 8 == 0 else 1
    wpx = nwg // nx
    ctr = [0] * nx
    st = [0] * total1
    dep = [0] * mt
    done = [0] * total
    started2 = []

    def wg(b):
        vx = [b % nx]

        def draw():
            v = ctr[vx[0]]
            ctr[vx[0]] += 1
            return v

        def pos_of(k):
            c = (k // wpx) * nwg + vx[0] * wpx + k % wpx
            tries = 1
            while c >= total and tries < nx:
                vx[0] = (vx[0] + 1) % nx
                k2 = draw()
                c = (k2 // wpx) * nwg + vx[0] * wpx + k2 % wpx
                tries += 1
            return c

        def take(t):
            old, st[t] = st[t], 1
            return old == 0

        nxt, pend, grab = draw(), -1, 0
        yield 1
        while True:
            cmd = total
            while True:
                if pend < 0:
                    k = nxt
                    while True:
                        c = pos_of(k)
                        if c >= total or c >= total1 or take(c):
                            break
                        k = draw()
                        yield 1
                    if c >= total:
                        break
                    grab = draw()
                    if c < total1:
                        cmd = c
                        break
                    pend = c
                mi = mtile_of(pend - total1, nb2, mt)
                if dep[mi] < nb1:
                    steal = next((t1 for t1 in (tile_at(mi, n, nb1, mt) for n in range(nb1))
                                  if st[t1] == 0 and take(t1)), -1)
                    if steal >= 0:
                        cmd = steal
                        break
                    spins = 0
                    while dep[mi] < nb1:     # only tiles that someone runs
                        spins += 1
                        assert spins < 20000, "a waiter waits on a tile nobody runs"
                        yield 1
                cmd, pend = pend, -1
                break
            if cmd >= total:
                return
            if cmd >= total1:
                mi = mtile_of(cmd - total1, nb2, mt)
                assert all(done[tile_at(mi, n, nb1, mt)] == 1 for n in range(nb1))
                started2.append(cmd)
                yield rnd.randint(8, 12)
                done[cmd] += 1
            else:
                yield rnd.randint(20, 45)
                done[cmd] += 1
                dep[mtile_of(cmd, nb1, mt)] += 1
            nxt = grab

    start = {b: (late(b) if late else 0) for b in range(nwg)}
    gens = {b: wg(b) for b in range(nwg)}
    wake = dict(start)
    now = 0
    while gens:
        now += 1
        for b in list(gens):
            if wake[b] <= now:
                try:
                    wake[b] = now + next(gens[b])
                except StopIteration:
                    del gens[b]
        assert now < 10 ** 6
    assert done == [1] * total
    assert sorted(started2) == list(range(total1, total))


SHAPES = [(43, 16, 30), (1, 1, 1), (9, 2, 3), (8, 16, 30), (17, 4, 2), (3, 16, 30), (100, 2, 30)]


@pytest.mark.parametrize("mt,nb1,nb2", SHAPES)
@pytest.mark.parametrize("nwg", [256, 16, 8])
def test_every_tile_once_in_dependency_order(mt, nb1, nb2, nwg):
    for seed in range(2):
        run(mt, nb1, nb2, nwg, seed, late=lambda b: random.Random(b).choice([0, 0, 0, 50, 400]))


@pytest.mark.parametrize("mt,nb1,nb2", [(43, 16, 30), (9, 2, 3), (100, 2, 30)])
def test_an_absent_xcd_does_not_stall_the_others(mt, nb1, nb2):
    # XCD 3's workgroups start only after the others could have finished:
    # its gate/up tiles are taken over by the waiting down tiles, and no
    # waiter spins long (the model asserts a bounded spin)
    run(mt, nb1, nb2, 256, 0, late=lambda b: 30000 if b % 8 == 3 else 0)
