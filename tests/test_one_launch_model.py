"""A CPU model of the one-launch chain call's work distribution.

The one-launch call runs the statistics chunks and the sampling workgroups of
every sequence in one grid. Sampling roles wait (spin) until every chunk of
their sequence has been counted. Roles are not tied to block indices: a
workgroup of sequence b's block range takes the next ticket of b's queue when
it starts, tickets 0 .. cps-1 stream chunks, later tickets sample.

This model dispatches the grid's workgroups in an arbitrary order into a
limited number of slots (resident workgroups), with slots also held by
another launch's spinning workgroups, and checks that every workgroup
finishes: a sampling role only ever waits for chunks whose tickets were taken
by running workgroups, and those wait for nothing. A planted mistake (roles
by block index, as a plain grid would assign them) must deadlock for some
dispatch orders: the model is able to see the failure it rules out.
"""
import numpy as np
import pytest


def _simulate(B, cps, nblk, slots, order, by_ticket, foreign=0, rng=None, max_steps=200_000):
    """Run one launch. Returns True if every workgroup finished, False on a
    deadlock (nothing can run, work remains). `order` is the dispatch order
    of the block indices; `foreign` slots are held for the whole run by
    workgroups of another launch that never finish (the worst case)."""
    rng = rng or np.random.default_rng(0)
    n = B * (cps + nblk)
    nstats = B * cps

    def seq_of(blk):
        return blk // cps if blk < nstats else (blk - nstats) // nblk

    ticket = [0] * B
    done = [0] * B
    pending = list(order)
    running = []  # [role, b, remaining_work]
    free = slots - foreign
    finished = 0
    for _ in range(max_steps):
        # dispatch into free slots, in the given order
        while free > 0 and pending:
            blk = pending.pop(0)
            b = seq_of(blk)
            if by_ticket:
                t = ticket[b]
                ticket[b] += 1
            else:
                t = blk % cps if blk < nstats else cps + (blk - nstats) % nblk
            role = "stats" if t < cps else "sample"
            running.append([role, b, int(rng.integers(1, 4))])
            free -= 1
        if not running:
            return finished == n
        progressed = False
        for w in list(running):
            role, b, left = w
            if role == "sample" and done[b] < cps:
                continue  # spinning
            w[2] -= 1
            progressed = True
            if w[2] == 0:
                running.remove(w)
                free += 1
                finished += 1
                if role == "stats":
                    done[b] += 1
        if not progressed:
            return False
    raise AssertionError("model did not settle")


@pytest.mark.parametrize("B,cps,nblk,slots", [(4, 6, 3, 5), (8, 11, 4, 12), (3, 2, 5, 4), (16, 4, 4, 9)])
def test_tickets_finish_in_any_dispatch_order(B, cps, nblk, slots):
    rng = np.random.default_rng(1000 + B * cps + nblk)
    n = B * (cps + nblk)
    orders = [np.arange(n)[::-1], np.concatenate([np.arange(B * cps, n), np.arange(B * cps)])]
    orders += [rng.permutation(n) for _ in range(300)]
    for order in orders:
        for foreign in (0, slots - 1):
            assert _simulate(B, cps, nblk, slots, list(order), by_ticket=True, foreign=foreign, rng=rng)


def test_roles_by_block_index_can_deadlock():
    # planted mistake: sampling roles fixed by block index; dispatching the
    # sampling blocks first fills every slot with spinning workgroups
    B, cps, nblk, slots = 4, 6, 3, 5
    n = B * (cps + nblk)
    sampling_first = list(np.concatenate([np.arange(B * cps, n), np.arange(B * cps)]))
    assert not _simulate(B, cps, nblk, slots, sampling_first, by_ticket=False)
    # and the in-order dispatch the block layout is designed for finishes
    assert _simulate(B, cps, nblk, slots, list(range(n)), by_ticket=False)
