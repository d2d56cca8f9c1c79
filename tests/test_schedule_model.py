"""Slot-by-slot model of the full-attention kernel's ping-pong schedule.

The 8-wave full pass runs two 4-wave groups half a tile apart: each wave
alternates an MFMA phase X(j) (V^T P^T of tile j-1, then S^T of tile j) and
a softmax phase Y(j), a workgroup barrier ends every phase, and the second
group takes one extra barrier at the start. K and V tiles each rotate through
three LDS buffers (tile t in buffer t % 3). Y(j) issues the loads of K(j+2)
and V(j+1), and each wave waits for its share before the barrier that ends
Y(j). The prologue loads K(0), K(1) and V(0) and waits before the first
barrier.

Barriers split time into slots: slot s lies between barrier instances s and
s+1 for every wave at once. The model lists, for every tile count, each
group's LDS reads and writes per slot and checks that no buffer is written
while another tile in it may still be read, and that every tile is complete
before any wave reads it. It models the protocol, not the hardware: the GPU
tests check the kernel's results.
"""
import pytest

NBUF = 3


def schedule(ntiles):
    """Per group, the slots of its phases and its barrier count."""
    groups = {}
    for g, off in (("early", 0), ("late", 1)):
        x_slot = {j: 2 * j + off for j in range(ntiles + 1)}   # X(0..n); X(n) is V^T P^T only
        y_slot = {j: 2 * j + 1 + off for j in range(ntiles)}   # Y(0..n-1)
        # prologue barrier, the late group's extra one, one per phase, the early group's extra one
        barriers = 1 + (1 if off else 0) + (2 * ntiles + 1) + (0 if off else 1)
        groups[g] = dict(x=x_slot, y=y_slot, barriers=barriers)
    return groups


def events(ntiles):
    """(kind, tensor, tile, buffer, slot) for every LDS read and load, all groups."""
    ev = []
    # Prologue: every wave loads its share before barrier 0 ("slot -1").
    for g in ("early", "late"):
        ev.append(("write", "K", 0, 0, -1))
        if ntiles > 1:
            ev.append(("write", "K", 1, 1, -1))
        ev.append(("write", "V", 0, 0, -1))
    for g, sch in schedule(ntiles).items():
        for j, s in sch["x"].items():
            if j < ntiles:
                ev.append(("read", "K", j, j % NBUF, s))
            if j >= 1:
                ev.append(("read", "V", j - 1, (j - 1) % NBUF, s))
        for j, s in sch["y"].items():
            if j + 2 < ntiles:
                ev.append(("write", "K", j + 2, (j + 2) % NBUF, s))
            if j + 1 < ntiles:
                ev.append(("write", "V", j + 1, (j + 1) % NBUF, s))
    return ev


@pytest.mark.parametrize("ntiles", list(range(1, 14)) + [512])
def test_barrier_counts_match(ntiles):
    sch = schedule(ntiles)
    assert sch["early"]["barriers"] == sch["late"]["barriers"]


@pytest.mark.parametrize("ntiles", list(range(1, 14)) + [512])
def test_loads_complete_before_first_read(ntiles):
    ev = events(ntiles)
    for tensor in ("K", "V"):
        for t in range(ntiles):
            writes = [s for k, x, tt, b, s in ev if k == "write" and x == tensor and tt == t]
            reads = [s for k, x, tt, b, s in ev if k == "read" and x == tensor and tt == t]
            assert len(writes) == 2, (tensor, t)        # one share per group
            assert reads, (tensor, t)
            # A write in slot s has landed by barrier s+1; every read needs a later slot.
            assert max(writes) < min(reads), (tensor, t, writes, reads)


@pytest.mark.parametrize("ntiles", list(range(1, 14)) + [512])
def test_no_buffer_overwritten_while_read(ntiles):
    ev = events(ntiles)
    for tensor in ("K", "V"):
        for t_new in range(NBUF, ntiles):
            buf = t_new % NBUF
            t_old = t_new - NBUF
            old_reads = [s for k, x, tt, b, s in ev if k == "read" and x == tensor and tt == t_old and b == buf]
            new_writes = [s for k, x, tt, b, s in ev if k == "write" and x == tensor and tt == t_new and b == buf]
            assert old_reads and new_writes
            # Reads in slot s are consumed within it; a load may start only in a later slot.
            assert max(old_reads) < min(new_writes), (tensor, t_new, old_reads, new_writes)


@pytest.mark.parametrize("ntiles", list(range(1, 14)))
def test_groups_run_opposite_phases(ntiles):
    sch = schedule(ntiles)
    early_x = set(sch["early"]["x"].values())
    late_y = set(sch["late"]["y"].values())
    early_y = set(sch["early"]["y"].values())
    late_x = set(sch["late"]["x"].values())
    # Whenever both groups are inside their loops, one runs X while the other runs Y.
    both = set(range(1, 2 * ntiles))
    for s in both:
        assert (s in early_x and s in late_y) or (s in early_y and s in late_x), s
