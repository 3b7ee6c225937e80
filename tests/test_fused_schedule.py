"""The scheduling protocol of the one-launch pooled selection, simulated on the CPU.

Each (b, h) belongs to one work queue, (b*H + h) mod the number of XCDs; a
queue holds its heads' pooling items and then their selection items, and a
selection item of head h waits until every pooling item of h has finished. The
grid is persistent: a workgroup serves the queue of the XCD it runs on, taking
items by an atomic ticket until that queue is drained, and the last workgroup
to leave runs, in order, every queue that no workgroup took. This model replays
the protocol under any placement of workgroups on XCDs (including XCDs that get
none), any dispatch order and any limit on resident workgroups per XCD: every
run ends with all items done exactly once. It also shows why the ticket is
needed: waits on a fixed item per workgroup can leave every resident slot
waiting on pooling that is never dispatched.
"""
import random

import pytest


def queue_items(n_heads, n_queues, pool_per_head, sel_per_head, q):
    """Items of queue q in ticket order: ("pool", head) then ("sel", head)."""
    heads = list(range(q, n_heads, n_queues))
    return ([("pool", h) for h in heads for _ in range(pool_per_head)] +
            [("sel", h) for h in heads for _ in range(sel_per_head)])


def simulate(n_heads, n_queues, pool_per_head, sel_per_head, grid, resident, seed):
    """True if every item runs exactly once and every wait ends."""
    rng = random.Random(seed)
    # placement of the grid's workgroups on XCDs; some XCDs may get none
    used = rng.sample(range(n_queues), rng.randint(1, n_queues))
    xcd_of = [rng.choice(used) for _ in range(grid)]
    queues = [queue_items(n_heads, n_queues, pool_per_head, sel_per_head, q) for q in range(n_queues)]
    ticket = [0] * n_queues
    done = [0] * n_heads
    ran = [0] * n_queues
    pending = list(range(grid))         # workgroups not yet dispatched
    rng.shuffle(pending)
    running = {}                        # workgroup -> [queue, item or None, remaining work]
    exits = 0
    while pending or running:
        # dispatch up to `resident` workgroups per XCD
        for wg in list(pending):
            x = xcd_of[wg]
            if sum(1 for v in running.values() if v[0] == x) < resident:
                pending.remove(wg)
                running[wg] = [x, None, 0]
        moved = False
        for wg, slot in list(running.items()):
            x, item, left = slot
            if item is None:            # take a ticket from its queue
                t = ticket[x]
                ticket[x] += 1
                if t >= len(queues[x]):
                    del running[wg]     # drained: leave
                    exits += 1
                    moved = True
                    if exits == grid:   # the last one runs untaken queues in order
                        for q in range(n_queues):
                            while ticket[q] < len(queues[q]):
                                kind, h = queues[q][ticket[q]]
                                ticket[q] += 1
                                if kind == "sel" and done[h] < pool_per_head:
                                    return False
                                if kind == "pool":
                                    done[h] += 1
                                ran[q] += 1
                    continue
                slot[1], slot[2] = t, rng.randint(1, 4)
                moved = True
                continue
            kind, h = queues[x][item]
            if kind == "sel" and done[h] < pool_per_head:
                continue                # waiting on its head's pooling
            moved = True
            slot[2] -= 1
            if slot[2] == 0:
                if kind == "pool":
                    done[h] += 1
                ran[x] += 1
                slot[1] = None
        if not moved and not pending:
            return False
        if not moved and pending and all(
                sum(1 for v in running.values() if v[0] == xcd_of[wg]) >= resident for wg in pending):
            return False
    return ran == [len(q) for q in queues]


@pytest.mark.parametrize("resident", [1, 2, 3, 7, 64])
def test_queue_tickets_always_finish(resident):
    for seed in range(200):
        heads = 1 + seed % 5
        queues = 1 + seed % 8
        grid = 1 + (seed * 7) % 20
        assert simulate(heads, queues, 1 + seed % 5, 1 + (seed // 3) % 4, grid, resident, seed), \
            (resident, seed)


def simulate_fixed(n_heads, pool_per_head, sel_per_head, resident, seed):
    """One workgroup per item, item = workgroup index (no ticket), one queue:
    True if every item finishes."""
    rng = random.Random(seed)
    npool = n_heads * pool_per_head
    total = npool + n_heads * sel_per_head
    order = list(range(total))
    rng.shuffle(order)
    done = [0] * n_heads
    running = []
    finished = 0
    while finished < total:
        while order and len(running) < resident:
            running.append([order.pop(), rng.randint(1, 4)])
        moved = False
        for slot in list(running):
            item, left = slot
            if item >= npool and done[(item - npool) // sel_per_head] < pool_per_head:
                continue
            moved = True
            slot[1] = left - 1
            if slot[1] == 0:
                running.remove(slot)
                finished += 1
                if item < npool:
                    done[item // pool_per_head] += 1
        if not moved:
            return False
    return True


def test_block_index_order_can_stall():
    stalls = sum(not simulate_fixed(2, 3, 2, 2, seed) for seed in range(200))
    assert stalls > 0
