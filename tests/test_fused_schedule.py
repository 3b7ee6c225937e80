"""The scheduling protocol of the one-launch pooled selection, simulated on the CPU.

The kernel's grid holds pooling items (head-major) and then selection items
(head-major). A workgroup takes one item by an atomic ticket when it starts,
and a selection item of head h waits until every pooling item of h has
finished. This model replays that protocol under any dispatch order the
hardware may choose and any limit on resident workgroups. Every run ends with
all items done. It also shows why the ticket is needed: the same waits with
item = workgroup index can leave every resident slot waiting on pooling that
is never dispatched.
"""
import random

import pytest


def simulate(n_heads, pool_per_head, sel_per_head, resident, seed, ticketed=True):
    """True if every item finishes; False if no resident workgroup can move."""
    rng = random.Random(seed)
    npool = n_heads * pool_per_head
    total = npool + n_heads * sel_per_head
    order = list(range(total))          # the order in which workgroups get dispatched
    rng.shuffle(order)
    next_ticket = 0
    done = [0] * n_heads
    running = []                        # [item, remaining work]
    finished = 0
    while finished < total:
        while order and len(running) < resident:
            wg = order.pop()
            item = next_ticket if ticketed else wg
            next_ticket += 1
            running.append([item, rng.randint(1, 4)])
        moved = False
        for slot in list(running):
            item, left = slot
            if item >= npool:
                h = (item - npool) // sel_per_head
                if done[h] < pool_per_head:
                    continue            # waiting on its head's pooling
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


@pytest.mark.parametrize("resident", [1, 2, 3, 7, 64])
def test_ticket_order_always_finishes(resident):
    for seed in range(200):
        heads = 1 + seed % 4
        assert simulate(heads, 1 + seed % 5, 1 + (seed // 3) % 4, resident, seed), (resident, seed)


def test_block_index_order_can_stall():
    stalls = sum(not simulate(2, 3, 2, 2, seed, ticketed=False) for seed in range(200))
    assert stalls > 0
    assert all(simulate(2, 3, 2, 2, seed, ticketed=True) for seed in range(200))
