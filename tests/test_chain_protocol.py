"""CPU model of the synchronisation protocol of the chained GEMV kernel.

The kernel (layer_sliced_quantized_amd/csrc/chain.hip) runs several
dependent products in one launch.  Workgroup index i picks the product and
its (row group, split): the first indices belong to product 0, the next to
product 1, and so on.  The hardware hands the launch's workgroups to the 8
XCDs in turn (index i to XCD i mod 8), and each XCD starts its share in index
order as room frees up.  A workgroup first reads the launch number k - 1 from
copy (i mod 64) of the last product's ready flag; a workgroup of product
p > 0 then waits until copy (i mod 64) of product p - 1's ready flag reaches
k.  The last split of each row group counts the row group as done, and the
row groups are counted in groups of ceil(row_groups / 32) on one counter
each; the workgroup that completes a group counts it on the product's
counter, and the one that brings that to k * groups sets every copy of the
ready flag to k.

This model replays that protocol step by step under adversarial schedules:
at most R workgroups resident on each XCD (down to one), the resident ones
advanced in random order, several launches of the same chain.  It checks
what the kernel relies on: the launch always drains (no workgroup waits on
one that cannot start), every workgroup reads the right launch number, a
product starts only after the previous one has finished, and the counters
stay consistent across launches.
"""
import random

import pytest


class Chain:
    def __init__(self, products):
        # products: [(row_groups, splits)]
        self.products = products
        self.nwg = [rg * ks for rg, ks in products]
        self.grid = sum(self.nwg)
        self.done = [0] * len(products)
        self.ready = [[0] * 64 for _ in products]
        self.split_tickets = [dict() for _ in products]
        self.group_done = [dict() for _ in products]

    def place(self, id_):
        p = 0
        while p + 1 < len(self.nwg) and id_ >= self.nwg[p]:
            id_ -= self.nwg[p]
            p += 1
        return p, id_


def run_launches(products, launches, resident, seed, xcds=8, reverse=False):
    rng = random.Random(seed)
    ch = Chain(products)
    copies = 64
    last = len(products) - 1
    for launch in range(launches):
        queues = [[i for i in range(ch.grid) if i % xcds == x] for x in range(xcds)]
        if reverse:   # a dispatcher that starts the highest indices first (not what the hardware does)
            queues = [q[::-1] for q in queues]
        running = [[] for _ in range(xcds)]
        completed_products = []
        product_rows_done = [0] * len(products)
        steps = 0
        while any(queues) or any(running):
            for x in range(xcds):
                while queues[x] and len(running[x]) < resident:
                    i = queues[x].pop(0)
                    epoch = ch.ready[last][i % copies] + 1
                    assert epoch == launch + 1, "a workgroup read another launch's number"
                    p, pid = ch.place(i)
                    running[x].append({"p": p, "id": pid, "i": i, "epoch": epoch, "state": "wait" if p > 0 else "work"})
            busy = [x for x in range(xcds) if running[x]]
            assert busy, "no workgroup can run: the launch cannot drain"
            x = rng.choice(busy)
            wg = rng.choice(running[x])
            steps += 1
            assert steps < 20_000_000, "the model did not finish"
            p, epoch = wg["p"], wg["epoch"]
            if wg["state"] == "wait":
                if ch.ready[p - 1][wg["i"] % copies] - epoch >= 0:
                    assert product_rows_done[p - 1] == products[p - 1][0], "started before its input was complete"
                    wg["state"] = "work"
                else:
                    # a deadlock: no resident workgroup can proceed and no XCD has room to start one
                    def can_go(w):
                        return w["state"] == "work" or ch.ready[w["p"] - 1][w["i"] % copies] - w["epoch"] >= 0
                    stuck = not any(can_go(w) for r in running for w in r) and \
                        not any(queues[y] and len(running[y]) < resident for y in range(xcds))
                    assert not stuck, "every resident workgroup waits and none that could help can start"
                continue
            rgs, ks = products[p]
            rg, k = divmod(wg["id"], ks)
            cnt = ch.split_tickets[p].get(rg, 0)
            running[x].remove(wg)
            if cnt + 1 < ks:
                ch.split_tickets[p][rg] = cnt + 1
                continue
            ch.split_tickets[p][rg] = 0
            product_rows_done[p] += 1
            # two-level count: groups of gsize row groups, then the groups
            gsize = (rgs + 31) // 32
            g = rg // gsize
            ngroups = (rgs + gsize - 1) // gsize
            in_group = min(gsize, rgs - g * gsize)
            old = ch.group_done[p].get(g, 0)
            ch.group_done[p][g] = (old + 1) % 2**32
            if (old + 1) % 2**32 != (epoch * in_group) % 2**32:
                continue
            old = ch.done[p]
            ch.done[p] = (old + 1) % 2**32
            if (old + 1) % 2**32 == (epoch * ngroups) % 2**32:
                assert product_rows_done[p] == rgs
                for c in range(copies):
                    ch.ready[p][c] = epoch
                completed_products.append(p)
        assert completed_products == list(range(len(products))), completed_products
        assert all(f == launch + 1 for r in ch.ready for f in r)


# the chains of the hybrid's layers at hidden 5120 (row groups, splits): mixer
# output, gate/up, down, next input projections; scaled down 8x in row groups so
# the model runs quickly, with the same split counts
SHAPES = {
    "deltanet_layer": [(10, 4), (68, 2), (10, 8), (33, 4)],
    "deltanet_layer_with_update": [(16, 1), (10, 4), (68, 2), (10, 8), (33, 4)],
    "attention_layer": [(10, 4), (68, 2), (10, 8), (32, 4)],
    "last_layer": [(10, 4), (68, 2), (10, 8)],
    "no_ffn": [(3, 1), (5, 2)],
    # a launch over a run of DeltaNet layers: each layer's update waits for the
    # input projections before it, in the same launch
    "three_deltanet_layers": [(16, 1), (10, 4), (68, 2), (10, 8), (33, 4)] * 3,
    "attention_then_deltanet_layers": [(10, 4), (68, 2), (10, 8), (33, 4)] +
                                      [(16, 1), (10, 4), (68, 2), (10, 8), (33, 4)] * 3,
    "many_row_groups": [(70, 1), (300, 2), (33, 3)],
}


@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("resident", [1, 2, 7, 64, 10_000])
@pytest.mark.parametrize("xcds", [1, 8])
def test_chain_protocol_drains_in_order(shape, resident, xcds):
    run_launches(SHAPES[shape], launches=3, resident=resident, seed=resident * 7 + xcds, xcds=xcds)


def test_counters_wrap_safely():
    # 32-bit counters wrap: the done target is compared modulo 2^32
    rgs = 257
    epoch = (2**32 // rgs) + 5
    done_before = ((epoch - 1) * rgs) % 2**32
    assert (done_before + rgs) % 2**32 == (epoch * rgs) % 2**32
    # the ready compare is wrap-safe: (flag - epoch) as a signed 32-bit value
    def reached(flag, ep):
        d = (flag - ep) % 2**32
        return d < 2**31
    assert reached(5, 5) and not reached(4, 5)
    assert reached(2, 2**32 - 1) and not reached(2**32 - 1, 3)     # across the wrap


def test_model_detects_the_deadlock_of_another_dispatch_order():
    """With the highest indices started first and little room, waiting
    workgroups of later products fill the machine: the model must see it."""
    with pytest.raises(AssertionError, match="none that could help"):
        run_launches(SHAPES["deltanet_layer"], launches=1, resident=2, seed=3, reverse=True)
