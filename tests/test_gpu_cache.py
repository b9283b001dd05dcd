"""GPU tests of the routed-expert cache (experts in pinned host memory, a
bounded set of expert slots in device memory).

The cache only changes where the expert bytes are read from, so every call
through it must give bitwise the outputs of the resident-expert decode call
on the same inputs; those are themselves checked against the oracle in
test_gpu_parity.py, and here once more on the first call.  The slot
policy (least recently used, ties to the lower slot, never a slot the batch
uses) is checked by replaying the routed expert sets through a plain Python
model of that policy and comparing the hit and miss counts.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

from test_gpu_parity import TOL_Y, per_token_err

pytestmark = pytest.mark.gpu


def _q():
    import quantized_routed_moe_router_amd as q
    return q


def lru_counts(n_slots, batches):
    """Hits and misses of the slot policy over batches of distinct experts
    (each in ascending order, the order the cache plans them in)."""
    slot_e = [-1] * n_slots
    stamp = [0] * n_slots
    where = {}
    hits = misses = 0
    for step, used in enumerate(batches, start=1):
        for e in used:
            if e in where:
                stamp[where[e]] = step
        for e in used:
            if e in where:
                hits += 1
                continue
            v = min((stamp[s], s) for s in range(n_slots) if stamp[s] != step)[1]
            if slot_e[v] >= 0:
                del where[slot_e[v]]
            slot_e[v], stamp[v], where[e] = e, step, v
            misses += 1
    return hits, misses


class SlotModel:
    """Plain model of the slot policy.  A call's used experts (ascending)
    split into the hits and the misses; the misses go through the slots in
    batches: batch 0 is the hits and the first S - hits misses, every later
    batch the next S misses.  Each batch is one step; its hits take the step
    as their stamp first, then each miss, in order, takes the slot with the
    smallest (stamp, slot) among those the step has not stamped.  A decode
    call is the one-batch case."""

    def __init__(self, n_slots):
        self.S = n_slots
        self.slot_e = [-1] * n_slots
        self.stamp = [0] * n_slots
        self.where = {}
        self.step = 0
        self.hits = self.misses = 0

    def call(self, used):
        S = self.S
        hit = [e for e in used if e in self.where]
        miss = [e for e in used if e not in self.where]
        room = S - len(hit)
        batches = [miss[:room]] + [miss[i:i + S] for i in range(room, len(miss), S)]
        for j, part in enumerate(batches):
            self.step += 1
            if j == 0:
                for e in hit:
                    self.stamp[self.where[e]] = self.step
            for e in part:
                v = min((self.stamp[s], s) for s in range(S) if self.stamp[s] != self.step)[1]
                if self.slot_e[v] >= 0:
                    del self.where[self.slot_e[v]]
                self.slot_e[v], self.stamp[v], self.where[e] = e, self.step, v
        self.hits += len(hit)
        self.misses += len(miss)
        return len(batches)


def _run_sequence(L0, dl, cache, Ts, seed_batch0=1):
    """Cached and resident decode over fresh batches of sizes Ts: bitwise
    equal outputs and routing; returns the routed expert sets."""
    q = _q()
    used = []
    for i, T in enumerate(Ts):
        x = dl.x_tensor(synth.make_x(L0.wl, L0.seed, T, batch=seed_batch0 + i))
        r1, r2 = dl.routing_buffers(T), dl.routing_buffers(T)
        y_res = dl.forward(x, q.MODE_DECODE, routing=r1)
        y_c = cache.forward(x, routing=r2)
        torch.cuda.synchronize()
        assert torch.equal(y_res.view(torch.int32), y_c.view(torch.int32)), f"call {i} T={T}"
        for k in r1:
            assert torch.equal(r1[k], r2[k]), (i, k)
        used.append(sorted(set(r1["topk_idx"].cpu().numpy().reshape(-1).tolist())))
    return used


def _mid(E=64, k=4, bits=2, bits_down=0, I=256):
    return synth.Workload("mid_cache", 0, T=1, H=512, E=E, I=I, k=k, x_dtype="f32", router_dtype="f32",
                          router_sigma=0.05, layer_id=0, bits=bits, bits_down=bits_down)


@pytest.mark.parametrize("bits,bits_down", [(2, 0), (4, 0), (2, 4), (4, 2), (5, 6)])
def test_cache_matches_resident_with_evictions(bits, bits_down):
    """E = 64, k = 4, 16 slots: batches of 1-4 tokens evict all the time
    (also with the down matrices in the other code width)."""
    q = _q()
    L0 = synth.make_layer(_mid(bits=bits, bits_down=bits_down))
    dl = q.from_layer_inputs(L0)
    cache = q.ExpertCache(dl, 16)
    # the first call also against the oracle
    bufs = dl.routing_buffers(1)
    y = cache.forward(dl.x_tensor(L0.x), routing=bufs)
    torch.cuda.synchronize()
    ref, _, _ = oracle.layer_inputs(L0)
    assert per_token_err(y.cpu().numpy(), ref) <= TOL_Y
    first = sorted(set(bufs["topk_idx"].cpu().numpy().reshape(-1).tolist()))
    Ts = [1, 2, 4, 3, 1, 4, 4, 2, 1, 3, 4, 4, 1, 2]
    used = _run_sequence(L0, dl, cache, Ts)
    calls, hits, misses = cache.stats()
    h, m = lru_counts(16, [first] + used)
    print(f"bits={bits}: {calls} calls, {hits} hits, {misses} misses")
    assert (calls, hits, misses) == (len(Ts) + 1, h, m)
    assert misses > 16  # evictions happened


def test_cache_t16_and_reset():
    """T = 16 (the register-pipeline decode kernels) with exactly T*k slots,
    then a reset: the counters restart and the first calls miss again."""
    q = _q()
    L0 = synth.make_layer(_mid(E=128, k=4))
    dl = q.from_layer_inputs(L0)
    cache = q.ExpertCache(dl, 64)
    used = _run_sequence(L0, dl, cache, [16, 16, 8, 16, 5, 16])
    calls, hits, misses = cache.stats()
    assert (calls, hits, misses) == (6, *lru_counts(64, used))
    cache.reset()
    used = _run_sequence(L0, dl, cache, [16, 3], seed_batch0=40)
    calls, hits, misses = cache.stats()
    assert (calls, hits, misses) == (2, *lru_counts(64, used))
    assert misses >= len(used[0])


def test_cache_all_slots_hit():
    """With a slot per expert, every expert misses once and then always hits."""
    q = _q()
    L0 = synth.make_layer(_mid(E=32, k=4))
    dl = q.from_layer_inputs(L0)
    cache = q.ExpertCache(dl, 32)
    used = _run_sequence(L0, dl, cache, [4] * 10)
    calls, hits, misses = cache.stats()
    assert misses == len(set().union(*map(set, used)))
    assert hits == sum(len(u) for u in used) - misses


@pytest.mark.parametrize("T", [2, 12])
def test_cache_with_shared_expert(T):
    """Routed experts through the cache beside a resident bf16 shared expert."""
    q = _q()
    wl = synth.Workload("cache_sh", 0, T=T, H=512, E=64, I=256, k=4, Is=96, x_dtype="bf16", router_dtype="bf16",
                        router_sigma=0.05, layer_id=0)
    L0 = synth.make_layer(wl)
    dl = q.from_layer_inputs(L0)
    cache = q.ExpertCache(dl, 48)
    used = _run_sequence(L0, dl, cache, [T] * 5)
    assert cache.stats() == (5, *lru_counts(48, used))


def test_cache_rejects_device_pointers():
    """Expert pointers that are not pinned host memory are refused before
    anything is launched."""
    q = _q()
    L0 = synth.make_layer(_mid())
    dl = q.from_layer_inputs(L0)
    cache = q.ExpertCache(dl, 16)
    x = dl.x_tensor(L0.x)
    with pytest.raises(q.Ds4MoeError) as ei:
        cache.forward(x, weights=dl.weights())  # device pointers
    assert ei.value.status == q.binding.DS4MOE_ERR_HOSTMEM
    with pytest.raises(q.Ds4MoeError) as ei:
        cache.forward(dl.x_tensor(synth.make_x(L0.wl, L0.seed, 5)))  # 5*4 = 20 experts > 16 slots
    assert ei.value.status == q.binding.DS4MOE_ERR_SHAPE


def test_cache_full_decode1():
    """Full-size layer (256 experts of 2048 x 4096, k = 8), 204 slots (80 %
    of the experts): decode calls bitwise equal to resident experts."""
    q = _q()
    L0 = synth.make_layer("prefill")
    dl = q.from_layer_inputs(L0)
    cache = q.ExpertCache(dl, 204)
    wl = synth.WORKLOADS["decode1"]
    used = []
    for b in range(8):
        x = dl.x_tensor(synth.make_x(wl, L0.seed, 1, batch=b))
        r1, r2 = dl.routing_buffers(1), dl.routing_buffers(1)
        y_res = dl.forward(x, q.MODE_DECODE, routing=r1)
        y_c = cache.forward(x, routing=r2)
        torch.cuda.synchronize()
        assert torch.equal(y_res.view(torch.int32), y_c.view(torch.int32)), b
        used.append(sorted(r1["topk_idx"].cpu().numpy().reshape(-1).tolist()))
    assert cache.stats() == (8, *lru_counts(204, used))


# ------------------------------------------------------------- prefill through the cache

def _run_prefill_sequence(L0, dl, cache, Ts, seed_batch0=1, model=None):
    """Cached and resident prefill over fresh batches of sizes Ts: bitwise
    equal outputs and routing; the slot model follows each call."""
    q = _q()
    nbs = []
    for i, T in enumerate(Ts):
        x = dl.x_tensor(synth.make_x(L0.wl, L0.seed, T, batch=seed_batch0 + i))
        r1, r2 = dl.routing_buffers(T), dl.routing_buffers(T)
        y_res = dl.forward(x, q.MODE_PREFILL, routing=r1)
        y_c = cache.forward_prefill(x, routing=r2)
        torch.cuda.synchronize()
        assert torch.equal(y_res.view(torch.int32), y_c.view(torch.int32)), f"call {i} T={T}"
        for k in r1:
            assert torch.equal(r1[k], r2[k]), (i, k)
        if model is not None:
            nbs.append(model.call(sorted(set(r1["topk_idx"].cpu().numpy().reshape(-1).tolist()))))
    return nbs


@pytest.mark.parametrize("bits,bits_down", [(2, 0), (4, 0), (2, 4), (4, 2), (5, 6)])
def test_prefill_cache_matches_resident(bits, bits_down):
    """E = 64, k = 4, 16 slots: batches of 1..700 tokens use up to all 64
    experts, so most calls stream their experts through the slots in several
    batches (80-token tiles); outputs bitwise those of resident experts, the
    first call also against the oracle, and the counters those of the slot
    model."""
    q = _q()
    L0 = synth.make_layer(_mid(bits=bits, bits_down=bits_down), T=200)
    dl = q.from_layer_inputs(L0)
    cache = q.ExpertCache(dl, 16)
    bufs = dl.routing_buffers(200)
    y = cache.forward_prefill(dl.x_tensor(L0.x), routing=bufs)
    torch.cuda.synchronize()
    ref, _, _ = oracle.layer_inputs(L0)
    assert per_token_err(y.cpu().numpy(), ref) <= TOL_Y
    model = SlotModel(16)
    model.call(sorted(set(bufs["topk_idx"].cpu().numpy().reshape(-1).tolist())))
    nbs = _run_prefill_sequence(L0, dl, cache, [300, 50, 1, 700, 128, 17, 300], model=model)
    assert cache.stats() == (8, model.hits, model.misses)
    assert max(nbs) >= 4 and min(nbs) == 1


@pytest.mark.parametrize("S", [1, 5, 63, 64])
def test_prefill_cache_slot_counts(S):
    """One slot (every expert its own batch) up to a slot per expert."""
    q = _q()
    L0 = synth.make_layer(_mid())
    dl = q.from_layer_inputs(L0)
    cache = q.ExpertCache(dl, S)
    model = SlotModel(S)
    _run_prefill_sequence(L0, dl, cache, [96, 3, 257], model=model)
    assert cache.stats() == (3, model.hits, model.misses)


def test_prefill_cache_64_token_tiles():
    """Intermediate size 128 (below 256): the 64-token GEMM kernels with the
    padded down projection, through the slots."""
    q = _q()
    L0 = synth.make_layer(_mid(I=128))
    dl = q.from_layer_inputs(L0)
    cache = q.ExpertCache(dl, 12)
    model = SlotModel(12)
    _run_prefill_sequence(L0, dl, cache, [130, 64, 1000], model=model)
    assert cache.stats() == (3, model.hits, model.misses)


def test_prefill_and_decode_share_the_cache():
    """Decode and prefill calls on one cache buffer: one slot policy, one
    set of counters; outputs bitwise those of resident experts."""
    q = _q()
    L0 = synth.make_layer(_mid())
    dl = q.from_layer_inputs(L0)
    cache = q.ExpertCache(dl, 16)
    model = SlotModel(16)
    for i, (mode, T) in enumerate([("p", 400), ("d", 4), ("d", 1), ("p", 33), ("d", 2), ("p", 900), ("d", 3)]):
        if mode == "p":
            _run_prefill_sequence(L0, dl, cache, [T], seed_batch0=60 + i, model=model)
        else:
            for used in _run_sequence(L0, dl, cache, [T], seed_batch0=60 + i):
                model.call(used)
    assert cache.stats() == (7, model.hits, model.misses)


def test_prefill_cache_with_shared_expert():
    """bf16 activations and router, a resident bf16 shared expert beside the
    routed experts streamed through the slots."""
    q = _q()
    wl = synth.Workload("cache_sh", 0, T=1, H=512, E=64, I=256, k=4, Is=96, x_dtype="bf16", router_dtype="bf16",
                        router_sigma=0.05, layer_id=0)
    L0 = synth.make_layer(wl)
    dl = q.from_layer_inputs(L0)
    cache = q.ExpertCache(dl, 20)
    model = SlotModel(20)
    _run_prefill_sequence(L0, dl, cache, [500, 70], model=model)
    assert cache.stats() == (2, model.hits, model.misses)


def test_prefill_cache_rejects_device_pointers():
    q = _q()
    L0 = synth.make_layer(_mid())
    dl = q.from_layer_inputs(L0)
    cache = q.ExpertCache(dl, 16)
    with pytest.raises(q.Ds4MoeError) as ei:
        cache.forward_prefill(dl.x_tensor(synth.make_x(L0.wl, L0.seed, 100)), weights=dl.weights())
    assert ei.value.status == q.binding.DS4MOE_ERR_HOSTMEM


def test_prefill_cache_full_size():
    """Full-size layer (256 experts of 2048 x 4096, k = 8), 204 slots (80 %
    of the experts), 2048-token prefills: every call uses all 256 experts,
    so it streams them in two batches; outputs bitwise those of resident
    experts, counters those of the slot model (after the first call 52
    experts are copied per call)."""
    q = _q()
    L0 = synth.make_layer("prefill")
    dl = q.from_layer_inputs(L0)
    cache = q.ExpertCache(dl, 204)
    model = SlotModel(204)
    nbs = _run_prefill_sequence(L0, dl, cache, [2048, 2048, 2048], model=model)
    assert nbs == [2, 2, 2]
    assert cache.stats() == (3, model.hits, model.misses)
    assert model.misses == 256 + 2 * 52
