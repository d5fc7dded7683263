"""CPU checks of the expert tier's replacement policy (md_expert_cache_plan)
against a model written here from its documented rule, and of the tier entry
points' argument checks (nothing is enqueued on these paths)."""
import ctypes

import numpy as np
import pytest

import moe_decode_amd as md

FAKE = 0x7F0000000000


class PolicyModel:
    """Hits keep their slots; each missed expert, in order of first
    appearance, takes the lowest empty slot, else the slot with the fewest
    uses (ties: least recently used, then lowest index) not used this step."""

    def __init__(self, E, S):
        self.slot_of = [-1] * E
        self.held = [-1] * S
        self.uses = [0] * S
        self.last = [0] * S
        self.step = 0
        self.hits = self.misses = 0

    def plan(self, idx):
        distinct = list(dict.fromkeys(int(e) for e in idx))
        self.step += 1
        for e in distinct:
            s = self.slot_of[e]
            if s >= 0:
                self.uses[s] += 1
                self.last[s] = self.step
                self.hits += 1
        misses = []
        for e in distinct:
            if self.slot_of[e] >= 0:
                continue
            empty = [s for s in range(len(self.held)) if self.held[s] < 0]
            if empty:
                v = empty[0]
            else:
                cand = [s for s in range(len(self.held)) if self.last[s] != self.step]
                v = min(cand, key=lambda s: (self.uses[s], self.last[s], s))
            if self.held[v] >= 0:
                self.slot_of[self.held[v]] = -1
            self.held[v] = e
            self.slot_of[e] = v
            self.uses[v] = 1
            self.last[v] = self.step
            self.misses += 1
            misses.append((e, v))
        return [self.slot_of[int(e)] for e in idx], misses


@pytest.mark.parametrize("E,S,k,T", [(12, 5, 2, 1), (8, 8, 2, 3), (64, 20, 8, 2), (256, 64, 8, 1), (40, 12, 3, 4)])
def test_policy_matches_model(E, S, k, T):
    rng = np.random.default_rng([E, S, k, T])
    c = md.ExpertCache(E, S)
    m = PolicyModel(E, S)
    # a skewed choice of experts so that hits, misses and evictions all occur
    w = rng.zipf(1.5, E).astype(np.float64)
    w /= w.sum()
    for step in range(200):
        idx = np.stack([rng.choice(E, size=k, replace=False, p=w) for _ in range(T)]).reshape(-1)
        if len(set(idx.tolist())) > S:
            continue
        slots, misses = c.plan(idx)
        slots_m, misses_m = m.plan(idx)
        assert slots.tolist() == slots_m and misses == misses_m, step
        assert c.hits == m.hits and c.misses == m.misses
    assert c.hits > 0 and (c.misses > S or E == S)      # evictions happened (when they can)
    # invariants of the state
    held = c.expert_in_slot
    for s, e in enumerate(held.tolist()):
        if e >= 0:
            assert c.slot_of_expert[e] == s


def test_plan_errors_leave_the_state_alone():
    c = md.ExpertCache(8, 3)
    c.plan(np.array([1, 2], dtype=np.int32))
    before = (c.slot_of_expert.copy(), c.expert_in_slot.copy(), c.uses.copy(), c.state.step)
    with pytest.raises(md.MDError) as ei:
        c.plan(np.array([1, 9], dtype=np.int32))
    assert ei.value.name == "MD_ERR_INVALID_ARG"
    with pytest.raises(md.MDError) as ei:
        c.plan(np.array([0, 3, 4, 5], dtype=np.int32))      # 4 distinct experts, 3 slots
    assert ei.value.name == "MD_ERR_UNSUPPORTED"
    after = (c.slot_of_expert, c.expert_in_slot, c.uses, c.state.step)
    assert all(np.array_equal(a, b) for a, b in zip(before[:3], after[:3])) and before[3] == after[3]
    # repeated ids in one step count once
    slots, misses = c.plan(np.array([2, 2, 7], dtype=np.int32))
    assert misses == [(7, 2)] and slots.tolist() == [1, 1, 2]


def _layer(E, **kw):
    d = md.MoELayerDesc()
    d.H, d.F, d.E, d.k, d.act, d.type = 256, 512, E, 2, 0, md.Q8_0
    d.gate_q = d.up_q = d.down_q = d.W_r = FAKE
    for a, v in kw.items():
        setattr(d, a, v)
    return d


def test_fill_and_forward_argument_checks():
    L = md.lib()
    src, dst = _layer(8), _layer(4)
    me = (ctypes.c_int32 * 2)(1, 2)
    ms = (ctypes.c_int32 * 2)(0, 4)                          # slot 4 of 4
    assert md.STATUS[L.md_expert_cache_fill(ctypes.byref(src), ctypes.byref(dst), me, ms, 2, None)] == \
        "MD_ERR_INVALID_ARG"
    bad = _layer(4, F=768)
    ms = (ctypes.c_int32 * 2)(0, 1)
    assert md.STATUS[L.md_expert_cache_fill(ctypes.byref(src), ctypes.byref(bad), me, ms, 2, None)] == "MD_ERR_SHAPE"
    sz = ctypes.c_size_t(0)
    assert L.md_moe_cached_workspace_size(ctypes.byref(src), ctypes.byref(dst), 3, ctypes.byref(sz)) == 0
    assert sz.value > 0
    c = md.ExpertCache(8, 3)                                 # 3 slots, but dst has 4
    assert md.STATUS[L.md_moe_cached_forward(ctypes.byref(src), ctypes.byref(dst), ctypes.byref(c.state), FAKE, 1,
                                             FAKE, None, None, FAKE, 1 << 30, None, None, None)] == "MD_ERR_SHAPE"
    c4 = md.ExpertCache(8, 4)
    assert md.STATUS[L.md_moe_cached_forward(ctypes.byref(src), ctypes.byref(dst), ctypes.byref(c4.state), FAKE, 1,
                                             FAKE, None, None, FAKE, 1 << 30, None, FAKE, None)] == \
        "MD_ERR_INVALID_ARG"                                # a copy stream without its event
    sh = _layer(4, has_shared=1)
    assert md.STATUS[L.md_moe_experts_forward(ctypes.byref(sh), FAKE, 1, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)] in \
        ("MD_ERR_UNSUPPORTED", "MD_ERR_INVALID_ARG")
    d = _layer(4)
    assert md.STATUS[L.md_moe_experts_forward(ctypes.byref(d), FAKE, 1, None, FAKE, FAKE, FAKE, 1 << 30, None)] == \
        "MD_ERR_INVALID_ARG"
