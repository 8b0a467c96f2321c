"""CPU model of the attention kernel's two-group barrier schedule (k_sparse_attn in
csrc/attention.hip).

A workgroup holds two work items (groups g = 0, 1 of four waves) with n0 and n1 kept tiles.  Each
group runs its own loop; the loops must meet the same workgroup barriers (s_barrier counts waves, not
program locations), so a miscount would hang the GPU.  The model below follows the kernel's control
flow event by event -- the prologue DMA, the group-1 idle phase, the MFMA and VALU phases, the two
barrier kinds and the padding loop up to P + 1 barriers with the kernel's P = max(2 n0 + 1, 2 n1 + 2)
-- and checks, for every pair of counts:
  * both groups pass the same number of barriers;
  * in no phase do both groups run their MFMA phase (the ping-pong alternation);
  * the LDS buffers (per group: K double buffer, one V^T buffer) are never read before the DMA that
    fills them has been waited for by a DMA barrier, and never refilled before a barrier that
    follows their last read (LDS reads drain at every barrier; DMA only at the DMA barrier).
"""
import numpy as np
import pytest


def kernel_P(n0, n1):
    return max(2 * n0 + 1, 2 * n1 + 2)


def group_events(g, n, n_other):
    """The kernel's control flow of group g with n kept tiles: a list of events
    ("bar", kind) | ("dma", buf) | ("read", buf) | ("stale", buf) | ("phase", kind); a stale read
    is one whose result is discarded."""
    n0, n1 = (n, n_other) if g == 0 else (n_other, n)
    P = kernel_P(n0, n1)
    ev = []
    if n > 0:
        ev.append(("dma", "k0"))                       # stage_k(K[0], tile 0)
    if g == 1:
        ev.append(("bar", "lds"))                      # B_-1: group 1's phase 0 is idle
    ev.append(("bar", "dma"))
    passed = 1 + g

    def mfma_phase(t):
        ev.append(("phase", "mfma"))
        if t >= 1:
            ev.append(("read", "v"))                   # pv_tile: V^T of tile t-1
        if t + 1 < n:
            ev.append(("dma", "k%d" % ((t + 1) & 1)))  # stage_k of tile t+1
        # qk_scores; at t = n its scores are never used and the buffer may hold anything
        ev.append(("read" if t < n else "stale", "k%d" % (t & 1)))

    if n > 0:
        mfma_phase(0)
        ev.append(("bar", "lds"))
        passed += 1
        for t in range(n):
            ev.append(("phase", "valu"))
            ev.append(("dma", "v"))                    # stage_vt of tile t
            ev.append(("bar", "dma"))
            mfma_phase(t + 1)
            ev.append(("bar", "lds"))
            passed += 2
    while passed < P + 1:
        ev.append(("bar", "lds"))
        passed += 1
    return ev


def check_pair(n0, n1):
    evs = [group_events(0, n0, n1), group_events(1, n1, n0)]
    bars = [[e for e in ev if e[0] == "bar"] for ev in evs]
    assert len(bars[0]) == len(bars[1]) == kernel_P(n0, n1) + 1, (n0, n1)

    # phase kind of each group between consecutive barriers (index = barriers passed before it)
    kinds = []
    for ev in evs:
        k, cur = [], "idle"
        for e in ev:
            if e[0] == "phase":
                cur = e[1]
            elif e[0] == "bar":
                k.append(cur)
                cur = "idle"
        kinds.append(k)
    for p, (a, b) in enumerate(zip(kinds[0], kinds[1])):
        assert not (a == "mfma" and b == "mfma"), f"({n0}, {n1}): both groups in MFMA before barrier {p}"

    # LDS hazards, per group (each group owns its buffers)
    for ev in evs:
        state = {}          # buf -> "landed" | "inflight" | None
        read_since_bar = set()
        for e in ev:
            if e[0] == "dma":
                assert e[1] not in read_since_bar, f"({n0}, {n1}): {e[1]} refilled before its reads drained"
                assert state.get(e[1]) != "inflight", f"({n0}, {n1}): {e[1]} refilled while in flight"
                state[e[1]] = "inflight"
            elif e[0] == "read":
                assert state.get(e[1]) == "landed", f"({n0}, {n1}): {e[1]} read before its DMA was waited for"
                read_since_bar.add(e[1])
            elif e[0] == "stale":
                read_since_bar.add(e[1])
            elif e[0] == "bar":
                read_since_bar.clear()
                if e[1] == "dma":
                    for b, s in state.items():
                        if s == "inflight":
                            state[b] = "landed"


def test_schedule_all_pairs_up_to_48():
    for n0 in range(49):
        for n1 in range(49):
            check_pair(n0, n1)


def test_schedule_large_and_sampled_pairs_up_to_1024():
    rng = np.random.default_rng(0)
    pairs = [(a, b) for a in (0, 1, 2, 511, 1023, 1024) for b in (0, 1, 2, 512, 1023, 1024)]
    pairs += [tuple(int(v) for v in rng.integers(0, 1025, size=2)) for _ in range(300)]
    for n0, n1 in pairs:
        check_pair(n0, n1)


def test_model_catches_a_short_padding():
    """A P one short of the kernel's (the padding loop ending a barrier early) is detected."""
    with pytest.raises(AssertionError):
        global kernel_P
        saved = kernel_P
        try:
            kernel_P = lambda n0, n1: max(2 * n0 + 1, 2 * n1 + 1)
            for n0 in range(4):
                for n1 in range(4):
                    check_pair(n0, n1)
        finally:
            kernel_P = saved
