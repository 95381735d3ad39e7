"""Host-side model of the DMA schedules of the ping-pong kernels.

The ping-pong attention kernel (attn_bf16_pp_kernel) and the attention-mass
kernel (mass_bf16_kernel) stream K (and V) tiles into LDS rings through
direct-to-LDS DMA issued by dedicated waves, with explicit vmcnt waits before
the barriers instead of a fence. Correctness rests on three invariants, checked
here by simulation for every tile count up to 64:

* a ring slot is refilled only after the last phase that reads its previous
  tile has ended (the issue happens after the barrier that opens a later slot);
* every tile has landed before the barrier that opens the first phase reading
  it: the issuing wave's vmcnt wait allows in flight only loads issued after
  that tile (vmcnt counts a wave's loads in issue order);
* a wave never needs more than 63 loads counted (the vmcnt field's range).

The constants mirror the kernels: 64-key tiles of d = 128 bf16 (16 DMA
instructions of 1 KB per K or V tile), K ring of 4 slots issued 3 tiles ahead
and V ring of 5 slots issued 3 tiles ahead in the attention kernel, K ring of 4
slots issued 3 tiles ahead by two waves (8 instructions each) in the mass
kernel. A slot is one phase: slot 2t opens the phase that reads tile t for the
leading half of the workgroup, slot 2t + 1 the same phase for the lagging half.
"""
import pytest


def _landed_ok(seq, need_tile, slot, allowed, ipt):
    """seq: this wave's issues as (slot, tile), in order. At the wait before
    the barrier that opens `slot`, the issues made so far are those with an
    issue slot < `slot`; the wait leaves `allowed` instructions in flight. The
    tile is landed iff every issue after it accounts for at least `allowed`."""
    done = [x for x in seq if x[0] < slot]
    pos = [i for i, x in enumerate(done) if x[1] == need_tile]
    assert pos, f"tile {need_tile} not issued before slot {slot}"
    after = (len(done) - 1 - pos[0]) * ipt
    return allowed <= after and allowed <= 63


def _attention_schedule(T, NSK=4, NSV=5, IPT=16, KA=None, VA=None):
    KA = NSK - 1 if KA is None else KA
    VA = NSV - 2 if VA is None else VA
    ok = lambda x: 0 <= x < T
    # prologue issues carry slot -1; K(t + KA) after the barrier of slot 2t,
    # V(t + VA) after the barrier of slot 2t + 1
    K = [(-1, t) for t in range(KA) if ok(t)] + [(2 * t, t + KA) for t in range(T + 1) if ok(t + KA)]
    V = [(-1, t) for t in range(VA) if ok(t)] + [(2 * t + 1, t + VA) for t in range(T + 1) if ok(t + VA)]
    # readers: K of tile t in slots 2t, 2t+1 (M(t) of each half), V of tile t
    # in slots 2t+2, 2t+3 (M(t+1), the PV part)
    reads = {"K": {t: [2 * t, 2 * t + 1] for t in range(T)},
             "V": {t: [2 * t + 2, 2 * t + 3] for t in range(T)}}

    def inst(a, b):  # the kernel's count of a wave's DMA instructions for tiles [a, b]
        lo, hi = max(a, 0), min(b, T - 1)
        return (hi - lo + 1) * IPT if hi >= lo else 0

    return K, V, reads, KA, VA, NSK, NSV, inst


@pytest.mark.parametrize("T", range(0, 65))
def test_attention_pp_schedule(T):
    K, V, reads, KA, VA, NSK, NSV, inst = _attention_schedule(T)
    for name, seq, ns in (("K", K, NSK), ("V", V, NSV)):
        issued = {t: q for q, t in seq}
        assert sorted(issued) == list(range(T)), name
        for q, t in seq:  # ring hazard: the previous occupant's last read ended
            if t - ns >= 0:
                assert max(reads[name][t - ns]) < q, (name, T, t)
        for t, slots in reads[name].items():  # issued before the barrier of its first reader
            assert issued[t] < min(slots)
    for t in range(T + 1):  # waits before the barrier of slot 2t
        if t < T:  # K issuer: K(t) landed, K(t+1 .. t+KA-1) may be in flight
            assert _landed_ok(K, t, 2 * t, inst(t + 1, t + KA - 1), 16)
        if t >= 1:  # V issuer: V(t-1) landed, V(t .. t+VA-1) may be in flight
            assert _landed_ok(V, t - 1, 2 * t, inst(t, t + VA - 1), 16)


@pytest.mark.parametrize("T", range(0, 65))
def test_mass_pp_schedule(T):
    NS, KA, IPW = 4, 3, 8
    ok = lambda x: 0 <= x < T
    # each of the two issuing waves: prologue tiles 0..KA-1, then tile u + KA
    # after the barrier of slot 2u
    seq = [(-1, u) for u in range(KA) if ok(u)] + [(2 * u, u + KA) for u in range(T + 1) if ok(u + KA)]
    reads = {u: [2 * u, 2 * u + 1] for u in range(T)}  # M(u) of the leading, then the lagging half
    issued = {u: q for q, u in seq}
    assert sorted(issued) == list(range(T))
    for q, u in seq:
        if u - NS >= 0:
            assert max(reads[u - NS]) < q, (T, u)
    for u, slots in reads.items():
        assert issued[u] < min(slots)

    def inst(a, b):
        lo, hi = max(a, 0), min(b, T - 1)
        return (hi - lo + 1) * IPW if hi >= lo else 0

    for u in range(T):
        assert _landed_ok(seq, u, 2 * u, inst(u + 1, u + KA - 1), IPW)
    # column sums of tile u: written in slot 2u+1 (leading half) and 2u+2
    # (lagging half) into buffer u % 2, read in slot 2u+3; the next writes to
    # that buffer (tile u+2) come in slots 2u+5 and 2u+6
    for u in range(T):
        writes, read = (2 * u + 1, 2 * u + 2), 2 * u + 3
        assert max(writes) < read
        if u + 2 < T:
            assert min(2 * (u + 2) + 1, 2 * (u + 2) + 2) > read


def test_schedule_model_catches_mistakes():
    # V issued three tiles ahead into a ring of four would overwrite the tile
    # the lagging half is still reading
    K, V, reads, KA, VA, NSK, NSV, inst = _attention_schedule(20, NSV=4, VA=3)
    assert any(t - NSV >= 0 and max(reads["V"][t - NSV]) >= q for q, t in V)
    # K issued four tiles ahead into a ring of four: the same for K
    K, V, reads, KA, VA, NSK, NSV, inst = _attention_schedule(20, KA=4)
    assert any(t - NSK >= 0 and max(reads["K"][t - NSK]) >= q for q, t in K)
    # a wait that allows one tile more in flight than issued after K(t)
    K, V, reads, KA, VA, NSK, NSV, inst = _attention_schedule(20)
    assert not _landed_ok(K, 5, 10, inst(6, 5 + KA - 1) + 16, 16)
