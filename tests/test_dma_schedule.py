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
instructions of 1 KB per K or V tile). In the attention kernel one wave (which
owns no rows) issues both K and V, two tiles ahead each, in the order K0, V0,
K1, V1, K2, ... (K(t + 2) after the barrier of slot 2t, V(t + 2) after that of
slot 2t + 1), into a K ring of 3 slots and a V ring of 4, and before each
16-instruction group it waits until at most 47 loads are counted. The mass
kernel has a K ring of 4 slots issued 3 tiles ahead by two waves (8
instructions each). A slot is one phase: slot 2t opens the phase that reads
tile t for the leading half of the workgroup, slot 2t + 1 the same phase for
the lagging half.
"""
import pytest


def _landed_ok(seq, need_tile, slot, allowed, ipt):  # (mass kernel: one name per sequence)
    """seq: this wave's issues as (slot, tile), in order. At the wait before
    the barrier that opens `slot`, the issues made so far are those with an
    issue slot < `slot`; the wait leaves `allowed` instructions in flight. The
    tile is landed iff every issue after it accounts for at least `allowed`."""
    done = [x for x in seq if x[0] < slot]
    pos = [i for i, x in enumerate(done) if x[1] == need_tile]
    assert pos, f"tile {need_tile} not issued before slot {slot}"
    after = (len(done) - 1 - pos[0]) * ipt
    return allowed <= after and allowed <= 63


def _attention_schedule(T, NSK=3, NSV=4, IPT=16, KA=2, VA=2):
    """The issuing wave's single sequence of (issue slot, name, tile): the
    prologue (slot -1) K0, V0, K1, V1, ..., then K(t + KA) after the barrier
    of slot 2t and V(t + VA) after that of slot 2t + 1."""
    ok = lambda x: 0 <= x < T
    seq = []
    for t in range(max(KA, VA)):
        if t < KA and ok(t):
            seq.append((-1, "K", t))
        if t < VA and ok(t):
            seq.append((-1, "V", t))
    for t in range(T + 1):
        if ok(t + KA):
            seq.append((2 * t, "K", t + KA))
        if ok(t + VA):
            seq.append((2 * t + 1, "V", t + VA))
    # readers: K of tile t in slots 2t, 2t+1 (M(t) of each half), V of tile t
    # in slots 2t+2, 2t+3 (M(t+1), the PV part)
    reads = {"K": {t: [2 * t, 2 * t + 1] for t in range(T)},
             "V": {t: [2 * t + 2, 2 * t + 3] for t in range(T)}}

    def after_k(t):  # the kernel's count of loads issued after K(t) when it waits for it
        return IPT * ((1 if t < T else 0) + (2 if t + 1 < T else 0))

    return seq, reads, NSK, NSV, after_k


def _outstanding_ok(seq, IPT, cap=47):
    """Before each group the wave waits until at most `cap` loads are counted,
    so that a group of IPT never takes the count past 63."""
    return cap + IPT <= 63


def _landed(seq, name, tile, slot, allowed, ipt):
    done = [x for x in seq if x[0] < slot]
    pos = [i for i, x in enumerate(done) if (x[1], x[2]) == (name, tile)]
    assert pos, f"{name}{tile} not issued before slot {slot}"
    after = (len(done) - 1 - pos[0]) * ipt
    return allowed <= after and allowed <= 63


@pytest.mark.parametrize("T", range(0, 65))
def test_attention_pp_schedule(T):
    seq, reads, NSK, NSV, after_k = _attention_schedule(T)
    assert _outstanding_ok(seq, 16)
    # issue order is one sequence: slots never go back
    assert [x[0] for x in seq] == sorted(x[0] for x in seq)
    for name, ns in (("K", NSK), ("V", NSV)):
        issued = {t: q for q, n, t in seq if n == name}
        assert sorted(issued) == list(range(T)), name
        for q, n, t in seq:  # ring hazard: the previous occupant's last read ended
            if n == name and t - ns >= 0:
                assert max(reads[name][t - ns]) < q, (name, T, t)
        for t, slots in reads[name].items():  # issued before the barrier of its first reader
            assert issued[t] < min(slots)
    for t in range(T):  # wait before the barrier of slot 2t: K(t) and V(t-1) landed
        assert _landed(seq, "K", t, 2 * t, after_k(t), 16)
        if t >= 1:
            assert _landed(seq, "V", t - 1, 2 * t, after_k(t), 16)


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
    # a V ring of three: V(t + 2) would overwrite V(t - 1) while the lagging
    # half still reads it
    seq, reads, NSK, NSV, after_k = _attention_schedule(20, NSV=3)
    assert any(n == "V" and t - NSV >= 0 and max(reads["V"][t - NSV]) >= q for q, n, t in seq)
    # K three tiles ahead into a ring of three: the same for K
    seq, reads, NSK, NSV, after_k = _attention_schedule(20, KA=3)
    assert any(n == "K" and t - NSK >= 0 and max(reads["K"][t - NSK]) >= q for q, n, t in seq)
    # a wait that allows one group more in flight than was issued after K(t)
    seq, reads, NSK, NSV, after_k = _attention_schedule(20)
    assert not _landed(seq, "K", 5, 10, after_k(5) + 16, 16)
    # no cap before the groups: four groups in flight would need 64 counts
    assert not _outstanding_ok(seq, 16, cap=48)
