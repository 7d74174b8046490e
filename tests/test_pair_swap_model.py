"""A model check, on the CPU, of the hand-off between the two workgroups of a
16-row block in the split form of the single-frame kernel.

Each half stores its partial sums, waits for all of its memory operations
(its reads of state_in included), then meets its partner at one 64-bit word:

- eager calls exchange the word for (epoch, half, XCD id) in one atomic
  operation; the one whose old value carries this call's epoch and the other
  half is the second;
- captured calls (a graph replays its epoch) flip a toggle tagged with a
  magic value by compare-and-swap: idle (or untagged) becomes waiting, and
  the one that finds the word waiting is the second, who leaves it idle.

The second alone writes the block's rows of state_out; the first polls the
word (bounded) until the second has been there.  This file writes the two
encodings out as the kernel defines them and runs every interleaving of the
two halves' word operations and polls, over sequences of calls that mix both
modes, starting from fresh memory, stale words of either kind and arbitrary
bits, with and without waits that run out.  Checked for every call:

- exactly one half writes state_out, and only after both halves have read
  state_in (so state_out may equal state_in);
- a half that uses its partner's sums uses this call's sums, stored before
  it looked;
- a half whose wait runs out uses no sums of its partner (its output is NaN)
  and does not write the state;
- the word a call leaves behind lets the next call of either mode do all of
  the above.
"""
import itertools

import pytest

pytestmark = pytest.mark.filterwarnings("ignore")

MAGIC = 0x9D3A61
MASK64 = (1 << 64) - 1


# ---- the two encodings, as the kernel writes and reads them ---------------
def eager_value(epoch, half, xcc):
    return (epoch | (half << 32) | (xcc << 40)) & MASK64


def eager_partner(word, epoch, half):
    want = epoch | ((1 - half) << 32)
    return (word & 0x1FFFFFFFF) == want and (word >> 40) < 256


def toggle_next(word, xcc):
    """The compare-and-swap's new value and whether the caller is second."""
    second = (word >> 40) == MAGIC and (word & 1) == 1
    return ((MAGIC << 40) | (xcc << 32) | (0 if second else 1)) & MASK64, second


def toggle_partner_done(word):
    return (word & 1) == 0


# ---- one call: the two halves as step generators ---------------------------
class Call:
    def __init__(self, mode, epoch, xcc, limits):
        self.mode, self.epoch, self.xcc, self.limits = mode, epoch, xcc, limits
        self.events = []          # (half, what)
        self.second = {}
        self.used_partner = {}
        self.sums_stored = set()

    def half(self, h, mem):
        # state_in read and sums stored (both precede the word operation)
        self.events.append((h, "read_state"))
        self.sums_stored.add(h)
        self.events.append((h, "stored"))
        yield
        if self.mode == "eager":
            old = mem["word"]
            mem["word"] = eager_value(self.epoch, h, self.xcc)
            second = eager_partner(old, self.epoch, h)
            seen = old
        else:
            while True:
                cur = mem["word"]
                nxt, second = toggle_next(cur, self.xcc)
                yield  # the load and the compare-and-swap may be split by the partner
                if mem["word"] == cur:
                    mem["word"] = nxt
                    break
            seen = cur
        self.second[h] = second
        ok = second
        polls = 0
        while not ok and polls < self.limits[h]:
            yield
            seen = mem["word"]
            polls += 1
            ok = eager_partner(seen, self.epoch, h) if self.mode == "eager" else toggle_partner_done(seen)
        if ok:
            # the partner's sums: stored before its word operation, which this
            # half has seen
            assert (1 - h) in self.sums_stored, "partner sums read before they were stored"
            self.used_partner[h] = True
        else:
            self.used_partner[h] = False
        if second:
            self.events.append((h, "write_state"))
        yield


def run_call(call, mem, order):
    """Advance the two halves in the given order of half ids (a schedule:
    either may run alone for a while, as a workgroup that starts late), then
    in turn until both are done."""
    gens = {0: call.half(0, mem), 1: call.half(1, mem)}
    live = {0: True, 1: True}
    for h in order:
        if live[h]:
            try:
                next(gens[h])
            except StopIteration:
                live[h] = False
    while live[0] or live[1]:  # then in turn
        for h in (0, 1):
            if live[h]:
                try:
                    next(gens[h])
                except StopIteration:
                    live[h] = False


def check_call(call):
    writes = [h for h, what in call.events if what == "write_state"]
    assert len(writes) == 1, f"{len(writes)} writers"
    w = call.events.index((writes[0], "write_state"))
    for h in (0, 1):
        assert call.events.index((h, "read_state")) < w, "state written before a half read it"
    for h in (0, 1):
        if not call.used_partner[h]:
            assert not call.second[h], "the second always has its partner's sums"


def schedules(n):
    """Every schedule of n steps over the two halves."""
    return [list(p) for p in itertools.product((0, 1), repeat=n)]


# Words a call can find: fresh memory (zeros or arbitrary bits), an idle
# toggle, an eager word of an earlier epoch.  (A toggle left waiting would
# take a call in which one half never ran.)
STARTS = [0, 1, (MAGIC << 40) | (3 << 32), eager_value(7, 0, 2), eager_value(7, 1, 2), (1 << 64) - 1,
          0x123456789ABCDEF0, (MAGIC - 1) << 40 | 1]


@pytest.mark.parametrize("start", STARTS, ids=lambda v: hex(v))
def test_every_interleaving_of_call_sequences(start):
    """Three calls in a row (every eager/captured mix), each under every
    schedule of its first 9 steps (then the halves take turns), from a word
    left in a given state."""
    epochs = iter(range(8, 10 ** 6))
    for modes in itertools.product(("eager", "captured"), repeat=3):
        for order in schedules(9):
            mem = {"word": start}
            for mode in modes:
                call = Call(mode, next(epochs), xcc=2, limits=(64, 64))
                run_call(call, mem, order)
                check_call(call)
                assert all(call.used_partner.values()), "a wait with a large limit ran out"


@pytest.mark.parametrize("mode", ["eager", "captured"])
def test_waits_that_run_out(mode):
    """Limits of 0 to 3 polls: the first may give up.  It then uses no sums of
    its partner and does not write the state; the second still writes it, and
    the calls after it work with ample limits."""
    epochs = iter(range(100, 10 ** 6))
    for lim0, lim1 in itertools.product(range(4), repeat=2):
        for order in schedules(8):
            mem = {"word": 0}
            call = Call(mode, next(epochs), xcc=5, limits=(lim0, lim1))
            run_call(call, mem, order)
            check_call(call)
            for h in (0, 1):
                if not call.used_partner[h]:
                    assert not call.second[h]
            for nxt in ("eager", "captured"):
                c2 = Call(nxt, next(epochs), xcc=5, limits=(64, 64))
                run_call(c2, mem, [0, 1] * 8)
                check_call(c2)
                assert all(c2.used_partner.values())


def test_encodings_cannot_be_confused():
    """An eager word never reads as a waiting toggle and a toggle word never
    reads as an eager partner; a wrong epoch or the same half never matches."""
    for epoch in (1, 2, 0xFFFFFFFF):
        for half in (0, 1):
            for xcc in range(8):
                w = eager_value(epoch, half, xcc)
                assert toggle_next(w, xcc)[1] is False
                assert eager_partner(w, epoch, 1 - half)
                assert not eager_partner(w, epoch, half)
                assert not eager_partner(w, epoch + 1 if epoch < 0xFFFFFFFF else 1, 1 - half)
    for xcc in range(8):
        for bit in (0, 1):
            w = (MAGIC << 40) | (xcc << 32) | bit
            for epoch in (0, 1, bit):
                for half in (0, 1):
                    assert not eager_partner(w, epoch, half)


def test_a_planted_mistake_is_caught():
    """The model catches a protocol in which the first of a pair also writes
    the state: two writers."""
    class TwoWriters(Call):
        def half(self, h, mem):
            gen = super().half(h, mem)
            for _ in gen:
                yield
            if not self.second[h]:
                self.events.append((h, "write_state"))
    call = TwoWriters("eager", 5, xcc=1, limits=(64, 64))
    run_call(call, {"word": 0}, [0, 1] * 6)
    with pytest.raises(AssertionError):
        check_call(call)


def test_a_toggle_without_its_tag_is_caught():
    """Without the tag, fresh memory whose low bit is set reads as a waiting
    partner: the first half to arrive takes itself for the second and reads
    sums that were never stored.  The model catches it."""
    global toggle_next
    real = toggle_next

    def untagged(word, xcc):
        second = (word & 1) == 1
        return ((MAGIC << 40) | (xcc << 32) | (0 if second else 1)) & MASK64, second
    toggle_next = untagged
    try:
        call = Call("captured", 5, xcc=1, limits=(64, 64))
        with pytest.raises(AssertionError):
            run_call(call, {"word": 1}, [0, 0, 0, 0, 1, 1, 1, 1])
            check_call(call)
    finally:
        toggle_next = real
