"""Token ids whose SplitMix64 stream holds a chosen output at a chosen draw.

Hash routing ("DeepSeek-V4-Flash-SI" card, 架构特性, MoE paragraph: experts of
the first layers follow from the token id) is read here as SplitMix64
(Steele, Lea and Flood, OOPSLA 2014) started from (seed << 32) xor token_id,
with draws r >= 2**64 - (2**64 mod E) rejected.  For E = 384 only the top 256
values of r are rejected, so random tokens never reach that branch.  This
module builds tokens that do: it inverts the generator's finalizer (each
xor-shift step is a bijection undone by repeated shifting, each multiply by
an odd constant is undone by its inverse modulo 2**64), steps the state back
by the additive increment, and xors the seed back out.

It is written from the generator's published definition, independently of
the oracle and of the GPU kernel, and is used by tests only.
"""

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15          # the golden-ratio increment
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB


def _finalize(z):
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def _undo_xorshift(y, s):
    """x with x ^ (x >> s) == y."""
    x = y
    for _ in range(64 // s + 1):
        x = y ^ (x >> s)
    return x


def _unfinalize(r):
    z = _undo_xorshift(r, 31)
    z = (z * pow(MIX2, -1, 1 << 64)) & MASK64
    z = _undo_xorshift(z, 27)
    z = (z * pow(MIX1, -1, 1 << 64)) & MASK64
    return _undo_xorshift(z, 30)


def draws(state, n):
    """The first n outputs from a 64-bit start state."""
    out = []
    for _ in range(n):
        state = (state + GAMMA) & MASK64
        out.append(_finalize(state))
    return out


def token_with_draw(seed, draw_index, value):
    """A token id (int64, two's complement) whose stream under `seed` has
    output number `draw_index` (0-based) equal to `value`."""
    s = _unfinalize(value)
    start = (s - (draw_index + 1) * GAMMA) & MASK64
    tid = start ^ (((seed & MASK64) << 32) & MASK64)
    assert draws(start, draw_index + 1)[draw_index] == value
    return tid - (1 << 64) if tid >= (1 << 63) else tid


def start_state(seed, token_id):
    return (((seed & MASK64) << 32) ^ (token_id & MASK64)) & MASK64


def rejection_tokens(seed, n_experts, k):
    """Tokens that put a draw right at and right below the rejection limit
    2**64 - (2**64 mod E), and one at the top of the range mid-stream.

    Returns a list of (token_id, expected experts in draw order, what it
    exercises).  The expected lists follow from the construction: a draw at
    or above the limit is dropped, one below it is kept; the other draws
    come from the forward generator.  Each case is chosen so that a slip in
    the comparison (> for >=, or a limit off by one either way) changes the
    expected experts."""
    E = n_experts
    limit = (1 << 64) - ((1 << 64) % E)
    assert limit < (1 << 64), "E is a power of two: nothing is rejected"

    def distinct(rs):
        out = []
        for r in rs:
            e = r % E
            if e not in out:
                out.append(e)
        return out[:k]

    cases = []
    # (forced values to try in order, rejected?, first draw index): a case is
    # kept at the first value and draw index at which it discriminates.  The
    # stream after a forced output is fixed by that output, so with few
    # experts the next draw can repeat its expert for every draw index; the
    # neighbouring values (still on the same side of the limit) are tried then.
    for values, rejected, first, what in [
            ([limit + j for j in range(8)], True, 0, "a draw at the limit"),
            ([limit - 1 - j for j in range(8)], False, 0, "a draw below the limit"),
            ([MASK64 - j for j in range(8)], True, 2, "a later draw at the top of the range")]:
        found = None
        for value in values:
            for idx in range(first, first + 8):
                tid = token_with_draw(seed, idx, value)
                rs = draws(start_state(seed, tid), 96)
                kept = [r for i, r in enumerate(rs) if not (i == idx and rejected)]
                expect = distinct(kept)
                flipped = distinct(rs if rejected else [r for i, r in enumerate(rs) if i != idx])
                if expect != flipped:
                    found = (tid, expect, f"{what}: 2**64 - {(1 << 64) - value} at draw {idx}")
                    break
            if found:
                break
        if found is None:
            raise AssertionError("construction does not discriminate")
        cases.append(found)
    return cases
