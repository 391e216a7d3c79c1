"""O(3) irreps strings (oracle side).

Follows e3nn-course Lesson 12a, section 21.2 ("Irreps, with the group written
down"): a string such as ``"32x0e + 32x1o"`` is a sum of terms
``MULxLP``, L the angular momentum, P the parity ``e`` (+1) or ``o`` (-1);
a term without ``MULx`` has multiplicity 1.  The dimension is
sum MUL * (2L + 1) (the page prints 128 for ``32x0e+32x1o``).
"""

import re

_TERM = re.compile(r"^(?:(\d+)\s*x\s*)?(\d+)\s*([eo])$")


def parse(s):
    """Return the list of blocks ``[(mul, l, p), ...]`` of an O(3) irreps
    string, p = +1 for ``e`` and -1 for ``o``.  An empty string means no
    blocks."""
    s = s.strip()
    if not s:
        return []
    out = []
    for term in s.split("+"):
        m = _TERM.match(term.strip())
        if m is None:
            raise ValueError(f"cannot parse irreps term {term!r} in {s!r}")
        mul = int(m.group(1)) if m.group(1) is not None else 1
        out.append((mul, int(m.group(2)), 1 if m.group(3) == "e" else -1))
    return out


def dim(blocks):
    """sum mul * (2l + 1) over the blocks."""
    return sum(mul * (2 * l + 1) for mul, l, _ in blocks)


def to_str(blocks):
    """Blocks back to the compact form the pages print (``32x0e+32x1o``)."""
    return "+".join(f"{mul}x{l}{'e' if p == 1 else 'o'}" for mul, l, p in blocks)


def type_key(l, p):
    """Order of output irrep types: by l, and within one l the natural
    parity (-1)^l first (0e, 0o, 1o, 1e, 2e, 2o, ...).  The pages only show
    0e before 1o (Lesson 12a, section 21.4); the rest is this oracle's
    reading of that order."""
    return (l, 0 if p == (-1) ** l else 1)


def parity_str(p):
    return "e" if p == 1 else "o"
