"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's source (a dropped term,
a wrong sign, index or bound, a transposed operand), loads the copy as a module
of its own, and runs the pins of tests/test_oracle_pins.py against it, in
order, until one fails. A mutant that passes every pin fails this test. Runs
on the CPU only; the oracle itself is never changed.
"""
import inspect
import types

import pytest

import tests.test_oracle_pins as P
from oracle import dsa_oracle as O

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")
SRC = inspect.getsource(O)

# (name, text in the oracle, replacement)
MUTATIONS = [
    ("slash offset 0 not forced",
     "S = topk_indices(s32, slash_topk, forced=(0,))", "S = topk_indices(s32, slash_topk)"),
    ("diagonal block not forced",
     "topk_indices(L32[a, : a + 1], topk, forced=(a,))", "topk_indices(L32[a, : a + 1], topk)"),
    ("merge gap strict", "d - intervals[-1][1] <= block", "d - intervals[-1][1] < block"),
    ("diagonal sum not reversed", "s[: i + 1] += p[::-1]", "s[: i + 1] += p"),
    ("causal mask off by one", "allowed = keys <= row_pos[r]", "allowed = keys < row_pos[r]"),
    ("no max subtraction in attention",
     "e = np.exp(lr - m)\n        p = e / e.sum()\n        out[r]", "e = np.exp(lr)\n        p = e / e.sum()\n        out[r]"),
    ("estimate unscaled", "logits = scale * (q[rows] @ k.T)", "logits = (q[rows] @ k.T)"),
    ("estimate window one row short", "rows = np.arange(n - lq, n)", "rows = np.arange(n - lq + 1, n)"),
    ("top-k ties to the highest index", "np.lexsort((np.arange(n), -key, ~is_forced))",
     "np.lexsort((-np.arange(n), -key, ~is_forced))"),
    ("NaN ranked first", "y[np.isnan(y)] = -np.inf", "y[np.isnan(y)] = np.inf"),
    ("slash range end off by one", "hi = min(n, r0 + BLOCK - d_lo)", "hi = min(n, r0 + BLOCK - d_lo - 1)"),
    ("slash range start off by one", "lo = max(0, r0 - d_hi)", "lo = max(0, r0 - d_hi + 1)"),
    ("vertical columns past the block end", "if j < end and not any", "if j <= end and not any"),
    ("ragged pool divides by 64", "x[a * BLOCK: min(n, (a + 1) * BLOCK)].mean(axis=0)",
     "x[a * BLOCK: min(n, (a + 1) * BLOCK)].sum(axis=0) / BLOCK"),
    ("block logits transposed", "scale * (f64(qp) @ f64(kp).T)", "scale * (f64(kp) @ f64(qp).T)"),
    ("streaming window one block wide", "if c < init_blocks or a - c < local_blocks]",
     "if c < init_blocks or a - c <= local_blocks]"),
    ("streaming sink one block short", "if c < init_blocks or a - c < local_blocks]",
     "if c + 1 < init_blocks or a - c < local_blocks]"),
    ("retention window one row short", "for i in range(n - w, n):", "for i in range(n - w + 1, n):"),
    ("retention unnormalised", "S[: i + 1] += e / e.sum()", "S[: i + 1] += e"),
    ("decode row placed before the last key", "np.array([n]), keys, k, v, scale)",
     "np.array([n - 2]), keys, k, v, scale)"),
    ("default scale 1/D", "return 1.0 / math.sqrt(head_dim)", "return 1.0 / head_dim"),
    ("pruning chunk score is the mean", "return s[x * c: min(limit, (x + 1) * c)].max()",
     "return s[x * c: min(limit, (x + 1) * c)].mean()"),
    ("pruning forced chunk dropped", "pick = topk_indices(scores, keep, forced=(forced,))",
     "pick = topk_indices(scores, keep)"),
    ("pruning later stages see every chunk",
     "cand = [y for x in kept for y in range(x * r, (x + 1) * r) if y * c < limit]",
     "cand = [y for y in range((limit + c - 1) // c)]"),
    ("pruning stage limit taken from the whole cache", "cand = list(range((limit + c - 1) // c))",
     "cand = list(range((len(k) + c - 1) // c))"),
    ("pruning forces the first chunk", "forced = cand.index((limit - 1) // c)", "forced = 0"),
]


def _cases():
    """Every pin of the pin module as (name, function, kwargs)."""
    for name, fn in list(vars(P).items()):
        if not (name.startswith("test_") and isinstance(fn, types.FunctionType)):
            continue
        params = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not params:
            yield name, fn, {}
            continue
        assert len(params) == 1, name
        argnames, values = params[0].args[:2]
        names = [s.strip() for s in argnames.split(",")] if isinstance(argnames, str) else list(argnames)
        for val in values:
            val = tuple(val) if len(names) > 1 else (val,)
            yield name, fn, dict(zip(names, val))


def _mutant(old, new):
    assert SRC.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    mod = types.ModuleType("dsa_oracle_mutant")
    mod.__dict__["__builtins__"] = __builtins__
    exec(compile(SRC.replace(old, new), "dsa_oracle_mutant", "exec"), mod.__dict__)
    return mod


def test_unmutated_oracle_passes_the_runner(monkeypatch):
    """The runner itself: with an exact copy of the oracle every pin passes."""
    mod = _mutant("def num_blocks(n: int) -> int:", "def num_blocks(n: int) -> int:")
    monkeypatch.setattr(P, "O", mod)
    for name, fn, kw in _cases():
        fn(**kw)


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(name, old, new, monkeypatch):
    mod = _mutant(old, new)
    monkeypatch.setattr(P, "O", mod)
    for pin, fn, kw in _cases():
        try:
            fn(**kw)
        except Exception:   # an assertion or any error the mistake causes
            return
    pytest.fail(f"no pin catches the mutation '{name}'")
