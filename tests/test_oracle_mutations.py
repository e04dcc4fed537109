"""The oracle's pins catch plausible mistakes: each case plants one mistake in a
copy of the oracle's source (oracle/gqa_ref.py), runs the CPU pin tests
(tests/test_oracle.py, tests/test_oracle_chunk.py, tests/test_oracle_paged.py,
tests/test_golden_pages.py) against that copy, and requires at least one of them
to fail.  The mistakes are planted in the oracle, on the CPU; nothing here runs
on a GPU."""

import importlib.util
import itertools
import os
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "gqa_ref.py")
PIN_MODULES = ("test_oracle.py", "test_oracle_chunk.py", "test_oracle_paged.py", "test_golden_pages.py")

# (name, [(text in the oracle, planted replacement), ...])
MUTATIONS = [
    ("rmsnorm drops eps", [("np.mean(x * x, axis=-1, keepdims=True) + float(eps))",
                            "np.mean(x * x, axis=-1, keepdims=True))")]),
    ("rmsnorm sums instead of averaging", [("np.mean(x * x, axis=-1, keepdims=True)",
                                             "np.sum(x * x, axis=-1, keepdims=True)")]),
    ("rope rotates the other way", [("[lo * c - hi * s, hi * c + lo * s]", "[lo * c + hi * s, hi * c - lo * s]")]),
    ("rope frequency exponent -i/d", [("-2.0 * i / float(d)", "-1.0 * i / float(d)")]),
    ("rope pairs adjacent elements", [("lo, hi = x[..., :h], x[..., h:]", "lo, hi = x[..., 0::2], x[..., 1::2]")]),
    ("norm after rope", [("""    if gamma is not None:
        y = rms_norm(y, gamma, eps)
    if theta is not None and theta > 0:
        y = rope(y, pos, theta)""", """    if theta is not None and theta > 0:
        y = rope(y, pos, theta)
    if gamma is not None:
        y = rms_norm(y, gamma, eps)""")]),
    ("no softmax scale", [("s = float(scale) * (q @ K.T)\n    if visible", "s = (q @ K.T)\n    if visible")]),
    ("keys in place of values", [("return p @ V, (m + np.log(z))[:, 0], p", "return p @ K, (m + np.log(z))[:, 0], p")]),
    ("query head h reads KV head h mod Hkv", [
        ("            Q = prologue(q[b, h * G:(h + 1) * G], q_norm_w, p, rope_theta, eps)\n"
         "            o, l, _ = attend(Q, K, V, sc)\n"
         "            out[b, h * G:(h + 1) * G] = o",
         "            Q = prologue(q[b, h::Hkv], q_norm_w, p, rope_theta, eps)\n"
         "            o, l, _ = attend(Q, K, V, sc)\n"
         "            out[b, h::Hkv] = o")]),
    ("decode re-rotates cached keys", [
        ("            K[L - 1] = prologue(K[L - 1], k_norm_w, p, rope_theta, eps)\n"
         "            Q = prologue(q[b, h * G:(h + 1) * G], q_norm_w, p, rope_theta, eps)\n"
         "            o, l, _ = attend(Q, K, V, sc)",
         "            K = prologue(K, k_norm_w, p - L + 1 + np.arange(L), rope_theta, eps)\n"
         "            Q = prologue(q[b, h * G:(h + 1) * G], q_norm_w, p, rope_theta, eps)\n"
         "            o, l, _ = attend(Q, K, V, sc)")]),
    ("decode ignores the position", [("        p = float(positions[b])\n        for h in range(Hkv):\n            K = _f64(k_cache[b, h, :L]).copy()\n            V = _f64(v_cache[b, h, :L])\n            K[L - 1] = prologue(K[L - 1], k_norm_w, p, rope_theta, eps)\n            Q = prologue(q[b, h * G:(h + 1) * G], q_norm_w, p, rope_theta, eps)\n            o, l, _ = attend(Q, K, V, sc)",
                                      "        p = 0.0\n        for h in range(Hkv):\n            K = _f64(k_cache[b, h, :L]).copy()\n            V = _f64(v_cache[b, h, :L])\n            K[L - 1] = prologue(K[L - 1], k_norm_w, p, rope_theta, eps)\n            Q = prologue(q[b, h * G:(h + 1) * G], q_norm_w, p, rope_theta, eps)\n            o, l, _ = attend(Q, K, V, sc)")]),
    ("merge weights inverted", [("share_a = np.exp(lse_a - lse)", "share_a = np.exp(lse - lse_a)")]),
    ("strict causal rule", [("vis = (np.arange(n)[None, :] <= rsel[:, None]) if causal else None",
                             "vis = (np.arange(n)[None, :] < rsel[:, None]) if causal else None")]),
    ("chunk causal mask aligned top-left", [("vis = (np.arange(n)[None, :] <= (P + tsel)[:, None]) if causal else None",
                                              "vis = (np.arange(n)[None, :] <= tsel[:, None]) if causal else None")]),
    ("lengths not clamped", [("    return int(min(max(int(L), 0), cap))", "    return int(L)")]),
]


def mutant(edits):
    src = open(ORACLE_SRC).read()
    for old, new in edits:
        assert src.count(old) >= 1, f"mutation site not found: {old[:60]!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "<oracle mutant>", "exec"), mod.__dict__)
    return mod


def pin_modules():
    mods = []
    for name in PIN_MODULES:
        spec = importlib.util.spec_from_file_location("pins_" + name[:-3], os.path.join(os.path.dirname(__file__), name))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mods.append(mod)
    return mods


def calls(fn):
    """Every argument set pytest would call fn with (its parametrize marks)."""
    sets = [{}]
    for mark in getattr(fn, "pytestmark", []):
        if mark.name != "parametrize":
            continue
        names, values = mark.args[0], mark.args[1]
        names = [n.strip() for n in names.split(",")] if isinstance(names, str) else list(names)
        new = []
        for base, val in itertools.product(sets, values):
            vals = val if len(names) > 1 else (val,)
            new.append(dict(base, **dict(zip(names, vals))))
        sets = new
    return sets


def first_failure(oracle_module):
    """Name of the first pin test that fails against `oracle_module`, or None."""
    for mod in pin_modules():
        mod.O = oracle_module
        for attr in sorted(dir(mod)):
            fn = getattr(mod, attr)
            if not attr.startswith("test_") or not callable(fn):
                continue
            for kw in calls(fn):
                try:
                    fn(**kw)
                except Exception:   # an assertion, or the mutant breaking outright
                    return f"{mod.__name__}.{attr}{kw or ''}"
    return None


def test_unmutated_oracle_passes_every_pin():
    import oracle as O
    assert first_failure(O) is None


@pytest.mark.filterwarnings("ignore::RuntimeWarning")   # a mutant may compute inf - inf
@pytest.mark.parametrize("name,edits", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(name, edits):
    caught = first_failure(mutant(edits))
    assert caught is not None, f"no pin fails when the oracle has: {name}"
