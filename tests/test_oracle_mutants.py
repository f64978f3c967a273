"""Plant mistakes in the oracle's source and check that its pins catch every one.

Each mutation below rewrites one spot of ``oracle/attention.py`` (on the CPU,
in a throw-away module: the real oracle is untouched) into a plausible slip:
a dropped term, a wrong sign, index, axis or operand, an off-by-one in the
mask or in the decode length, the wrong head grouping, the wrong page lookup.
The whole pin suite of ``tests/test_oracle.py`` is then run against the
mutant; at least one pin must fail.  A mutation that survives means the pins
leave that part of the oracle unchecked.
"""

import inspect
import itertools
import os
import types

import pytest

import tests.test_oracle as pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "attention.py")

MUTATIONS = {
    "head groups taken modulo": [("return h // (Hq // Hkv)", "return h % Hkv")],
    "scale dropped": [("s = scale * (qrows @ keys.T)", "s = qrows @ keys.T")],
    "scores transposed": [("s = scale * (qrows @ keys.T)", "s = scale * (keys @ qrows.T)")],
    "masked scores set to 0, not -inf": [("np.where(visible, s, -np.inf)", "np.where(visible, s, 0.0)")],
    "max over the wrong axis": [("m = s.max(axis=1, keepdims=True)", "m = s.max(axis=0, keepdims=True)")],
    "exponent sign flipped": [("e = np.exp(s - m)", "e = np.exp(m - s)")],
    "no normalisation": [("out = (e @ vals) / l", "out = (e @ vals)")],
    "probabilities transposed": [("out = (e @ vals) / l", "out = (e.T @ vals) / l")],
    "lse in base 2": [("lse = m[:, 0] + np.log(l[:, 0])", "lse = m[:, 0] + np.log2(l[:, 0])")],
    "lse drops the max": [("lse = m[:, 0] + np.log(l[:, 0])", "lse = np.log(l[:, 0])")],
    "diagonal excluded": [("np.tril(np.ones((T, T), dtype=bool), k=0)", "np.tril(np.ones((T, T), dtype=bool), k=-1)")],
    "one future key visible": [("np.tril(np.ones((T, T), dtype=bool), k=0)", "np.tril(np.ones((T, T), dtype=bool), k=1)")],
    "mask transposed": [("np.tril(np.ones((T, T), dtype=bool), k=0)", "np.triu(np.ones((T, T), dtype=bool), k=0)")],
    "V replaced by K": [("_attend(q[b, h], k[b, kv], v[b, kv], scale, visible)", "_attend(q[b, h], k[b, kv], k[b, kv], scale, visible)")],
    "row sampler sees one future key": [
        ("ks = _as64(k[b, kv, : i + 1])", "ks = _as64(k[b, kv, : i + 2])"),
        ("vs = _as64(v[b, kv, : i + 1])", "vs = _as64(v[b, kv, : i + 2])"),
        ("np.ones((1, i + 1), dtype=bool)", "np.ones((1, min(i + 2, k.shape[2])), dtype=bool)"),
    ],
    "page and slot swapped": [
        ("page_ids = np.asarray(table_row)[j // page_size]", "page_ids = np.asarray(table_row)[j % page_size]"),
        ("slots = j % page_size", "slots = j // page_size"),
    ],
    "block table ignored": [("page_ids = np.asarray(table_row)[j // page_size]", "page_ids = j // page_size")],
    "gather ignores the kv head": [("_as64(pages[page_ids, kvh, slots])", "_as64(pages[page_ids, 0, slots])")],
    "decode query misses its own token": [("L = int(sl[b])", "L = int(sl[b]) - 1")],
    "decode heads taken modulo": [
        ("            kv = kv_head_of(h, Hq, Hkv)\n            keys", "            kv = h % Hkv\n            keys"),
    ],
    "empty sequence lse 0": [("lse = np.full((B, Hq), -np.inf)", "lse = np.zeros((B, Hq))")],
    "chunk mask aligned top-left": [("pos = ctx - Tq + rows", "pos = rows")],
    "chunk sees one future key": [("pos = ctx - Tq + rows", "pos = ctx - Tq + rows + 1")],
    "chunk misses its own key": [("np.arange(ctx)[None, :] <= pos[:, None]", "np.arange(ctx)[None, :] < pos[:, None]")],
    "chunk heads taken modulo": [("kvh = kv_head_of(h, Hq, Hkv)", "kvh = h % Hkv")],
    "chunk reads the first rows' queries": [("_attend(q[b, h, rows]", "_attend(q[b, h, : rows.size]")],
    "append one position late": [("position = total - Tn + t", "position = total - Tn + t + 1")],
    "append at the sequence start": [("position = total - Tn + t", "position = t")],
    "append page and slot swapped": [
        ("page = int(bt[b, position // page_size])", "page = int(bt[b, position % page_size])"),
        ("k_out[page, :, position % page_size]", "k_out[page, :, position // page_size]"),
    ],
    "varlen keys from the batch start": [("_attend(q[first:last, h], k[first:last, g], v[first:last, g]",
                                          "_attend(q[first:last, h], k[:n, g], v[:n, g]")],
    "varlen mask not causal": [("seen = np.tril(np.ones((n, n), dtype=bool))", "seen = np.ones((n, n), dtype=bool)")],
    "varlen heads taken modulo": [("g = kv_head_of(h, Hq, Hkv)", "g = h % Hkv")],
    "fp8 exponent bias 8": [("(1.0 + m / 8.0) * 2.0 ** (e - 7)", "(1.0 + m / 8.0) * 2.0 ** (e - 8)")],
    "fp8 subnormals without the 2^-6": [("m / 8.0 * 2.0 ** -6", "m / 8.0 * 2.0 ** -7")],
    "fp8 sign ignored": [("sign = np.where(c & 0x80, -1.0, 1.0)", "sign = 1.0")],
    "fp8 value scale on the keys": [("vals = fp8_e4m3_value(v_codes) * float(v_scale)",
                                     "vals = fp8_e4m3_value(v_codes) * float(k_scale)")],
    "fused step attends before appending": [
        ("    k_after, v_after = kv_append(k_pages, v_pages, k_new, v_new, block_table, seq_lens, page_size)\n"
         "    out, lse = prefill_paged(q, k_after, v_after,",
         "    out, lse = prefill_paged(q, k_pages, v_pages,"),
        ("page_size, rows=rows)\n    return out, lse, k_after, v_after",
         "page_size, rows=rows)\n    k_after, v_after = kv_append(k_pages, v_pages, k_new, v_new, block_table, "
         "seq_lens, page_size)\n    return out, lse, k_after, v_after"),
    ],
    "fused step returns the old cache": [("rows=rows)\n    return out, lse, k_after, v_after",
                                          "rows=rows)\n    return out, lse, k_pages, v_pages")],
    "fused decode returns the old cache": [("scale, page_size)\n    return out, lse, k_after, v_after",
                                            "scale, page_size)\n    return out, lse, k_pages, v_pages")],
    "fused decode attends before appending": [
        ("    out, lse = decode_paged(q, k_after, v_after, block_table, seq_lens, scale, page_size)",
         "    out, lse = decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale, page_size)"),
    ],
    "fused decode appends the new token one slot late": [
        ("    some = np.nonzero(sl > 0)[0]\n    k_after, v_after = kv_append(k_pages, v_pages, kn[some], vn[some], "
         "np.asarray(block_table)[some], sl[some],",
         "    some = np.nonzero(sl > 0)[0]\n    k_after, v_after = kv_append(k_pages, v_pages, kn[some], vn[some], "
         "np.asarray(block_table)[some], sl[some] + 1,"),
    ],
    "append writes V into K": [("k_out[page, :, position % page_size] = np.asarray(k_new)[b, :, t]",
                                "k_out[page, :, position % page_size] = np.asarray(v_new)[b, :, t]")],
}


def _mutant(subs):
    src = open(SRC_PATH).read()
    for old, new in subs:
        assert src.count(old) == 1, f"mutation anchor must occur exactly once: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, SRC_PATH + " (mutant)", "exec"), mod.__dict__)
    return mod


def _pin_cases():
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            yield name, fn, {}
            continue
        axes = []
        for m in marks:
            argnames = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
            vals = [v if len(argnames) > 1 else (v,) for v in m.args[1]]
            axes.append([dict(zip(argnames, v)) for v in vals])
        for combo in itertools.product(*axes):
            kw = {}
            for part in combo:
                kw.update(part)
            yield name, fn, kw


def _failing_pins(mod):
    saved = pins.oracle
    pins.oracle = mod
    failed = []
    try:
        for name, fn, kw in _pin_cases():
            try:
                fn(**kw)
            except (Exception, pytest.fail.Exception) as exc:  # a failed check or a crash: caught
                failed.append((name, type(exc).__name__))
    finally:
        pins.oracle = saved
    return failed


def test_unmutated_oracle_passes_every_pin():
    import oracle

    assert _failing_pins(oracle) == []


# Pins that check values (the error-path test is not counted: a mutant must
# be caught by a wrong number, not only by a missing exception).
ERROR_PATH_TESTS = {"test_oracle_rejects_bad_shapes"}


@pytest.mark.parametrize("label", sorted(MUTATIONS))
def test_pins_catch_mutation(label):
    failed = [f for f in _failing_pins(_mutant(MUTATIONS[label])) if f[0] not in ERROR_PATH_TESTS]
    assert failed, f"mutation '{label}' survived every value pin"
