"""Pins of the oracle's step composition (oracle.step) against hand-worked
decode steps (tests/golden/step_hand_worked.json): which scale each K and V
value is quantised under (per tensor or per kv head, K's or V's), the query
head -> kv head map h // G, the latent row's first head_dim_v values as V,
and an aborted request's zero output and -inf lse. Expected outputs are
softmax attention over the hand-derived scores and dequantised values,
computed here with math.fsum / math.exp; planted mistakes in the step
composition must fail the comparison."""
import json
import math
import os
import types

import numpy as np
import pytest

from oracle import attention, step

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "step_hand_worked.json")))
TOL_ABS, TOL_REL = 1e-12, 1e-13


def _bf16_bits(x) -> np.ndarray:
    """Bit patterns of values that bf16 represents exactly (checked)."""
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "hand-made input is not a bf16 value"
    assert np.array_equal(u.view(np.float32).astype(np.float64), np.asarray(x, dtype=np.float64))
    return (u >> 16).astype(np.uint16)


class HandWorkload:
    """A workload whose values come from the fixture instead of a generator."""

    def __init__(self, spec, per_head: bool):
        sh = spec["shape"]
        self.batch = sh["batch"]
        self.num_q_heads = sh["num_q_heads"]
        self.num_kv_heads = sh["num_kv_heads"]
        self.head_dim_k = sh.get("head_dim_k", sh.get("head_dim"))
        self.head_dim_v = sh.get("head_dim_v", sh.get("head_dim"))
        self.page_size = sh["page_size"]
        self.sm_scale = sh["sm_scale"]
        self.latent = "v" not in spec["inputs"]
        self.per_head_scales = per_head
        self.seq_lens = np.array(spec["seq_lens"], dtype=np.int32)
        self.block_table = np.array(spec["block_table"], dtype=np.int32)
        self.page_tags = np.array(spec["page_tags"], dtype=np.uint32)
        self.expected_tags = np.array(spec["expected_tags"], dtype=np.uint32)
        self._k = [np.array(r, dtype=np.float64) for r in spec["inputs"]["k"]]
        self._v = None if self.latent else [np.array(r, dtype=np.float64) for r in spec["inputs"]["v"]]
        self._q = np.array(spec["inputs"]["q"], dtype=np.float64)

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads

    def amax(self, which, head=None):
        rows = self._k if which == "k" else self._v
        return float(max(np.abs(r if head is None else r[:, head]).max() for r in rows))

    def _sel(self, rows, b, heads, tokens):
        x = rows[b]
        if tokens is not None:
            x = x[np.asarray(tokens)]
        if heads is not None:
            x = x[:, np.asarray(heads)]
        return _bf16_bits(x)

    def k_bits(self, b, heads=None, tokens=None):
        return self._sel(self._k, b, heads, tokens)

    def v_bits(self, b, heads=None, tokens=None):
        if self.latent:
            raise ValueError("latent workloads have no separate V stream")
        return self._sel(self._v, b, heads, tokens)

    def q_bits(self):
        return _bf16_bits(self._q)


def _softmax_attention(scores, values):
    """o and lse of one head from hand-derived scores and value rows."""
    m = max(scores)
    e = [math.exp(s - m) for s in scores]
    den = math.fsum(e)
    o = [math.fsum(e[t] * values[t][d] for t in range(len(e))) / den for d in range(len(values[0]))]
    return np.array(o), m + math.log(den)


def _cases():
    out = []
    for name in ("fp8_per_head", "fp8_per_tensor", "bf16"):
        out.append(("gqa", name, "bf16" if name == "bf16" else "fp8", name != "fp8_per_tensor"))
    out.append(("latent", "fp8", "fp8", False))
    out.append(("latent", "fp8", "fp8", True))
    return out


CASES = _cases()
IDS = [f"{s}-{c}-{'head' if ph else 'tensor'}" for s, c, _, ph in CASES]


def _mismatches(spec_name, case_name, kv, per_head):
    """Every way the step's results differ from the hand-worked case (empty
    when they agree)."""
    spec = GOLDEN[spec_name]
    case = spec["cases"][case_name]
    w = HandWorkload(spec, per_head)
    bad = []
    ks, vs = step.scales(w, kv)
    if not (np.array_equal(ks, np.array(case["k_scale"], np.float32)) and
            np.array_equal(vs, np.array(case["v_scale"], np.float32))):
        bad.append(f"scales {ks} {vs}")
    res = step.run(w, kv)
    if not np.array_equal(res["flags"], np.array(spec["expected_abort"], np.uint8)):
        bad.append(f"flags {res['flags']}")
    for b in range(w.batch):
        o, lse = res["out"][b]
        if spec["expected_abort"][b]:
            if not (np.all(o == 0) and np.all(np.isneginf(lse))):
                bad.append(f"aborted request {b} not 0 / -inf")
            continue
        k, v = step.request_kv(w, b, kv, ks, vs)
        if not (np.array_equal(k, np.array(case["k_hat"][b])) and
                np.array_equal(v, np.array(case["v_hat"][b]))):
            bad.append(f"request {b} dequantised values")
        for h, hd in enumerate(case["heads"][str(b)]):
            vals = [case["v_hat"][b][t][hd["kv"]] for t in range(int(w.seq_lens[b]))]
            o_ref, lse_ref = _softmax_attention(hd["scores"], vals)
            if not (np.all(np.abs(o[h] - o_ref) <= TOL_ABS + TOL_REL * np.abs(o_ref)) and
                    abs(lse[h] - lse_ref) <= TOL_ABS):
                bad.append(f"request {b} head {h}: {o[h]} {lse[h]} vs {o_ref} {lse_ref}")
    return bad


@pytest.mark.parametrize("spec_name,case_name,kv,per_head", CASES, ids=IDS)
def test_step_matches_hand_worked_case(spec_name, case_name, kv, per_head):
    assert _mismatches(spec_name, case_name, kv, per_head) == []


def test_fixture_inputs_and_amax_are_as_stated():
    for name in ("gqa", "latent"):
        spec = GOLDEN[name]
        w = HandWorkload(spec, True)
        for i, a in enumerate(spec["amax"]["k"]):
            assert w.amax("k", i) == a
        assert w.amax("k") == spec["amax"]["k_tensor"]
        if not w.latent:
            for i, a in enumerate(spec["amax"]["v"]):
                assert w.amax("v", i) == a
            assert w.amax("v") == spec["amax"]["v_tensor"]


def test_selected_kv_heads_give_their_query_heads_in_order():
    """request_output for kv head 1 alone is the rows of q heads 2 and 3."""
    spec = GOLDEN["gqa"]
    w = HandWorkload(spec, True)
    ks, vs = step.scales(w, "fp8")
    full_o, full_l = step.request_output(w, 0, "fp8", ks, vs, False)
    o1, l1 = step.request_output(w, 0, "fp8", ks, vs, False, kv_heads=[1])
    assert np.array_equal(o1, full_o[2:4]) and np.array_equal(l1, full_l[2:4])
    o2, _ = step.request_output(w, 2, "fp8", ks, vs, True, kv_heads=[0, 1])
    assert o2.shape == (4, 2) and np.all(o2 == 0)


def test_codes_of_the_hand_worked_values():
    """The codes themselves: 448 * 1 -> 0x7E, 28 under 2^-4 -> 448 -> 0x7E,
    0.0068359375 under 2^-4 -> 0.109375 = 1.75 * 2^-4 -> exponent field 3,
    mantissa 6 -> 0x1E; under scale 1 it is the subnormal tie 3.5 * 2^-9 ->
    code 4 (even)."""
    spec = GOLDEN["gqa"]
    w = HandWorkload(spec, True)
    ks, vs = step.scales(w, "fp8")
    kc, vc = step.request_codes(w, 2, ks, vs)
    assert kc[0, 0, 0] == 0x7E and kc[1, 0, 0] == 0xFE and kc[0, 1, 0] == 0x7E
    assert vc[0, 0, 0] == 0x7E and vc[0, 1, 0] == 0x7E and vc[1, 1, 1] == 0xFE
    kc0, _ = step.request_codes(w, 0, ks, vs)
    assert kc0[0, 1, 0] == 0x1E
    w_t = HandWorkload(spec, False)
    kt, vt = step.scales(w_t, "fp8")
    kc_t, vc_t = step.request_codes(w_t, 0, kt, vt)
    assert kc_t[0, 1, 0] == 0x04 and vc_t[0, 1, 0] == 0x02


def test_bf16_widening_is_exact_bit_arithmetic():
    bits = np.array([0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x8000, 0x43E0, 0x7F80], dtype=np.uint16)
    got = step.bf16_bits_to_f64(bits)
    assert got[0] == 1.0 and got[1] == -1.0 and got[2] == 2.0 ** -133
    assert got[3] == float(np.float32(3.3895313892515355e38)) and got[5] == 448.0
    assert got[4] == 0.0 and np.signbit(got[4]) and np.isinf(got[6])


def test_oracle_imports_no_torch():
    import subprocess
    import sys
    code = ("import sys, oracle, oracle.step; "
            "sys.exit(1 if any(m == 'torch' or m.startswith('torch.') for m in sys.modules) else 0)")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root)
    assert r.returncode == 0


# ------------------------------------------------------------ planted mistakes
def _mutant_swap_scales(orig):
    return lambda w, kv="fp8": tuple(reversed(orig(w, kv)))


def _mutant_ignore_per_head(orig):
    def f(w, kv="fp8"):
        flat = types.SimpleNamespace(**{**w.__dict__, "per_head_scales": False})
        flat.amax = w.amax
        return orig(flat, kv)
    return f


def _mutant_head_map_mod(orig_attend):
    def attend(q, k, v, sm):
        g = q.shape[0] // k.shape[1]
        rows = [orig_attend(q[h:h + 1], k[:, [h % g]], v[:, [h % g]], sm) for h in range(q.shape[0])]
        return np.concatenate([r[0] for r in rows]), np.concatenate([r[1] for r in rows])
    return types.SimpleNamespace(attend=attend)


def _mutant_latent_tail(orig):
    def f(w, b, kv, ks, vs, heads=None):
        k, v = orig(w, b, kv, ks, vs, heads)
        return (k, k[..., -w.head_dim_v:]) if w.latent else (k, v)
    return f


def _mutant_abort_ignored(orig):
    return lambda w, b, kv, ks, vs, aborted, kv_heads=None, q=None: orig(w, b, kv, ks, vs, False,
                                                                          kv_heads, q)


def _mutant_q_of_request0(orig):
    def f(w, b, kv, ks, vs, aborted, kv_heads=None, q=None):
        return orig(w, b, kv, ks, vs, aborted, kv_heads, step.bf16_bits_to_f64(w.q_bits()[0]))
    return f


MUTANTS = {
    "swap_k_and_v_scales": ("scales", _mutant_swap_scales, [("gqa", "fp8_per_head", "fp8", True)]),
    "per_tensor_for_per_head": ("scales", _mutant_ignore_per_head,
                                [("gqa", "fp8_per_head", "fp8", True)]),
    "head_map_h_mod_G": ("attention", _mutant_head_map_mod, [("gqa", "fp8_per_head", "fp8", True)]),
    "latent_v_from_row_tail": ("request_kv", _mutant_latent_tail, [("latent", "fp8", "fp8", False)]),
    "abort_ignored": ("request_output", _mutant_abort_ignored, [("gqa", "fp8_per_head", "fp8", True)]),
    "query_of_wrong_request": ("request_output", _mutant_q_of_request0,
                               [("gqa", "fp8_per_head", "fp8", True)]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, make, cases = MUTANTS[name]
    if attr == "attention":
        monkeypatch.setattr(step, "attention", make(attention.attend))
    else:
        monkeypatch.setattr(step, attr, make(getattr(step, attr)))
    for c in cases:
        assert _mismatches(*c) != [], f"mutant {name} not caught on {c}"
