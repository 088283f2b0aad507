"""Mutation check of the oracle's pins (CPU only).

Each mutant is a copy of oracle/oracle.c with one plausible mistake planted
(an off-by-one window edge, a dropped sink term, a dropped scale, a wrong GQA
index, values swapped for keys, an ignored causal offset, a wrong sign in the
exponent, a reversed operand, a verify that hides the query's own token, an argmax
that breaks ties the other way, an acceptance that continues past a
rejection, a rotary embedding with the wrong pairing or sign, a backward without
the delta term or with the sink gradient's sign flipped, ...).
Each is compiled with gcc into a temporary library and every pin is run
against it: at least one pin must fail, or the pins would not detect that
mistake.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "window_edge_W_plus_1": ("long lo = i - (long)window + 1;", "long lo = i - (long)window;"),
    "sink_dropped_from_normaliser": ("double z = sink ? exp(*sink - m) : 0.0;", "double z = 0.0;"),
    "scale_dropped": ("sbuf[j] = scale * acc;", "sbuf[j] = acc;"),
    "gqa_modulo_grouping": ("int g = h / G;", "int g = h % Hkv;"),
    "keys_used_as_values": ("const float *vr = (j < nA) ? vA + j * strideA : vB + (j - nA) * strideB;",
                            "const float *vr = (j < nA) ? kA + j * strideA : kB + (j - nA) * strideB;"),
    "q_offset_ignored": ("long i = (long)q_offset + r;", "long i = r;"),
    "exponent_sign": ("z += exp(sbuf[j] - m);", "z += exp(m - sbuf[j]);"),
    "reversed_operand": ("acc += (double)qv[d] * (double)kr[d];",
                         "acc += (double)qv[d] * (double)kr[D - 1 - d];"),
    "sink_mass_unshifted": ("*psink_out = sink ? exp(*sink - m) / z : 0.0;",
                            "*psink_out = sink ? exp(*sink) / z : 0.0;"),
    "verify_hides_own_token": ("long nB = t - u0 + 1;", "long nB = t - u0;"),
    "verify_drops_oldest_key": ("long nA = lo < L ? L - lo : 0;", "long nA = lo < L ? L - lo - 1 : 0;"),
    "ring_slot_shifted": ("long slot = ring ? p % slots : p;", "long slot = ring ? (p + 1) % slots : p;"),
    "lse_without_max": ("*lse_out = m + log(z);", "*lse_out = log(z);"),
    "argmax_ties_to_highest": ("if (row[v] > row[best])", "if (row[v] >= row[best])"),
    "append_count_without_committed_row": ("n_append[b] = 1 + accepted;", "n_append[b] = accepted;"),
    "accept_after_rejection": ("for (t = 0; t + 1 < T && open; ++t) {", "for (t = 0; t + 1 < T; ++t) {"),
    "accept_compares_shifted_target": ("if (target[(size_t)b * T + t] == draft",
                                       "if (target[(size_t)b * T + t + 1] == draft"),
    "rope_interleaved_pairs": ("const double a = xr[i], b = xr[i + half];",
                               "const double a = xr[(2 * i) % rot], b = xr[(2 * i + 1) % rot];"),
    "rope_sign_flipped": ("orow[i] = a * c - b * s;", "orow[i] = a * c + b * s;"),
    "rope_frequency_over_head_dim": ("pow(base, -2.0 * i / rot)", "pow(base, -2.0 * i / D)"),
    "rope_tail_dropped": ("orow[i] = xr[i];", "orow[i] = i < rot ? xr[i] : 0.0;"),
    "backward_delta_dropped": ("const double ds = wbuf[j] * (dp - delta);", "const double ds = wbuf[j] * dp;"),
    "backward_dk_unscaled": ("dkr[d] += sm_scale * ds * (double)qv[d];", "dkr[d] += ds * (double)qv[d];"),
    "backward_dv_uses_ds": ("dvr[d] += wbuf[j] * (double)go[d];", "dvr[d] += ds * (double)go[d];"),
    "backward_dq_uses_values": ("dqv[d] += sm_scale * ds * (double)kr[d];",
                                "dqv[d] += sm_scale * ds * (double)vr[d];"),
    "backward_sink_sign": ("dsink_b[b * Hq + h] += -psink * delta;", "dsink_b[b * Hq + h] += psink * delta;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    count = text.count(old)
    assert count >= 1, f"mutation site for {name} not found in oracle.c"
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "mutant.c")
        with open(src, "w") as f:
            f.write(text.replace(old, new))
        lib = oracle.build(src, os.path.join(d, "libmutant.so"))
        monkeypatch.setattr(oracle, "_lib", oracle.load(lib))
        caught = []
        for pin in oracle_pins.ALL_PINS:
            try:
                pin()
            except (AssertionError, ValueError) as e:
                caught.append(pin.__name__)
        assert caught, f"no pin detects mutant {name}"
