"""Plant plausible mistakes in copies of the oracle source and check that the
pins catch every one of them (a mutant that passes all pins would mean the pins
do not constrain that part of the oracle)."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sage_oracle.c")

# (id, original text, planted mistake)
MUTANTS = [
    ("O_update_drops_alpha", "O[d] = alpha * O[d] + (float)acc;", "O[d] = O[d] + (float)acc;"),
    ("l_update_drops_alpha", "l = alpha * l + (float)psum;", "l = l + (float)psum;"),
    ("l_from_unrounded_p", "psum += (double)pq[t];",
     "psum += (double)(pv_mode == ORC_PV_FP8 ? p[t] * 448.0f : p[t]);"),
    ("alpha_wrong_sign", "expf(m - mnew)", "expf(mnew - m)"),
    ("p_wrong_sign", "expf(s[t] - mnew)", "expf(mnew - s[t])"),
    ("qk_transposed_out", "out[(size_t)i * S + n] = dot_i8", "out[(size_t)n * S + i] = dot_i8"),
    ("int8_range_128", "float inv = 127.0f / amax;", "float inv = 128.0f / amax;"),
    ("int8_scale_128", "*scale = amax / 127.0f;", "*scale = amax / 128.0f;"),
    ("no_k_smoothing", "ks[i] = k[i] - mean[i % D];", "ks[i] = k[i];"),
    ("mean_divides_by_D", "(float)(s / (double)S)", "(float)(s / (double)D)"),
    ("p_static_scale_240", "orc_e4m3_encode(p[t] * 448.0f)", "orc_e4m3_encode(p[t] * 240.0f)"),
    ("v_scale_wrong_channel", "v_scale[d] / l", "v_scale[0] / l"),
    ("v_quant_scale_240", "float inv = 448.0f / amax;", "float inv = 240.0f / amax;"),
    ("causal_masks_diagonal", "(is_causal && n > i)", "(is_causal && n >= i)"),
    ("round_ties_away", "return nearbyint(a / q) * q;", "return round(a / q) * q;"),
    ("e4m3_bias_8", "ldexp(1.0 + fr / 8.0, ex - 7)", "ldexp(1.0 + fr / 8.0, ex - 8)"),
    ("missing_sm_scale", "float c = (dq * k_scale[kg]) * sm_scale;", "float c = dq * k_scale[kg];"),
    ("k_scale_indexed_by_tile", "int kg = k_lane ? orc_lane_group(n) : n / blk_k;",
     "int kg = k_lane ? orc_lane_group(n) : n / tile_k;"),
    ("k_scale_first_block_only", "float c = (dq * k_scale[kg])", "float c = (dq * k_scale[0])"),
    ("k_lane_scale_by_block", "int kg = k_lane ? orc_lane_group(n) : n / blk_k;", "int kg = n / blk_k;"),
    ("lane_group_wrong_bit", "return 2 * (n >> 5) + ((n >> 2) & 1);", "return 2 * (n >> 5) + ((n >> 3) & 1);"),
    ("lane_group_no_subtile", "return 2 * (n >> 5) + ((n >> 2) & 1);", "return (n >> 5) + ((n >> 2) & 1);"),
    ("lane_k_not_smoothed", "for (size_t i = 0; i < n; ++i) ks[i] = k[i] - mean[i % D];\n    for (int g = 0;",
     "for (size_t i = 0; i < n; ++i) ks[i] = k[i];\n    for (int g = 0;"),
    ("q_scale_wrong_block", "float dq = qk ? 0.0f : q_scale[i / blk_q];", "float dq = qk ? 0.0f : q_scale[i / blk_k];"),
    ("exact_causal_off_by_one", "int nvis = is_causal ? (i + 1 < S ? i + 1 : S) : S;",
     "int nvis = is_causal ? (i < S ? (i > 0 ? i : 1) : S) : S;"),
    ("fp16_pv_no_rounding", "pq[t] = round_f16(p[t]);", "pq[t] = p[t];"),
    ("fp8_p_not_quantised", "pq[t] = orc_e4m3_decode(orc_e4m3_encode(p[t] * 448.0f));", "pq[t] = p[t] * 448.0f;"),
    ("smooth_v_mean_not_added", "o[d] = o[d] + v_mean[d];", "o[d] = o[d];"),
    ("smooth_v_not_subtracted", "vs[i] = v[i] - mean[i % D];", "vs[i] = v[i];"),
    ("e2m1_ties_away", "double v = round_to_format(fabs((double)x), 1, 0);",
     "double v = fabs((double)x) < 6.0 ? round(fabs((double)x) * 2.0) / 2.0 : 6.0;"),
    ("mx_scale_exponent_off_by_one", "e = fe - 1 - 2;", "e = fe - 1 - 1;"),
    ("mx_qk_first_block_scale", "ldexp(blk, (int)qe[(size_t)i * nb + b] - 127", "ldexp(blk, (int)qe[(size_t)i * nb] - 127"),
    ("mx_qk_scale_sign", "+ (int)ke[(size_t)n * nb + b] - 127);", "- (int)ke[(size_t)n * nb + b] + 127);"),
    ("fp4_scores_without_sm_scale", "s[t] = qk[(size_t)r * S + n] * sm_scale;", "s[t] = qk[(size_t)r * S + n];"),
    ("smooth_q_not_subtracted", "qs[(size_t)t * D + d] = q[(size_t)t * D + d] - qmean[(size_t)b * D + d];",
     "qs[(size_t)t * D + d] = q[(size_t)t * D + d];"),
    ("delta_wrong_block", "delta[(size_t)(i / blk_d) * S + n] * sm_scale", "delta[(size_t)(i / blk_k) * S + n] * sm_scale"),
    ("delta_without_sm_scale", "delta[(size_t)(i / blk_d) * S + n] * sm_scale;", "delta[(size_t)(i / blk_d) * S + n];"),
    ("delta_k_not_smoothed", "kc[i] = k[i] - kmean[i % D];", "kc[i] = k[i];"),
    ("fp4_smooth_q_not_subtracted",
     "qs[(size_t)t * D + d] = q[(size_t)t * D + d] - qmean[(size_t)b * D + d];\n    }\n    orc_mxfp4_quant_rows",
     "qs[(size_t)t * D + d] = q[(size_t)t * D + d];\n    }\n    orc_mxfp4_quant_rows"),
    ("pv_group_wrong_bit", "return 2 * (n >> 6) + ((n >> 2) & 1);", "return 2 * (n >> 6) + ((n >> 3) & 1);"),
    ("pv_group_contiguous", "return 2 * (n >> 6) + ((n >> 2) & 1);", "return 2 * (n >> 6) + ((n >> 5) & 1);"),
    ("fp4_p_exponent_off_by_one", "int e = mx_shared_exp(amax);\n                        for (int t = 0; t < tile_k; ++t)",
     "int e = mx_shared_exp(amax) + 1;\n                        for (int t = 0; t < tile_k; ++t)"),
    ("fp4_p_group_misaligned", "int g0 = orc_pv_group(n0);", "int g0 = orc_pv_group(n0) + 1;"),
    ("fp4_v_first_group_scale", "(int)v_e8m0[(size_t)orc_pv_group(n) * D + d] - 127", "(int)v_e8m0[(size_t)d] - 127"),
    ("fp4_v_not_smoothed", "vs[i] = v[i] - mean[i % D];\n    for (int g = 0; g < ng; ++g)",
     "vs[i] = v[i];\n    for (int g = 0; g < ng; ++g)"),
    ("fp4_v_mean_not_added", "if (v_mean && pv_mode == ORC_PV_FP4)\n                    for (int d = 0; d < D; ++d) o[d] = o[d] + v_mean[d];",
     "if (v_mean && pv_mode == ORC_PV_FP4)\n                    for (int d = 0; d < D; ++d) o[d] = o[d];"),
    ("f16_decode_bias", "ldexp(1.0 + fr / 1024.0, ex - 15)", "ldexp(1.0 + fr / 1024.0, ex - 14)"),
]

RUNNER = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, oracle_pins
with oracle.use_library({so!r}):
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except AssertionError:
            print("caught by", pin.__name__)
            sys.exit(0)
print("survived every pin")
sys.exit(3)
"""


@pytest.mark.parametrize("mid,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(orc, tmp_path, mid, old, new):
    src = open(SRC).read()
    code_only = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    assert code_only.count(old) >= 1, "mutation site vanished from the oracle code"
    # mutate the first occurrence that lies in code, not in a comment
    pos, start = -1, 0
    while True:
        pos = src.index(old, start)
        opened, closed = src.rfind("/*", 0, pos), src.rfind("*/", 0, pos)
        if opened <= closed:
            break
        start = pos + 1
    mutated = src[:pos] + new + src[pos + len(old):]
    c = tmp_path / "mutant.c"
    c.write_text(mutated)
    so = str(tmp_path / "libmutant.so")
    orc.build_variant(str(c), so)
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), so=so)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode != 3, f"mutant {mid} survived: {r.stdout[-500:]}"
    assert r.returncode == 0, f"mutant {mid} crashed the runner (rc={r.returncode}): {r.stderr[-800:]}"


# planted mistakes in the oracle's Python head bookkeeping (grouped-query attention)
PY_MUTANTS = [
    ("kv_head_modulo", lambda h, H, Hkv: h % Hkv),
    ("kv_head_first", lambda h, H, Hkv: 0),
]


@pytest.mark.parametrize("mid,fn", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_planted_python_mistake_is_caught(orc, monkeypatch, mid, fn):
    import oracle_pins

    monkeypatch.setattr(orc, "kv_head", fn)
    with pytest.raises(AssertionError):
        oracle_pins.pin_gqa_equals_replicated_kv()


# planted mistakes in the oracle's packed-batch bookkeeping, applied to the
# function's own source text
PY_SRC_MUTANTS = [
    ("varlen_k_uses_q_offsets", "attn_varlen", "(q0, q1), (k0, k1) = sq[b], sk[b]", "(q0, q1), (k0, k1) = sq[b], sq[b]"),
    ("varlen_v_uses_q_offsets", "attn_varlen", "v[None, k0:k1]", "v[None, q0:q1]"),
    ("varlen_start_off_by_one", "seq_slices", "return list(zip(cu[:-1], cu[1:]))",
     "return list(zip([c + (c > 0) for c in cu[:-1]], cu[1:]))"),
]


@pytest.mark.parametrize("mid,fname,old,new", PY_SRC_MUTANTS, ids=[m[0] for m in PY_SRC_MUTANTS])
def test_planted_python_source_mistake_is_caught(orc, monkeypatch, mid, fname, old, new):
    import inspect

    import oracle_pins

    src = inspect.getsource(getattr(orc, fname))
    assert src.count(old) == 1, "mutation site vanished from the oracle code"
    ns = dict(vars(orc))
    exec(compile(src.replace(old, new), f"<mutant {mid}>", "exec"), ns)
    monkeypatch.setattr(orc, fname, ns[fname])
    caught = None
    for pin in (oracle_pins.pin_varlen_matches_separate_sequences, oracle_pins.pin_no_keys_gives_zero):
        try:
            pin()
        except (AssertionError, ValueError, IndexError) as e:
            caught = (pin.__name__, type(e).__name__)
            break
    assert caught, f"mutant {mid} survived"
