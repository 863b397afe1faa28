"""Plant plausible mistakes in copies of the oracle source (on the CPU) and
require the pins to catch every one of them."""

import importlib.util
import os
import sys
import types

import pytest

import oracle_pins as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load_mutant(relpath, old, new, name):
    src = open(os.path.join(ROOT, relpath)).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1)
    mod = types.ModuleType(name)
    mod.__file__ = os.path.join(ROOT, relpath)
    sys.modules[name] = mod
    exec(compile(src, mod.__file__, "exec"), mod.__dict__)
    return mod


GDR_MUTANTS = {
    "dropped_decay": ("S = a[t][:, None, None] * S", "S = S"),
    "decay_after_write": ("S = a[t][:, None, None] * S\n", "S = S\n"),
    "wrong_sign": ("err = v[t] - pred", "err = v[t] + pred"),
    "dropped_beta": ("delta = b[t][:, None] * err", "delta = err"),
    "query_for_key": ('pred = np.einsum("hk,hkv->hv", kt, S)', 'pred = np.einsum("hk,hkv->hv", q[t], S)'),
    "transposed_state": ('pred = np.einsum("hk,hkv->hv", kt, S)', 'pred = np.einsum("hk,hvk->hv", kt, S)'),
    "output_uses_key": ('o[t] = scale * np.einsum("hk,hkv->hv", q[t], S)',
                        'o[t] = scale * np.einsum("hk,hkv->hv", kt, S)'),
    "dropped_scale": ('o[t] = scale * np.einsum', 'o[t] = 1.0 * np.einsum'),
    "prechunk_off_by_one": ("if t % chunk == 0:", "if t % chunk == 1:"),
    "compose_order": ("S = np.matmul(M[s], S) + S_loc[s]", "S = np.matmul(S, M[s]) + S_loc[s]"),
    "compose_drop_local": ("S = np.matmul(M[s], S) + S_loc[s]", "S = np.matmul(M[s], S)"),
    "segment_extra_to_last": ("nc = base + (1 if s < extra else 0)",
                              "nc = base + (1 if s >= n_segments - extra else 0)"),
    # batch wrapper: packing and head sampling
    "wrapper_h0_unsampled": ("np.array(h0[n][hs], dtype=np.float64)", "np.array(h0[n][:Hs], dtype=np.float64)"),
    "wrapper_beta_unsampled": ("beta[b, s:e][:, hs], S0, scale", "beta[b, s:e][:, :Hs], S0, scale"),
    "wrapper_h_rows_by_sequence": ("h[offsets[n]:offsets[n + 1]] = pre", "h[n:n + len(pre)] = pre"),
}


@pytest.mark.parametrize("mut", sorted(GDR_MUTANTS))
def test_gdr_pins_catch(mut):
    old, new = GDR_MUTANTS[mut]
    if mut == "decay_after_write":
        # move the decay after the write: S_t = a (S + b k (v - S^T k)^T)
        old = "        S = a[t][:, None, None] * S\n"
        new = "        pass\n"
        m = _load_mutant("oracle/gdr_ref.py", old, new, f"mut_{mut}")
        src_old = "        vnew[t] = delta\n"
        # re-load with the decay applied after the write instead
        src = open(os.path.join(ROOT, "oracle/gdr_ref.py")).read()
        src = src.replace(old, new, 1).replace(src_old, src_old + "        S = a[t][:, None, None] * S\n", 1)
        m = types.ModuleType(f"mut_{mut}")
        exec(compile(src, "gdr_ref_mut", "exec"), m.__dict__)
    else:
        m = _load_mutant("oracle/gdr_ref.py", old, new, f"mut_{mut}")
    failures = 0
    for check in P.GDR_CHECKS:
        try:
            check(m)
        except Exception:
            failures += 1
    assert failures > 0, f"no pin caught mutation {mut}"


ABC_MUTANTS = {
    "ratio_inverted": ("r = np.exp(z_prev - zt)", "r = np.exp(zt - z_prev)"),
    "unnormalised_weight": ("w = np.exp(s[t] - zt)", "w = np.exp(s[t] - z_prev)"),
    "missing_logaddexp": ("zt = np.logaddexp(z_prev, s[t])", "zt = np.maximum(z_prev, s[t])"),
    "hk_scaled_on_rows": ("Hk = Hk * r[:, None, :]", "Hk = Hk * r[:, :1, None]"),
    "hv_scaled_on_cols": ("Hv = Hv * r[:, :, None]", "Hv = Hv * r[:, None, :1]"),
    "prechunk_after_update": ("        if t % chunk == 0:\n            hk_pre.append(Hk.copy())",
                              "        if t % chunk == 1:\n            hk_pre.append(Hk.copy())"),
    "weighted_scan_sign": ("Hk = Hk * r[t][None, :] + np.outer(k[t], w[t])",
                           "Hk = Hk * r[t][None, :] - np.outer(k[t], w[t])"),
    "resume_ignores_normaliser": ("z_prev = np.full((H, M), -np.inf) if z0 is None else np.array(z0, dtype=np.float64)",
                                  "z_prev = np.full((H, M), -np.inf)"),
    "read_score_unscaled": ("score[t] = scale * np.einsum", "score[t] = np.einsum"),
    "read_value_with_scores": ('o[t] = np.einsum("hmv,hm->hv", Hv, pw[t])', 'o[t] = np.einsum("hmv,hm->hv", Hv, score[t])'),
    "read_softmax_unnormalised": ("pw[t] = e / e.sum(axis=-1, keepdims=True)", "pw[t] = e"),
    "read_query_for_key": ('score[t] = scale * np.einsum("hkm,hk->hm", Hk, q[t])',
                           'score[t] = scale * np.einsum("hkm,hk->hm", Hk, k[t])'),
    # batch wrappers: row and head sampling
    "wrapper_logits_unsampled": ("s[b][:, hs], chunk) for b in bs]", "s[b][:, :len(hs)], chunk) for b in bs]"),
    "wrapper_read_weights_unsampled": ("np.asarray(p[b], dtype=np.float64)[:, hs]",
                                       "np.asarray(p[b], dtype=np.float64)[:, :len(hs)]"),
    "wrapper_read_query_of_first_row": ("abc_readout_sequence(q[b][:, hs]", "abc_readout_sequence(q[bs[0]][:, hs]"),
}


@pytest.mark.parametrize("mut", sorted(ABC_MUTANTS))
def test_abc_pins_catch(mut):
    old, new = ABC_MUTANTS[mut]
    m = _load_mutant("oracle/abc_ref.py", old, new, f"mut_abc_{mut}")
    failures = 0
    for check in P.ABC_CHECKS + P.ABC_READ_CHECKS:
        try:
            check(m)
        except Exception:
            failures += 1
    assert failures > 0, f"no pin caught mutation {mut}"


BWD_MUTANTS = {
    "bwd_dropped_scale": ("G = carry + scale * q[t]", "G = carry + q[t]"),
    "bwd_no_end_gradient": ("carry = np.array(dS_end, dtype=np.float64)",
                            "carry = 0 * np.array(dS_end, dtype=np.float64)"),
    "bwd_jacobian_sign": ("(X - beta[t][:, None, None]", "(X + beta[t][:, None, None]"),
    "bwd_dropped_decay": ("return a[t][:, None, None] * (X", "return (X"),
    "bwd_boundary_includes_own_output": ("dh[t // chunk] = carry",
                                         "dh[t // chunk] = carry + scale * q[t][:, :, None] * do[t][:, None, :]"),
    "bwd_dv_untransposed": ("scale * (P.T @ dd)", "scale * (P @ dd)"),
    "bwd_dv_no_decay": ("np.exp(ga[-1] - ga)[:, None] * (kk @ dh[c, hh])", "(kk @ dh[c, hh])"),
    "bwd_dv_wrong_boundary": ("(kk @ dh[c, hh])", "(kk @ dh[max(c - 1, 0), hh])"),
    # batch wrapper: packing, final-gradient rows and head sampling
    "bwd_wrapper_dhT_first_sequence": ("np.array(dhT[n][hs], dtype=np.float64)",
                                       "np.array(dhT[0][hs], dtype=np.float64)"),
    "bwd_wrapper_dhT_unsampled": ("np.array(dhT[n][hs], dtype=np.float64)", "np.array(dhT[n][:Hs], dtype=np.float64)"),
    "bwd_wrapper_do_unsampled": ("do[b, s:e][:, hs], dS_end", "do[b, s:e][:, :Hs], dS_end"),
    "bwd_wrapper_dh_rows_by_sequence": ('out["dh"][offsets[n]:offsets[n + 1]] = dh', 'out["dh"][n:n + len(dh)] = dh'),
}


@pytest.mark.parametrize("mut", sorted(BWD_MUTANTS))
def test_bwd_pins_catch(mut):
    from oracle import chunked_ref, gdr_ref

    old, new = BWD_MUTANTS[mut]
    src = open(os.path.join(ROOT, "oracle/gdr_bwd_ref.py")).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1).replace("from .gdr_ref import", "from oracle.gdr_ref import")
    m = types.ModuleType(f"mut_{mut}")
    exec(compile(src, "gdr_bwd_ref_mut", "exec"), m.__dict__)
    failures = 0
    for check in P.BWD_CHECKS:
        try:
            P.run_bwd_check(check, m, gdr_ref, chunked_ref)
        except Exception:
            failures += 1
    assert failures > 0, f"no pin caught mutation {mut}"


ABC_BWD_MUTANTS = {
    "abc_bwd_no_end_gradient": ("ck = np.zeros((H, K, M)) if dhk_end is None else np.array(dhk_end, dtype=np.float64)",
                                "ck = np.zeros((H, K, M))"),
    "abc_bwd_boundary_includes_own_read": ("dhk[t // chunk] = ck", "dhk[t // chunk] = ck + scale * q[t][:, :, None] * dscore[t][:, None, :]"),
    "abc_bwd_dropped_scale": ("Gk = ck + scale * q[t]", "Gk = ck + q[t]"),
    "abc_bwd_ratio_inverted": ("r = np.exp(zp - z[t])", "r = np.exp(z[t] - zp)"),
    "abc_bwd_ratio_of_next_token": ("zp = z[t - 1] if t > 0 else z_before", "zp = z[t]"),
    "abc_bwd_value_uses_scores": ("Gv = cv + p[t][:, :, None] * do[t][:, None, :]",
                                  "Gv = cv + dscore[t][:, :, None] * do[t][:, None, :]"),
    "abc_bwd_value_ratio_on_columns": ("cv = Gv * r[:, :, None]", "cv = Gv * r[:, :1, None]"),
    "abc_bwd_key_ratio_on_rows": ("ck = Gk * r[:, None, :]", "ck = Gk * r[:, :1, None]"),
    # batch wrapper: final-gradient rows and head sampling
    "abc_bwd_wrapper_final_unsampled": ("np.asarray(dhk_final[b], dtype=np.float64)[hs]",
                                        "np.asarray(dhk_final[b], dtype=np.float64)[:len(hs)]"),
    "abc_bwd_wrapper_weights_unsampled": ("p[b][:, hs], dscore[b]", "p[b][:, :len(hs)], dscore[b]"),
    "abc_bwd_wrapper_final_first_row": ("np.asarray(dhv_final[b], dtype=np.float64)[hs]",
                                        "np.asarray(dhv_final[bs[0]], dtype=np.float64)[hs]"),
}


@pytest.mark.parametrize("mut", sorted(ABC_BWD_MUTANTS))
def test_abc_bwd_pins_catch(mut):
    from oracle import abc_ref

    old, new = ABC_BWD_MUTANTS[mut]
    m = _load_mutant("oracle/abc_bwd_ref.py", old, new, f"mut_abc_bwd_{mut}")
    failures = 0
    for check in P.ABC_BWD_CHECKS:
        try:
            P.run_abc_bwd_check(check, m, abc_ref)
        except Exception:
            failures += 1
    assert failures > 0, f"no pin caught mutation {mut}"


KDA_MUTANTS = {
    "channel_averaged_decay": ("S = a[t][:, :, None] * S", "S = a[t].mean(axis=1)[:, None, None] * S"),
    "dropped_beta": ("delta = b[t][:, None] * (v[t] - pred)", "delta = v[t] - pred"),
    "wrong_sign": ("delta = b[t][:, None] * (v[t] - pred)", "delta = b[t][:, None] * (v[t] + pred)"),
    "decay_after_write": ("        S = a[t][:, :, None] * S\n", "        pass\n"),
    "w_without_decay": ("W = T @ (beta[:, None] * k * np.exp(Gam))", "W = T @ (beta[:, None] * k)"),
    "kg_wrong_reference": ("Kg = k * np.exp(Gam[-1][None, :] - Gam)", "Kg = k * np.exp(-Gam)"),
    "a_includes_diagonal": ('A = np.tril(beta[:, None] * np.einsum("td,id,tid->ti", k, k, dec), -1)',
                            'A = np.tril(beta[:, None] * np.einsum("td,id,tid->ti", k, k, dec), 0)'),
    "output_strictly_causal": ("causal = np.tril(np.ones((n, n), dtype=bool))[:, :, None]",
                               "causal = np.tril(np.ones((n, n), dtype=bool), -1)[:, :, None]"),
    "state_decay_first_token": ("return Gam, W, U, Kg, np.exp(Gam[-1])", "return Gam, W, U, Kg, np.exp(Gam[0])"),
}


@pytest.mark.parametrize("mut", sorted(KDA_MUTANTS))
def test_kda_pins_catch(mut):
    from oracle import gdr_ref

    old, new = KDA_MUTANTS[mut]
    src = open(os.path.join(ROOT, "oracle/kda_ref.py")).read()
    assert src.count(old) == 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1)
    if mut == "decay_after_write":
        anchor = "        vnew[t] = delta\n"
        src = src.replace(anchor, anchor + "        S = a[t][:, :, None] * S\n", 1)
    src = src.replace("from .gdr_ref import _sequences, chunk_counts", "from oracle.gdr_ref import _sequences, chunk_counts")
    m = types.ModuleType(f"kda_mut_{mut}")
    exec(compile(src, "kda_ref_mut", "exec"), m.__dict__)
    checks = [lambda: c(m) for c in P.KDA_CHECKS]
    checks += [lambda: P.check_kda_scalar_reduction(m, gdr_ref), lambda: P.check_kda_chunk_algebra(m)]
    failures = 0
    for check in checks:
        try:
            check()
        except Exception:
            failures += 1
    assert failures > 0, f"no pin caught mutation {mut}"
