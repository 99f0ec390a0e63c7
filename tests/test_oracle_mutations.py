"""Planted mistakes in the oracle (CPU only): each plausible slip in the forward
(a dropped term, a wrong base, a mis-mapped head, a mask or partition off by one,
unnormalised merge weights, a reversed ring) and in the backward (a dropped D
term, a flipped sign, a wrong operand or scale, a gradient off by 1e-4, GQA
groups not summed) is put into the oracle by monkeypatching, and at least one of
its pins must then fail. Without a planted mistake every pin passes.

The mistakes are planted in the oracle only, on the CPU. The pins compare it with
independent references (the pure-Python brute force, torch's fp64 SDPA, closed
forms, the hand-computed golden case, invariants), so each row here shows that a
mistake of that kind cannot go unnoticed.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.attention as att
import oracle.partition as part_mod
from tests import test_oracle_attention as pins

_orig_rows = att.attention_rows
_orig_positions = part_mod.positions
_orig_visible = part_mod.visible_matrix
_orig_merge = att.lse_merge


def _rows_no_scale(q, pq, k, v, pk, cu, S, causal=True, scale=None):
    return _orig_rows(q, pq, k, v, pk, cu, S, causal, 1.0 if scale is None else scale)


def _rows_lse_log2(*a, **kw):
    O, L = _orig_rows(*a, **kw)
    return O, L / math.log(2.0)


def _rows_heads_interleaved(q, pq, k, v, pk, cu, S, causal=True, scale=None):
    # query head h reads KV head h % hkv instead of h // (hq / hkv)
    hq, hkv = np.shape(q)[1], np.shape(k)[1]
    sel = [h % hkv for h in range(hq)]
    return _orig_rows(q, pq, np.asarray(k)[:, sel], np.asarray(v)[:, sel], pk, cu, S, causal, scale)


def _visible_strict(pos_q, pos_k, cu, S, causal):
    vis = _orig_visible(pos_q, pos_k, cu, S, causal)
    if causal:
        vis &= np.asarray(pos_k)[None, :] != np.asarray(pos_q)[:, None]  # a row misses its own key
    return vis


def _visible_no_docs(pos_q, pos_k, cu, S, causal):
    return _orig_visible(pos_q, pos_k, None, S, causal)


def _positions_mirror_off(partition, S, cp, rank, cu=None):
    if partition != "zigzag":
        return _orig_positions(partition, S, cp, rank, cu)
    half = S // (2 * cp)
    mirror = (2 * cp - rank) % (2 * cp)  # off by one: should be 2 cp - 1 - rank
    return np.concatenate([np.arange(rank * half, (rank + 1) * half), np.arange(mirror * half, (mirror + 1) * half)])


def _positions_striped_blocked(partition, S, cp, rank, cu=None):
    if partition == "striped":
        return _orig_positions("contiguous", S, cp, rank, cu)
    return _orig_positions(partition, S, cp, rank, cu)


def _merge_unnormalised(o_a, lse_a, o_b, lse_b):
    # weights e^{LSE_a}, e^{LSE_b} without dividing by e^{LSE}
    o, lse = _orig_merge(o_a, lse_a, o_b, lse_b)
    wa = np.exp(np.asarray(lse_a)).T[:, :, None]
    wb = np.exp(np.asarray(lse_b)).T[:, :, None]
    return wa * np.asarray(o_a) + wb * np.asarray(o_b), lse


def _ring_reversed(cp, rank):
    return [(rank + t) % cp for t in range(cp)]


MISTAKES = {
    "softmax scale dropped": [(att, "attention_rows", _rows_no_scale)],
    "LSE in base 2": [(att, "attention_rows", _rows_lse_log2)],
    "GQA heads interleaved": [(att, "attention_rows", _rows_heads_interleaved)],
    "causal mask off by one": [(att, "visible_matrix", _visible_strict), (part_mod, "visible_matrix", _visible_strict)],
    "documents ignored": [(att, "visible_matrix", _visible_no_docs), (part_mod, "visible_matrix", _visible_no_docs)],
    "zigzag mirror chunk off by one": [(att, "positions", _positions_mirror_off)],
    "striped read as contiguous": [(att, "positions", _positions_striped_blocked)],
    "merge weights unnormalised": [(att, "lse_merge", _merge_unnormalised), (oracle, "lse_merge", _merge_unnormalised)],
    "ring direction reversed": [(att, "ring_chunk_order", _ring_reversed), (oracle, "ring_chunk_order", _ring_reversed)],
}

PINS = {
    "brute force, zigzag GQA with documents": lambda: pins.test_dense_matches_brute_force("zigzag", 2, True, 4, 2, True),
    "brute force, striped non-causal": lambda: pins.test_dense_matches_brute_force("striped", 4, False, 4, 1, False),
    "brute force, contiguous": lambda: pins.test_dense_matches_brute_force("contiguous", 2, False, 2, 2, True),
    "torch SDPA, GQA": lambda: pins.test_cp1_equals_torch_sdpa(True, 8, 2),
    "documents as separate sequences": pins.test_documents_equal_independent_sequences,
    "one token per rank (golden)": pins.test_one_token_per_rank_golden,
    "closed forms": pins.test_closed_forms,
    "I1 chunk and merge": lambda: pins.test_I1_chunk_and_merge_equals_unchunked("zigzag", True),
    "merge hand example": pins.test_merge_hand_example,
    "ring passing": pins.test_ring_chunk_order_follows_the_send_to_next_ring,
}


def _failing_pins():
    failed = []
    for name, pin in PINS.items():
        try:
            pin()
        except AssertionError:
            failed.append(name)
    return failed


def test_every_pin_passes_on_the_oracle_as_written():
    assert _failing_pins() == []


@pytest.mark.parametrize("mistake", list(MISTAKES))
def test_planted_mistake_fails_a_pin(mistake, monkeypatch):
    for module, name, fn in MISTAKES[mistake]:
        monkeypatch.setattr(module, name, fn)
    failed = _failing_pins()
    assert failed, f"no pin notices: {mistake}"


# ---------------------------------------------------------------------------
# The backward oracle: attention_rank_backward goes through
# attention_rows_backward, whose chain-rule steps are restated below with one
# slip each (ring_step_gradients keeps its own, unchanged copy, so the pins that
# compare the two also see the slip).
# ---------------------------------------------------------------------------
import oracle.backward as bwd_mod  # noqa: E402
from tests import test_oracle_backward as bwd_pins  # noqa: E402


def _rows_backward_with(slip):
    def f(q_rows, pos_q, k_rows, v_rows, pos_k, dout, cu_seqlens, s_total, causal=True, scale=None):
        q_rows, k_rows, v_rows, dout = (np.asarray(x, dtype=np.float64) for x in (q_rows, k_rows, v_rows, dout))
        R, hq, d = q_rows.shape
        K, hkv, _ = k_rows.shape
        group = hq // hkv
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        dq, dk, dv = np.zeros((R, hq, d)), np.zeros((K, hkv, d)), np.zeros((K, hkv, d))
        vis = part_mod.visible_matrix(np.asarray(pos_q), np.asarray(pos_k), cu_seqlens, s_total, causal)
        any_vis = vis.any(axis=1)
        for h in range(hq):
            g = h // group
            s = np.where(vis, (q_rows[:, h] @ k_rows[:, g].T) * scale, -np.inf)
            m = np.where(any_vis, s.max(axis=1), 0.0)
            e = np.exp(s - m[:, None])
            P = np.where(any_vis[:, None], e / np.where(any_vis, e.sum(axis=1), 1.0)[:, None], 0.0)
            dO = dout[:, h]
            dP = dO @ v_rows[:, g].T
            D = (P * dP).sum(axis=1)[:, None]
            dS = {"D term dropped": P * dP, "dS sign flipped": P * (D - dP)}.get(slip, P * (dP - D))
            dq[:, h] = scale * (dS @ (v_rows[:, g] if slip == "dQ against V" else k_rows[:, g]))
            dk_h = (1.0 if slip == "scale dropped on dK" else scale) * (dS.T @ q_rows[:, h])
            dv_h = (dS if slip == "dV from dS" else P).T @ dO * (1 + 1e-4 if slip == "dV off by 1e-4" else 1.0)
            if slip == "GQA group not summed":
                dk[:, g], dv[:, g] = dk_h, dv_h
            else:
                dk[:, g] += dk_h
                dv[:, g] += dv_h
        return dq, dk, dv
    return f


BWD_SLIPS = ["D term dropped", "dS sign flipped", "dQ against V", "scale dropped on dK", "dV from dS",
             "dV off by 1e-4", "GQA group not summed"]

BWD_PINS = {
    "autograd, zigzag GQA with documents": lambda: bwd_pins.test_backward_matches_torch_autograd(
        "zigzag", 2, True, (4, 1), True),
    "autograd, striped non-causal": lambda: bwd_pins.test_backward_matches_torch_autograd(
        "striped", 4, False, (2, 2), False),
    "golden one token per rank": bwd_pins.test_backward_golden_one_token_per_rank,
    "closed forms": bwd_pins.test_backward_closed_forms,
    "identities": lambda: bwd_pins.test_backward_identities("zigzag"),
    "ring steps partition the sums": lambda: bwd_pins.test_ring_steps_partition_the_sums("contiguous"),
}


def _failing_bwd_pins():
    failed = []
    for name, pin in BWD_PINS.items():
        try:
            pin()
        except AssertionError:
            failed.append(name)
    return failed


def test_every_backward_pin_passes_on_the_oracle_as_written():
    assert _failing_bwd_pins() == []


def test_the_restated_chain_rule_without_a_slip_passes(monkeypatch):
    monkeypatch.setattr(bwd_mod, "attention_rows_backward", _rows_backward_with(None))
    assert _failing_bwd_pins() == []


@pytest.mark.parametrize("slip", BWD_SLIPS)
def test_planted_backward_slip_fails_a_pin(slip, monkeypatch):
    monkeypatch.setattr(bwd_mod, "attention_rows_backward", _rows_backward_with(slip))
    assert _failing_bwd_pins(), f"no pin notices: {slip}"
