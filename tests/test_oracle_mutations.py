"""Planted mistakes in the oracle (CPU only): each plausible slip in the forward
(a dropped term, a wrong base, a mis-mapped head, a mask or partition off by one,
unnormalised merge weights, a reversed ring) and in the backward (a dropped D
term, a flipped sign, a wrong operand or scale, a gradient off by 1e-4, GQA
groups not summed) and in the layouts (Ulysses head or token order, a reorder
inverse off by a rank, ragged tiles, the per-document zigzag's bounds and pair
rotation) and in the Ulysses x Ring hybrid (head slices, key positions) is put
into the oracle by monkeypatching, and at least one of its pins
must then fail. Without a planted mistake every pin passes.

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


# ---------------------------------------------------------------------------
# Layouts, classification and the per-document zigzag map.
# ---------------------------------------------------------------------------
import oracle.classify as cls_mod  # noqa: E402
import oracle.layouts as lay_mod  # noqa: E402
from tests import test_oracle_doc_zigzag as doc_pins  # noqa: E402
from tests import test_oracle_layouts as lay_pins  # noqa: E402

_orig_ulysses = lay_mod.ulysses_permute
_orig_reorder = lay_mod.cp_reorder
_orig_classify = cls_mod.classify_tiles
_orig_bounds = part_mod.doc_zigzag_piece_bounds
_orig_runs = part_mod.doc_zigzag_rank_runs


def _ulysses_heads_interleaved(x, n, inverse=False):
    # device rho takes heads rho, rho + n, ... instead of the block [rho H/n, (rho+1) H/n)
    x = np.asarray(x)
    if inverse:
        return _orig_ulysses(x, n, inverse)
    N, sl, H, d = x.shape
    perm = [h2 * n + rho for rho in range(n) for h2 in range(H // n)]
    return _orig_ulysses(x[:, :, perm], n)


def _ulysses_tokens_by_local_index(x, n, inverse=False):
    # tokens ordered by local index, then source rank
    y = _orig_ulysses(x, n, inverse)
    if inverse:
        return y
    N, S = y.shape[:2]
    sl = S // n
    order = [j * sl + i for i in range(sl) for j in range(n)]
    return y[:, order]


def _reorder_inverse_shifted(x, cp, partition, inverse=False, cu_seqlens=None, s_total=None):
    # the inverse takes rank r's rows from rank r - 1's slot
    if not inverse:
        return _orig_reorder(x, cp, partition, inverse, cu_seqlens, s_total)
    return _orig_reorder(np.roll(np.asarray(x), 1, axis=0), cp, partition, True, cu_seqlens, s_total)


def _classify_edges_as_full_tiles(s_total, cp, rank, partition, cu_seqlens, bm, bn, causal=True,
                                  return_counts=False):
    # edge tiles compared with a whole bm x bn tile: a fully visible ragged tile reads PARTIAL
    cls, counts = _orig_classify(s_total, cp, rank, partition, cu_seqlens, bm, bn, causal, True)
    cls = np.where(counts == 0, 0, np.where(counts == bm * bn, 2, 1)).astype(np.int8)
    return (cls, counts) if return_counts else cls


def _bounds_rounded_down(L, cp, g=part_mod.DOC_GRANULE):
    n = 2 * cp
    k = np.arange(n + 1, dtype=np.int64)
    b = np.minimum(g * ((k * L) // (n * g)), L)
    b[n] = L
    return b


def _runs_pairs_not_rotated(cu_seqlens, s_total, cp, rank, g=part_mod.DOC_GRANULE):
    # every document gives rank r the same pair (r, 2CP-1-r): no rotation by document
    cu = np.asarray([0, s_total] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    runs = []
    for j in range(len(cu) - 1):
        b = part_mod.doc_zigzag_piece_bounds(int(cu[j + 1] - cu[j]), cp, g)
        for piece in (rank, 2 * cp - 1 - rank):
            n_tok = int(b[piece + 1] - b[piece])
            if n_tok > 0:
                runs.append((int(cu[j] + b[piece]), n_tok, g * -(-n_tok // g)))
    return runs


LAYOUT_MISTAKES = {
    "Ulysses heads interleaved": [(lay_mod, "ulysses_permute", _ulysses_heads_interleaved),
                                  (oracle, "ulysses_permute", _ulysses_heads_interleaved)],
    "Ulysses tokens by local index": [(lay_mod, "ulysses_permute", _ulysses_tokens_by_local_index),
                                      (oracle, "ulysses_permute", _ulysses_tokens_by_local_index)],
    "cp_reorder inverse reads the wrong rank": [(lay_mod, "cp_reorder", _reorder_inverse_shifted),
                                                (oracle, "cp_reorder", _reorder_inverse_shifted)],
    "edge tiles classified as whole tiles": [(cls_mod, "classify_tiles", _classify_edges_as_full_tiles),
                                             (oracle, "classify_tiles", _classify_edges_as_full_tiles)],
    "doc-zigzag bounds rounded down": [(part_mod, "doc_zigzag_piece_bounds", _bounds_rounded_down),
                                       (doc_pins, "doc_zigzag_piece_bounds", _bounds_rounded_down)],
    "doc-zigzag pairs not rotated by document": [(part_mod, "doc_zigzag_rank_runs", _runs_pairs_not_rotated),
                                                 (doc_pins, "doc_zigzag_rank_runs", _runs_pairs_not_rotated)],
}

LAYOUT_PINS = {
    "Ulysses worked layout (golden)": lay_pins.test_ulysses_worked_layout_golden,
    "Ulysses element indexing": lambda: lay_pins.test_ulysses_inverse_roundtrip_and_indexing(4, 6, 8, 3),
    "cp_reorder against brute positions": lambda: lay_pins.test_cp_reorder_against_brute_positions("zigzag", 4),
    "classification against brute force": lambda: lay_pins.test_classify_matches_brute_force(
        "striped", 2, True, (3, 5), True),
    "classification of ragged tiles": lambda: lay_pins.test_classify_matches_brute_force(
        "contiguous", 2, False, (3, 5), False),
    "doc-zigzag positions against brute force": lambda: doc_pins.test_positions_match_brute_force_and_cover_once(
        5, 2),
    "doc-zigzag piece bounds": lambda: doc_pins.test_piece_bounds(5000, 3),
    "doc-zigzag balance": doc_pins.test_doc_zigzag_balances_packed_documents,
}


def _failing_layout_pins():
    failed = []
    for name, pin in LAYOUT_PINS.items():
        try:
            pin()
        except AssertionError:
            failed.append(name)
    return failed


def test_every_layout_pin_passes_on_the_oracle_as_written():
    assert _failing_layout_pins() == []


@pytest.mark.parametrize("mistake", list(LAYOUT_MISTAKES))
def test_planted_layout_mistake_fails_a_pin(mistake, monkeypatch):
    for module, name, fn in LAYOUT_MISTAKES[mistake]:
        monkeypatch.setattr(module, name, fn)
    assert _failing_layout_pins(), f"no pin notices: {mistake}"


# ---------------------------------------------------------------------------
# The Ulysses x Ring hybrid: usp_forward restated with one slip each.
# ---------------------------------------------------------------------------
import oracle.usp as usp_mod  # noqa: E402
from tests import test_oracle_usp as usp_pins  # noqa: E402


def _usp_with(slip):
    def f(gq, gk, gv, cu_seqlens, U, R, partition, causal=True, scale=None):
        S, hq, d = gq.shape
        sl = S // R
        Yq = [lay_mod.ulysses_permute(s, U) for s in usp_mod.usp_device_shards(gq, U, R, partition)]
        Yk = [lay_mod.ulysses_permute(s, U) for s in usp_mod.usp_device_shards(gk, U, R, partition)]
        Yv = [lay_mod.ulysses_permute(s, U) for s in usp_mod.usp_device_shards(gv, U, R, partition)]
        pos = [part_mod.positions(partition, S, R, r) for r in range(R)]
        O = np.zeros((R, U, sl, hq // U, d))
        L = np.full((R, U, hq // U, sl), -np.inf)
        for r in range(R):
            for u in range(U):
                o = lse = None
                for s in att.ring_chunk_order(R, r):
                    uk = (U - 1 - u) if slip == "KV head slice mirrored" else u
                    pk = pos[r] if slip == "key positions of the query group" else pos[s]
                    o_t, l_t = _orig_rows(Yq[r][u], pos[r], Yk[s][uk], Yv[s][uk], pk, cu_seqlens, S, causal, scale)
                    o, lse = (o_t, l_t) if o is None else _orig_merge(o, lse, o_t, l_t)
                O[r, u], L[r, u] = o, lse
        out = np.stack([lay_mod.ulysses_permute(O[r], U, inverse=True) for r in range(R)])
        return out, L
    return f


USP_SLIPS = [None, "KV head slice mirrored", "key positions of the query group"]
USP_PINS = {
    "global attention, U = R = 2, zigzag with documents": lambda: usp_pins.test_usp_equals_global_attention(
        2, 2, "zigzag", True),
    "global attention, U = 4, R = 2, striped": lambda: usp_pins.test_usp_equals_global_attention(4, 2, "striped", False),
    "corner cases": usp_pins.test_usp_corner_cases_reduce_to_ring_and_ulysses,
}


@pytest.mark.parametrize("slip", USP_SLIPS)
def test_planted_usp_slip_fails_a_pin(slip, monkeypatch):
    monkeypatch.setattr(usp_mod, "usp_forward", _usp_with(slip))
    monkeypatch.setattr(oracle, "usp_forward", _usp_with(slip))
    failed = []
    for name, pin in USP_PINS.items():
        try:
            pin()
        except AssertionError:
            failed.append(name)
    if slip is None:
        assert failed == [], failed  # the restatement without a slip passes every pin
    else:
        assert failed, f"no pin notices: {slip}"
