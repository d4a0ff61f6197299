"""CPU tests: the oracle against its pins, and planted mistakes that the pins catch."""

import importlib.util
import os
import sys
import types

import pytest

import oracle
import oracle.moba_oracle as om
from tests import oracle_pins as P

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "moba_oracle.py")


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(om)


def test_package_exports():
    for name in ("moba_ref", "select_blocks", "pooled_keys", "sparsity", "attended_pairs_closed_form"):
        assert hasattr(oracle, name)


# Each mutation plants one plausible mistake in a copy of the oracle's source.
MUTATIONS = {
    "no_forced_current_block": ("sorted(order[i, :topk - 1].tolist() + [int(j)])",
                                "sorted(order[i, :topk].tolist())"),
    "gate_chunk_offset_dropped": ("sel[h, c0 + i, :len(row)] = row", "sel[h, i, :len(row)] = row"),
    "dense_chunk_drops_last_row": ("idx = in_j[c0:c0 + max_rows_chunk]", "idx = in_j[c0:c0 + max_rows_chunk - 1]"),
    "lists_include_own_block": ("                if 0 <= b < j:\n                    lists[h][b].append(t)",
                                "                if 0 <= b <= j:\n                    lists[h][b].append(t)"),
    "lists_descending": ("for t in range(N):                      # ascending t: every list comes out ascending",
                         "for t in range(N - 1, -1, -1):"),
    "lists_block_major": ("    for h in range(H):\n        for b in range(n):\n            qidx.extend(lists[h][b])",
                          "    for b in range(n):\n        for h in range(H):\n            qidx.extend(lists[h][b])"),
    "causal_mask_off_by_one": ("chosen[:, key_block] & (key_pos[None, :] <= t[:, None])",
                               "chosen[:, key_block] & (key_pos[None, :] < t[:, None] + 2)"),
    "future_blocks_compete": ("neg[np.arange(n)[None, :] >= jj[:, None]] = np.inf",
                              "neg[np.arange(n)[None, :] > jj[:, None]] = np.inf"),
    "ascending_scores": ("neg = -sc.astype(np.float64)", "neg = sc.astype(np.float64)"),
    "scale_1_over_d": ("    scale = 1.0 / math.sqrt(D)\n    R = rows.shape[0]", "    scale = 1.0 / D\n    R = rows.shape[0]"),
    "pool_sum_not_mean": ("return np.ascontiguousarray((total / block_size).transpose(1, 0, 2))",
                          "return np.ascontiguousarray(total.transpose(1, 0, 2))"),
    "pool_wrong_axis": ("total += k64[:, r]", "total += k64[:, r][:, ::-1]"),
    "unstable_ties": ('order = np.argsort(neg, axis=1, kind="stable")',
                      'order = np.argsort(neg[:, ::-1], axis=1, kind="stable"); order = neg.shape[1] - 1 - order'),
    "lse_base2": ("return p / l, (m + np.log(l))[..., 0]", "return p / l, (m + np.log2(l))[..., 0]"),
    "own_block_full": ("parts.append(np.arange(j * block_size, t + 1))",
                       "parts.append(np.arange(j * block_size, (j + 1) * block_size))"),
    "no_fp32_gate_rounding": ("return s.astype(np.float32)", "return s"),
    "pool_fp32_not_rounded": ("return pooled_keys(k, block_size, pooling, weights).astype(np.float32)",
                              "return pooled_keys(k, block_size, pooling, weights).astype(np.float16).astype(np.float32)"),
    "pad_with_zero": ("sel = np.full((H, R, topk), -1, dtype=np.int32)",
                      "sel = np.full((H, R, topk), 0, dtype=np.int32)"),
    "transposed_scores": ("s = np.asarray(q_rows, np.float64) @ np.asarray(kbar32_h, np.float64).T",
                          "s = (np.asarray(q_rows, np.float64)[:, ::-1] @ np.asarray(kbar32_h, np.float64).T)"),
    "softmax_without_max": ("p = np.exp(logits - m)", "p = np.exp(logits - m * 0.5)"),
    "blocks_causal_off_by_one": ("lg[own] = np.where(kpos[None, :] <= rows[ridx][own][:, None], lg[own], -np.inf)",
                                 "lg[own] = np.where(kpos[None, :] < rows[ridx][own][:, None], lg[own], -np.inf)"),
    "blocks_drops_denominator_terms": ("l[ridx] += p.sum(axis=1)", "l[ridx] = p.sum(axis=1)"),
    "rowwise_wrong_head": ("kh = np.asarray(k[keys, h, :], np.float64)",
                           "kh = np.asarray(k[keys, (h + 1) % H, :], np.float64)"),
    "decode_token_off_by_one": ("    t = N - 1\n    j = t // block_size\n    if sel is None:",
                                "    t = N - 1\n    j = t // block_size\n    t = max(t - 1, 0)\n    if sel is None:"),
    "decode_means_reversed": ("kbar32 = pooled_keys_fp32(k[:j * block_size], block_size)",
                                   "kbar32 = pooled_keys_fp32(k[:j * block_size], block_size)[:, ::-1]"),
    "decode_wrong_query_head": ("logits = (k_att @ np.asarray(q_new[h], np.float64)) * inv_sqrt_d",
                                "logits = (k_att @ np.asarray(q_new[(h + 1) % H], np.float64)) * inv_sqrt_d"),
    "decode_scale_1_over_d": ("inv_sqrt_d = 1.0 / math.sqrt(D)", "inv_sqrt_d = 1.0 / D"),
    "pool_max_is_min": ("return np.ascontiguousarray(k64.max(axis=1).transpose(1, 0, 2))",
                        "return np.ascontiguousarray(k64.min(axis=1).transpose(1, 0, 2))"),
    "weighted_not_normalised": ("total / safe[:, :, None], 0.0)", "total, 0.0)"),
    "weighted_weights_of_wrong_head": ("wb = w64.reshape(H, n, block_size).transpose(1, 2, 0)",
                                       "wb = w64[::-1].reshape(H, n, block_size).transpose(1, 2, 0)"),
    "dynamic_k_rounds_up": ("round((1.0 - sparsity) * N / block_size)", "math.ceil((1.0 - sparsity) * N / block_size)"),
    "varlen_local_block_indices": ("sel[:, a:b] = np.where(s >= 0, s + a // block_size, -1)",
                                   "sel[:, a:b] = s"),
    "varlen_sequences_share_context": ("o, l, s = moba_ref(q[a:b], k[a:b], v[a:b], block_size, topk)",
                                       "o, l, s = moba_ref(q[:b], k[:b], v[:b], block_size, topk); "
                                       "o, l, s = o[a:], l[:, a:], s[:, a:]"),
    "varlen_backward_wrong_segment": ("dq, dk, dv, _ = moba_backward_ref(q[a:b], k[a:b], v[a:b], dout[a:b], block_size, topk, sel=s)",
                                      "dq, dk, dv, _ = moba_backward_ref(q[a:b], k[a:b], v[a:b], dout[::-1][a:b], block_size, topk, sel=s)"),
    "backward_scale_1_over_d": ("softmax_scale = 1.0 / math.sqrt(D)", "softmax_scale = 1.0 / D"),
    "backward_drops_row_sum": ("dl = p * (dp - np.sum(p * dp, axis=1, keepdims=True))", "dl = p * dp"),
    "backward_dk_unscaled": ("dk[:nk, oh] += scale * (dl.T @ qh)", "dk[:nk, oh] += dl.T @ qh"),
    "backward_dq_against_v": ("dq[t, oh] = scale * (dl @ kh)", "dq[t, oh] = scale * (dl @ vh)"),
    "backward_dv_uses_logit_grad": ("dv[:nk, oh] += p.T @ doh", "dv[:nk, oh] += dl.T @ doh"),
    "backward_mask_off_by_one": ("mask = chosen[:, key_pos // B] & (key_pos[None, :] <= t[:, None])",
                                 "mask = chosen[:, key_pos // B] & (key_pos[None, :] < t[:, None])"),
    "backward_blocks_delta_last_block_only": ("delta[ridx] += np.sum(p * (doh[ridx] @ vb.T), axis=1)",
                                              "delta[ridx] = np.sum(p * (doh[ridx] @ vb.T), axis=1)"),
    "backward_blocks_dk_from_dout": ("dk[b * B:(b + 1) * B, oh] += scale * (dl.T @ qh[ridx])",
                                     "dk[b * B:(b + 1) * B, oh] += scale * (dl.T @ doh[ridx])"),
}


def _mutant(name, old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutation {name} no longer applies"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    mod.__file__ = ORACLE_SRC
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(name, *MUTATIONS[name])
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError, or a crash caused by the mistake
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin catches the planted mistake {name}"
