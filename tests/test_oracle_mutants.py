"""Each plausible mistake planted in a copy of the oracle fails some pin.

The oracle's source is copied, one edit is applied to the copy (a dropped
term, a wrong sign, a wrong index or axis, a transposed operand), the copy is
loaded as a separate module on the CPU, and the full pin battery must reject it.
The real oracle is never modified.
"""
import os
import types

import pytest

from tests import oracle_checks as oc

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
SRC = os.path.join(ORACLE_DIR, "attention.py")

MUTANTS = {
    "dropped_scale": ("s = sc * (q @ k.T)", "s = (q @ k.T)"),
    "mask_direction": ("return np.tril(np.ones((n, n), dtype=bool))",
                       "return np.triu(np.ones((n, n), dtype=bool))"),
    "mask_strict": ("return np.tril(np.ones((n, n), dtype=bool))",
                    "return np.tril(np.ones((n, n), dtype=bool), -1) | (np.arange(n) == 0)[None, :]"),
    "lse_dropped_max": ("lse = m[:, 0] + np.log(l[:, 0])", "lse = np.log(l[:, 0])"),
    "lse_log2": ("lse = m[:, 0] + np.log(l[:, 0])", "lse = m[:, 0] + np.log2(l[:, 0])"),
    "sum_wrong_axis": ("l = e.sum(axis=1, keepdims=True)\n    p = e / l",
                       "l = e.sum(axis=0, keepdims=True)\n    p = e / l"),
    "pv_transposed": ("return p @ v, lse", "return p.T @ v, lse"),
    "dv_untransposed": ("dv = p.T @ do", "dv = p @ do"),
    "dp_transposed": ("dp = do @ v.T", "dp = (do @ v.T).T"),
    "ds_sign": ("ds = p * (dp - dvec)", "ds = p * (dp + dvec)"),
    "ds_dropped_d": ("ds = p * (dp - dvec)", "ds = p * dp"),
    "d_wrong_axis": ("dvec = (p * dp).sum(axis=1, keepdims=True)",
                     "dvec = (p * dp).sum(axis=0, keepdims=True)"),
    "dq_transposed": ("dq = sc * (ds @ k)", "dq = sc * (ds.T @ k)"),
    "dk_untransposed": ("dk = sc * (ds.T @ q)", "dk = sc * (ds @ q)"),
    "dk_dropped_scale": ("dk = sc * (ds.T @ q)", "dk = (ds.T @ q)"),
    "rows_mask_strict": ("s = np.where(j <= np.asarray(rows)[:, None], s, -np.inf)",
                         "s = np.where(j < np.asarray(rows)[:, None] + (j == 0), s, -np.inf)"),
    "recurrence_no_rescale": ("l = l * alpha + float(np.exp(t - m_new).sum())",
                              "l = l + float(np.exp(t - m_new).sum())"),
    "recurrence_alpha_sign": ("alpha = 0.0 if m == -np.inf else np.exp(m - m_new)",
                              "alpha = 0.0 if m == -np.inf else np.exp(m_new - m)"),
    "decode_shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "gqa_interleaved_groups": ("return h // (H // Hkv)", "return h % Hkv"),
    "gqa_dk_overwritten": ("dk[b, g] += dk_h", "dk[b, g] = dk_h"),
    "gqa_dv_overwritten": ("dv[b, g] += dv_h", "dv[b, g] = dv_h"),
    "mass_row_sums": ("mass[b] += p.sum(axis=0)", "mass[b] += p.sum(axis=1)"),
    "mass_last_head_only": ("mass[b] += p.sum(axis=0)", "mass[b] = p.sum(axis=0)"),
    "mass_kv_head_by_query_head": ("p, _ = head_probs(q[b, h], k[b, kv_head(h, H, Hkv)], causal, scale)",
                                   "p, _ = head_probs(q[b, h], k[b, h % Hkv], causal, scale)"),
    # FP8 path (oracle/fp8.py)
    "e4m3_round_half_up": ("fp8", "r = np.round(a / step) * step", "r = np.floor(a / step + 0.5) * step"),
    "e4m3_subnormal_step": ("fp8", "expo = np.maximum(ex - 1, -6)          # binade",
                            "expo = np.maximum(ex - 1, -7)          # binade"),
    "e4m3_encode_mantissa": ("fp8", "np.where(normal, 8.0, 1.0)", "np.where(normal, 16.0, 1.0)"),
    "block_exponent_strict": ("fp8", "e = np.where(m <= 0.875, ex - 9, ex - 8)",
                              "e = np.where(m < 0.875, ex - 9, ex - 8)"),
    "block_exponent_floor": ("fp8", "e = np.where(m <= 0.875, ex - 9, ex - 8)", "e = ex - 9"),
    "block_amax_whole_rows": ("fp8", "e = block_exponent(np.abs(blk).max(axis=(1, 2)))",
                              "e = block_exponent(np.abs(x[:, rows, :]).max(axis=(1, 2)))"),
    "dequant_without_scale": ("fp8", "deq[:, rows, cols] = np.ldexp(v, e[:, None, None])",
                              "deq[:, rows, cols] = v"),
    "fp8_forward_unquantised_k": ("fp8", "return attention_forward(qd.reshape(q.shape), kd.reshape(k.shape), v, causal, scale)",
                                  "return attention_forward(qd.reshape(q.shape), k, v, causal, scale)"),
    "rows32_amax_whole_row": ("fp8", "e = block_exponent(np.abs(blk).max(axis=3))            # [R, N, nb]",
                              "e = block_exponent(np.abs(blk).max(axis=(2, 3)))[..., None] + 0 * np.abs(blk).max(axis=3).astype(np.int64)"),
    "rows32_blocks_of_16": ("fp8", "blk = x.reshape(R, N, nb, MX_BLOCK)", "blk = x.reshape(R, N, 2 * nb, 16)[:, :, ::2, :].repeat(1, axis=2).reshape(R, N, nb, 16).repeat(2, axis=3)"),
    "rows32_dequant_without_scale": ("fp8", "deq = np.ldexp(v, e[..., None]).reshape(R, N, d)",
                                     "deq = v.reshape(R, N, d)"),
    "mx_forward_unquantised_q": ("fp8", "return attention_forward(qd, kd, v, causal, scale)",
                                 "return attention_forward(q, kd, v, causal, scale)"),
    "f16_decoded_as_bf16": ("return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)",
                            "return bf16_bits_to_f64(bits)"),
}


def _load_mutant(name, *spec):
    """The oracle with one edit planted: a namespace holding every oracle
    function, those of the edited module taken from the edited copy."""
    import oracle
    fname, old, new = spec if len(spec) == 3 else ("attention", *spec)
    with open(os.path.join(ORACLE_DIR, fname + ".py")) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation {name} does not match oracle/{fname}.py exactly once"
    mod = types.ModuleType(f"oracle.mutant_{name}")
    mod.__package__ = "oracle"  # relative imports resolve to the real package
    exec(compile(text.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    ns = {k: getattr(oracle, k) for k in dir(oracle) if not k.startswith("_")}
    ns.update({k: v for k, v in mod.__dict__.items() if not k.startswith("_")})
    return types.SimpleNamespace(**ns)


def _battery_fails(mod):
    for check in oc.ALL_CHECKS:
        try:
            check(mod)
        except Exception:
            return check.__name__
    return None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _load_mutant(name, *MUTANTS[name])
    caught_by = _battery_fails(mod)
    assert caught_by is not None, f"planted mistake {name!r} passed every pin"


@pytest.mark.parametrize("fname,anchor", [("attention", "def key_mass("), ("fp8", "def e4m3_round(")])
def test_unmutated_copy_passes(fname, anchor):
    # the same loading path with an edit that changes nothing
    assert _battery_fails(_load_mutant("identity", fname, anchor, anchor)) is None
