"""Plant plausible mistakes in the oracle (on the CPU, in a private copy of
its source) and check that the pins catch every one of them: a dropped term,
a wrong index or sign, a transposed or reversed operand, an off-by-one mask."""
import importlib.util
import os
import types

import pytest

import oracle
import test_oracle_backward as bpins
import test_oracle_layered as lpins
import test_oracle_pages as ppins
import test_oracle_pins as pins
import test_oracle_quant_append_counts as qpins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

ATTENTION_MUTANTS = [
    ("g = h // group", "g = h % hkv"),                                   # wrong GQA head map
    ("p = ctx - q_len + i", "p = i"),                                    # top-left causal alignment
    ("vis &= j <= p", "vis &= j < p"),                                   # diagonal masked
    ("vis &= (p - j) <= window_left", "vis &= (p - j) < window_left"),   # window one short
    ("s = scale * (q_rows @ keys.T)", "s = q_rows @ keys.T"),            # dropped scale
    ("num = e @ values", "num = e @ values[::-1]"),                      # wrong value index
    ("slot = t % page_size", "slot = (t + 1) % page_size"),              # wrong slot
    ("phys = block_row[t // page_size]", "phys = block_row[(t // page_size) // 2]"),  # wrong page
    ("lse[ok] = m_safe[ok] + np.log(denom[ok])", "lse[ok] = m_safe[ok] - np.log(denom[ok])"),  # sign
    ("e = np.exp(s - m_safe[:, None])", "e = np.exp(s - m_safe[:, None] / 2)"),  # max not subtracted fully
    ("(1.0 / np.sqrt(d))", "(1.0 / d)"),                                 # wrong default scale
    ("q_rows @ keys.T", "q_rows @ keys[::-1].T"),                        # reversed keys
]

QUANT_MUTANTS = [
    ("np.float32(127.0)", "np.float32(128.0)"),
    ("np.rint(y)", "np.floor(y)"),
    ("np.abs(x).max(axis=(1, 3))", "x.max(axis=(1, 3))"),
    ("axis=(1, 3)", "axis=(1, 2)"),
]


DEQUANT_MUTANTS = [
    ("[:, None, :, None]\n", "[None, :, :, None]\n"),                  # scale of the slot's index, not the page's
    ("np.asarray(codes, dtype=np.float64) *", "np.asarray(codes, dtype=np.float64).clip(-64, 64) *"),  # codes clipped
]


APPEND_MUTANTS = [
    ("* scales[phys, hk]\n", "\n"),                                      # old codes not dequantised
    ("amax = np.abs(vals).max()", "amax = np.abs(new).max() if new.size else np.float32(0)"),  # old rows out of absmax
    ("n_old = max(0, min(s0, p0 + page_size) - p0)", "n_old = 0"),      # old rows ignored
    ("first_row = r0 + (p0 + n_old - s0)", "first_row = r0 + max(0, p0 - s0 - 1)"),  # wrong input row
    ("hi = min(end, p0 + page_size) - p0", "hi = min(end + 1, p0 + page_size) - p0"),  # one slot past the end
]


LAYERED_MUTANTS = [
    ("for part, n in ((hi, n_hi), (lo, n_lo)):", "for part, n in ((hi, n_hi), (lo, max(0, n_lo - 1))):"),  # last int8 key dropped
    ('part.get("v_scales"), row', 'part.get("k_scales"), row'),          # V read back with K's scales
    ("keys = np.concatenate(parts_k, axis=0)", "keys = np.concatenate(parts_k[::-1], axis=0)"),  # K/V paired across parts
    ('row = np.asarray(part["block_table"])[b]', 'row = np.asarray(hi["block_table"])[b]'),  # second part through the first's table
    ("phys = np.asarray(block_row)[np.arange(n_tokens) // page_size]", "phys = np.arange(n_tokens) // page_size"),  # scale of the logical page
]


PAGES_MUTANTS = [
    ("and self.refcount[row[have - 1]] > 1)", "and False)"),                 # no copy-on-write
    ("length % self.page_size != 0", "True"),                                # copy also at a page boundary
    ("        self.rows[seq] = []\n", "        pass\n"),                    # release keeps the table row
    ("            self.refcount[p] += 1\n", "            pass\n"),            # fork does not count holders
    ("p = min(self.free_pages())", "p = max(self.free_pages())"),            # highest id first
    ("k[d], v[d] = k[s], v[s]", "k[d], v[d] = k[s], v[d]"),                  # V page not copied
]


BACKWARD_MUTANTS = [
    ("ds = p * (dp - (doh * o).sum(axis=1)[:, None])", "ds = p * dp"),           # softmax Jacobian term dropped
    ("dq[q0:q1, h, :] = scale * (ds @ kh)", "dq[q0:q1, h, :] = ds @ kh"),         # scale dropped in dQ
    ("dk[:, g, :] += scale * (ds.T @ qh)", "dk[:, g, :] = scale * (ds.T @ qh)"),  # GQA heads not summed
    ("dv[:, g, :] += p.T @ doh", "dv[:, g, :] += p.T @ doh[::-1]"),              # rows of dO misaligned
    ("dp = doh @ vh.T", "dp = doh @ kh.T"),                                     # dP from K instead of V
    ("g = h // group", "g = h % hkv"),                                          # wrong GQA head map
]


def _load_mutant(filename, old, new):
    src = open(os.path.join(ORACLE_DIR, filename)).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant_" + filename[:-3])
    exec(compile(src, filename + " (mutant)", "exec"), mod.__dict__)
    return mod


def _attention_battery():
    for kw in pins.CASES:
        pins.test_oracle_matches_brute_force(kw)
    for args in [(4, 4, True, -1), (8, 2, True, -1), (6, 3, False, -1), (4, 2, True, 4)]:
        pins.test_oracle_matches_torch_sdpa(*args)
    pins.test_closed_form_example()
    pins.test_causal_row0_and_zero_query()
    pins.test_window_special_cases()
    pins.test_decode_equals_prefill_row()


def _quant_battery():
    qpins.test_int8_quantiser_bounds_and_roundtrip()
    qpins.test_int8_quantiser_matches_per_element_fp32_loop()
    qpins.test_int8_half_way_rounds_to_even()


def _dequant_battery():
    qpins.test_int8_dequantiser_matches_per_element_loop()
    qpins.test_int8_quantiser_bounds_and_roundtrip()


def _append_battery():
    qpins.test_int8_append_of_a_whole_page_is_the_page_quantiser()
    qpins.test_int8_append_with_smaller_rows_keeps_scale_and_old_codes()
    qpins.test_int8_append_error_bound_on_old_and_new_rows()
    qpins.test_int8_append_matches_scalar_loop()


def _layered_battery():
    lpins.test_layered_split_equals_whole_cache()
    lpins.test_layered_with_an_empty_part_is_the_plain_decode()
    lpins.test_layered_int8_part_matches_brute_force()
    lpins.test_layered_sequence_without_keys()


def _pages_battery():
    ppins.test_hand_worked_scenario()
    ppins.test_out_of_pages_changes_nothing()
    for seed in range(6):
        ppins.test_random_scripts_keep_invariants_and_contents(seed)
    ppins.test_copy_pages_is_a_page_copy()


def _backward_battery():
    for case in bpins.CASES:
        bpins.test_backward_matches_torch_autograd(case)
    bpins.test_gqa_gradient_is_the_sum_over_repeated_heads()
    bpins.test_keys_no_query_sees_get_zero_gradient()


def test_battery_passes_on_the_real_oracle():
    _attention_battery()
    _quant_battery()
    _dequant_battery()
    _append_battery()
    _layered_battery()
    _pages_battery()
    _backward_battery()


@pytest.mark.parametrize("old,new", ATTENTION_MUTANTS)
def test_attention_mutant_is_caught(monkeypatch, old, new):
    mut = _load_mutant("attention.py", old, new)
    for name in ("attention_paged", "decode_paged", "visible_mask", "gather_sequence"):
        monkeypatch.setattr(oracle, name, getattr(mut, name))
    with pytest.raises(AssertionError):
        _attention_battery()


@pytest.mark.parametrize("old,new", QUANT_MUTANTS)
def test_quant_mutant_is_caught(monkeypatch, old, new):
    mut = _load_mutant("quant.py", old, new)
    monkeypatch.setattr(oracle, "quantize_int8_pages", mut.quantize_int8_pages)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        _quant_battery()


@pytest.mark.parametrize("old,new", DEQUANT_MUTANTS)
def test_dequant_mutant_is_caught(monkeypatch, old, new):
    mut = _load_mutant("quant.py", old, new)
    monkeypatch.setattr(oracle, "dequantize_int8_pages", mut.dequantize_int8_pages)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        _dequant_battery()


@pytest.mark.parametrize("old,new", APPEND_MUTANTS)
def test_int8_append_mutant_is_caught(monkeypatch, old, new):
    mut = _load_mutant("quant.py", old, new)
    monkeypatch.setattr(oracle, "append_int8_pages", mut.append_int8_pages)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        _append_battery()


@pytest.mark.parametrize("old,new", LAYERED_MUTANTS)
def test_layered_mutant_is_caught(monkeypatch, old, new):
    mut = _load_mutant("attention.py", old, new)
    monkeypatch.setattr(oracle, "decode_layered", mut.decode_layered)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        _layered_battery()


@pytest.mark.parametrize("old,new", PAGES_MUTANTS)
def test_pages_mutant_is_caught(monkeypatch, old, new):
    from oracle import pages
    mut = _load_mutant("pages.py", old, new)
    monkeypatch.setattr(pages, "PagePoolModel", mut.PagePoolModel)
    monkeypatch.setattr(pages, "copy_pages", mut.copy_pages)
    with pytest.raises((AssertionError, ValueError, IndexError, TypeError)):
        _pages_battery()


@pytest.mark.parametrize("old,new", BACKWARD_MUTANTS)
def test_backward_mutant_is_caught(monkeypatch, old, new):
    from oracle import backward
    src = open(os.path.join(ORACLE_DIR, "backward.py")).read()
    assert src.count(old) == 1, old
    src = src.replace(old, new).replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType("oracle_mutant_backward")
    exec(compile(src, "backward.py (mutant)", "exec"), mod.__dict__)
    monkeypatch.setattr(backward, "attention_backward_paged", mod.attention_backward_paged)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        _backward_battery()
