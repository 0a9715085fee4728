"""The traffic model: byte counts per launch and the capacity chooser (CPU only)."""
import ctypes

import pytest

import recurrent_state_updates_amd as dl
from recurrent_state_updates_amd import _binding as B
from recurrent_state_updates_amd import traffic


def _predict_py(op, Bsz, H, d, C, read, copy, dv=0):
    sh = traffic.Shape(op, Bsz, H, d, 2, dv)
    us = sum(traffic.append_bytes(sh, L) for L in range(C - 1)) / (read * 1e3)
    us += traffic.merge_bytes(sh, C) / (copy * 1e3)
    return us / C


@pytest.mark.parametrize("op,d", [("gdn", 128), ("kda", 128), ("rwkv6", 64), ("gdn", 32)])
@pytest.mark.parametrize("C", [1, 2, 5, 8, 32])
def test_library_model_matches_the_python_byte_model(op, d, C):
    cfg = dl.make_config(op, "bf16", 96, 32, d, d, C)
    got = dl.dl_predict_token_us(cfg, 6000.0, 5000.0)
    assert got == pytest.approx(_predict_py(op, 96, 32, d, C, 6000.0, 5000.0), rel=1e-12)


@pytest.mark.parametrize("op,dk,dv", [("gdn", 64, 128), ("kda", 128, 32), ("rwkv6", 32, 64)])
def test_model_with_distinct_key_and_value_widths(op, dk, dv):
    cfg = dl.make_config(op, "bf16", 16, 8, dk, dv, 8)
    got = dl.dl_predict_token_us(cfg, 6000.0, 5000.0)
    assert got == pytest.approx(_predict_py(op, 16, 8, dk, 8, 6000.0, 5000.0, dv), rel=1e-12)
    sh = traffic.Shape(op, 16, 8, dk, 2, dv)
    assert sh.base() == 4 * dk * dv
    assert traffic.eager_bytes(sh) == 16 * 8 * (8 * dk * dv + sh.token_in() + 4 * dv) + sh.shared()


def test_default_bandwidths_and_argmin():
    cfg = dl.make_config("gdn", "bf16", 128, 32, 128, 128, 8)
    assert dl.dl_predict_token_us(cfg) == pytest.approx(_predict_py("gdn", 128, 32, 128, 8, 6760, 5580))
    for max_c in (1, 4, 8, 32):
        best = dl.dl_choose_capacity(cfg, max_c)
        preds = {C: dl.dl_predict_token_us(dl.make_config("gdn", "bf16", 128, 32, 128, 128, C))
                 for C in range(1, max_c + 1)}
        assert best == min(preds, key=preds.get)


def test_eager_equivalent_and_interval_tradeoff():
    # C = 1 moves exactly the eager bytes; larger C first saves dense writes, then replay grows
    sh = traffic.Shape("gdn", 128, 32, 128, 2)
    assert traffic.cycle_bytes(sh, 1) == traffic.eager_bytes(sh)
    per = [traffic.per_token_bytes(sh, C) for C in range(1, 33)]
    assert per[0] > per[3] > per[7]
    assert per[-1] > min(per)
    # the headline workload: 321.1 MB per token at C = 8 against 542.1 MB eager
    assert traffic.per_token_bytes(sh, 8) / 1e6 == pytest.approx(321.09, abs=0.01)
    assert traffic.eager_bytes(sh) / 1e6 == pytest.approx(542.15, abs=0.01)


def test_rejects_invalid():
    with pytest.raises(dl.DeltaLogError):
        dl.dl_predict_token_us(B.Config(0, 1, 0, 32, 128, 128, 8))
    with pytest.raises(dl.DeltaLogError):
        dl.dl_choose_capacity(dl.make_config("gdn", "bf16", 1, 1, 128, 128, 8), 33)
    with pytest.raises(dl.DeltaLogError):
        dl.dl_choose_capacity(dl.make_config("gdn", "bf16", 1, 1, 128, 128, 8), 0)


def test_call_bytes_of_segmented_launches():
    """A call that fits the log moves what one chunk moves; a call that passes
    the log's end moves the chunks it splits into, less the base reads that
    the later segments take from registers."""
    from recurrent_state_updates_amd import traffic as T
    for op, d, s in (("gdn", 128, 2), ("kda", 64, 4), ("rwkv6", 32, 2)):
        sh = T.Shape(op, 3, 2, d, s)
        for C in (4, 8, 13):
            for L in range(C):
                for K in range(1, 9):
                    got = T.call_bytes(sh, L, K, C)
                    parts, l, left = [], L, K
                    while left > 0:
                        k = min(left, C - l)
                        parts.append(T.chunk_bytes(sh, l, k, l + k == C))
                        l = 0 if l + k == C else l + k
                        left -= k
                    want = sum(parts) - (len(parts) - 1) * (sh.heads * sh.base() + sh.shared())
                    assert got == want, (op, C, L, K)
    sh = T.Shape("gdn", 128, 32, 128, 2)
    assert T.multi_token_bytes(sh, 8, 8, 16) == 2 * T.chunk_bytes(sh, 0, 8, True)


def _family(C):
    return 0 if C <= 8 else (1 if C <= 16 else 2)


@pytest.mark.parametrize("op,d", [("gdn", 128), ("kda", 128), ("rwkv6", 64)])
def test_family_rates_price_each_capacity_with_its_own_kernels(op, d):
    """Each capacity is priced at the rates of the kernels it runs: the ones
    built for 8, 16 or 32 entries.  With one rate for all three the model is
    dl_predict_token_us."""
    read, copy = (6100.0, 5900.0, 5200.0), (5000.0, 4800.0, 4300.0)
    for C in (1, 7, 8, 9, 13, 16, 17, 32):
        cfg = dl.make_config(op, "bf16", 64, 32, d, d, C)
        f = _family(C)
        assert dl.dl_predict_token_us_bounds(cfg, read, copy) == pytest.approx(
            _predict_py(op, 64, 32, d, C, read[f], copy[f]), rel=1e-12)
        assert dl.dl_predict_token_us_bounds(cfg, (6000.0,) * 3, (5000.0,) * 3) == \
            dl.dl_predict_token_us(cfg, 6000.0, 5000.0)


def test_family_rates_move_the_pick_to_the_kernels_that_run_faster():
    """The 64 x 64 heads at B=128: with one rate for every capacity the byte
    model picks a capacity of the 16-entry family; with that family 3 % slower
    (as measured for RWKV6) the pick stays with the 8-entry kernels.  Both
    picks are the argmin of the Python model priced the same way."""
    cfg = dl.make_config("rwkv6", "bf16", 128, 32, 64, 64, 8)
    one = dl.dl_choose_capacity(cfg, dl.DL_MAX_CAPACITY, 8000.0, 6000.0)
    assert 8 < one <= 16
    read, copy = (8000.0, 0.97 * 8000.0, 0.97 * 8000.0), (6000.0, 0.97 * 6000.0, 0.97 * 6000.0)
    got = dl.dl_choose_capacity_bounds(cfg, read, copy)
    preds = {C: _predict_py("rwkv6", 128, 32, 64, C, read[_family(C)], copy[_family(C)]) for C in range(1, 33)}
    assert got == min(preds, key=preds.get) == 8
    assert dl.dl_choose_capacity_bounds(cfg, (8000.0,) * 3, (6000.0,) * 3) == one
    # max_c caps the search as for the one-rate chooser
    assert dl.dl_choose_capacity_bounds(cfg, (8000.0,) * 3, (6000.0,) * 3, max_c=4) == \
        dl.dl_choose_capacity(cfg, 4, 8000.0, 6000.0)


def test_family_rates_reject_invalid():
    cfg = dl.make_config("gdn", "bf16", 1, 1, 128, 128, 8)
    with pytest.raises(ValueError):
        dl.dl_choose_capacity_bounds(cfg, (1.0, 2.0), (1.0, 2.0, 3.0))
    with pytest.raises(dl.DeltaLogError):
        dl.dl_choose_capacity_bounds(cfg, (1.0,) * 3, (1.0,) * 3, max_c=33)
    with pytest.raises(dl.DeltaLogError):
        dl.dl_predict_token_us_bounds(B.Config(0, 1, 0, 32, 128, 128, 8), (1.0,) * 3, (1.0,) * 3)
    lib = dl.load_library()
    assert lib.dl_predict_token_us_bounds(ctypes.byref(cfg), None, None) < 0
    assert lib.dl_choose_capacity_bounds(ctypes.byref(cfg), 8, None, None) == B.DL_ERR_ARG
