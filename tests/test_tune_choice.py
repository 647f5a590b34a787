"""The tuner's final choice (host logic, no GPU): fastest configuration that
matches the oracle, with two-pass splits held to a 10% margin."""
from latency_decode_gemm_amd import tune
from latency_decode_gemm_amd._capi import SkgConfig

MK = SkgConfig.make
ONE = MK(inner=2, split_k=1, row_tiles=1, waves_k=4, depth=2)
SPLIT1 = MK(backend=1, inner=2, split_k=4, row_tiles=1, waves_k=4, depth=2)
TWO = MK(backend=2, inner=5, split_k=4, row_tiles=1, waves_n=3, depth=3)


def test_fastest_passing_config_wins():
    assert tune.choose({ONE: 10.0, SPLIT1: 9.0}, lambda c: True) == SPLIT1
    assert tune.choose({ONE: 10.0, SPLIT1: 9.0}, lambda c: c != SPLIT1) == ONE
    assert tune.choose({ONE: 10.0}, lambda c: False) is None


def test_two_pass_needs_a_ten_percent_lead():
    # 2% faster by graph time: the single dispatch is kept
    assert tune.choose({ONE: 11.8, TWO: 11.56}, lambda c: True) == ONE
    # more than 10% faster: the two-pass split is taken
    assert tune.choose({ONE: 11.8, TWO: 10.5}, lambda c: True) == TWO
    # only two-pass candidates: the fastest of them
    other = MK(backend=2, inner=2, split_k=2, row_tiles=1, waves_k=2, depth=2)
    assert tune.choose({TWO: 8.0, other: 7.5}, lambda c: True) == other


def test_input_timings_untouched():
    timed = {ONE: 11.8, TWO: 11.56}
    tune.choose(timed, lambda c: True)
    assert timed[TWO] == 11.56


def test_crossover_is_the_last_m_of_the_winning_prefix():
    from latency_decode_gemm_amd.tune import crossover_max_m
    assert crossover_max_m({16: (1, 2), 24: (1, 2), 32: (3, 2), 40: (1, 2)}) == 24
    assert crossover_max_m({16: (3, 2), 24: (1, 2)}) == 0
    assert crossover_max_m({16: (1, 2), 64: (1, 2)}) == 64
