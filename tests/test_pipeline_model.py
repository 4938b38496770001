"""The max-plus pipeline model (EStream section 3.4, Eq. 5) against closed
forms of its special cases."""
import pytest

from routed_expert_ffn_top_amd.pipeline_model import predict, schedule


def test_io_bound_flow_shop():
    # loads back to back (q = 1, enough banks), executions shorter than loads:
    # the last execution starts when the last load lands
    K, l, x = 6, 10.0, 3.0
    r = predict([1] * K, [l] * K, [x] * K, B=K, q=1, T_ne=1.0, T_route=1.0)
    assert r["t_pipe"] == pytest.approx(K * l + x)


def test_exec_bound():
    K, l, x = 5, 2.0, 7.0
    r = predict([1] * K, [l] * K, [x] * K, B=K, q=1, T_ne=0.0, T_route=0.0)
    assert r["t_pipe"] == pytest.approx(l + K * x)


def test_one_bank_serialises_everything():
    L = [4.0, 5.0, 6.0, 7.0]
    X = [1.0, 2.0, 3.0, 4.0]
    r = predict([1] * 4, L, X, B=1, q=1, T_ne=0.0, T_route=0.0)
    assert r["t_pipe"] == pytest.approx(sum(L) + sum(X))


def test_two_banks_by_hand():
    # g0, g1 load before routing; g2 reuses bank 0 after g0 runs, g3 bank 1
    r = predict([1, 1, 1, 1], [10, 10, 10, 10], [1, 1, 1, 1], B=2, q=1, T_ne=0.5, T_route=0.5)
    assert r["t_pipe"] == pytest.approx(41.0)
    # non-expert work longer than the first load delays the first execution
    r = predict([1, 1], [1, 1], [1, 1], B=2, q=2, T_ne=5.0, T_route=5.0)
    assert r["t_pipe"] == pytest.approx(7.0)


def test_routing_delays_late_loads_only():
    # without prefetch every load waits for routing
    r = predict([1, 1], [3, 3], [1, 1], B=2, q=1, T_ne=2.0, T_route=2.0, prefetch=False)
    assert r["t_pipe"] == pytest.approx(2 + 3 + 3 + 1)
    r = predict([1, 1], [3, 3], [1, 1], B=2, q=1, T_ne=2.0, T_route=2.0, prefetch=True)
    assert r["t_pipe"] == pytest.approx(3 + 3 + 1)


def test_empty_groups():
    s = schedule([0, 1, 0, 1, 1], B=2, prefetch=True)
    assert [(x["group"], x["bank"], x["early"], x["executed"]) for x in s] == [
        (0, 0, True, False), (1, 1, True, True), (3, 0, False, True), (4, 1, False, True)]
    # group 0 was loaded for nothing: its bank is free at once, so group 3's
    # load waits only for the loader (and routing)
    r = predict([0, 1, 0, 1, 1], [2, 2, 2, 2], [1, 1, 1], B=2, q=1, T_ne=0.0, T_route=0.0)
    assert r["t_pipe"] == pytest.approx(2 + 2 + 2 + 2 + 1)
    s = schedule([0, 0, 3], B=2, prefetch=False)
    assert [(x["group"], x["bank"]) for x in s] == [(2, 0)]


def _profile(g, n_exp, l_e, x_per_group, T_ne=0.0):
    ng = n_exp // g
    return {"routed": [1] * ng, "group_size": [g] * ng, "routed_experts": [g] * ng, "l_expert": l_e,
            "X": [x_per_group] * ng, "T_ne": T_ne, "T_tail": 0.0}


def test_configure_prefers_overlap_within_budget():
    from routed_expert_ffn_top_amd.pipeline_model import configure
    # 16 experts, load 1 per expert, execution 3 per group whatever its size:
    # one big group cannot overlap anything; many small groups overlap loads
    # with execution but pay the per-group execution time more often
    profiles = {16: _profile(16, 16, 1.0, 3.0), 4: _profile(4, 16, 1.0, 3.0), 1: _profile(1, 16, 1.0, 3.0)}
    res = configure(profiles, max_slots=16)
    t = res["table"]
    assert t[(16, 1)] == pytest.approx(16 + 3)            # load everything, then run
    assert t[(4, 1)] == pytest.approx(4 * (4 + 3))        # one bank: no overlap
    assert t[(4, 2)] == pytest.approx(4 + 4 + 4 + 4 + 3)  # two banks: loads back to back
    assert t[(1, 16)] == pytest.approx(1 + 16 * 3)        # execution-bound
    assert (res["G"], res["B"]) == (4, 2) and res["t_pipe"] == pytest.approx(19.0)
    # a budget of 4 slots rules out g = 16 and leaves g = 4 with one bank
    res = configure(profiles, max_slots=4)
    assert (16, 1) not in res["table"] and res["G"] in (1, 4)
