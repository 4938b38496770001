"""Max-plus model of the paged layer's loading/execution pipeline (EStream,
section 3.4, "Automatic Pipeline Configuration", Eq. 5).

Groups are loaded into B banks by a loader that keeps at most q loads in
flight and executed one after another by the compute stream. For load i (in
loading order) with service time L_i and execution k (in execution order)
with service time X_k:

    a_i = max(d_{i-q}, f_{prev(bank_i)}, r_i)   load start
    d_i = a_i + L_i                              load done
    s_k = max(d_{load(k)}, T_ne, f_{k-1})        execution start
    f_k = s_k + X_k                              execution done

with d_j = f_j = 0 for j <= 0. f_{prev(bank)} is the completion of the last
execution that used the bank the load overwrites (0 if none), r_i is the
earliest time the loader may issue load i (0 for loads issued before routing,
the routing time for loads chosen after it), and T_ne is the completion of
the work that precedes every group's execution (router, top-k, route counts).
The prediction of the layer time is f_K plus whatever follows the last group
(the combine).

The bank of each load follows the library's schedule: the first B groups in
group order go to banks 0..B-1 before routing (when `prefetch`); a group with
no routes is never executed and frees its bank at once; every later group with
routes takes the bank released longest ago.
"""
from __future__ import annotations

from collections import deque
from typing import Dict, List, Sequence


def schedule(routed: Sequence[int], B: int, prefetch: bool) -> List[dict]:
    """Loads in loading order: {group, bank, early}, where early = issued
    before routing. `routed[g]` is group g's route count."""
    loads = []
    ng = len(routed)
    npre = min(B, ng) if prefetch else 0
    for g in range(npre):
        loads.append({"group": g, "bank": g, "early": True})
    banks = deque() if prefetch else deque(range(B))
    exec_bank: Dict[int, int] = {}
    for g in range(ng):
        pre = g < npre
        if routed[g] == 0:
            if pre:
                banks.appendleft(g)
            continue
        if pre:
            bank = g
        else:
            bank = banks.popleft()
            loads.append({"group": g, "bank": bank, "early": False})
        exec_bank[g] = bank
        banks.append(bank)
    for ld in loads:
        ld["executed"] = ld["group"] in exec_bank
    return loads


def predict(routed: Sequence[int], L: Sequence[float], X: Sequence[float], B: int, q: int,
            T_ne: float, T_route: float, T_tail: float = 0.0, prefetch: bool = True) -> dict:
    """Evaluate the recurrence. L: service time of each load in loading order;
    X: service time of each executed group in execution (group) order."""
    loads = schedule(routed, B, prefetch)
    assert len(L) == len(loads), (len(L), len(loads))
    executed = [g for g in range(len(routed)) if routed[g] > 0]
    assert len(X) == len(executed), (len(X), len(executed))
    d = []                       # load completions in loading order
    load_of_group = {}
    f_exec = {}                  # group -> execution completion
    last_user = {}               # bank -> group whose execution last used it
    exec_order = iter(range(len(executed)))
    f_prev = 0.0
    # Loads and executions interleave in time; the loader issues loads in
    # order and an execution needs its own load, so evaluate loads first and
    # executions as soon as their load is known, in order.
    k = 0
    pending = list(executed)
    for i, ld in enumerate(loads):
        a = d[i - q] if i - q >= 0 else 0.0
        prev = last_user.get(ld["bank"])
        if prev is not None:
            # the execution that last used this bank must finish first; it is
            # earlier in execution order, so evaluate executions up to it
            while prev not in f_exec:
                g = pending.pop(0)
                s = max(d[load_of_group[g]], T_ne, f_prev)
                f_prev = s + X[k]
                f_exec[g] = f_prev
                k += 1
            a = max(a, f_exec[prev])
        if not ld["early"]:
            a = max(a, T_route)
        d.append(a + L[i])
        load_of_group[ld["group"]] = i
        if ld["executed"]:
            last_user[ld["bank"]] = ld["group"]
        else:
            last_user.pop(ld["bank"], None)
    while pending:
        g = pending.pop(0)
        s = max(d[load_of_group[g]], T_ne, f_prev)
        f_prev = s + X[k]
        f_exec[g] = f_prev
        k += 1
    t_io = sum(L)
    t_exec = sum(X) + T_ne + T_tail
    t_pipe = f_prev + T_tail
    return {"t_pipe": t_pipe, "t_io": t_io, "t_exec": t_exec,
            "bubble": 1.0 - max(t_io, t_exec) / t_pipe if t_pipe > 0 else 0.0,
            "loads": len(loads)}


def predict_from_profile(prof: dict, b: int) -> dict:
    """Prediction for bank count b from one profiled run at group size g:
    prof = {routed: per-group route counts, experts: per-group expert ids
    with routes (counts), g, l_expert: load time per expert, X: execution
    time per executed group (group order), T_ne, T_tail}. A load copies every
    expert of its group when issued before routing, else only the experts
    with routes."""
    loads = schedule(prof["routed"], b, prefetch=True)
    L = [prof["l_expert"] * (prof["group_size"][ld["group"]] if ld["early"] else prof["routed_experts"][ld["group"]])
         for ld in loads]
    return predict(prof["routed"], L, prof["X"], B=b, q=1, T_ne=prof["T_ne"], T_route=prof["T_ne"],
                   T_tail=prof["T_tail"], prefetch=True)


def configure(profiles: Dict[int, dict], max_slots: int) -> dict:
    """The nested search of the pages' configuration step: for every profiled
    group size g, the bank counts b with g*b <= max_slots (the arena's memory
    budget) are evaluated with the max-plus model and the best b kept (inner
    optimisation); the group size whose best configuration predicts the
    shortest layer wins (outer optimisation)."""
    table = {}
    best = None
    for g, prof in sorted(profiles.items()):
        inner = None
        for b in range(1, max_slots // g + 1):
            t = predict_from_profile(prof, b)["t_pipe"]
            table[(g, b)] = t
            if inner is None or t < inner[1] - 1e-12:
                inner = (b, t)
        if inner is not None and (best is None or inner[1] < best[2] - 1e-12):
            best = (g, inner[0], inner[1])
    return {"G": best[0], "B": best[1], "t_pipe": best[2], "table": table}
