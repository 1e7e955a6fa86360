"""The oracle's chunked-prefill planner against what the page fixes and
what its reading implies ([ttlab] "llm-kv-cache-02-serving-engine-kv",
section "3. 연속 배칭: 빈 자리를 걸음마다 채우기").

  * the page's own measurement: a 3,500-token input under caps of 512,
    1,024, 2,048 and 8,192 tokens; at 8,192 it is "effectively 3,500" --
    the whole input in one step;
  * a step never processes more tokens than its budget, decodes included;
  * chunks of one prompt are consecutive and cover its prompt exactly once;
  * waiting prompts are served in arrival order (a later prompt gets no
    chunk while an earlier one is unfinished and the budget ran out);
  * brute force on small cases: the plan is the unique one that gives each
    prompt, in order, as many tokens as the budget still allows.
"""

import itertools

import pytest

from oracle.scheduler import plan_step, run_schedule


@pytest.mark.parametrize("cap,steps", [(512, 7), (1024, 4), (2048, 2), (8192, 1)])
def test_page_caps_on_a_3500_token_input(cap, steps):
    """With no other request running, the input needs ceil(3,500 / cap)
    steps; at 8,192 the cap is never reached (one chunk of 3,500)."""
    plan = run_schedule(cap, 0, [3500])
    assert len(plan) == steps
    assert [c[0][2] for c in plan][:-1] == [cap] * (steps - 1)
    assert sum(c[0][2] for c in plan) == 3500
    if cap == 8192:
        assert plan == [[(0, 0, 3500)]]


@pytest.mark.parametrize("cap", [512, 1024, 2048, 8192])
def test_decodes_count_against_the_budget(cap):
    """63 running decodes take 63 tokens of every step's cap; the prompt gets
    the rest, chunk after chunk, positions consecutive."""
    plan = run_schedule(cap, 63, [3500])
    pos = 0
    for chunks in plan:
        (i, cb, t), = chunks
        assert i == 0 and cb == pos and 0 < t <= cap - 63
        pos += t
    assert pos == 3500
    assert len(plan) == -(-3500 // (cap - 63))


def test_budget_below_the_decodes_leaves_no_prefill():
    assert plan_step(40, 40, [(100, 0)]) == []
    assert plan_step(39, 40, [(100, 0)]) == []
    with pytest.raises(ValueError):
        run_schedule(10, 10, [5])


def test_prompts_in_arrival_order_and_chunk_limit():
    prompts = [(30, 30), (50, 10), (20, 0), (5, 0)]  # the first is finished
    assert plan_step(60, 0, prompts) == [(1, 10, 40), (2, 0, 20)]
    assert plan_step(45, 0, prompts) == [(1, 10, 40), (2, 0, 5)]
    assert plan_step(100, 0, prompts) == [(1, 10, 40), (2, 0, 20), (3, 0, 5)]
    assert plan_step(100, 0, prompts, max_chunks=2) == [(1, 10, 40), (2, 0, 20)]


def _brute(budget, n_decode, prompts, max_chunks):
    """Every assignment of 0..rest tokens per prompt; keep those within the
    budget that serve prompts in order (a prompt gets tokens only if every
    earlier unfinished prompt got all of its rest) and at most max_chunks
    prompts; the plan gives the most tokens."""
    rests = [max(0, n - d) for n, d in prompts]
    best = None
    for take in itertools.product(*[range(r + 1) for r in rests]):
        if sum(take) + n_decode > budget or sum(1 for t in take if t) > max_chunks:
            continue
        ok = all(take[j] == rests[j] for i in range(len(take)) if take[i] for j in range(i))
        if ok and (best is None or sum(take) > sum(best)):
            best = take
    return [(i, prompts[i][1], t) for i, t in enumerate(best) if t] if best else []


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_small_cases(seed):
    import numpy as np

    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 4))
    prompts = []
    for _ in range(n):
        length = int(rng.integers(0, 6))
        prompts.append((length, int(rng.integers(0, length + 1))))
    budget, n_dec = int(rng.integers(0, 12)), int(rng.integers(0, 4))
    max_chunks = int(rng.integers(1, 4))
    assert plan_step(budget, n_dec, prompts, max_chunks) == _brute(budget, n_dec, prompts, max_chunks)
