"""Chunked prefill under a per-step token budget (test infrastructure only).

[ttlab] "llm-kv-cache-02-serving-engine-kv", section "3. 연속 배칭: 빈 자리를
걸음마다 채우기", part "새 문제: 긴 프리필이 디코드를 멈춘다": a long prompt's
prefill processed in one step stalls every running request's next token, so
the prompt is cut into chunks that ride along with the decode tokens of each
step, under a cap on the tokens a step may process.  The page measures caps
of 512, 1,024, 2,048 and 8,192 tokens with a 3,500-token input (the largest
cap is "effectively 3,500": the whole input fits in one step).

Reading of "budget" (the page gives the cap, not its accounting): the cap
counts every token a step processes.  Each running decode takes one token
and is never postponed; the waiting prompts then take, in arrival order,
chunks of their remaining prompt tokens until the budget is spent.  A prompt
gets a chunk only after every earlier waiting prompt has had its chunk this
step, so at most one prompt per step gets a partial chunk, and a prompt's
chunks are consecutive positions: chunk k of a prompt starts where chunk
k-1 ended (its ``ctx_before``).  At most ``max_chunks`` prompts get a chunk
in one step.
"""


def plan_step(budget, n_decode, prompts, max_chunks=32):
    """One step's prefill chunks.

    budget: tokens the step may process; n_decode: running decodes (one
    token each); prompts: waiting prompts in arrival order, each
    (prompt_len, computed) with computed = prompt tokens already prefilled.
    Returns [(prompt index, ctx_before, T)] in prompt order.
    """
    left = budget - n_decode
    out = []
    for i, (length, done) in enumerate(prompts):
        if left <= 0 or len(out) == max_chunks:
            break
        rest = length - done
        if rest <= 0:
            continue
        t = min(rest, left)
        out.append((i, done, t))
        left -= t
    return out


def run_schedule(budget, n_decode, prompt_lens, max_chunks=32):
    """Steps until every prompt is prefilled, with n_decode decodes running
    throughout: the list of each step's chunks."""
    done = [0] * len(prompt_lens)
    steps = []
    while any(d < n for d, n in zip(done, prompt_lens)):
        chunks = plan_step(budget, n_decode, list(zip(prompt_lens, done)), max_chunks)
        before = sum(done)
        for i, cb, t in chunks:
            done[i] = cb + t
        if sum(done) <= before:
            raise ValueError("the budget leaves no room for prefill")
        steps.append(chunks)
    return steps
