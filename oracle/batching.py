"""Batching and cache-utilisation model -- TEST INFRASTRUCTURE ONLY (oracle).

What is modelled (pages cited by title and section):
  * neuralialabs "Tornar a inferencia barata", batching passage: a fixed (static) batch runs
    until its longest member finishes and every finished member keeps its place until then;
    continuous batching treats the batch as a set of places, and a place freed by a finished
    request admits the next queued request at the very next step.
  * chatgpz.de "Aufmerksamkeit", paged-attention article, SECTION 1: the naive cache reserves
    max_seq_len tokens per request up front; SECTION 2: pages are taken on demand, one when
    the token count crosses a page boundary, and return to the pool when released;
    SECTION 4: utilisation = tokens written / tokens reserved, naive (reserve max_seq per
    request) against paged (ceil(tokens / page) pages per request).

Readings (the pages leave the step rules open):
  * every request is queued at step 0, in index order (first in, first out);
  * at the start of a step, free places admit queued requests in order -- under the static
    policy only when no place is occupied (the previous batch has been returned); admission
    takes the request's prompt tokens (paged) or max_seq_len tokens (naive) from the pool,
    and stops at the first request the pool cannot hold;
  * in a step every admitted request that has not finished produces one token; a paged
    request whose token needs a new page the pool cannot give stalls for that step;
  * a request finishes in the step that produces its last token; under the continuous
    policy it is returned at once and its place and pages are free for the next step; under
    the static policy the whole batch is returned, and its pages released, when its last
    member finishes.  A request's latency is the number of the step that returns it
    (counting from 1, from the common arrival at step 0); its service time counts the steps
    from its admission to its return (the passage's "a request done in four steps waits for
    its 231-token neighbour");
  * when the admitted requests all wait for pages and none can be admitted, the pool is too
    small for the schedule (there is no preemption): an error.
  * utilisation after a step = tokens resident in admitted requests / tokens of the pages
    they hold; the simulation reports its mean over steps.
The pure-Python loops here are the definition; the library's scheduler (kvp_sched.cpp)
must reproduce every integer result and the utilisation.
"""
import math

import numpy as np

STATIC, CONTINUOUS = 0, 1
PAGED, NAIVE = 0, 1


def simulate(prompt_lens, output_lens, slots, policy, alloc, max_seq_len, block_size, num_blocks):
    """Returns a dict: steps, tokens, busy_slot_steps (requests that produced a token, summed
    over steps), padding_slot_steps (places held by finished requests of a static batch),
    latency and service (per request, in steps), mean_latency, mean_service, max_latency,
    peak_blocks,
    mean_utilisation, deferrals (admissions stopped by a full pool), stalls (tokens delayed
    by a full pool)."""
    n = len(prompt_lens)
    assert len(output_lens) == n
    assert all(o >= 1 for o in output_lens) and all(p >= 0 for p in prompt_lens)
    if alloc == NAIVE:
        assert all(p + o <= max_seq_len for p, o in zip(prompt_lens, output_lens))
    pages = lambda t: -(-t // block_size)
    free = num_blocks
    queue = 0                  # next request to admit
    active = []                # admitted, not yet returned: [req, tokens, blocks, generated, done]
    latency = [0] * n
    admitted_at = [0] * n
    step = 0
    busy = padding = 0
    peak = 0
    util_sum = 0.0
    deferrals = stalls = 0
    returned = 0
    while returned < n:
        progress = 0
        # admission
        if policy == CONTINUOUS or not active:
            while len(active) < slots and queue < n:
                r = queue
                need = pages(prompt_lens[r]) if alloc == PAGED else pages(max_seq_len)
                if need > free:
                    deferrals += 1
                    break
                free -= need
                active.append([r, prompt_lens[r], need, 0, False])
                admitted_at[r] = step
                queue += 1
                progress += 1
        # one token for every unfinished admitted request
        for a in active:
            if a[4]:  # finished in an earlier step, holding its place (static policy)
                padding += 1
                continue
            if alloc == PAGED and pages(a[1] + 1) > a[2]:
                if free == 0:
                    stalls += 1
                    continue
                free -= 1
                a[2] += 1
            a[1] += 1
            a[3] += 1
            busy += 1
            progress += 1
            if a[3] == output_lens[a[0]]:
                a[4] = True
        step += 1
        # statistics after the step (before returns)
        held = sum(a[2] for a in active)
        peak = max(peak, held)
        resident = sum(a[1] for a in active)
        util_sum += resident / (held * block_size) if held else 0.0
        # returns
        if policy == CONTINUOUS:
            keep = []
            for a in active:
                if a[4]:
                    latency[a[0]] = step
                    free += a[2]
                    returned += 1
                else:
                    keep.append(a)
            active = keep
        elif active and all(a[4] for a in active):
            for a in active:
                latency[a[0]] = step
                free += a[2]
                returned += 1
            active = []
        if progress == 0 and active and not all(a[4] for a in active):
            raise RuntimeError("the pool cannot hold the admitted requests")
    return {
        "steps": step, "tokens": int(sum(output_lens)), "busy_slot_steps": busy,
        "padding_slot_steps": padding, "latency": latency, "mean_latency": sum(latency) / n,
        "service": [latency[i] - admitted_at[i] for i in range(n)],
        "mean_service": sum(latency[i] - admitted_at[i] for i in range(n)) / n,
        "max_latency": max(latency), "peak_blocks": peak, "mean_utilisation": util_sum / step,
        "deferrals": deferrals, "stalls": stalls,
    }


def naive_utilisation(tokens, max_seq):
    """Tokens written / tokens reserved when every request reserves max_seq (SECTION 4)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    return tokens.sum() / (max_seq * len(tokens)) * 100.0


def paged_utilisation(tokens, page):
    """Tokens written / tokens of the pages taken, ceil(t / page) pages per request."""
    tokens = np.asarray(tokens, dtype=np.int64)
    pages = -(-tokens // page)
    return tokens.sum() / (pages * page).sum() * 100.0


def response_lengths(n, seed, avg=500, std=200, lo=200, hi=2048):
    """The SECTION 4 recipe: normal(avg, std) token counts truncated to integers and clipped
    to [lo, hi] (a seeded generator stands in for the page's unseeded one)."""
    rng = np.random.default_rng(seed)
    return np.clip(rng.normal(avg, std, n).astype(np.int64), lo, hi)
