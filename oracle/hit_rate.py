"""Cache hit rate and its Theorem 3.1 optimum (oracle).

SGLang explainer, section 04 ("cache hit rate" formula): the hit rate is
token-weighted, the sum over requests of cached prefill tokens divided by
the sum of prefill tokens.

SGLang explainer, section 04, Theorem 3.1 formulas (and the paper summary,
appendix A.3): with T the prefix tree of all requests and |e| the token count
of edge e, any schedule computes C >= sum_e |e| tokens, depth-first order
reaches C_DFS = sum_e |e|, and the optimal hit rate is 1 - C_DFS / sum of
prefill tokens.  sum_e |e| equals the number of distinct non-empty token
prefixes among the requests, which is what ``distinct_prefix_tokens``
counts.
"""

from fractions import Fraction


def hit_rate(cached_tokens, prefill_tokens):
    """Exact ratio of two integer sums (Fraction)."""
    if prefill_tokens == 0:
        return Fraction(0)
    return Fraction(cached_tokens, prefill_tokens)


def distinct_prefix_tokens(prompts):
    """Number of distinct non-empty prefixes, counted in an uncompressed
    token trie built from nested dicts (one trie node per prefix)."""
    trie, count = {}, 0
    for p in prompts:
        node = trie
        for t in p:
            if t not in node:
                node[t] = {}
                count += 1
            node = node[t]
    return count


def optimal_hit_rate(prompts):
    total = sum(len(p) for p in prompts)
    if total == 0:
        return Fraction(0)
    return 1 - Fraction(distinct_prefix_tokens(prompts), total)
