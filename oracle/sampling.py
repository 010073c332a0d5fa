"""Plain CPU oracle for chain speculative-sampling acceptance.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it.

Source: PR #362 "Support speculative-decode verify on ROCm, and stop auto
routing short-query prefill to AITER" (AMD-Ecosystem FlashInfer fork),
Summary and Architecture / design notes: the verify step feeds an acceptance
sampler, chain_speculative_sampling, over (batch_size, num_speculate_tokens);
drafts are one linear chain per request.  The pages name the step but do not
spell it out; the reading taken is standard speculative (rejection) sampling:

  for draft position t = 0, 1, ... of request b, with drafted token x:
      accept x when u_t * q_t(x) < p_t(x)       (u_t uniform in [0, 1),
                                                  q = draft, p = target probs)
      otherwise emit one token drawn from the residual max(p_t - q_t, 0)
      (normalised; p_t itself if the residual is all zero) and stop;
  if every draft token is accepted, emit a bonus token drawn from p_n.

Draws use inverse-CDF sampling with one extra uniform s per request: the
smallest k whose running sum of the weights exceeds s * (sum of all
weights); if none does, the last k with a positive weight.  Randomness is an
input (u [B, n], s [B]), so the result is a function.  The accept test is a
single float32 product and compare, taken exactly as the kernel takes it.
The draw is taken on the float32 weights with float64 running sums (exact
for any vocabulary here); a float32 implementation, whose sums round at
each step, can land on a neighbouring index when s * total falls within its
summation error of a boundary -- the tests accept such a draw only when it
is valid within that error bound.
"""
from __future__ import annotations

import numpy as np


def inverse_cdf(weights, s):
    """Index drawn from non-negative float32 weights by the uniform s."""
    w = np.asarray(weights, dtype=np.float32)
    c = np.cumsum(w, dtype=np.float64)
    thr = float(np.float32(s)) * c[-1]
    hit = np.nonzero(c > thr)[0]
    if hit.size:
        return int(hit[0])
    pos = np.nonzero(w > 0)[0]
    return int(pos[-1]) if pos.size else len(w) - 1


def chain_speculative_sampling(draft_probs, draft_token_ids, target_probs, accept_u, sample_u):
    """Accept/reject a chain of drafts per request.

    draft_probs [B, n, V], draft_token_ids [B, n], target_probs [B, n + 1, V],
    accept_u [B, n], sample_u [B].  Returns (output_token_ids [B, n + 1],
    int64, -1 after the last emitted token; num_accepted [B]).
    """
    q_all = np.asarray(draft_probs, dtype=np.float32)
    p_all = np.asarray(target_probs, dtype=np.float32)
    B, n, V = q_all.shape
    assert p_all.shape == (B, n + 1, V)
    out = np.full((B, n + 1), -1, dtype=np.int64)
    accepted = np.zeros(B, dtype=np.int64)
    for b in range(B):
        for t in range(n):
            x = int(draft_token_ids[b, t])
            if np.float32(accept_u[b, t]) * q_all[b, t, x] < p_all[b, t, x]:
                out[b, t] = x
                accepted[b] += 1
                continue
            resid = np.maximum(p_all[b, t] - q_all[b, t], np.float32(0))
            w = resid if resid.sum(dtype=np.float64) > 0 else p_all[b, t]
            out[b, t] = inverse_cdf(w, sample_u[b])
            break
        else:
            out[b, n] = inverse_cdf(p_all[b, n], sample_u[b])
    return out, accepted
