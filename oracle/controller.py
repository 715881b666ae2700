"""Oracle of the bandwidth-adaptive chunk-version choice — TEST INFRASTRUCTURE ONLY.

Only ``tests/`` may import this module.  It is a plain Python
transcription of the selection rule of the CacheGen blog (section 2.2, the
bandwidth-adaptive selection formula): each chunk of a context exists in three
pre-encoded versions H, M, L; with B the bandwidth measured while streaming and
SLO the service-level objective, a version's score is

    (SLO - T_decode(Q)) / T_transmit(Q, B).

Reading taken (the printed formula is an argmax, which read literally would
always pick the smallest version): the score is the factor by which the
version's transfer fits in the time the SLO leaves after decoding, so

* SLO is what is left of the context's objective when the chunk is sent,
* T_transmit(Q, B) = bytes of this and all later chunks at Q / B,
* T_decode(Q) = the decode time of the same chunks at Q,
* the choice is the highest quality whose score is >= 1 (it fits), and when
  no version fits, the one that is done soonest (smallest T_transmit + T_decode;
  an argmax of negative scores would pick the largest version instead).

B is the throughput the previous chunk of the context saw; the caller gives a
prior for the first chunk.

Parity status: the rule is pinned by closed-form cases and by monotonicity in
bandwidth and budget (tests/test_oracle_controller.py); the pages give no
worked example, and their 81% -> 8% SLO-violation result needs their network
traces, so the simulated violation rates are context only.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

H, M, L = 0, 1, 2


def choose_version(budget_ms: float, bandwidth_bpms: float, bytes_left: Sequence[int],
                   decode_ms_left: Sequence[float]) -> Tuple[int, List[float]]:
    """(version, scores) for the next chunk.  bytes_left[q] = 0 marks a version
    that does not exist; its score is reported as 0."""
    if not (bandwidth_bpms > 0.0) or math.isinf(bandwidth_bpms):
        raise ValueError("bandwidth must be positive and finite")
    if math.isnan(budget_ms):
        raise ValueError("budget is NaN")
    scores = [0.0, 0.0, 0.0]
    fits = []
    ends = []
    for q in (H, M, L):
        d = float(decode_ms_left[q])
        if not (d >= 0.0) or math.isinf(d):
            raise ValueError("bad decode time")
        if int(bytes_left[q]) == 0:
            continue
        t_send = float(int(bytes_left[q])) / bandwidth_bpms
        scores[q] = (budget_ms - d) / t_send
        if scores[q] >= 1.0:
            fits.append(q)
        ends.append((t_send + d, q))
    if not ends:
        raise ValueError("no version of the chunk")
    if fits:
        return fits[0], scores
    best_end = min(e for e, _ in ends)
    return [q for e, q in ends if e == best_end][0], scores


def stream_context(sizes: Sequence[Sequence[int]], decode_ms: Sequence[Sequence[float]],
                   slo_ms: float, send, prior_bpms: float, policy: str = "adaptive"):
    """One context streamed chunk by chunk over a simulated link.

    sizes[c][q] / decode_ms[c][q]: bytes and decode time of chunk c at version q.
    send(nbytes) -> milliseconds the link takes for nbytes from the current
    clock (it advances the clock).  policy: "adaptive", or "H" / "M" / "L" for a
    fixed version.  Decoding of a chunk overlaps the transfer of the next ones;
    the context is loaded when the last chunk is decoded.

    Returns (load time in ms, versions chosen, bandwidths used)."""
    n = len(sizes)
    t = 0.0          # transfer clock since the request
    decoded = 0.0    # when the last decode finished
    bw = prior_bpms
    versions = []
    used = []
    for c in range(n):
        if policy == "adaptive":
            left = [sum(int(sizes[j][q]) for j in range(c, n)) for q in (H, M, L)]
            dleft = [sum(float(decode_ms[j][q]) for j in range(c, n)) for q in (H, M, L)]
            q, _ = choose_version(slo_ms - t, bw, left, dleft)
        else:
            q = "HML".index(policy)
        used.append(bw)
        dt = send(int(sizes[c][q]))
        t += dt
        bw = int(sizes[c][q]) / dt
        decoded = max(decoded, t) + float(decode_ms[c][q])
        versions.append(q)
    return decoded, versions, used
