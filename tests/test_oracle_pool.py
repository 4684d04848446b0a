"""The worker-process plumbing of the full-size parity tests (CPU): a unit
computed in a spawned worker equals the same oracle calls made in this
process."""
import numpy as np

import oracle
import oracle_pool


def _bits(rng, shape):
    return (rng.standard_normal(shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_workers_match_direct_oracle_calls():
    rng = np.random.default_rng(5)
    n, G, D, topk = 200, 4, 64, 5
    P = -(-n // 16)
    kbits, vbits, qbits = _bits(rng, (P, 16, D)), _bits(rng, (P, 16, D)), _bits(rng, (G, D))
    kbits[P - 1, n - (P - 1) * 16:] = 0x7FC0  # NaN slots past the last token: never read
    chosen = np.array([0, 3, 7, P - 1])
    with oracle_pool.pool() as ex:
        got = dict(oracle_pool.map_bounded(ex, oracle_pool.quest_unit,
                                           [(0, (kbits, vbits[chosen], qbits, n, 0.125, chosen, D, False))]))
        qw, kw = _bits(rng, (G, 8, D)), _bits(rng, (300, D))
        pooled = dict(oracle_pool.map_bounded(ex, oracle_pool.snapkv_unit, [(1, (qw, kw, 300, 0.125, 7))]))[1]
    mins, maxs, A, out, vmax = got[0]
    kp = oracle.gather_unit_pages(kbits[:, None], np.arange(P), 0, n)
    m2, M2 = oracle.unit_summaries(kp, n)
    qf = oracle.bf16_to_f64(qbits)
    A2 = oracle.unit_kv_head_score(oracle.unit_page_bounds(qf, m2, M2, 0.125))
    vp = np.full((P, 16, D), np.nan)
    vp[chosen] = oracle.bf16_to_f64(vbits[chosen])
    vp[P - 1, n - (P - 1) * 16:] = np.nan
    keys, vals = oracle.unit_selected_tokens(kp, chosen, n), oracle.unit_selected_tokens(vp, chosen, n)
    assert (mins == m2).all() and (maxs == M2).all() and (A == A2).all()
    assert (out == oracle.unit_attention(qf, keys, vals, 0.125)).all() and vmax == np.abs(vals).max()
    S, _, _ = oracle.snapkv_unit_votes(oracle.bf16_to_f64(qw), oracle.bf16_to_f64(kw), 300, 0.125)
    assert (pooled == oracle.maxpool1d(S, 7)).all()
