"""The algorithmic bytes bench.py divides by: a Quest decode step moves q,
the summaries of every valid page, the page table, the valid tokens of the
kept pages (K and V, or the latent row once when V is a prefix of K) and the
output.  The totals for the 32K and 128K workloads are worked out by hand
from their shapes."""
import bench


def test_128k_workload_step_and_scorer_bytes():
    # B32, Hq32, Hkv4, D128, 131072 tokens = 8192 pages, 256 kept
    a = bench.quest_algorithmic_bytes([131072] * 32, 32, 4, 128, 128, False, 256, 256)
    assert a["q"] == 32 * 32 * 128 * 2 == 256 * 1024
    assert a["summaries"] == 32 * 8192 * 4 * 512 == 512 * 2 ** 20
    assert a["page_table"] == 32 * 8192 * 4 == 2 ** 20
    assert a["kv"] == 32 * 4 * 256 * 16 * 512 == 256 * 2 ** 20
    assert a["out"] == 32 * 32 * 128 * 4 == 512 * 1024
    assert a["step"] == 807_141_376  # 769.75 MiB
    # q, summaries and page table; the page scores written are an intermediate
    assert a["scorer_launch"] == 256 * 1024 + 512 * 2 ** 20 + 2 ** 20 == 538_181_632


def test_32k_workload_step_bytes():
    # B8, Hq32, Hkv8, D128, 32768 tokens = 2048 pages, 128 kept
    a = bench.quest_algorithmic_bytes([32768] * 8, 32, 8, 128, 128, False, 128, 128)
    assert a["step"] == 134_479_872  # 128.25 MiB


def test_partial_last_page_and_latent_rows():
    # one MLA request of 40 tokens (3 pages, the last with 8 tokens), all
    # pages kept: 40 latent rows of 1152 bytes, V counted inside them
    a = bench.quest_algorithmic_bytes([40], 32, 1, 576, 512, True, 8, 8)
    assert a["kv"] == 40 * 1152
    assert a["summaries"] == 3 * 2 * 576 * 2
    assert a["page_table"] == 3 * 4
    # a long request keeping 2 of 3 pages without forced recent pages: two
    # whole pages; with recent pages forced the partial last page counts its
    # valid tokens
    b = bench.quest_algorithmic_bytes([40], 4, 1, 128, 128, False, 2, 2)
    assert b["kv"] == 32 * 512
    c = bench.quest_algorithmic_bytes([40], 4, 1, 128, 128, False, 1, 2, recent=1)
    assert c["kv"] == (16 + 8) * 512


def test_nothing_scored_reads_only_the_kept_page_table_entries():
    a = bench.quest_algorithmic_bytes([160] * 2, 8, 2, 128, 128, False, 0, 3)
    assert a["summaries"] == 0
    assert a["page_table"] == 2 * 3 * 4


def test_snapkv_workload_bytes():
    # B16, Hq32, Hkv8, D128, 32768-token prompts, window 32, 2,080 rows kept,
    # 64 decode steps
    ev, dec, votes = bench.snapkv_algorithmic_bytes(16, 32, 8, 128, 32768, 32, 2080, 64)
    q_win = 16 * 32 * 32 * 128 * 2                 # 4.2 MB
    k_once = 16 * 8 * 32768 * 256                  # 1,073.7 MB
    kept_rw = 2 * 2 * 16 * 8 * 2080 * 256          # K and V rows read and written, 272.6 MB
    assert ev == q_win + k_once + kept_rw + 16 * 8 * 2080 * 4
    assert round(ev / 1e6) == 1352
    # step s attends 2081 + s rows: 136.4 MB at the first step
    first = 16 * 8 * 2081 * 512 + 16 * 32 * 128 * 6
    assert dec == sum(16 * 8 * (2081 + s) * 512 for s in range(64)) + 64 * 16 * 32 * 128 * 6
    assert dec > 64 * first
    assert votes == q_win + k_once  # the votes written are an intermediate
