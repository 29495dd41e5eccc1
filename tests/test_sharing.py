"""The sharing-savings harness (paged_kv_cache_82_amd.sharing) on the CPU: closed forms on
deterministic lengths, no saving without sharing, monotone savings, and paged waste within
its bound of one partly filled block per sequence ([PA-summary] "Results")."""
import math

from paged_kv_cache_82_amd import sharing


def test_parallel_sampling_closed_form():
    # prompt of 32 tokens = 2 full blocks of 16, two samples of 16 tokens: at every step the
    # shared pool holds 2 prompt blocks + 1 block per sample = 4, private copies hold 2 * 3
    r = sharing.parallel_sampling(2, requests=1, block_size=16, prompt_median=32,
                                  output_median=16, sigma=0.0)
    assert r["shared_block_steps"] == 16 * 4 and r["private_block_steps"] == 16 * 6
    assert math.isclose(r["saving"], 1 / 3)


def test_beam_search_closed_form():
    # two beams over a 32-token prompt for one step: whichever parents survive, the two prompt
    # blocks are shared and each beam starts one new block: 4 blocks against 2 * 3
    r = sharing.beam_search(2, requests=1, block_size=16, prompt_median=32, output_median=1,
                            sigma=0.0)
    assert (r["shared_block_steps"], r["private_block_steps"]) == (4, 6)


def test_no_sharing_no_saving_and_savings_grow():
    assert sharing.parallel_sampling(1, requests=8)["saving"] == 0.0
    assert sharing.beam_search(1, requests=4)["saving"] == 0.0
    s = [sharing.parallel_sampling(n, requests=16)["saving"] for n in (2, 4)]
    b = [sharing.beam_search(k, requests=8)["saving"] for k in (2, 4)]
    assert 0 < s[0] < s[1] < 1 and 0 < b[0] < b[1] < 1


def test_waste_paged_vs_contiguous():
    r = sharing.waste(requests=128, block_size=16, max_len=2048)
    assert 0 <= r["paged_waste"] <= r["paged_waste_bound"]
    assert r["contiguous_waste"] > 0.5 > r["paged_waste"]
