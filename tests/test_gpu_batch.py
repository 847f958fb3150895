"""GPU parity of batch decode steps (several sequences per step) against the oracle.

A batch plan runs the dense projections as MFMA tiles over all sequences, a
router/top-k task per sequence and expert tasks shared by the sequences
routed to them; each expert task takes an equal share of the rows of the
experts the routing chose (one case keeps a fixed expert part per task). Each case compares every sequence of one step with the
oracle exactly as the batch-1 cases do (greedy token, logits, hidden state
after every residual, new K/V in the pool, top-k ids, counters), on ragged
contexts that include an empty one and a single token.
"""
import pytest

from test_gpu_step import greedy_agreement, run_step_parity

pytestmark = pytest.mark.gpu


def test_tiny_dense_batch3():
    # contexts 128, 0, 47: a full page set, an empty cache and a ragged tail
    run_step_parity("tiny_dense_b3")


def test_small_moe_batch5():
    # contexts 2048, 1, 517, 1300, 16
    run_step_parity("small_moe_b5")


def test_small_moe_batch32_ragged():
    # 32 sequences, contexts uniform in [1, 1024]: both MFMA column blocks
    run_step_parity("small_moe_b32")


def test_small_moe_batch5_greedy_16():
    greedy_agreement("small_moe_b5", 16)


def test_small_moe_batch5_fixed_expert_parts():
    # every expert task on one fixed (expert, part), not shares of the
    # experts the routing chose
    import decode_megakernel_persistent_amd as mk
    run_step_parity("small_moe_b5", plan_flags=mk.MK_PLAN_NO_EXPERT_SHARE)


def test_batch_attention_split_queue():
    # the batch's attention splits pulled from one shared queue (longest
    # first, from the plan's split table) instead of dealt to fixed units
    import decode_megakernel_persistent_amd as mk
    run_step_parity("small_moe_b5", plan_flags=mk.MK_PLAN_ATTN_QUEUE)
    run_step_parity("small_moe_b32", plan_flags=mk.MK_PLAN_ATTN_QUEUE)
