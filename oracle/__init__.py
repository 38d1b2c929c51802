"""CPU oracle for the RocketKV hot path.  Test infrastructure only: imported by
the tests, ``__graft_entry__.smoke()`` and the cpu_baseline leg of bench.py,
never by the library or its binding."""

from .rocketkv_oracle import *  # noqa: F401,F403
from .rocketkv_oracle import (attention, block_scores, block_select, build_aux,
                              channel_select, hsa_decode, hsa_decode_mt_unit,
                              hsa_unit, pool, pool_max, pool_sum, selected_tokens, snapkv_evict,
                              snapkv_select, split, table1_storage_traffic,
                              topk_lower_index, window_scores, SELECT_METHODS, select_plan,
                              exact_topk_scores, quest_page_scores, sparq_channels, sparq_scores,
                              select_decode_unit, adakv_select, adakv_evict)
