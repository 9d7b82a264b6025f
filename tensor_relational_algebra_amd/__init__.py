"""MI355X-native executor for extended EinSum as tensor-relational algebra.

The compute path is the C-ABI library libtra (include/tra.h: tra_plan,
tra_execute, tra_repartition, tra_choose, ...) with hand-written gfx950 HIP
kernels; this package is its thin Python binding (torch supplies device
memory and streams) plus the seeded synthetic workloads.
"""
from ._binding import (  # noqa: F401
    CHOOSE_TIME, GRAPH_CHOOSE_TIME, GRAPH_FUSE_ATTENTION, GRAPH_OVERLAP_COPIES, LIB_PATH, Graph, Plan, TraError,
    from_relation, lib, to_relation, tra_canonical_labels, tra_choose, tra_choose_cache_clear, tra_choose_cache_stats,
    tra_cost, tra_d_from_operand_form, tra_execute, tra_execute_chain, tra_execute_contract_chain, tra_execute_static,
    tra_graph_execute, tra_graph_plan, tra_probe_mfma_loop, tra_static_scratch_bytes,
    tra_graph_plan_cap, tra_graph_plan_ex, tra_graph_run_node, tra_plan, tra_predict_ns, tra_predict_repartition_ns,
    tra_repartition)
from .attention import AttentionLayer  # noqa: F401
