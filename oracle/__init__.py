"""fp64 CPU oracle of the Switch FFN layer forward pass.

Test infrastructure only: tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import it; the library never does.
"""
from .switch_oracle import (  # noqa: F401
    Aux, LayerResult, Routing, Slots, aux_loss, capacity, combine, dispatch,
    expert_ffn, expert_rows, layer_dense_onehot, layer_forward, layer_per_token,
    router_logits, router_z_loss, slot_scan, softmax_top1, ZLoss,
    AuxG, LayerResultG, RoutingK, SlotsG, aux_loss_grouped, assignment_order, combine_topk,
    group_capacity, layer_forward_grouped, layer_per_token_topk, slot_scan_grouped, softmax_topk,
    LayerGrads, layer_backward, layer_objective,
)
