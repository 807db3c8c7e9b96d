"""CPU oracle of the Sparse-BitLinear operator.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.
"""
from .sparse_bitlinear import (CODE_MINUS, CODE_PLUS, CODE_ZERO, abs_sum_exact, act_quant,  # noqa: F401
                               adamw_repack, adamw_update, f64_to_bf16_bits, mask_flips, unpack_mask,
                               rmsnorm_act_quant, rmsnorm_bf16, rmsnorm_rstd, mean_square_f32, rsqrt_rn32,
                               square_sum_exact, pack_sparse24, unpack_sparse24, pack_pairs, unpack_pairs,
                               pair_index, PAIR_CODES,
                               backward, backward_stop_gradient, bf16_to_f64, dequant_act,
                               effective_weight, forward_acc, forward_y, gamma_f32, mask_from_quantized,
                               mask_grad, nm_mask,
                               pack_codes, pack_mask, quant_mask_pack, round_rational_to_f32,
                               sparse_bitlinear_step, ternary, unpack_codes)
