"""The CPU oracle against its pins (closed forms, brute force, second formulations,
hand-worked fixtures, published generator outputs).  CPU only."""
import numpy as np
import pytest

import oracle_pins as P


@pytest.fixture
def rng():
    return np.random.default_rng(20241203)


@pytest.mark.parametrize("name", ["switch_top1_worked.json", "top2_priority_worked.json"])
def test_worked_fixture(name):
    P.check_worked_fixture(name)


def test_capacity_values():
    P.check_capacity_values()


def test_capacity_bruteforce(rng):
    P.check_capacity_bruteforce(rng)


def test_logits_exact(rng):
    P.check_logits_exact(rng)


def test_logits_bias(rng):
    P.check_logits_bias(rng)


def test_softmax(rng):
    P.check_softmax(rng)


def test_topk_rank(rng):
    P.check_topk_rank(rng)


def test_gate_raw(rng):
    P.check_gate_raw(rng)


def test_splitmix_reference():
    P.check_splitmix_reference()


def test_rre(rng):
    P.check_rre(rng)


def test_dispatch_invariants(rng):
    P.check_dispatch_invariants(rng)


def test_dispatch_no_drop(rng):
    P.check_dispatch_no_drop(rng)


def test_choice_priority(rng):
    P.check_choice_priority(rng)


def test_gelu_values():
    P.check_gelu_values()


def test_dense_equals_sparse(rng):
    P.check_dense_equals_sparse(rng)


def test_forward_rows(rng):
    P.check_forward_rows(rng)


def test_route_and_dispatch(rng):
    P.check_route_and_dispatch(rng)


def test_glu_coordinate_gate(rng):
    P.check_glu_coordinate_gate(rng)


def test_glu_linear_in_v(rng):
    P.check_glu_linear_in_v(rng)


def test_single_expert_is_mlp(rng):
    P.check_single_expert_is_mlp(rng)


def test_k_equals_E_is_softmax_mixture(rng):
    P.check_k_equals_E_is_softmax_mixture(rng)


def test_expert_permutation(rng):
    P.check_expert_permutation(rng)


def test_aux_loss(rng):
    P.check_aux_loss(rng)


def test_backward_autograd(rng):
    P.check_backward_autograd(rng)


def test_backward_finite_differences(rng):
    P.check_backward_finite_differences(rng)


def test_backward_single_expert_is_mlp(rng):
    P.check_backward_single_expert_is_mlp(rng)


def test_backward_rre(rng):
    P.check_backward_rre_no_router_grad(rng)


def test_sparse_clip(rng):
    P.check_sparse_clip(rng)
