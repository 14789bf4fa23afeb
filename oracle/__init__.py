"""CPU oracle for content-adaptive block-sparse attention (ASA / ASA_G).

TEST INFRASTRUCTURE ONLY.  A plain, slow, float64 (and exact-rational, for the
mask) implementation of what the GPU path computes, written from the method's
description and sharing no code with the HIP library.  Only tests, the smoke
check and the CPU-baseline leg of the bench may import it; the product path
never does.

Modules: perm (curve and cuboid orders), reorder (gather / scatter), estimator
(sampled block importance), mask (cumulative-threshold mask), mask_rules
(the top-k and statistical-threshold alternatives), attention
(block-masked attention with optional global tokens), attention_bwd (its
gradients, plain ASA, and the key-to-query block lists), query_prune (BSA
query pruning and token filling), pooled (MEAN / TripPool block estimators
and the SICS aggregation score), accounting (sparsity and FLOP).  Every function is pinned by CPU tests against closed forms, invariants
and brute force (tests/test_oracle_*.py).
"""
