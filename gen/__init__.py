"""Seeded synthetic inputs for absorbed-MLA tree-verify attention.

This package only draws random numbers and lays them out (shapes, trees, page
tables). It holds none of the attention arithmetic, so the CPU oracle and the
HIP library can both consume it without sharing any of the method.
"""
from .configs import CONFIGS, VerifyConfig, get_config
from .inputs import VerifyInputs, make_accept_tokens, make_inputs, make_tree_parents

__all__ = ["CONFIGS", "VerifyConfig", "get_config", "VerifyInputs", "make_accept_tokens", "make_inputs",
           "make_tree_parents"]
