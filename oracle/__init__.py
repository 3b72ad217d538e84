"""Test infrastructure: the fp64 CPU oracle. Never imported by the product path."""

from .beam_oracle import *  # noqa: F401,F403
