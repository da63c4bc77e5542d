"""CPU oracle of the MoE feed-forward layer (test infrastructure; see ref.py)."""
from .ref import *  # noqa: F401,F403
