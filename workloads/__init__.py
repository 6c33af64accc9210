"""Seeded synthetic link workloads: configs and input generators (no link arithmetic)."""
from .configs import CONFIGS, CONFIG_ORDER, MODEL_LINK, MODEL_SHAPES, LinkConfig, ModelShape
from . import gen

__all__ = ["CONFIGS", "CONFIG_ORDER", "MODEL_LINK", "MODEL_SHAPES", "LinkConfig", "ModelShape", "gen"]
