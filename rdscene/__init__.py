"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

Holds scene geometry and the raw-echo simulator only; none of the focusing arithmetic."""
from .configs import C1, C2, C3, C4, C5, CONFIGS, C_LIGHT, SceneConfig  # noqa: F401
from .simulate import Scene, cached_scene, make_scene  # noqa: F401
