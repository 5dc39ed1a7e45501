"""Offline launch-shape sweep for gfx950 (see sweep.py)."""
