"""Routed bit-sliced linear layers (MoBiQuant-style elastic weight quantization) for MI355X."""
