"""Activation-sparse ReLU-gated FFN (TwELL) on MI355X: HIP kernels behind a C-ABI."""
