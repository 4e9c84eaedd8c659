"""Seeded synthetic inputs for the packed ternary-weight product.

This package makes the inputs that both the HIP path and the CPU oracle
consume: trit planes, per-group / per-tensor scales, codebook indices,
balanced-ternary digits and activations.  It holds no part of the product
itself (no packing, no quantisation, no dot products): it only draws random
numbers and rounds them to the storage types the workloads name.

`gen` is the host (numpy) generator.  `device` drives the same generator
compiled for the GPU (`synth_kernels.hip`) so that multi-gigabyte inputs can be
made in HBM; both sides evaluate the same sequence of IEEE basic operations
and agree bit for bit.
"""
