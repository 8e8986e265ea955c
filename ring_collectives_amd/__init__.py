"""ring_collectives_amd -- ring collectives for P virtual ranks held in one
MI355X's HBM (gfx950), behind a C-ABI library of hand-written HIP kernels.

The Python layer only marshals arguments (device pointers, sizes, the HIP
stream) into the C ABI; every step of the collectives runs in the kernels.
"""
