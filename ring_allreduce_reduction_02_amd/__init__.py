"""Collective reduction schedules (ring / halving-doubling / butterfly AllReduce,
ReduceScatter, AllGather, Broadcast, AllToAll(v)) for N logical ranks held as
rank-strided buffers in one MI355X's HBM.

The compute path is the C-ABI library ``libcc.so`` (HIP kernels for gfx950);
``ccgpu`` is its ctypes binding.  Importing this package loads nothing.
"""
__all__ = ["ccgpu", "synth"]
