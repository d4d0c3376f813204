"""LatentIndex decode indexer for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``liblatentindex.so`` built from the HIP
sources in ``csrc/``; ``ops`` is its thin Python binding.  ``workloads`` draws
the seeded synthetic inputs.  Importing the package loads nothing native.
"""
