"""BF16 DiT row epilogues for MI355X (gfx950): a C-ABI HIP library and its
Python binding.  The binding is loaded lazily on the first call."""
