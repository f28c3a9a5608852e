"""Lynx split-stream KV codec and anchor-only decode attention for AMD MI355X (gfx950).

The compute lives in the HIP library liblynx.so (C ABI in include/lynx.h);
`decode_attention_lynx_amd.lynx` is the thin ctypes binding.  Importing the
package loads nothing; the binding loads the library on first use and raises
if it is missing.
"""
