"""kv_cache_bit_amd: NSNQuant KV-cache vector quantisation and compressed-cache
decode attention for MI355X (gfx950).  The compute lives in the HIP library
``libnsnq.so``; :mod:`kv_cache_bit_amd.nsnq` is its ctypes binding."""
