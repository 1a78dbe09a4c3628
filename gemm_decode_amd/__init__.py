"""Weight-only quantized linear (W8A16 / W4A16) for AMD MI355X (gfx950).

* ``gemm_decode_amd.csrc``  -- HIP kernels and the C ABI (include/wq.h), built
  into ``libwq.so`` by ``gemm_decode_amd.build``;
* ``gemm_decode_amd.wq``    -- the Python binding (ctypes, argument marshalling
  only; importing it raises ImportError when libwq.so is not built).
"""
