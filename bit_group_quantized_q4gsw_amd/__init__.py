"""q4gsw for AMD MI355X: the 4-bit group-symmetric weight-quantized linear layer.

dequant(W[n, k]) = (code[n, k] - 8) * scale[k / group_size, n]
  forward         y   = x . dequant(W)^T
  input gradient  d_x = d_out . dequant(W)           (contracting over N)
  fused QKV       three forwards of one activation, three distinct outputs

All computation runs in the HIP library libq4gsw.so (C ABI: include/q4gsw.h);
this package only marshals arguments.  Importing it loads the library and raises
if it has not been built.
"""
from .binding import (  # noqa: F401
    BF16, F16, F32, OP_BWD_INPUT, OP_DQ8CA, OP_FWD, OP_QKV, ROUTES, PackedWeight, Q4gswError, WeightDesc,
    adamw_step, adapter_bwd, adapter_fwd, adapter_workspace_bytes, build_info, dq8ca_quantize, embedding, linear_dq8ca, forced_plan, forced_route, lib, linear_bwd_input, linear_fwd, linear_fwd_noalloc, pack, packed_bytes, qkv_fused,
    plan, qkv_workspace_bytes, route, route_name, status_str, unpack, workspace_bytes,
)

lib()
