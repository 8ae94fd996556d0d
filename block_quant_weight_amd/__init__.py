"""Block-quantized (Q4_0 / Q8_0) weight matrix x activation products on one
MI355X (gfx950): a C-ABI HIP library (include/qmv.h, csrc/) and its thin
Python binding (qmv.py).  synth.py draws the seeded synthetic inputs."""
from .qmv import (EXPORTS, QMV_Q4_0, QMV_Q8_0, QmvError, QmvHandle,  # noqa: F401
                  qmv_block_dots, qmv_class_wtype, qmv_create, qmv_destroy,
                  qmv_embed_rows, qmv_gemm, qmv_gemv, qmv_gemv_group, qmv_quantize_q8,
                  qmv_span, qmv_status_str, qmv_upload)
