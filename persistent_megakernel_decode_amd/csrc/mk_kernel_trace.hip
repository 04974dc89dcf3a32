// The traced kernels (mk_megakernel_b*_trace): the same megakernel with per-op timing stamps
// (start, inputs in hand, end) written to KArgs::trace.  Chosen by mk_create under MK_TRACE=1.
#define MK_TRACE_STAMPS 1
#include "mk_kernel.hip"
