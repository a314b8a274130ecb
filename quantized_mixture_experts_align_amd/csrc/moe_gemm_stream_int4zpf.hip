// Instantiation of the streaming decode GEMM for asymmetric int4 weights with float16 zero points
// (one translation unit per format so the kernel variants compile in parallel).
#include "moe_gemm_stream.h"

namespace moe {
template int launch_gemm_stream<MOE_Q_INT4ZPF_G128>(bool, int, const GemmArgs&, const moe_gemm_config&, int, int, hipStream_t);
}  // namespace moe
