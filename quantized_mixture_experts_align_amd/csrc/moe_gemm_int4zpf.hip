// Instantiation of the grouped GEMM kernels for asymmetric int4 weights with float16 zero points
// (one translation unit per format so the kernel variants compile in parallel).
#include "moe_gemm_decode.h"
#include "moe_gemm_mfma.h"

namespace moe {
template int launch_gemm_decode<MOE_Q_INT4ZPF_G128>(bool, int, const GemmArgs&, const moe_gemm_config&, int, int, hipStream_t);
template int launch_gemm_mfma<MOE_Q_INT4ZPF_G128>(bool, int, const GemmArgs&, const moe_gemm_config&, int, hipStream_t);
template int mfma_residency<MOE_Q_INT4ZPF_G128>(bool, bool, int, int*);
}  // namespace moe
