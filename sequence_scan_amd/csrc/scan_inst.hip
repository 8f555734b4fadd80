// One set of instances of the chunked scan kernel (scan_kernel.h), chosen by
// the build: input dtype SSM_INST_TIN and output dtype SSM_INST_TOUT (float,
// or uint16_t for bfloat16 bit patterns), and the input coefficient
// SSM_INST_ZOH (0: Mamba's dt; 1: the exact zero-order hold (e^{dt A} - 1) / A
// of "Модуль 8. Альтернативы Transformer", vladkulikov.com, section 4).  The
// build compiles this unit once per combination, in parallel, each defining
// the launcher named SSM_INST_FN (declared in internal.h).
#include "scan_kernel.h"

#if !defined(SSM_INST_TIN) || !defined(SSM_INST_TOUT) || !defined(SSM_INST_ZOH) || !defined(SSM_INST_FN)
#error "scan_inst.hip is compiled with SSM_INST_TIN, SSM_INST_TOUT, SSM_INST_ZOH and SSM_INST_FN defined"
#endif

namespace ssm {

hipError_t SSM_INST_FN(const ScanArgs& a, int ns, hipStream_t s) {
  return launch_scan_ns<SSM_INST_TIN, SSM_INST_TOUT, (SSM_INST_ZOH != 0)>(a, ns, s);
}

}  // namespace ssm
