// Kernel launchers for the host-sanitizer build of libbsattn: the host
// sources (argument checks, block-index builder, calibration, workspace
// layout) are built with AddressSanitizer and UndefinedBehaviorSanitizer
// and linked against these stand-ins instead of the device code, so the
// library loads and runs its host paths on a machine without a GPU.  Every
// launch reports "no device".  Test infrastructure only.
#include <hip/hip_runtime_api.h>

#include "../../block_sparse_attention_flash_amd/csrc/internal.h"

namespace bsattn {

int launch_prefill_bf16(const PrefillParams&, void*) { return hipErrorNoDevice; }
int launch_prefill_f32(const PrefillParams&, void*) { return hipErrorNoDevice; }
int launch_prefill_bwd(const BwdParams&, void*) { return hipErrorNoDevice; }
int launch_decode(const DecodeParams&, void*) { return hipErrorNoDevice; }
int noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  return hipErrorNoDevice;
}

}  // namespace bsattn
