// Stand-ins for the device-side launchers, for the host-code sanitizer build only: the
// harness drives the C ABI through its host checks, gates and file handling, which return
// before any kernel would be launched, so none of these is ever called.
#include "qd_common.h"

namespace qd {
#define QD_STUB return hipErrorInvalidValue
hipError_t launch_quantize_rows(const float*, int, int, int8_t*, float*, int, int, hipStream_t) { QD_STUB; }
hipError_t launch_rope_table(float2*, int, int, float, hipStream_t) { QD_STUB; }
hipError_t launch_fill_i32(int*, int, int, hipStream_t) { QD_STUB; }
hipError_t launch_set_positions(int*, const int*, const int*, int, hipStream_t) { QD_STUB; }
hipError_t launch_iota(int*, int, hipStream_t) { QD_STUB; }
hipError_t launch_embed(const int*, int, const int8_t*, const float*, int, int, bf16_t*, hipStream_t,
                        int*, const int*) { QD_STUB; }
hipError_t launch_rmsnorm(const bf16_t*, int, int, const float*, float, bf16_t*, hipStream_t) { QD_STUB; }
hipError_t launch_resid_norm(bf16_t*, int, int, const float*, int, const float*, const float*, float,
                             bf16_t*, hipStream_t) { QD_STUB; }
hipError_t launch_gemv(const GemvArgs&, int, hipStream_t) { QD_STUB; }
hipError_t launch_skinny(const GemvArgs&, int, hipStream_t) { QD_STUB; }
bool skinny_norm_ok(int, int, int, int) { return false; }
hipError_t launch_gemm(const GemmArgs&, hipStream_t, int*, int*) { QD_STUB; }
hipError_t launch_qk_rope(const RopeArgs&, hipStream_t) { QD_STUB; }
hipError_t launch_sample(const SampleArgs&, int, hipStream_t) { QD_STUB; }
hipError_t sample_scratch_address(void**) { QD_STUB; }
hipError_t launch_reset_seq(int*, int*, const int*, int, int, hipStream_t) { QD_STUB; }
hipError_t launch_attention_decode(const AttnDecArgs&, hipStream_t) { QD_STUB; }
hipError_t attention_decode_residency(int, int, int, int*) { QD_STUB; }
hipError_t launch_flash_prefill(const FlashArgs&, int, int, hipStream_t) { QD_STUB; }
}  // namespace qd
