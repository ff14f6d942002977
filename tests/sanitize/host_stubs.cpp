// host_stubs.cpp -- stand-ins for the kernel launchers of libcakv, for a
// host-only build of the C ABI layer (csrc/api.cpp) under AddressSanitizer
// and UndefinedBehaviorSanitizer (tests/sanitize/run_host_sanitizers.py).
//
// TEST BUILD ONLY: nothing here launches anything. Every launcher returns
// hipErrorNotSupported, so a call that gets past argument validation fails
// loudly instead of pretending to compute; the two geometry queries return
// the values of the real kernels (waves per workgroup, rows per fp32
// workgroup) because the validation layer sizes grids with them.
#include <hip/hip_runtime.h>

#include "bwd_args.h"
#include "decode_args.h"
#include "fwd_args.h"

namespace cakv {

static int no_launch() { return (int)hipErrorNotSupported; }

int launch_fwd_bf16(const FwdArgs&, int, void*) { return no_launch(); }
int launch_fwd_f32(const FwdArgs&, int, void*) { return no_launch(); }
int fwd_bf16_waves(int D, int G, long long tasks) {
    return (D == 64 || (G == 1 && tasks < 256LL * 8)) ? 4 : 8;
}
int fwd_f32_wg_rows() { return 64; }
int launch_state_init(float*, float*, float*, long long, int, void*) { return no_launch(); }
int launch_counter_add(unsigned long long*, unsigned long long, void*) { return no_launch(); }
int launch_mfma_burn(int, int, float*, void*) { return no_launch(); }
int launch_finalize(const float*, const float*, const float*, void*, int, float*, int, int, int,
                    int, void*) {
    return no_launch();
}
int launch_lse_merge(const float*, const float*, const float*, const float*, float*, float*, int,
                     int, int, int, void*) {
    return no_launch();
}
int launch_decode_split(const DecArgs&, int, void*) { return no_launch(); }
int launch_decode_merge(const DecArgs&, int, void*) { return no_launch(); }
int decode_scratch_address(void**) { return no_launch(); }
int launch_bwd(const BwdArgs&, int, void*) { return no_launch(); }

}  // namespace cakv
