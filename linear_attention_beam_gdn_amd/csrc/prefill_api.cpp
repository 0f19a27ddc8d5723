// Host side of the context-free prefill (declared in onela.h: onela_prefill).
#include <stdint.h>

#include "../../include/onela.h"
#include "onela_internal.h"

namespace {

bool pf_aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

extern "C" onela_status onela_prefill(int32_t n_seq, int32_t num_heads, int32_t d_k, int32_t d_v, int32_t seq_len,
                                      const uint16_t* k, const uint16_t* v, const float* alpha, const float* beta,
                                      const float* S_init, float* S_out, void* hip_stream) {
    if (n_seq < 1 || num_heads < 1 || seq_len < 0 || !S_out) return ONELA_E_INVALID_ARG;
    if (seq_len > 0 && (!k || !v || !alpha || !beta)) return ONELA_E_INVALID_ARG;
    if (!pf_aligned(k, 16) || !pf_aligned(v, 16) || !pf_aligned(alpha, 4) || !pf_aligned(beta, 4) ||
        !pf_aligned(S_init, 16) || !pf_aligned(S_out, 16))
        return ONELA_E_INVALID_ARG;
    if (!onela::step_supported(d_k, d_v)) return ONELA_E_UNSUPPORTED;
    if ((int64_t)n_seq * num_heads >= INT32_MAX) return ONELA_E_UNSUPPORTED;   // one workgroup each
    onela::PrefillParams p{};
    p.k = k;
    p.v = v;
    p.alpha = alpha;
    p.beta = beta;
    p.s_init = S_init;
    p.s_out = S_out;
    p.planes = nullptr;
    p.n_seq = n_seq;
    p.H = num_heads;
    p.L = seq_len;
    const hipError_t e = onela::launch_prefill(d_k, d_v, false, p, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? ONELA_OK : ONELA_E_HIP;
}
