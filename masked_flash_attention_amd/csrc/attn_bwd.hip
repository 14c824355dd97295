// Backward of masked attention (two passes). Placeholder exports until the
// kernels land: every call reports MFA_E_UNSUPPORTED.
#include "common.hpp"

extern "C" {
mfa_status mfa_attn_bwd_preprocess(const mfa_attn_bwd_args*, hipStream_t) { return MFA_E_UNSUPPORTED; }
mfa_status mfa_attn_bwd_dkdv(const mfa_attn_bwd_args*, const mfa_mask*, float, hipStream_t) { return MFA_E_UNSUPPORTED; }
mfa_status mfa_attn_bwd_dq(const mfa_attn_bwd_args*, const mfa_mask*, float, hipStream_t) { return MFA_E_UNSUPPORTED; }
}
