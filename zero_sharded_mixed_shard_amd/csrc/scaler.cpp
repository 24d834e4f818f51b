// Skip-or-apply decision and dynamic loss scale: host-only, no device access.
//
// A step whose unscaled gradients overflow is skipped and the loss scale is
// reduced; clean steps advance the applied-update counter that the bias
// corrections use ("Training models too big for one GPU: ZeRO & FSDP",
// "Mixed-precision training").  Halving on overflow and doubling after a run
// of clean steps is the usual dynamic rule.
#include <cmath>

#include "zero_shard.h"

extern "C" int zero_scaler_update(zero_scaler *s, int32_t found_inf, int32_t *apply) {
    if (s == nullptr || apply == nullptr) return ZERO_EINVAL;
    if (!(s->loss_scale > 0.0f) || !std::isfinite(s->loss_scale)) return ZERO_EINVAL;
    if (found_inf != 0) {
        s->loss_scale = s->loss_scale * 0.5f;
        s->clean_steps = 0;
        *apply = 0;
        return ZERO_OK;
    }
    s->step += 1;
    s->clean_steps += 1;
    if (s->growth_interval != 0 && s->clean_steps >= s->growth_interval) {
        const float grown = s->loss_scale * 2.0f;
        if (std::isfinite(grown)) s->loss_scale = grown;
        s->clean_steps = 0;
    }
    *apply = 1;
    return ZERO_OK;
}
