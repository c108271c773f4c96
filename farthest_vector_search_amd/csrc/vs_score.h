// vs_score.h -- a query's reported result from its merged packed key.
//
// The scans leave, per query, the minimum packed key over its candidates
// (ranking value high, index low).  The winner's index is unpacked and its
// score rebuilt: squared L2 adds the query's own squared norm qn back
// (|q|^2 + |c|^2 - 2 q.c) and clamps at 0; cosine reports q.c.  No key
// means no candidate: index -1, score NaN.  Every finalize of the dense
// search writes its results through this one routine.
#pragma once

#include "vs_internal.h"

namespace vs {

template <int M>
__device__ __forceinline__ void write_result(uint64_t k, float qn, int32_t *idx, float *score) {
    if (k == kNoKey) {
        *idx = -1;
        if (score) *score = __builtin_nanf("");
        return;
    }
    *idx = (int32_t)(uint32_t)(k & 0xffffffffu);
    if (score) {
        const float e = float_of_ord((uint32_t)(k >> 32));
        const float key = metric_is_max(M) ? -e : e;
        float s;
        if constexpr (metric_is_l2(M)) {
            s = qn + key;
            s = s > 0.0f ? s : 0.0f;
        } else {
            s = key;
        }
        *score = s;
    }
}

}  // namespace vs
