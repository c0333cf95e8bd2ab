// HIP-event bracketing of individual kernel launches for twomamba_fwd_timed.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace twm {

void ktimer_begin(KTimer* t, const char* name, void* stream) {
    if (!t || t->n >= KTimer::kMax) return;
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
        t->error = 1;
        return;
    }
    t->ev[2 * t->n] = a;
    t->ev[2 * t->n + 1] = b;
    t->names[t->n] = name;
    if (hipEventRecord(a, (hipStream_t)stream) != hipSuccess) t->error = 1;
}

void ktimer_end(KTimer* t, void* stream) {
    if (!t || t->n >= KTimer::kMax) return;
    if (hipEventRecord((hipEvent_t)t->ev[2 * t->n + 1], (hipStream_t)stream) != hipSuccess) t->error = 1;
    t->n++;
}

// Waits for the recorded launches, writes their durations and frees the events.
int ktimer_collect(KTimer* t, float* ms, const char** names, int cap) {
    int status = t->error ? TWOMAMBA_ERR_DEVICE : TWOMAMBA_OK;
    for (int i = 0; i < t->n; ++i) {
        hipEvent_t a = (hipEvent_t)t->ev[2 * i], b = (hipEvent_t)t->ev[2 * i + 1];
        float x = -1.f;
        if (hipEventSynchronize(b) != hipSuccess || hipEventElapsedTime(&x, a, b) != hipSuccess)
            status = TWOMAMBA_ERR_DEVICE;
        if (i < cap) {
            if (ms) ms[i] = x;
            if (names) names[i] = t->names[i];
        }
        hipEventDestroy(a);
        hipEventDestroy(b);
    }
    return status;
}

}  // namespace twm
