// Stream capture for the decode graph bucket set: the HIP runtime calls behind
// gattn_decode_graphs_create / _launch / _destroy (the bucket logic and every argument check
// live in gattn.cpp). A graph is captured on a private stream of the current device, with the
// default priority, in thread-local capture mode (no other capture-unsafe call of this thread
// may run meanwhile; the decode enqueue makes none), then instantiated once.
#include "kernels.h"

namespace gattn {

hipError_t graph_capture_begin(hipStream_t *s) {
    *s = nullptr;
    hipError_t e = hipStreamCreateWithFlags(s, hipStreamNonBlocking);
    if (e != hipSuccess)
        return e;
    e = hipStreamBeginCapture(*s, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) {
        (void)hipStreamDestroy(*s);
        *s = nullptr;
    }
    return e;
}

hipError_t graph_capture_end(hipStream_t s, void **exec) {
    *exec = nullptr;
    hipGraph_t g = nullptr;
    hipError_t e = hipStreamEndCapture(s, &g);
    if (e == hipSuccess && !g)
        e = hipErrorInvalidValue;
    if (e == hipSuccess) {
        hipGraphExec_t x = nullptr;
        e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
        if (e == hipSuccess)
            *exec = (void *)x;
    }
    if (g)
        (void)hipGraphDestroy(g);
    const hipError_t d = hipStreamDestroy(s);
    return e != hipSuccess ? e : d;
}

hipError_t graph_launch(void *exec, hipStream_t s) { return hipGraphLaunch((hipGraphExec_t)exec, s); }

void graph_free(void *exec) {
    if (exec)
        (void)hipGraphExecDestroy((hipGraphExec_t)exec);
}

}  // namespace gattn
