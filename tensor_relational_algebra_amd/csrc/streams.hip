// streams.hip -- host-side stream and event helpers for the graph executor
// (the planner sources are plain C++ compiled without the HIP headers).
//
// The overlapped graph executor runs the repartition copies between nodes on
// a second stream of the same device while the nodes run on the caller's
// stream, ordered by events: the copy-compute overlap that the EinDecomp
// page's closing remarks list among the costs a deployment should model.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "graph.h"

namespace tra {

int current_device(int *dev) { return (int)hipGetDevice(dev); }

// One non-blocking side stream per device, created on first use and kept for
// the life of the process (default priority).
int side_stream(void **out)
{
    static std::mutex mu;
    static std::map<int, hipStream_t> streams;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    std::lock_guard<std::mutex> lock(mu);
    auto it = streams.find(dev);
    if (it == streams.end()) {
        hipStream_t s = nullptr;
        e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
        if (e != hipSuccess) return (int)e;
        it = streams.emplace(dev, s).first;
    }
    *out = (void *)it->second;
    return 0;
}

int events_create(int n, void **ev)
{
    for (int i = 0; i < n; ++i) {
        hipEvent_t e = nullptr;
        hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
        if (r != hipSuccess) {
            events_destroy(i, ev);
            return (int)r;
        }
        ev[i] = (void *)e;
    }
    return 0;
}

void events_destroy(int n, void **ev)
{
    for (int i = 0; i < n; ++i)
        if (ev[i]) {
            (void)hipEventDestroy((hipEvent_t)ev[i]);
            ev[i] = nullptr;
        }
}

int event_record(void *ev, void *stream) { return (int)hipEventRecord((hipEvent_t)ev, (hipStream_t)stream); }

int stream_wait_event(void *stream, void *ev)
{
    return (int)hipStreamWaitEvent((hipStream_t)stream, (hipEvent_t)ev, 0);
}

}  // namespace tra
