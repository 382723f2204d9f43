// C ABI bookkeeping: status strings, thread-local last error and dispatch
// name, version.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "ls_common.hpp"

namespace {
thread_local char g_last_error[512] = "";
thread_local char g_last_dispatch[128] = "";
thread_local hipEvent_t g_time_start = nullptr;   // events for the next timed launch
thread_local hipEvent_t g_time_stop = nullptr;
}  // namespace

namespace ls {

// Armed timing events live for one operator call: every call ends through
// fail(), launch_status() or set_dispatch(), and each of them disarms.
static void disarm() { g_time_start = g_time_stop = nullptr; }

int fail(int status, const char* fmt, ...) {
    disarm();
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

void set_dispatch(const char* name) {
    disarm();
    std::snprintf(g_last_dispatch, sizeof(g_last_dispatch), "%s", name);
}

void clear_hip_error() { (void)hipGetLastError(); }

bool take_launch_events(hipEvent_t* start, hipEvent_t* stop) {
    if (!g_time_start) return false;
    *start = g_time_start;
    *stop = g_time_stop;
    g_time_start = g_time_stop = nullptr;
    return true;
}

int launch_status(const char* what) {
    disarm();
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(LS_ERR_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
    g_last_error[0] = '\0';
    return LS_OK;
}

}  // namespace ls

extern "C" {

const char* ls_status_string(int status) {
    switch (status) {
        case LS_OK: return "ok";
        case LS_ERR_NULL: return "null pointer";
        case LS_ERR_SHAPE: return "invalid shape";
        case LS_ERR_PARAM: return "invalid parameter";
        case LS_ERR_WORKSPACE: return "workspace too small";
        case LS_ERR_UNSUPPORTED: return "unsupported shape";
        case LS_ERR_HIP: return "HIP runtime error";
        case LS_ERR_UNIMPLEMENTED: return "not implemented";
        default: return "unknown status";
    }
}

int ls_time_next_launch(void* start_event, void* stop_event) {
    if (!start_event || !stop_event) {
        g_time_start = g_time_stop = nullptr;
        return ls::fail(LS_ERR_NULL, "ls_time_next_launch: null event");
    }
    g_time_start = static_cast<hipEvent_t>(start_event);
    g_time_stop = static_cast<hipEvent_t>(stop_event);
    return LS_OK;
}

int ls_time_armed(void) { return g_time_start != nullptr ? 1 : 0; }

const char* ls_last_error(void) { return g_last_error; }
const char* ls_last_dispatch(void) { return g_last_dispatch; }
const char* ls_version(void) { return "ls_mi355 0.1.0 (gfx950)"; }
int ls_dropout_decision_bits(void) { return ls::kDropoutBits; }

}  // extern "C"
