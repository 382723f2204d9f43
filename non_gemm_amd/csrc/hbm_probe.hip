// Reference streaming kernels for the attainable-bandwidth figure that the
// operator kernels are compared with (the roofline argument of [CS336]
// sec. 2.2 needs the bandwidth a kernel can actually reach, next to the
// 8 TB/s data-sheet peak).
//
// Both use the access pattern of the elementwise operators: one 16-byte
// non-temporal access per lane, one 256-thread block per 4 KiB, no loop.
#include "ls_common.hpp"

namespace ls {
namespace {

constexpr int kBlock = 256;

__global__ __launch_bounds__(kBlock) void probe_copy_kernel(float4v* out, const float4v* in, uint64_t n) {
    const uint64_t i = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(in + i), out + i);
}

// Every wave folds its 1 KiB into one float, which lane 0 writes: 4 bytes of
// output per 1024 read keep the loads live at 0.4 % extra traffic.
__global__ __launch_bounds__(kBlock) void probe_read_kernel(float* sink, const float4v* in, uint64_t n) {
    const uint64_t i = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x;
    float s = 0.0f;
    if (i < n) {
        const float4v v = __builtin_nontemporal_load(in + i);
        s = (v[0] + v[1]) + (v[2] + v[3]);
    }
    s = group_sum<kWave>(s);
    if ((threadIdx.x & (kWave - 1)) == 0 && i < n) sink[i / kWave] = s;
}

int probe_check(const char* name, const void* a, const void* b, int64_t bytes) {
    if (bytes < 0 || bytes % 16 != 0)
        return fail(LS_ERR_SHAPE, "%s: bytes must be a non-negative multiple of 16", name);
    if (bytes > 0 && (!a || !b)) return fail(LS_ERR_NULL, "%s: null pointer", name);
    if (bytes > 0 && (!aligned16(a) || !aligned16(b)))
        return fail(LS_ERR_PARAM, "%s: pointers must be 16-byte aligned", name);
    if (bytes / 16 / kBlock >= (1ll << 31)) return fail(LS_ERR_SHAPE, "%s: too large", name);
    return LS_OK;
}

}  // namespace
}  // namespace ls

extern "C" {

int ls_probe_copy(void* dst, const void* src, int64_t bytes, void* stream) {
    using namespace ls;
    const char* name = "ls_probe_copy";
    if (int rc = probe_check(name, dst, src, bytes)) return rc;
    if (bytes == 0) {
        set_dispatch("empty");
        return LS_OK;
    }
    clear_hip_error();
    const uint64_t n = static_cast<uint64_t>(bytes) / 16;
    const unsigned grid = static_cast<unsigned>((n + kBlock - 1) / kBlock);
    probe_copy_kernel<<<grid, kBlock, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<float4v*>(dst), static_cast<const float4v*>(src), n);
    set_dispatch("probe_copy/vec16_nt");
    return launch_status(name);
}

int ls_probe_read(float* sink, const void* src, int64_t bytes, void* stream) {
    using namespace ls;
    const char* name = "ls_probe_read";
    if (int rc = probe_check(name, sink, src, bytes)) return rc;
    if (bytes == 0) {
        set_dispatch("empty");
        return LS_OK;
    }
    clear_hip_error();
    const uint64_t n = static_cast<uint64_t>(bytes) / 16;
    const unsigned grid = static_cast<unsigned>((n + kBlock - 1) / kBlock);
    probe_read_kernel<<<grid, kBlock, 0, static_cast<hipStream_t>(stream)>>>(
        sink, static_cast<const float4v*>(src), n);
    set_dispatch("probe_read/vec16_nt");
    return launch_status(name);
}

}  // extern "C"
