// Measurement helpers for the benchmark (not part of the cache library), built as libkvq_probe.so: a plain
// streaming read of a device buffer (the achievable HBM read bandwidth of the box, reported next to the published
// peak) and an engine-clock probe that runs beside the timed calls.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kWaves = 2048;   // one 64-lane workgroup per wavefront, 8 per CU; one contiguous segment each
constexpr int kVec = 3;        // 1 KB loads in flight per wavefront

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Wavefront w reads its contiguous segment of src (a multiple of 1 KB, the last one shorter) with 16-byte
// non-temporal loads, kVec consecutive kilobytes per iteration, folded by XOR into one word per lane, which is
// written so the loads are kept. (A shape sweep on MI355X over 1.6 GB, 2048..4096 wavefronts with 3, 4 or 8 loads in
// flight: 6.7-7.1 TB/s with non-temporal loads, best at 2048 wavefronts and 3 loads; 6.0-6.2 TB/s with plain loads.
// An earlier plain-load sweep up to 65536 wavefronts and 16 loads gave 5.7-6.1 TB/s, and a grid-stride order with
// 8 MB between a wavefront's loads 5.5.)
__global__ __launch_bounds__(64) void hbm_read_kernel(const uint4 *src, size_t n16, size_t per, uint32_t *sink) {
    const size_t beg = (size_t)blockIdx.x * per;
    const size_t end = beg + per < n16 ? beg + per : n16;
    uint32_t acc = 0;
    size_t i = beg + threadIdx.x;
    const u32x4 *s4 = reinterpret_cast<const u32x4 *>(src);
    for (; i + (kVec - 1) * 64 < end; i += kVec * 64) {
        uint4 b[kVec];
#pragma unroll
        for (int k = 0; k < kVec; ++k) b[k] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(s4 + i + k * 64));
#pragma unroll
        for (int k = 0; k < kVec; ++k) acc ^= b[k].x ^ b[k].y ^ b[k].z ^ b[k].w;
    }
    for (; i < end; i += 64) {
        const uint4 a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    sink[(size_t)blockIdx.x * 64 + threadIdx.x] = acc;
}

constexpr int kClockWaves = 8;   // consecutive workgroups are dispatched to the eight XCDs in turn

// Engine clock over a window of wall time: each wavefront reads the shader cycle counter and the constant-rate
// counter, sleeps in short steps until `ticks` of the constant-rate counter have passed (every wavefront leaves the
// loop by then), and reads both again. One wavefront per XCD, a few VGPRs and no LDS: it shares its SIMD with the
// timed kernels' wavefronts and issues almost nothing itself.
__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t ticks, unsigned long long *out) {
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    uint64_t r1 = r0;
    while (r1 - r0 < ticks) {
        __builtin_amdgcn_s_sleep(32);
        r1 = __builtin_amdgcn_s_memrealtime();
    }
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        out[2 * blockIdx.x] = c1 - c0;
        out[2 * blockIdx.x + 1] = r1 - r0;
    }
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) size_t kvq_probe_clock_words(void) { return 2 * kClockWaves; }

// Rate of the constant-rate counter in kHz (0 if the runtime does not report it).
__attribute__((visibility("default"))) int kvq_probe_wall_clock_khz(void) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
    return khz;
}

// Enqueues the clock probe for `ticks` constant-rate ticks on `stream`. out: device, at least
// kvq_probe_clock_words() uint64 words: per wavefront (shader cycles, constant-rate ticks) elapsed. Returns 0, -1
// on bad arguments (nothing launched, ticks limited to 10^9), -8 on a launch error.
__attribute__((visibility("default"))) int kvq_probe_clock(uint64_t ticks, unsigned long long *out, size_t out_words,
                                                            void *stream) {
    if (!out || out_words < (size_t)(2 * kClockWaves) || ticks == 0 || ticks > 1000000000ull) return -1;
    hipLaunchKernelGGL(clock_probe_kernel, dim3(kClockWaves), dim3(64), 0, static_cast<hipStream_t>(stream), ticks,
                       out);
    return hipGetLastError() == hipSuccess ? 0 : -8;
}

__attribute__((visibility("default"))) size_t kvq_probe_sink_words(void) { return (size_t)kWaves * 64; }

// src: device, 16-byte aligned, bytes a positive multiple of 16; sink: device, at least kvq_probe_sink_words()
// uint32 words. Returns 0 on success, -1 on bad arguments (nothing launched), -8 on a launch error.
__attribute__((visibility("default"))) int kvq_probe_hbm_read(const void *src, size_t bytes, uint32_t *sink,
                                                               size_t sink_words, void *stream) {
    if (!src || !sink || bytes == 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15u) != 0 ||
        sink_words < (size_t)kWaves * 64)
        return -1;
    const size_t n16 = bytes / 16;
    const size_t per = ((n16 + kWaves - 1) / kWaves + 63) / 64 * 64;   // 16-byte units per wavefront
    const unsigned grid = (unsigned)((n16 + per - 1) / per);            // <= kWaves
    hipLaunchKernelGGL(hbm_read_kernel, dim3(grid), dim3(64), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4 *>(src), n16, per, sink);
    return hipGetLastError() == hipSuccess ? 0 : -8;
}

}  // extern "C"
