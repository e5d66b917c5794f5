// bandwidth.hip — memory-bandwidth probes in the pipeline kernels' access patterns (see
// include/zero_probe.h).  Trivial arithmetic, the same launch shape as the pipeline: a one-shot
// grid of 256-thread blocks, each thread one 16-byte chunk per stream, global (not flat)
// 16-byte accesses.  Every load and store instruction of a wavefront covers 1 KB of whole cache
// lines, and all of them are nontemporal: the fastest form of each pattern on this part (the
// pipeline kernels use the same form wherever their data is aligned that way).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zero_probe.h"

namespace {

constexpr int kBlock = 256;
constexpr int64_t kMaxBlocks = int64_t(1) << 23;  // fewer than 2^32 work-items per dispatch

// Blocks resident per CU, capped by reserving dynamic LDS that the kernels do not touch (a CU
// has 160 KB).  Measured on MI355X: the write stream is fastest at four blocks per CU (6% over
// full occupancy), the Adam stream mix at two (3%); the read and copy streams at full occupancy
// (four blocks: 8-40% slower).
constexpr unsigned kLdsPerCu = 160 * 1024;
constexpr unsigned kFourBlocksLds = 36 * 1024, kTwoBlocksLds = 60 * 1024;
static_assert(4 * kFourBlocksLds <= kLdsPerCu && 5 * kFourBlocksLds > kLdsPerCu, "four blocks per CU");
static_assert(2 * kTwoBlocksLds <= kLdsPerCu && 3 * kTwoBlocksLds > kLdsPerCu, "two blocks per CU");
#define ZP_GLOBAL __attribute__((address_space(1)))
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld(const void* p) { return __builtin_nontemporal_load((const ZP_GLOBAL u32x4*)p); }
__device__ __forceinline__ void st(void* p, u32x4 v) { __builtin_nontemporal_store(v, (ZP_GLOBAL u32x4*)p); }
__device__ __forceinline__ f32x4 ldf(const float* p) { return __builtin_nontemporal_load((const ZP_GLOBAL f32x4*)p); }
__device__ __forceinline__ void stf(float* p, f32x4 v) { __builtin_nontemporal_store(v, (ZP_GLOBAL f32x4*)p); }

// chunks: 16-byte chunks of the stream; one per thread per iteration of the grid-stride loop
__global__ __launch_bounds__(kBlock) void probe_read_kernel(const u32x4* __restrict__ src, int64_t chunks,
                                                            u32x4* __restrict__ sink) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t c = blockIdx.x * int64_t(kBlock) + threadIdx.x; c < chunks; c += int64_t(gridDim.x) * kBlock)
        acc ^= ld(src + c);
    if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u) st(sink, acc);
}

__global__ __launch_bounds__(kBlock) void probe_write_kernel(u32x4* __restrict__ dst, int64_t chunks) {
    for (int64_t c = blockIdx.x * int64_t(kBlock) + threadIdx.x; c < chunks; c += int64_t(gridDim.x) * kBlock) {
        const uint32_t w = uint32_t(c);
        const u32x4 v = {w, w ^ 0x55555555u, w ^ 0xaaaaaaaau, ~w};
        st(dst + c, v);
    }
}

__global__ __launch_bounds__(kBlock) void probe_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                            int64_t chunks) {
    for (int64_t c = blockIdx.x * int64_t(kBlock) + threadIdx.x; c < chunks; c += int64_t(gridDim.x) * kBlock)
        st(dst + c, ld(src + c));
}

// groups: spans of 2048 columns; a block takes one span, and in each of two passes its threads
// take consecutive 4-column groups of one half (Adam's lane-strided layout: every instruction of
// a wavefront covers whole lines of each stream, 8 bytes per lane for the 16-bit stream)
__global__ __launch_bounds__(kBlock) void probe_adam_streams_kernel(const float* __restrict__ g,
                                                                    float* __restrict__ p, float* __restrict__ m,
                                                                    float* __restrict__ v, uint16_t* __restrict__ lp,
                                                                    int64_t spans) {
    for (int64_t sp = blockIdx.x; sp < spans; sp += gridDim.x) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t x = sp * (8 * kBlock) + h * (4 * kBlock) + 4 * int64_t(threadIdx.x);
            const f32x4 g0 = ldf(g + x);
            f32x4 p0 = ldf(p + x), m0 = ldf(m + x), v0 = ldf(v + x);
            p0 += g0, m0 += g0, v0 += g0;
            stf(p + x, p0), stf(m + x, m0), stf(v + x, v0);
            const u32x4 a = __builtin_bit_cast(u32x4, p0);
            const uint64_t w = uint64_t((a.x >> 16) | (a.y & 0xffff0000u)) |
                               (uint64_t((a.z >> 16) | (a.w & 0xffff0000u)) << 32);
            __builtin_nontemporal_store(w, (ZP_GLOBAL uint64_t*)(lp + x));
        }
    }
}

int grid(int64_t threads) {
    const int64_t blocks = (threads + kBlock - 1) / kBlock;
    return int(blocks < 1 ? 1 : blocks < kMaxBlocks ? blocks : kMaxBlocks);
}

bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

zero_status launched() { return hipGetLastError() == hipSuccess ? ZERO_OK : ZERO_EHIP; }

}  // namespace

extern "C" zero_status zero_probe_read(const void* d_src, int64_t bytes, void* d_sink, void* stream) {
    if (!d_src || !d_sink || bytes <= 0 || bytes % 16 || !a16(d_src) || !a16(d_sink)) return ZERO_EINVAL;
    const int64_t chunks = bytes / 16;
    probe_read_kernel<<<grid(chunks), kBlock, 0, (hipStream_t)stream>>>(static_cast<const u32x4*>(d_src), chunks,
                                                                        static_cast<u32x4*>(d_sink));
    return launched();
}

extern "C" zero_status zero_probe_write(void* d_dst, int64_t bytes, void* stream) {
    if (!d_dst || bytes <= 0 || bytes % 16 || !a16(d_dst)) return ZERO_EINVAL;
    const int64_t chunks = bytes / 16;
    probe_write_kernel<<<grid(chunks), kBlock, kFourBlocksLds, (hipStream_t)stream>>>(static_cast<u32x4*>(d_dst),
                                                                                      chunks);
    return launched();
}

extern "C" zero_status zero_probe_copy(const void* d_src, void* d_dst, int64_t bytes, void* stream) {
    if (!d_src || !d_dst || bytes <= 0 || bytes % 16 || !a16(d_src) || !a16(d_dst)) return ZERO_EINVAL;
    const char* s = static_cast<const char*>(d_src);
    const char* d = static_cast<const char*>(d_dst);
    if (s < d + bytes && d < s + bytes) return ZERO_EINVAL;  // overlapping buffers
    const int64_t chunks = bytes / 16;
    probe_copy_kernel<<<grid(chunks), kBlock, 0, (hipStream_t)stream>>>(static_cast<const u32x4*>(d_src),
                                                                        static_cast<u32x4*>(d_dst), chunks);
    return launched();
}

extern "C" zero_status zero_probe_adam_streams(const float* d_g, float* d_p, float* d_m, float* d_v, uint16_t* d_lp,
                                               int64_t n, void* stream) {
    if (!d_g || !d_p || !d_m || !d_v || !d_lp || n <= 0 || n % (8 * kBlock)) return ZERO_EINVAL;
    if (!a16(d_g) || !a16(d_p) || !a16(d_m) || !a16(d_v) || !a16(d_lp)) return ZERO_EINVAL;
    const int64_t spans = n / (8 * kBlock);
    const int g = int(spans < kMaxBlocks ? spans : kMaxBlocks);
    probe_adam_streams_kernel<<<g, kBlock, kTwoBlocksLds, (hipStream_t)stream>>>(d_g, d_p, d_m, d_v, d_lp, spans);
    return launched();
}
