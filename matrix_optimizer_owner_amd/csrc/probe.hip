// probe.hip - measurement support: the bf16 MFMA rate this GPU sustains with
// given operand data.
//
// The Newton-Schulz contractions are dense bf16 products, so their roofline
// is the MFMA pipes.  The dense peak is reached only at the top shader clock,
// and the clock the part holds under load depends on how many operand bits
// toggle: register-only MFMA loops run near the top clock on zero operands
// and well below it on Gaussian data.  This kernel measures that ceiling
// with the caller's operands (for example the same Gaussian bf16 data the
// contractions see), so a benchmark can report a contraction's rate against
// both the published peak and this measured one.
#include "device_util.h"
#include "mfsdp.h"
#include "plan_internal.h"

namespace mfsdp {
namespace {

constexpr int kProbeWaves = 4;  // one wave per SIMD
constexpr int kProbeFrags = 16; // 8 A and 8 B fragments per lane, 16 bytes each

// Each wave holds 16 accumulators of 32 x 32 (256 AGPRs, as the contraction
// kernels do) and issues v_mfma_f32_32x32x16_bf16 back to back, alternating
// between two sets of 4 A x 4 B operand fragments loaded once per lane.
__global__ __launch_bounds__(64 * kProbeWaves, 1) void k_probe_mfma(const u32x4_t* ops, int n_ops, int iters,
                                                                    float* sink) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gw = blockIdx.x * kProbeWaves + wave;
    u32x4_t f[kProbeFrags];
#pragma unroll
    for (int i = 0; i < kProbeFrags; ++i) f[i] = ops[(int64_t(gw) * kProbeFrags * 64 + i * 64 + lane) % n_ops];
    f32x16_t acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = f32x16_t{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int n = 0; n < 4; ++n)
                    acc[m * 4 + n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8_t, f[s * 8 + m]), __builtin_bit_cast(bf16x8_t, f[s * 8 + 4 + n]),
                        acc[m * 4 + n], 0, 0, 0);
    }
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
        for (int e = 0; e < 16; ++e) sum += acc[k][e];
    sum = wave_sum(sum);
    if (lane == 0) sink[gw] = sum;  // keeps the products live
}

}  // namespace
}  // namespace mfsdp

using namespace mfsdp;

extern "C" mfsdp_status mfsdp_probe_mfma_bf16(const void* operands, uint64_t operand_bytes, int32_t blocks,
                                              int32_t iters, float* sink, void* stream, double* flops) {
    clear_error();
    if (!operands || !sink) return fail(MFSDP_ERR_INVALID_ARGUMENT, "NULL operands or sink");
    if (operand_bytes < 1024 || operand_bytes % 16 != 0 || reinterpret_cast<uintptr_t>(operands) % 16 != 0)
        return fail(MFSDP_ERR_INVALID_ARGUMENT, "operands: at least 1024 bytes, 16-byte aligned, a multiple of 16");
    if (blocks < 1 || blocks > 65536 || iters < 1) return fail(MFSDP_ERR_INVALID_ARGUMENT, "blocks in 1..65536, iters >= 1");
    const uint64_t n_ops = operand_bytes / 16;
    if (n_ops > uint64_t(INT32_MAX)) return fail(MFSDP_ERR_INVALID_ARGUMENT, "operands above 32 GiB");
    k_probe_mfma<<<dim3(blocks), dim3(64 * kProbeWaves), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4_t*>(operands), int(n_ops), iters, sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MFSDP_ERR_HIP, std::string("probe launch: ") + hipGetErrorString(e));
    if (flops) *flops = double(blocks) * kProbeWaves * double(iters) * 32.0 * (32.0 * 32.0 * 16.0 * 2.0);
    return MFSDP_OK;
}

// ---------------------------------------------------------------------------
// HBM streaming rates: read only, write only, and copy (half read, half
// written), 16-byte accesses: each block walks contiguous 32 KB chunks
// (chunk b, b + blocks, ...), each thread 8 accesses in flight, a wave's
// access covering 1 KB of consecutive bytes.  The elementwise phases move as many bytes in as out (momentum:
// 6 B read and 6 B written per bf16 element), so the copy rate is their
// ceiling on this part, below the published 8 TB/s.
namespace mfsdp {
namespace {

constexpr int kHbmBlocks = 2048, kHbmThreads = 256, kHbmUnroll = 8;

__global__ __launch_bounds__(kHbmThreads) void k_probe_hbm(u32x4_t* dst, const u32x4_t* src, int64_t n, int mode,
                                                            float* sink) {
    constexpr int64_t kChunk = int64_t(kHbmThreads) * kHbmUnroll;  // 16-byte words per block chunk
    const int64_t t = threadIdx.x;
    uint32_t acc = 0;
    for (int64_t base = int64_t(blockIdx.x) * kChunk; base < n; base += int64_t(gridDim.x) * kChunk) {
        u32x4_t v[kHbmUnroll];
#pragma unroll
        for (int u = 0; u < kHbmUnroll; ++u) {
            const int64_t i = base + u * kHbmThreads + t;
            if (mode != 1 && i < n) v[u] = src[i];
        }
#pragma unroll
        for (int u = 0; u < kHbmUnroll; ++u) {
            const int64_t i = base + u * kHbmThreads + t;
            if (i >= n) continue;
            if (mode == 0)
                acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
            else if (mode == 1)
                dst[i] = u32x4_t{uint32_t(i), 0u, 0u, 0u};
            else
                dst[i] = v[u];
        }
    }
    // keeps the reads live: one value per wave
    const float f = float(acc & 0xffffu);
    const float s = wave_sum(f);
    if ((threadIdx.x & 63) == 0) sink[(blockIdx.x * kHbmThreads + threadIdx.x) / 64] = s;
}

}  // namespace
}  // namespace mfsdp

extern "C" mfsdp_status mfsdp_probe_hbm(void* dst, const void* src, uint64_t bytes, int32_t mode, float* sink,
                                        void* stream) {
    clear_error();
    if (mode < 0 || mode > 2) return fail(MFSDP_ERR_INVALID_ARGUMENT, "mode must be 0 (read), 1 (write) or 2 (copy)");
    if (!sink || (mode != 1 && !src) || (mode != 0 && !dst))
        return fail(MFSDP_ERR_INVALID_ARGUMENT, "NULL buffer");
    if (bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(dst) % 16 != 0)
        return fail(MFSDP_ERR_INVALID_ARGUMENT, "bytes a nonzero multiple of 16, buffers 16-byte aligned");
    k_probe_hbm<<<dim3(kHbmBlocks), dim3(kHbmThreads), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<u32x4_t*>(dst), static_cast<const u32x4_t*>(src), int64_t(bytes / 16), mode, sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MFSDP_ERR_HIP, std::string("probe launch: ") + hipGetErrorString(e));
    return MFSDP_OK;
}
