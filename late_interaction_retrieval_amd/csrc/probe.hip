// probe.hip -- sustained MFMA rate on this GPU with given operand data, and
// the vector-ALU issue rate.
//
// A measurement aid, not part of MaxSim: every wave of every workgroup runs
// four independent accumulation chains of the same MFMA instruction the
// MaxSim kernels use, on operands read once from a caller buffer, for `iters`
// rounds of eight k-steps.  With random operands the chip's power limit
// lowers the clock well below the one the published peak assumes, so the
// rate measured here is the practical ceiling for the MaxSim contractions.
#include <hip/hip_runtime.h>

#include "maxsim_probe.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 4;
constexpr int kSteps = 8;
constexpr int kThreads = 512;

template <int KIND>
__global__ __launch_bounds__(kThreads) void mfma_loop(const u32x4* ops, float* sink, int iters) {
    const int wave = blockIdx.x * (kThreads / 64) + threadIdx.x / 64;
    const int l = threadIdx.x % 64;
    const u32x4* w = ops + (size_t)wave * 64 * (kSteps + kChains);
    u32x4 a[kSteps], b[kChains];
    for (int s = 0; s < kSteps; ++s) a[s] = w[64 * s + l];
    for (int c = 0; c < kChains; ++c) b[c] = w[64 * (kSteps + c) + l];
    float out = 0.f;
    if constexpr (KIND == MAXSIM_PROBE_I8) {
        i32x4 acc[kChains];
        for (int c = 0; c < kChains; ++c) acc[c] = i32x4{0, 0, 0, 0};
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int s = 0; s < kSteps; ++s)
#pragma unroll
                for (int c = 0; c < kChains; ++c)
                    acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a[s]),
                                                                   __builtin_bit_cast(i32x4, b[c]), acc[c], 0, 0, 0);
        for (int c = 0; c < kChains; ++c)
            for (int e = 0; e < 4; ++e) out += (float)acc[c][e];
    } else {
        f32x16 acc[kChains];
        for (int c = 0; c < kChains; ++c)
            for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int s = 0; s < kSteps; ++s)
#pragma unroll
                for (int c = 0; c < kChains; ++c) {
                    if constexpr (KIND == MAXSIM_PROBE_F16) {
                        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[s]),
                                                                        __builtin_bit_cast(f16x8, b[c]), acc[c], 0, 0, 0);
                    } else {
                        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[s]),
                                                                         __builtin_bit_cast(bf16x8, b[c]), acc[c], 0, 0, 0);
                    }
                }
        for (int c = 0; c < kChains; ++c)
            for (int e = 0; e < 16; ++e) out += acc[c][e];
    }
    sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = out;
}

// Vector-ALU issue rate: every thread runs kValuChains independent chains of
// fp32 fused multiply-adds (one v_fmac_f32 each, no packed instructions).
constexpr int kValuChains = 8;

__global__ __launch_bounds__(kThreads) void valu_loop(const float* ops, float* sink, int iters) {
    const size_t t = (size_t)blockIdx.x * kThreads + threadIdx.x;
    const float a = ops[t & 1023], b = ops[(t + 512) & 1023];
    float x[kValuChains];
#pragma unroll
    for (int c = 0; c < kValuChains; ++c) x[c] = ops[(t + 64 * c) & 1023];
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
#pragma unroll
            for (int c = 0; c < kValuChains; ++c) x[c] = __builtin_fmaf(x[c], a, b);
    float out = 0.f;
#pragma unroll
    for (int c = 0; c < kValuChains; ++c) out += x[c];
    sink[t] = out;
}

// Plain streaming read: every thread reads 16-byte chunks t, t + nthreads, ...
// of the buffer and writes the XOR of what it read to `sink` (so no load is
// dropped).
__global__ __launch_bounds__(256) void read_loop(const u32x4* buf, long long n16, unsigned* sink) {
    const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long stride = (long long)gridDim.x * 256;
    u32x4 x = u32x4{0u, 0u, 0u, 0u};
    for (long long k = t; k < n16; k += stride) x ^= buf[k];
    sink[t] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

}  // namespace

extern "C" {

int maxsim_probe_read(const void* buf, size_t bytes, int32_t blocks, unsigned* sink, void* stream) {
    if (!buf || !sink) return 1;
    if (blocks < 1 || bytes < 16 || (bytes & 15)) return 2;
    hipLaunchKernelGGL(read_loop, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(buf), (long long)(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}

double maxsim_probe_valu_lane_ops_per_launch(int32_t blocks, int32_t iters) {
    if (blocks < 1 || iters < 1) return 0.0;
    return (double)blocks * kThreads * iters * kSteps * kValuChains;
}

int maxsim_probe_valu(const float* operands, int32_t blocks, int32_t iters, float* sink, void* stream) {
    if (!operands || !sink) return 1;
    if (blocks < 1 || iters < 1) return 2;
    hipLaunchKernelGGL(valu_loop, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), operands, sink,
                       iters);
    return hipGetLastError() == hipSuccess ? 0 : 6;
}

size_t maxsim_probe_operand_bytes(int32_t blocks) {
    if (blocks < 1) return 0;
    return (size_t)blocks * (kThreads / 64) * 64 * (kSteps + kChains) * sizeof(u32x4);
}

double maxsim_probe_ops_per_launch(int32_t kind, int32_t blocks, int32_t iters) {
    if (blocks < 1 || iters < 1) return 0.0;
    // 32x32x16 and 16x16x64 are both 16384 multiply-adds per instruction
    (void)kind;
    return (double)blocks * (kThreads / 64) * iters * kSteps * kChains * 2.0 * 16384.0;
}

int maxsim_probe_mfma(int32_t kind, const void* operands, int32_t blocks, int32_t iters, float* sink, void* stream) {
    if (!operands || !sink) return 1;
    if (blocks < 1 || iters < 1) return 2;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4* ops = static_cast<const u32x4*>(operands);
    switch (kind) {
        case MAXSIM_PROBE_F16:
            hipLaunchKernelGGL(mfma_loop<MAXSIM_PROBE_F16>, dim3(blocks), dim3(kThreads), 0, s, ops, sink, iters);
            break;
        case MAXSIM_PROBE_BF16:
            hipLaunchKernelGGL(mfma_loop<MAXSIM_PROBE_BF16>, dim3(blocks), dim3(kThreads), 0, s, ops, sink, iters);
            break;
        case MAXSIM_PROBE_I8:
            hipLaunchKernelGGL(mfma_loop<MAXSIM_PROBE_I8>, dim3(blocks), dim3(kThreads), 0, s, ops, sink, iters);
            break;
        default:
            return 3;
    }
    return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // extern "C"
