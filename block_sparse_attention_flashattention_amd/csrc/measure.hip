// What the matrix cores of this device sustain on data shaped like the
// attention operands, for the roofline that the forward is reported against.
//
// The published dense bf16 peak assumes the top shader clock. Under a long
// run of v_mfma_f32_32x32x16_bf16 the clock is set by the power the chip
// draws, and that depends on the operand bits: all-zero operands keep the top
// clock, operands drawn from N(0,1) (as Q, K, V are here) do not. These
// kernels measure it directly:
//   mode 0  every wave issues MFMAs back to back on random bf16 operands
//           (eight operand pairs per wave, four independent accumulators,
//           two waves per SIMD);
//   mode 1  the same with all-zero operands;
//   mode 2  the phase split of the ping-pong forward kernels: on every SIMD
//           one wave issues the MFMAs of mode 0 while the other issues
//           softmax-shaped vector work (fma, exp2, add, max and a bf16 pack,
//           about 4.5 instructions per MFMA of its partner).
// Each wave records its shader cycles (s_memtime) and the constant 100 MHz
// real-time counter (s_memrealtime) around its loop; the host averages the
// ratio into a clock.
#include <hip/hip_runtime.h>

#include <vector>

#include "device_common.h"
#include "vsa_internal.h"

namespace vsa {
namespace {

using namespace dev;

constexpr int kMeasureFragments = 16;  // bf16x8 operand fragments per lane (A and B of 8 pairs)

template <bool ZERO>
__global__ __launch_bounds__(256, 2) void mfma_rate_kernel(const bf16x8* __restrict__ frag,
                                                           unsigned long long* __restrict__ out, int iters) {
    const int tid = threadIdx.x, lane = tid & 63;
    bf16x8 a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = ZERO ? bf16x8{} : frag[(2 * i) * 64 + lane];
        b[i] = ZERO ? bf16x8{} : frag[(2 * i + 1) * 64 + lane];
    }
    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[i], acc[i & 3], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[i][r];
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    const int w = blockIdx.x * 4 + (tid >> 6);
    if (lane == 0) {
        out[3 * w] = c1 - c0;
        out[3 * w + 1] = r1 - r0;
        out[3 * w + 2] = s == 12345.0f;  // keeps the sums, and so every MFMA, alive
    }
}

__global__ __launch_bounds__(512, 1) void mfma_pingpong_kernel(const bf16x8* __restrict__ frag,
                                                               unsigned long long* __restrict__ out, int iters) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float s = 0.0f;
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    if (wave < 4) {
        bf16x8 a[8], b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = frag[(2 * i) * 64 + lane];
            b[i] = frag[(2 * i + 1) * 64 + lane];
        }
        f32x16 acc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[i], acc[i & 3], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += acc[i][r];
    } else {
        // eight scores per iteration: scale and shift, exponential, row sum,
        // row max, and a bf16 pack of every second pair
        float x[8], sum[4] = {0.0f, 0.0f, 0.0f, 0.0f}, mx = -1e30f;
        const float shift = 0.001f * (float)(lane & 7);
        unsigned pk = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = 0.01f * (float)((lane * 7 + k * 13) & 63) - 0.3f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float t = fmaf(x[k], 0.9990234375f, shift);
                const float p = fast_exp2(t - 1.0f);
                sum[k & 3] += p;
                mx = fmaxf(mx, t);
                x[k] = t;
                if (k & 1) pk ^= pack_bf16x2(p, t);
            }
        }
        s = sum[0] + sum[1] + sum[2] + sum[3] + mx + (float)(pk & 1u);
    }
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    const int w = blockIdx.x * 8 + wave;
    if (lane == 0) {
        out[3 * w] = c1 - c0;
        out[3 * w + 1] = r1 - r0;
        out[3 * w + 2] = s == 12345.0f;
    }
}

// bf16 bits of N(0,1) draws (xorshift64 and Box-Muller), round to nearest even
std::vector<uint16_t> normal_bf16(size_t n) {
    std::vector<uint16_t> v(n);
    uint64_t x = 0x9E3779B97F4A7C15ull;
    auto next = [&]() {
        x ^= x << 13;
        x ^= x >> 7;
        x ^= x << 17;
        return (double)(x >> 11) * (1.0 / 9007199254740992.0);
    };
    for (size_t i = 0; i < n; ++i) {
        const double u1 = next() + 1e-300, u2 = next();
        const float f = (float)(__builtin_sqrt(-2.0 * __builtin_log(u1)) * __builtin_cos(6.283185307179586 * u2));
        uint32_t u;
        __builtin_memcpy(&u, &f, 4);
        v[i] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
    }
    return v;
}

}  // namespace

hipError_t measure_mfma(int mode, int iters, hipStream_t stream, float* tflops, float* clock_mhz) {
    const int cus = device_cu_count();
    const int grid = mode == 2 ? cus : 2 * cus;
    const int threads = mode == 2 ? 512 : 256;
    const int waves = grid * threads / 64;
    const int mfma_waves = mode == 2 ? waves / 2 : waves;
    const std::vector<uint16_t> host = normal_bf16((size_t)kMeasureFragments * 64 * 8);
    bf16x8* frag = nullptr;
    unsigned long long* out = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t e = hipMalloc((void**)&frag, host.size() * 2);
    if (e == hipSuccess) e = hipMalloc((void**)&out, (size_t)waves * 3 * sizeof(unsigned long long));
    if (e == hipSuccess) e = hipMemcpy(frag, host.data(), host.size() * 2, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    if (e == hipSuccess) e = hipEventRecord(e0, stream);
    if (e == hipSuccess) {
        if (mode == 2) hipLaunchKernelGGL(mfma_pingpong_kernel, dim3(grid), dim3(threads), 0, stream, frag, out, iters);
        else if (mode == 1) hipLaunchKernelGGL(mfma_rate_kernel<true>, dim3(grid), dim3(threads), 0, stream, frag, out, iters);
        else hipLaunchKernelGGL(mfma_rate_kernel<false>, dim3(grid), dim3(threads), 0, stream, frag, out, iters);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e1, stream);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    std::vector<unsigned long long> h((size_t)waves * 3);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e == hipSuccess) e = hipMemcpy(h.data(), out, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost);
    if (e == hipSuccess) {
        double clk = 0.0;
        int n = 0;
        for (int w = 0; w < waves; ++w) {
            if (h[3 * w + 1] == 0) continue;
            clk += (double)h[3 * w] / ((double)h[3 * w + 1] * 1e-8);  // cycles per second
            ++n;
        }
        const double flops = (double)mfma_waves * iters * 8 * 32768.0;
        *tflops = ms > 0.0f ? (float)(flops / (ms * 1e-3) / 1e12) : 0.0f;
        *clock_mhz = n > 0 ? (float)(clk / n / 1e6) : 0.0f;
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (out) (void)hipFree(out);
    if (frag) (void)hipFree(frag);
    return e;
}

}  // namespace vsa
