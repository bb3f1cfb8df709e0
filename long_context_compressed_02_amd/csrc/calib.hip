// calib.hip -- on-device calibration kernels for the benchmark's roofline
// (measurement infrastructure, built as its own library libdsv4calib.so; the
// attention library neither links nor calls it).
//
//   copy   dst <- src, 16 bytes per thread per iteration (grid-stride)
//   read   a wave-reduced XOR of src (each byte read once; one word per
//          wave written so the reads are not removed)
//   mfma   every wave issues back-to-back independent matrix instructions on
//          register operands: bf16 16x16x32, fp8 (E4M3) 16x16x128 and fp4
//          (E2M1) 16x16x128 through the scaled f8f6f4 instruction
//
// Each entry point launches, waits for the device and returns the measured
// rate; the time is taken with HIP events around the launches (the first
// launch is an untimed warm-up).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void k_calib_copy(const uint4 *__restrict__ src, uint4 *__restrict__ dst, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void k_calib_read(const uint4 *__restrict__ src, int64_t n, uint32_t *sink) {
    uint32_t x = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const uint4 v = src[i];
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    for (int o = 32; o >= 1; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
    if ((threadIdx.x & 63) == 0) sink[(blockIdx.x * 4 + (threadIdx.x >> 6)) & 1023] = x;
}

// kind 0: bf16 16x16x32 (16384 flop), 1: fp8 16x16x128 (65536 flop),
// 2: fp4 16x16x128 (65536 flop), 3: bf16 32x32x16 (32768 flop), 4: fp8
// 32x32x64 (131072 flop).  8 independent accumulators per wave.
template <int KIND>
__global__ __launch_bounds__(256) void k_calib_mfma(float *out, int iters, int seed) {
    const int lane = threadIdx.x & 63;
    f32x4 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (KIND == 0) {
        bf16x8 a, b;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            a[j] = (__bf16)(float)((lane + j + seed) & 7);
            b[j] = (__bf16)(float)((lane * 3 + j) & 7);
        }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
        }
    } else {
        i32x8 a, b;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            a[j] = 0x38383838 ^ ((lane + j + seed) & 0x07070707);
            b[j] = 0x30303030 ^ ((lane * 3 + j) & 0x07070707);
        }
        constexpr int FMT = KIND == 1 ? 0 : 4;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[i], FMT, FMT, 0, 127, 0, 127);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

template <int KIND>
__global__ __launch_bounds__(256) void k_calib_mfma32(float *out, int iters, int seed) {
    const int lane = threadIdx.x & 63;
    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[i][j] = 0.0f;
    if constexpr (KIND == 3) {
        bf16x8 a, b;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            a[j] = (__bf16)(float)((lane + j + seed) & 7);
            b[j] = (__bf16)(float)((lane * 3 + j) & 7);
        }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
        }
    } else {
        i32x8 a, b;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            a[j] = 0x38383838 ^ ((lane + j + seed) & 0x07070707);
            b[j] = 0x30303030 ^ ((lane * 3 + j) & 0x07070707);
        }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[i], 0, 0, 0, 127, 0, 127);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 16; ++j) s += acc[i][j];
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

static float time_ms(hipEvent_t a, hipEvent_t b) {
    float ms = 0.0f;
    hipEventSynchronize(b);
    hipEventElapsedTime(&ms, a, b);
    return ms;
}

extern "C" {

// GB/s of a copy of `bytes` (a multiple of 16; bytes read + bytes written
// counted), best of `reps` timed launches.  Returns < 0 on a HIP error.
double dsv4calib_copy_gbs(const void *src, void *dst, int64_t bytes, int reps) {
    const int64_t n = bytes / 16;
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return -1.0;
    const int grid = 256 * 8;
    double best = 0.0;
    for (int r = 0; r <= reps; ++r) {
        hipEventRecord(a, 0);
        hipLaunchKernelGGL(k_calib_copy, dim3(grid), dim3(256), 0, 0, (const uint4 *)src, (uint4 *)dst, n);
        hipEventRecord(b, 0);
        const float ms = time_ms(a, b);
        if (hipGetLastError() != hipSuccess) return -1.0;
        if (r > 0 && ms > 0.0f) {
            const double gbs = 2.0 * (double)bytes / (ms * 1e-3) / 1e9;
            best = gbs > best ? gbs : best;
        }
    }
    hipEventDestroy(a);
    hipEventDestroy(b);
    return best;
}

// GB/s of reading `bytes` once (sink: 4096 bytes of device scratch).
double dsv4calib_read_gbs(const void *src, int64_t bytes, void *sink, int reps) {
    const int64_t n = bytes / 16;
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return -1.0;
    const int grid = 256 * 8;
    double best = 0.0;
    for (int r = 0; r <= reps; ++r) {
        hipEventRecord(a, 0);
        hipLaunchKernelGGL(k_calib_read, dim3(grid), dim3(256), 0, 0, (const uint4 *)src, n, (uint32_t *)sink);
        hipEventRecord(b, 0);
        const float ms = time_ms(a, b);
        if (hipGetLastError() != hipSuccess) return -1.0;
        if (r > 0 && ms > 0.0f) {
            const double gbs = (double)bytes / (ms * 1e-3) / 1e9;
            best = gbs > best ? gbs : best;
        }
    }
    hipEventDestroy(a);
    hipEventDestroy(b);
    return best;
}

// TFLOP/s of back-to-back matrix instructions: kind 0 bf16, 1 fp8, 2 fp4
// (16x16), 3 bf16, 4 fp8 (32x32);
// `blocks` workgroups of 4 waves (out: blocks*256 floats of device scratch).
double dsv4calib_mfma_tflops(int kind, int blocks, int iters, void *out, int reps) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return -1.0;
    const double per = kind == 0 ? 16384.0 : kind == 3 ? 32768.0 : kind == 4 ? 131072.0 : 65536.0;
    double best = 0.0;
    for (int r = 0; r <= reps; ++r) {
        hipEventRecord(a, 0);
        if (kind == 0) hipLaunchKernelGGL(k_calib_mfma<0>, dim3(blocks), dim3(256), 0, 0, (float *)out, iters, r);
        else if (kind == 1) hipLaunchKernelGGL(k_calib_mfma<1>, dim3(blocks), dim3(256), 0, 0, (float *)out, iters, r);
        else if (kind == 2) hipLaunchKernelGGL(k_calib_mfma<2>, dim3(blocks), dim3(256), 0, 0, (float *)out, iters, r);
        else if (kind == 3) hipLaunchKernelGGL(k_calib_mfma32<3>, dim3(blocks), dim3(256), 0, 0, (float *)out, iters, r);
        else hipLaunchKernelGGL(k_calib_mfma32<4>, dim3(blocks), dim3(256), 0, 0, (float *)out, iters, r);
        hipEventRecord(b, 0);
        const float ms = time_ms(a, b);
        if (hipGetLastError() != hipSuccess) return -1.0;
        if (r > 0 && ms > 0.0f) {
            const double tf = (double)blocks * 4.0 * iters * 8.0 * per / (ms * 1e-3) / 1e12;
            best = tf > best ? tf : best;
        }
    }
    hipEventDestroy(a);
    hipEventDestroy(b);
    return best;
}

}  // extern "C"
