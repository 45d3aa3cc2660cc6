// fz_probe.hip -- measured integer VALU issue rates of the GPU
// (libfz_probe.so).
//
// The extension and local kernels are bound by integer VALU issue (adds,
// maxima, compares; no matrix cores): 32-bit lanes, or two 16-bit values
// per lane in the packed layouts of the extension.  Their roofline uses the
// peak from unit counts and clock (256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz,
// twice that for packed 16-bit operations); this probe measures what a
// plain add/max stream reaches on the part, so the two can be compared.
// Each lane runs eight independent chains of v_add_u32 / v_max_i32, or of
// v_pk_add_u16 / v_pk_max_i16 (two operations each), written in inline
// assembly (the compiler cannot fold them), eight waves per SIMD, timed
// with HIP events.  Not part of the alignment library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int PROBE_BLOCK = 256;
constexpr int OPS_PER_ITER = 16;

template <bool PK>
__global__ __launch_bounds__(PROBE_BLOCK) void valu_probe_kernel(int iters, uint32_t seed, uint32_t *out)
{
    uint32_t a0 = threadIdx.x ^ seed, a1 = a0 + 1, a2 = a0 + 2, a3 = a0 + 3;
    uint32_t a4 = a0 + 4, a5 = a0 + 5, a6 = a0 + 6, a7 = a0 + 7;
    const uint32_t b = blockIdx.x | 1u;
    for (int i = 0; i < iters; ++i) {
        if (PK) {
            asm volatile(
                "v_pk_add_u16 %0, %0, %8\n\t"
                "v_pk_add_u16 %1, %1, %8\n\t"
                "v_pk_add_u16 %2, %2, %8\n\t"
                "v_pk_add_u16 %3, %3, %8\n\t"
                "v_pk_add_u16 %4, %4, %8\n\t"
                "v_pk_add_u16 %5, %5, %8\n\t"
                "v_pk_add_u16 %6, %6, %8\n\t"
                "v_pk_add_u16 %7, %7, %8\n\t"
                "v_pk_max_i16 %0, %0, %1\n\t"
                "v_pk_max_i16 %1, %1, %2\n\t"
                "v_pk_max_i16 %2, %2, %3\n\t"
                "v_pk_max_i16 %3, %3, %4\n\t"
                "v_pk_max_i16 %4, %4, %5\n\t"
                "v_pk_max_i16 %5, %5, %6\n\t"
                "v_pk_max_i16 %6, %6, %7\n\t"
                "v_pk_max_i16 %7, %7, %0"
                : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
                : "v"(b));
            continue;
        }
        asm volatile(
            "v_add_u32 %0, %0, %8\n\t"
            "v_add_u32 %1, %1, %8\n\t"
            "v_add_u32 %2, %2, %8\n\t"
            "v_add_u32 %3, %3, %8\n\t"
            "v_add_u32 %4, %4, %8\n\t"
            "v_add_u32 %5, %5, %8\n\t"
            "v_add_u32 %6, %6, %8\n\t"
            "v_add_u32 %7, %7, %8\n\t"
            "v_max_i32 %0, %0, %1\n\t"
            "v_max_i32 %1, %1, %2\n\t"
            "v_max_i32 %2, %2, %3\n\t"
            "v_max_i32 %3, %3, %4\n\t"
            "v_max_i32 %4, %4, %5\n\t"
            "v_max_i32 %5, %5, %6\n\t"
            "v_max_i32 %6, %6, %7\n\t"
            "v_max_i32 %7, %7, %0"
            : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7)
            : "v"(b));
    }
    out[(size_t)blockIdx.x * PROBE_BLOCK + threadIdx.x] = a0 ^ a1 ^ a2 ^ a3 ^ a4 ^ a5 ^ a6 ^ a7;
}

template <bool PK>
int run_probe(int device, int waves_per_simd, int iters, float *ms, double *lane_ops)
{
    if (hipSetDevice(device) != hipSuccess) return -1;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return -1;
    const int blocks = prop.multiProcessorCount * waves_per_simd;     // 4 waves per block: one per SIMD
    uint32_t *out = nullptr;
    if (hipMalloc(&out, (size_t)blocks * PROBE_BLOCK * sizeof(uint32_t)) != hipSuccess) return -1;
    hipEvent_t e0, e1;
    (void)hipEventCreate(&e0);
    (void)hipEventCreate(&e1);
    valu_probe_kernel<PK><<<blocks, PROBE_BLOCK>>>(iters / 8 + 1, 1u, out);     // warm-up
    (void)hipEventRecord(e0, nullptr);
    valu_probe_kernel<PK><<<blocks, PROBE_BLOCK>>>(iters, 1u, out);
    (void)hipEventRecord(e1, nullptr);
    const hipError_t err = hipEventSynchronize(e1);
    float t = 0.f;
    (void)hipEventElapsedTime(&t, e0, e1);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    (void)hipFree(out);
    if (err != hipSuccess) return -1;
    *ms = t;
    *lane_ops = (double)blocks * PROBE_BLOCK * (double)iters * OPS_PER_ITER * (PK ? 2 : 1);
    return 0;
}

}  // namespace

extern "C" {

// Runs the probe on `device` (waves_per_simd waves on every SIMD, `iters`
// loop trips of 16 instructions per lane) and reports the kernel's time and
// the operations it issued (32-bit lane operations).  Returns 0, or -1 on a
// HIP error.
int fz_probe_valu(int device, int waves_per_simd, int iters, float *ms, double *lane_ops)
{
    return run_probe<false>(device, waves_per_simd, iters, ms, lane_ops);
}

// The same with packed 16-bit instructions; *ops counts 16-bit operations
// (two per lane per instruction).
int fz_probe_valu_pk16(int device, int waves_per_simd, int iters, float *ms, double *ops)
{
    return run_probe<true>(device, waves_per_simd, iters, ms, ops);
}

}  // extern "C"
