// Calibration kernel for the benchmark: how fast can an MI355X run the GEMM's
// inner loop -- v_mfma_f32_16x16x32_f16 fed by ds_read_b128 fragment reads,
// one wave per SIMD -- with no global memory traffic at all, for random and
// for constant fp16 operands?  The board's power limit sets the answer for
// random data (page "6. Register Reallocation, Multicast, and a Persistent
// Kernel" of the Tilus "Hopper matmul" pages warns, in its Warning, that an
// 8192^3 fp16 GEMM runs against the board's power budget): the ratio of the
// GEMM's throughput to this loop's is the share of the reachable rate it
// attains.  Not part of the GEMM library (libgemm_f16_calib.so).
//
// Each wave owns an FB x FB grid of 16x16 result blocks (FB = 4: 16 MFMAs
// per K step from 8 fragment reads, 64 accumulators; FB = 8: 64 MFMAs from
// 16 reads, all 256 AGPRs, the ratio of the GEMM's 128 x 128 wave tile).
// Fragments for the next K step are read while the current step's MFMAs
// run, from eight fragment sets in LDS (FB A and FB B fragments of 1 KB
// each) that the steps cycle through, so every MFMA sees new operands.  The LDS holds random fp16 values, uniform in
// [-1, 1) / sqrt(8192) like the benchmark's inputs, or one constant value of
// that size.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace gemm_f16_calib {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int LDS_BYTES = 128 * 1024;  // more than half the CU's LDS: one workgroup per CU
constexpr int SETS = 8;                 // fragment sets the K steps cycle through

__device__ __forceinline__ uint32_t mix(uint32_t h)
{
    h ^= h >> 16;
    h *= 0x7feb352du;
    h ^= h >> 15;
    h *= 0x846ca68bu;
    h ^= h >> 16;
    return h;
}

template <int FB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_loop_kernel(float *out, int32_t iters, int32_t constant)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];
    // operand values: SETS sets x (FB A + FB B fragments) x 64 lanes x 16 B
    constexpr int FRAG_BYTES = 64 * 16;
    constexpr int SET_SPAN = 2 * FB * FRAG_BYTES;
    static_assert(SETS * SET_SPAN <= LDS_BYTES, "fragment sets fit the LDS");
    _Float16 *h = reinterpret_cast<_Float16 *>(lds);
    for (int e = threadIdx.x; e < SETS * SET_SPAN / 2; e += blockDim.x) {
        float v = 0.011048543f;   // 1 / sqrt(8192)
        if (!constant) {
            const uint32_t r = mix(static_cast<uint32_t>(e) * 2654435761u + blockIdx.x * 40503u);
            v *= static_cast<float>(static_cast<int32_t>(r)) * (1.0f / 2147483648.0f);
        }
        h[e] = static_cast<_Float16>(v);
    }
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // each wave starts on its own set, so the four SIMDs do not read alike
    auto frag = [&](int set, int which, int i) {
        return *reinterpret_cast<const half8_t *>(
            lds + ((set + wave) % SETS) * SET_SPAN + (which * FB + i) * FRAG_BYTES + lane * 16);
    };
    f32x4_t acc[FB][FB];
#pragma unroll
    for (int i = 0; i < FB; ++i)
#pragma unroll
        for (int j = 0; j < FB; ++j) {
            acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            asm volatile("" : "+a"(acc[i][j]));
        }
    asm volatile("s_nop 4");   // VALU writes of the accumulators -> first MFMA
    half8_t af[2][FB], bf[2][FB];
#pragma unroll
    for (int i = 0; i < FB; ++i) {
        af[0][i] = frag(0, 0, i);
        bf[0][i] = frag(0, 1, i);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int kk = 0; kk < SETS; ++kk) {
            const int cur = kk & 1, nxt = cur ^ 1;
            constexpr int NM = FB * FB;
#pragma unroll
            for (int t = 0; t < NM; ++t) {
                // column by column, boustrophedon: consecutive MFMAs share B
                const int j = t / FB;
                const int i = (j & 1) ? FB - 1 - t % FB : t % FB;
                asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0"
                             : "+a"(acc[i][j]) : "v"(bf[cur][j]), "v"(af[cur][i]));
                // next step's fragments over the first half of the step
                const int r = t * 2 * FB / (NM / 2);
                if (t < NM / 2 && (t * 2 * FB) % (NM / 2) == 0) {
                    if (r < FB)
                        af[nxt][r] = frag(kk + 1, 0, r);
                    else
                        bf[nxt][r - FB] = frag(kk + 1, 1, r - FB);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");   // last MFMA -> reads of its result
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < FB; ++i)
#pragma unroll
        for (int j = 0; j < FB; ++j) {
            asm volatile("" : "+a"(acc[i][j]));
            s += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
        }
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace gemm_f16_calib

// fb: 4 or 8 (result blocks per wave side); constant: 0 random operands, 1
// one constant value; iters: trips of 8 K steps; grid workgroups of 256
// threads (4 waves, one per SIMD; one workgroup per CU); out: device buffer of
// grid * 256 floats (the accumulators' sums, so no work is dead).  Returns 0,
// 1 for bad arguments, 3 if the launch fails.  Flops per launch:
// grid * 4 * iters * 8 * fb * fb * 16384.
extern "C" int gemm_f16_calib_mfma_loop(int32_t fb, int32_t constant, int32_t iters, int32_t grid,
                                        float *out, hipStream_t stream)
{
    if ((fb != 4 && fb != 8) || iters < 1 || grid < 1 || !out) return 1;
    void *args[] = {&out, &iters, &constant};
    const void *fn = fb == 4 ? reinterpret_cast<const void *>(&gemm_f16_calib::mfma_loop_kernel<4>)
                             : reinterpret_cast<const void *>(&gemm_f16_calib::mfma_loop_kernel<8>);
    return hipLaunchKernel(fn, dim3(grid), dim3(256), args, 0, stream) == hipSuccess ? 0 : 3;
}
