// k_rf.hip -- positive random features of liblinattn.
//
// For rows x_i in R^d and projections w_r in R^d (r < m):
//   f_i[r] = exp(w_r . x_i - |x_i|^2 / 2) / sqrt(m)
// so that f(q) . f(k) estimates exp(q . k) without bias when the w_r are standard normal, with
// every feature positive ("Linear Attention Math", section "Feature maps: elu+1 and positive
// random features"; "线性注意力从头到尾讲清楚", section 9 on Performer). Attention over the
// features is the identity-phi form of the attention kernels. The projections are an input:
// the library draws no random numbers.
//
// Matrix-core kernel (bf16, d in {64, 128}, m in {64, 128, 256}): the dots W x_i are one
// [m x d] x [d x rows] product. Wave w of a 4-wave workgroup keeps the bf16 fragments of its
// m/4 projections in registers for the whole launch and sweeps blocks of 64 rows; the x rows are
// read straight from HBM as the B operand (lane li reads row li, 16 bytes per k block), so no
// LDS is needed. |x_i|^2 is summed in float32 from the same registers. The exponent runs as
// exp2 with log2(e) folded into one fused multiply-add per feature.
#include "la_device.h"
#include "la_launch.h"

#include <math.h>

namespace la {
namespace {

constexpr int RB = 64; // rows per block of the sweep

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D, int M>
__global__ __launch_bounds__(256) void k_rf_mfma(const uint16_t *__restrict__ x,
                                                 const uint16_t *__restrict__ W,
                                                 uint16_t *__restrict__ f, long rows,
                                                 float neg_half_log2m)
{
    constexpr int NKB = D / 32;     // k blocks of 32 features
    constexpr int MT = M / 64;      // 16-projection tiles per wave
    constexpr float LOG2E = 1.44269504088896341f;
    const int l = threadIdx.x & 63, li = l & 15, g = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int f0 = w * (M / 4);

    // A operand: projection row f0 + 16 mt + li, k-slots 8g..8g+7 of block kk
    bf16x8 wa[MT][NKB];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk)
            wa[mt][kk] = *reinterpret_cast<const bf16x8 *>(W + (size_t)(f0 + 16 * mt + li) * D + 32 * kk + 8 * g);

    const long nblk = (rows + RB - 1) / RB;
    for (long blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        const long r0 = blk * RB;
        // B operand of the four 16-row tiles: row r0 + 16s + li (clamped to the last row, so
        // every load is in bounds), k-slots 8g..8g+7 of block kk
        u32x4 xb[4][NKB];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const long r = min(r0 + 16 * s + li, rows - 1);
#pragma unroll
            for (int kk = 0; kk < NKB; ++kk)
                xb[s][kk] = *reinterpret_cast<const u32x4 *>(x + r * D + 32 * kk + 8 * g);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            float n = 0.f;
#pragma unroll
            for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const float a = bf_lo(xb[s][kk][h]), b = bf_hi(xb[s][kk][h]);
                    n = fmaf(a, a, n);
                    n = fmaf(b, b, n);
                }
            n += __shfl_xor(n, 16, 64);
            n += __shfl_xor(n, 32, 64);
            // exponent in base 2: (dot - n / 2) log2(e) - log2(m) / 2
            const float bias = fmaf(-0.5f * LOG2E, n, neg_half_log2m);
            const long r = r0 + 16 * s + li;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < NKB; ++kk)
                    c = mfma16(wa[mt][kk], __builtin_bit_cast(bf16x8, xb[s][kk]), c);
                // c[j] = w_{f0 + 16 mt + 4g + j} . x_r
                float e[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    e[j] = __builtin_amdgcn_exp2f(fmaf(c[j], LOG2E, bias));
                if (r < rows) {
                    const u32x2 o = {pack_bf2(e[0], e[1]), pack_bf2(e[2], e[3])};
                    *reinterpret_cast<u32x2 *>(f + r * M + f0 + 16 * mt + 4 * g) = o;
                }
            }
        }
    }
}

// Any dtype and shape (d <= 256): a block of 32 rows, x staged in LDS as float32, one output
// element per thread step with consecutive threads on consecutive features (coalesced
// stores); projections read from global memory (L1/L2-resident: m x d elements shared by all
// blocks). float32 arithmetic, accurate expf.
constexpr int GR = 32;
constexpr int DMAX = 256;

template <typename T>
__global__ __launch_bounds__(256) void k_rf_generic(const T *__restrict__ x, const T *__restrict__ W,
                                                    T *__restrict__ f, long rows, int d, int m,
                                                    float inv_sqrt_m)
{
    __shared__ float sx[GR][DMAX + 1];
    __shared__ float sn[GR];
    const int tid = threadIdx.x;
    const long r0 = (long)blockIdx.x * GR;
    const int nr = (int)min((long)GR, rows - r0);
    for (int e = tid; e < nr * d; e += 256) {
        const int i = e / d, j = e % d;
        sx[i][j] = Elem<T>::ld(x, (size_t)(r0 + i) * d + j);
    }
    __syncthreads();
    if (tid < nr) {
        float n = 0.f;
        for (int j = 0; j < d; ++j)
            n = fmaf(sx[tid][j], sx[tid][j], n);
        sn[tid] = n;
    }
    __syncthreads();
    for (long e = tid; e < (long)nr * m; e += 256) {
        const int i = (int)(e / m), r = (int)(e % m);
        float dot = 0.f;
        for (int j = 0; j < d; ++j)
            dot = fmaf(Elem<T>::ld(W, (size_t)r * d + j), sx[i][j], dot);
        Elem<T>::st(f, (size_t)(r0 + i) * m + r, expf(dot - 0.5f * sn[i]) * inv_sqrt_m);
    }
}

template <int D, int M>
void launch_rf(const void *x, const void *W, void *f, long rows, hipStream_t st)
{
    const long nblk = (rows + RB - 1) / RB;
    const unsigned grid = (unsigned)(nblk < 2048 ? nblk : 2048);
    hipLaunchKernelGGL((k_rf_mfma<D, M>), dim3(grid), dim3(256), 0, st,
                       static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(W),
                       static_cast<uint16_t *>(f), rows, -0.5f * log2f((float)M));
}

} // namespace

bool rf_mfma_ok(bool bf16, int d, int m)
{
    return bf16 && (d == 64 || d == 128) && (m == 64 || m == 128 || m == 256);
}

int rf_max_d() { return DMAX; }

hipError_t rf_features(bool bf16, const void *x, const void *W, void *f, long rows, int d, int m,
                       hipStream_t st)
{
    if (rf_mfma_ok(bf16, d, m)) {
#define LA_RF(DD, MM)                                                                           \
    if (d == DD && m == MM) {                                                                   \
        launch_rf<DD, MM>(x, W, f, rows, st);                                                   \
        return hipGetLastError();                                                               \
    }
        LA_RF(64, 64) LA_RF(64, 128) LA_RF(64, 256) LA_RF(128, 64) LA_RF(128, 128) LA_RF(128, 256)
#undef LA_RF
    }
    const dim3 grid((unsigned)((rows + GR - 1) / GR));
    const float s = 1.0f / sqrtf((float)m);
    if (bf16)
        hipLaunchKernelGGL(k_rf_generic<bf16_t>, grid, dim3(256), 0, st,
                           static_cast<const bf16_t *>(x), static_cast<const bf16_t *>(W),
                           static_cast<bf16_t *>(f), rows, d, m, s);
    else
        hipLaunchKernelGGL(k_rf_generic<float>, grid, dim3(256), 0, st,
                           static_cast<const float *>(x), static_cast<const float *>(W),
                           static_cast<float *>(f), rows, d, m, s);
    return hipGetLastError();
}

} // namespace la
