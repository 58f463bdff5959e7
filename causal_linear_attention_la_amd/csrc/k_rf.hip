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
// [m x d] x [d x rows] product. Each workgroup copies W into LDS once, in fragment order (the
// 16 bytes lane l reads for projection tile mt and k block kk sit at ((mt * NKB + kk) * 64 + l)
// * 16, so every operand read is one contiguous, conflict-free 1 KiB). The projections are
// placed in the tiles so that lane group g of the product holds features (m/4) g .. (m/4) g +
// m/4 - 1 of its row: two tiles give 8 consecutive features, one 16-byte store. Each wave then
// sweeps tiles of 16 rows: it reads the rows straight from HBM as the B operand (lane li reads
// row li, 16 bytes per k block; the next tile is loaded while the current one is computed), so
// every row is read from HBM once and by one wave, and computes all m features of its rows.
// |x_i|^2 is summed in float32 from the same registers. The exponent runs as exp2 with log2(e)
// folded into one fused multiply-add per feature. A wave's 16 x m feature tile goes through a
// wave-private LDS tile before it is stored, so each store instruction writes whole rows (1 KiB
// of consecutive memory) rather than 16-byte pieces of 16 rows: stored straight from the
// product, the pieces kept the texture addresser waiting on the L1 and the kernel took 37 us
// per 2 x 16 x 8192 x 128 tensor instead of 29 (measured on MI355X).
#include "la_device.h"
#include "la_launch.h"

#include <math.h>

namespace la {
namespace {

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D, int M, int NTH>
__global__ __launch_bounds__(NTH) void k_rf_mfma(const uint16_t *__restrict__ x,
                                                 const uint16_t *__restrict__ W,
                                                 uint16_t *__restrict__ f, long rows,
                                                 float neg_half_log2m)
{
    constexpr int NKB = D / 32;     // k blocks of 32 features
    constexpr int MT = M / 16;      // 16-projection tiles
    constexpr float LOG2E = 1.44269504088896341f;
    constexpr int FS = M + 8;       // row stride (elements) of a wave's feature tile
    constexpr int LPR = M / 8;      // lanes per row when a tile is stored (16 bytes each)
    constexpr int NW = NTH / 64;    // waves per workgroup
    __shared__ __attribute__((aligned(16))) uint16_t sW[M * D];
    __shared__ __attribute__((aligned(16))) uint16_t sF[NW][16 * FS];
    const int tid = threadIdx.x, l = tid & 63, li = l & 15, g = l >> 4;
    uint16_t *tileF = sF[tid >> 6];

    const long ntile = (rows + 15) / 16;
    const long nwave = (long)gridDim.x * NW;
    const long w0 = (long)blockIdx.x * NW + (tid >> 6);
    // B operand of a 16-row tile: row 16 t + li (clamped to the last row: every load is in
    // bounds), k-slots 8g..8g+7 of block kk
    auto load = [&](u32x4 (&dst)[NKB], long t) {
        const long r = min(16 * t + li, rows - 1);
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk)
            dst[kk] = *reinterpret_cast<const u32x4 *>(x + r * D + 32 * kk + 8 * g);
    };
    u32x4 xb[NKB], xn[NKB];
    load(xb, min(w0, ntile - 1));
    // W (row-major [M][D]) -> LDS in fragment order: granule (row r, columns 8c..8c+7) is lane
    // (c % 4) * 16 + (row of r in its tile) of fragment (tile of r, kk = c / 4)
    for (int e = tid; e < M * D / 8; e += NTH) {
        const int r = e / (D / 8), c = e % (D / 8);
        // projection r = (M/4) g + 4 mt + j sits in row 4g + j of tile mt, so that lane group g
        // of the product holds the M/4 consecutive features (M/4) g .. of its row
        const int gq = r / (M / 4), mt = (r % (M / 4)) / 4, j = r % 4;
        const int frag = mt * NKB + c / 4, lane = (c % 4) * 16 + 4 * gq + j;
        *reinterpret_cast<u32x4 *>(sW + (frag * 64 + lane) * 8) =
            *reinterpret_cast<const u32x4 *>(W + (size_t)r * D + 8 * c);
    }
    __syncthreads();

    for (long t = w0; t < ntile; t += nwave) {
        load(xn, min(t + nwave, ntile - 1)); // next tile (a re-read of the last one at the end)
        float n = 0.f;
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk)
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float a = bf_lo(xb[kk][h]), b = bf_hi(xb[kk][h]);
                n = fmaf(a, a, n);
                n = fmaf(b, b, n);
            }
        n += __shfl_xor(n, 16, 64);
        n += __shfl_xor(n, 32, 64);
        // exponent in base 2: (dot - n / 2) log2(e) - log2(m) / 2
        const float bias = fmaf(-0.5f * LOG2E, n, neg_half_log2m);
        // two projection tiles per step: enough independent work per wave without holding
        // every W fragment in registers at once
#pragma unroll 1
        for (int s = 0; s < MT / 2; ++s) {
            uint32_t o[4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int mt = 2 * s + h;
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < NKB; ++kk)
                    c = mfma16(*reinterpret_cast<const bf16x8 *>(sW + ((mt * NKB + kk) * 64 + l) * 8),
                               __builtin_bit_cast(bf16x8, xb[kk]), c);
                // c[j] = w_{(M/4) g + 4 mt + j} . x_r
                float e[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    e[j] = __builtin_amdgcn_exp2f(fmaf(c[j], LOG2E, bias));
                o[2 * h] = pack_bf2(e[0], e[1]);
                o[2 * h + 1] = pack_bf2(e[2], e[3]);
            }
            *reinterpret_cast<u32x4 *>(tileF + li * FS + (M / 4) * g + 8 * s) = u32x4{o[0], o[1], o[2], o[3]};
        }
        // the tile back as whole rows (this wave's LDS only: its accesses stay in order)
#pragma unroll
        for (int i = 0; i < 16 / (64 / LPR); ++i) {
            const int row = (64 / LPR) * i + l / LPR, col = 8 * (l % LPR);
            const u32x4 v = *reinterpret_cast<const u32x4 *>(tileF + row * FS + col);
            if (16 * t + row < rows)
                *reinterpret_cast<u32x4 *>(f + (16 * t + row) * M + col) = v;
        }
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk)
            xb[kk] = xn[kk];
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

// Waves per workgroup: 4, or 8 where W takes more than 32 KiB of LDS. With the larger W only
// one workgroup fits a CU (W plus one 16-row feature tile per wave), and 8 waves keep as many
// row loads in flight as two 4-wave workgroups do on the other shapes: measured on MI355X at
// d = 128, m = 256 over 2 x 16 x 8192 rows, 44 us with 8 waves against 57 with 4 (at m = 128 a
// second 8-wave workgroup per CU gained nothing: 26.5 against 25.7 us).
template <int D, int M> constexpr int rf_threads() { return M * D * 2 > 32768 ? 512 : 256; }

template <int D, int M>
void launch_rf(const void *x, const void *W, void *f, long rows, hipStream_t st)
{
    // workgroups: as many as fit the CUs at once, at most two per CU. Every workgroup copies
    // W from L2 first, all at the same time; measured on MI355X (d = m = 128), more workgroups
    // than this make the copies cost more than the extra waves bring.
    constexpr int NTH = rf_threads<D, M>();
    constexpr long LDS = (long)M * D * 2 + (NTH / 64) * 16L * (M + 8) * 2;
    static_assert(LDS <= 160 * 1024, "feature kernel LDS");
    const long ntile = (rows + 15) / 16;
    const long cap = 256L * (2 * LDS <= 160 * 1024 ? 2 : 1);
    const long want = (ntile + NTH / 64 - 1) / (NTH / 64);
    const unsigned grid = (unsigned)(want < cap ? want : cap);
    hipLaunchKernelGGL((k_rf_mfma<D, M, NTH>), dim3(grid), dim3(NTH), 0, st,
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
