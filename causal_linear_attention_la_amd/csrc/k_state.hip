// k_state.hip -- state kernels of liblinattn: the joins between sequence segments and the
// single-token decode step.
//
// Segment joins. The causal state is a prefix sum over tokens ("Linear Attention: From
// Pairwise Reads to a Recurrent State", section "A recurrence need not force token-serial
// training"), so the state before segment p is the initial state plus the sums of segments
// 0..p-1; the global state is the sum of all segments ("Linear Attention Math", section "The
// associativity trick, written out"). Each lane owns four consecutive floats of the
// E = d*d_v + d floats of a head's state; the prefix walks the P segment slots in order, the
// total adds them in an order fixed by P (either way the result does not depend on
// scheduling).
//
// Decode step ("Linear Attention Math", section "The recurrent form"): for each head,
// S' = S + phi(k) v^T and z' = z + phi(k) are written back in place, then
// out = phi(q)^T S' / phi(q)^T z' (F_IDENTITY: q, k are the features; F_UNNORM: no
// division). One workgroup per head streams the float32 state once in and once out with
// 16-byte accesses; the read phi(q)^T S' reuses the updated values while
// they are in registers, so each state byte crosses HBM exactly twice. The state accesses are
// non-temporal: the state is touched once per step, and on gfx950 an in-place stream with
// non-temporal loads and stores sustains about 8 % more bandwidth than with cached ones.
#include "la_device.h"
#include "la_launch.h"

namespace la {
namespace {

constexpr int NT = 256;

// Slots are read in batches of SB independent loads, each batch's stores issued before the
// next batch's loads, so the stores of early slots stream out while later slots are read.
// Measured on MI355X for the 8-segment prefill (32 heads): 10.3 us with all slots loaded
// before any store, 9.7 us with batches of 4, 9.3 us with batches of 2 (9.3-9.4 with 1).
constexpr int SB = 2;

// Four consecutive floats per thread (16-byte accesses): d and d_v are multiples of 16 and every
// state buffer is 16-byte aligned (the entry points reject anything else), so a group of four
// never straddles the end of S.
__global__ __launch_bounds__(NT) void k_seg_scan(float *__restrict__ ws, const float *__restrict__ S0,
                                                  const float *__restrict__ z0, int P, int d,
                                                  int dv, int blocks_per_head,
                                                  const float *__restrict__ gamma, int H, int L)
{
    const int E = d * dv + d;
    const int bh = blockIdx.x / blocks_per_head;
    const int e = 4 * ((blockIdx.x % blocks_per_head) * NT + threadIdx.x);
    if (e >= E)
        return;
    float4 run = {0.f, 0.f, 0.f, 0.f};
    if (S0)
        run = e < d * dv ? *reinterpret_cast<const float4 *>(S0 + (size_t)bh * d * dv + e)
                         : *reinterpret_cast<const float4 *>(z0 + (size_t)bh * d + (e - d * dv));
    float *slot = ws + (size_t)bh * P * E + e;
    const float fL = gamma ? decay_pow(decay_log2(gamma, bh, H), L) : 1.f;
    for (int p0 = 0; p0 < P - 1; p0 += SB) {
        float4 t[SB];
#pragma unroll
        for (int i = 0; i < SB; ++i)
            if (p0 + i < P - 1)
                t[i] = *reinterpret_cast<const float4 *>(slot + (size_t)(p0 + i) * E);
#pragma unroll
        for (int i = 0; i < SB; ++i)
            if (p0 + i < P - 1) {
                *reinterpret_cast<float4 *>(slot + (size_t)(p0 + i) * E) = run;
                if (gamma) {
                    run.x = fmaf(run.x, fL, t[i].x);
                    run.y = fmaf(run.y, fL, t[i].y);
                    run.z = fmaf(run.z, fL, t[i].z);
                    run.w = fmaf(run.w, fL, t[i].w);
                } else {
                    run.x += t[i].x;
                    run.y += t[i].y;
                    run.z += t[i].z;
                    run.w += t[i].w;
                }
            }
    }
    *reinterpret_cast<float4 *>(slot + (size_t)(P - 1) * E) = run;
}

// The global state of a head, the sum of its P segment states, in an order fixed by P alone:
// wave w of a workgroup adds segments w, w + 4, w + 8, ... (lane l owns four consecutive floats,
// and a lane's loads are independent of one another, TB of them issued together), and the four
// waves' partial sums are then added in wave order. A single in-order walk per thread waited for
// each pair of loads before the next (measured on MI355X, 8 heads of 32 segments at
// d = d_v = 128: 7.6 us).
constexpr int TB = 8;

__global__ __launch_bounds__(NT) void k_seg_total(const float *__restrict__ ws, float *__restrict__ S,
                                                  float *__restrict__ z, int P, int d, int dv,
                                                  int blocks_per_head)
{
    constexpr int NW = NT / 64;
    __shared__ f32x4 part[NW][64];
    const int E4 = (d * dv + d) / 4;
    const int bh = blockIdx.x / blocks_per_head, w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int e4 = (blockIdx.x % blocks_per_head) * 64 + l;
    f32x4 run = {0.f, 0.f, 0.f, 0.f};
    if (e4 < E4) {
        const f32x4 *slot = reinterpret_cast<const f32x4 *>(ws + (size_t)bh * P * E4 * 4) + e4;
        for (int p0 = w; p0 < P; p0 += NW * TB) {
            f32x4 t[TB];
#pragma unroll
            for (int i = 0; i < TB; ++i)
                t[i] = p0 + NW * i < P ? slot[(size_t)(p0 + NW * i) * E4] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < TB; ++i)
                run += t[i];
        }
    }
    part[w][l] = run;
    __syncthreads();
    if (w != 0 || e4 >= E4)
        return;
#pragma unroll
    for (int i = 1; i < NW; ++i)
        run += part[i][l];
    const int e = 4 * e4;
    if (e < d * dv)
        *reinterpret_cast<f32x4 *>(S + (size_t)bh * d * dv + e) = run;
    else
        *reinterpret_cast<f32x4 *>(z + (size_t)bh * d + (e - d * dv)) = run;
}

// One workgroup per head. Thread layout over the [D, DV] state: CG = DV/4 column groups of 4
// floats, RP row phases; thread (rp, cg) owns rows rp, rp+RP, ... of columns 4cg..4cg+3. RP is
// D/4 (four rows per thread), at least one wave and at most 1024 threads in all: at
// d = d_v = 128 that is sixteen waves per head, which keep more of the state's loads in flight per
// CU than four (measured on MI355X, 256 x 32 heads: 186.0 -> 176.9 us per step; 512 threads:
// 183.8 us), while at d = d_v = 64 one row per thread over 1024 threads was slower than four rows
// over 256 (512 x 64 heads: 4.17 against 3.83 us).
template <int D, int DV> struct DecCfg {
    static constexpr int CG = DV / 4;
    static constexpr int RPW = D / 4 > 64 / CG ? D / 4 : 64 / CG;
    static constexpr int RP = 1024 / CG < RPW ? 1024 / CG : RPW;
    static constexpr int THREADS = CG * RP;
    static constexpr int RPT = (D + RP - 1) / RP;
    static_assert(THREADS % 64 == 0 && THREADS >= D && THREADS >= DV, "decode block");
};

template <typename T, int D, int DV>
__global__ __launch_bounds__((DecCfg<D, DV>::THREADS)) void k_decode(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, T *__restrict__ out,
    float *__restrict__ S, float *__restrict__ z, int flags, const float *__restrict__ gamma, int H)
{
    const bool ident = flags & F_IDENTITY;
    using G = DecCfg<D, DV>;
    constexpr int CG = G::CG, RP = G::RP, RPT = G::RPT, NTH = G::THREADS;
    __shared__ float skf[D], sqf[D];
    __shared__ float red[RP][DV + 4];
    __shared__ float sden[NTH / 64];

    const int tid = threadIdx.x, cg = tid % CG, rp = tid / CG;
    const size_t bh = blockIdx.x;
    f32x4 *Sh = reinterpret_cast<f32x4 *>(S + bh * D * DV);
    // decay of the carried state (1 without gamma): S' = gd S + phi(k) v^T, z' = gd z + phi(k)
    const float gd = decay_gamma(gamma, (long)bh, H);

    // the head's state rows, all loads in flight before any use
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rp + RP * i;
        if (r < D)
            s[i] = __builtin_nontemporal_load(Sh + r * CG + cg);
    }

    float part = 0.f;
    if (tid < D) {
        const float kf = feature(Elem<T>::ld(k, bh * D + tid), ident);
        const float qf = feature(Elem<T>::ld(q, bh * D + tid), ident);
        skf[tid] = kf;
        sqf[tid] = qf;
        const float zn = fmaf(gd, z[bh * D + tid], kf);
        z[bh * D + tid] = zn;
        part = qf * zn;
    }
    part = wave_sum(part);
    if ((tid & 63) == 0)
        sden[tid >> 6] = part;
    f32x4 vv;
#pragma unroll
    for (int c = 0; c < 4; ++c)
        vv[c] = Elem<T>::ld(v, bh * DV + 4 * cg + c);
    __syncthreads();

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rp + RP * i;
        if (r < D) {
            const float kf = skf[r], qf = sqf[r];
            f32x4 sn;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                sn[c] = fmaf(gd, s[i][c], kf * vv[c]);
                acc[c] += qf * sn[c];
            }
            __builtin_nontemporal_store(sn, Sh + r * CG + cg);
        }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
        red[rp][4 * cg + c] = acc[c];
    __syncthreads();
    if (tid < DV) {
        float num = 0.f;
#pragma unroll
        for (int i = 0; i < RP; ++i)
            num += red[i][tid];
        float den = 0.f;
#pragma unroll
        for (int w = 0; w < NTH / 64; ++w)
            den += sden[w];
        Elem<T>::st(out, bh * DV + tid, (flags & F_UNNORM) ? num : num / den);
    }
}

template <typename T>
hipError_t decode_t(int flags, const void *q, const void *k, const void *v, void *out, float *S,
                    float *z, int BH, int d, int dv, const float *gamma, int H, hipStream_t st)
{
    const dim3 grid((unsigned)BH);
    const T *qq = static_cast<const T *>(q), *kk = static_cast<const T *>(k),
            *vv = static_cast<const T *>(v);
    T *oo = static_cast<T *>(out);
#define LA_DEC(DD, VV)                                                                          \
    if (d == DD && dv == VV) {                                                                  \
        hipLaunchKernelGGL((k_decode<T, DD, VV>), grid, dim3(DecCfg<DD, VV>::THREADS), 0, st, qq, kk, \
                           vv, oo, S, z, flags, gamma, H);                                      \
        return hipGetLastError();                                                               \
    }
#define LA_DEC_ROW(DD) LA_DEC(DD, 16) LA_DEC(DD, 32) LA_DEC(DD, 64) LA_DEC(DD, 128)
    LA_DEC_ROW(16)
    LA_DEC_ROW(32)
    LA_DEC_ROW(64)
    LA_DEC_ROW(128)
#undef LA_DEC_ROW
#undef LA_DEC
    return hipErrorInvalidValue;
}

} // namespace

hipError_t seg_exclusive_scan(float *ws, const float *S0, const float *z0, int BH, int P, int d,
                              int dv, const float *gamma, int H, int L, hipStream_t st)
{
    const int E = d * dv + d;
    auto a16 = [](const void *p) { return ((uintptr_t)p & 15) == 0; };
    if (d % 4 || dv % 4 || !a16(ws) || (S0 && (!a16(S0) || !a16(z0))))
        return hipErrorInvalidValue;
    const int bph = (E / 4 + NT - 1) / NT;
    hipLaunchKernelGGL(k_seg_scan, dim3((unsigned)(BH * bph)), dim3(NT), 0, st, ws, S0, z0, P, d,
                       dv, bph, gamma, H, L);
    return hipGetLastError();
}

hipError_t seg_total(const float *ws, float *S, float *z, int BH, int P, int d, int dv,
                     hipStream_t st)
{
    if (d % 4 || dv % 4 || ((uintptr_t)ws & 15) || ((uintptr_t)S & 15) || ((uintptr_t)z & 15))
        return hipErrorInvalidValue;
    const int E4 = (d * dv + d) / 4, bph = (E4 + 63) / 64;
    hipLaunchKernelGGL(k_seg_total, dim3((unsigned)(BH * bph)), dim3(NT), 0, st, ws, S, z, P, d,
                       dv, bph);
    return hipGetLastError();
}

hipError_t decode_step(bool bf16, int flags, const void *q, const void *k, const void *v,
                       void *out, float *S, float *z, int BH, int d, int dv, const float *gamma,
                       int H, hipStream_t st)
{
    return bf16 ? decode_t<bf16_t>(flags, q, k, v, out, S, z, BH, d, dv, gamma, H, st)
                : decode_t<float>(flags, q, k, v, out, S, z, BH, d, dv, gamma, H, st);
}

} // namespace la
