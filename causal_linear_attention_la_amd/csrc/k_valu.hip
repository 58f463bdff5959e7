// k_valu.hip -- vector-ALU kernels of liblinattn for the shapes the matrix-core kernels do not
// take: float32 inputs (all arithmetic stays in float32) and any d, d_v in {16, 32, 64, 128}
// with either input dtype. One workgroup of 512 or 1024 threads per (segment, head); the float32
// state of the head lives in LDS; chunks of CH in {16, 32} tokens (64 and 128 when asked for).
// A short causal sequence (at most 64 tokens, d and d_v in {16, 32}, no decay) takes k_short
// instead, the whole sequence as one chunk (at the end of this file).
//
// Per chunk, with Qf = phi(Q_c), Kf = phi(K_c) and the state S, z before the chunk:
//   A[i][j] = Qf_i . Kf_j for j <= i (inclusive causal mask), 0 otherwise
//   den_i   = sum_j A[i][j] + Qf_i . z,   num_i = sum_j A[i][j] v_j + Qf_i^T S
//   out_i   = num_i / den_i;   then S += Kf^T V_c, z += colsum(Kf)
// -- the recurrence of "Linear Attention Math", section "The recurrent form: a running KV
// state", grouped by chunk. With causal = false the kernel is the global read
// out_i = Qf_i^T S / Qf_i . z of section "The associativity trick, written out".
// Flags: F_IDENTITY takes q and k as the features themselves; F_UNNORM stores num_i (no
// division). With a per-head decay gamma (causal only; the retention recurrence
// S_t = gamma S_{t-1} + Kf_t V_t^T), A[i][j] carries gamma^(i - j), the carried S and z reach
// row i scaled by gamma^(i + 1), and the update is S = gamma^n S + sum_j gamma^(n - 1 - j)
// Kf_j V_j^T over the chunk's n tokens.
#include "la_device.h"
#include "la_launch.h"

namespace la {
namespace {

// Threads of the chunked kernels' workgroups: 1024 for heads with d d_v >= 4096, 512 below
// (measured on MI355X against 256: causal B=1 H=4 N=1024 d=128 float32 at chunk 16 128.0 ->
// 74.8 us; B=1 H=8 N=4096 d=32 68.2 -> 60.0 us at 512 and 68.6 at 1024; B=2 H=4 N=1024 d=16
// d_v=64 32.8 -> 30.3 at 512 and 33.3 at 1024).
__host__ __device__ constexpr int valu_threads(int d, int dv) { return d * dv >= 4096 ? 1024 : 512; }
// threads of the short-sequence kernel: one per (row, quarter of the value columns)
constexpr int SNT = 256;

// The sum s + term(0) + ... + term(n - 1) in increasing order, n a multiple of 16 (every head
// size and chunk is): blocks of 16 terms are unrolled so that their LDS reads leave together
// instead of one dependent read per step (measured on MI355X: B=1 H=1 N=64 d=16 float32 as two
// segments 22.8 -> 18.8 us per call, B=1 H=8 N=4096 d=32 float32 92 -> 68 us, B=1 H=4 N=1024
// d=128 bf16 at chunk 16 206 -> 126 us). Sums over a chunk's keys run over the whole chunk: its rows past the end
// and the scores above the diagonal are stored as zeros, so the extra terms add exact zeros.
template <typename Term> __device__ __forceinline__ float sum16(int n, Term term, float s = 0.f)
{
    for (int j0 = 0; j0 < n; j0 += 16) {
#pragma unroll
        for (int j = j0; j < j0 + 16; ++j)
            s += term(j);
    }
    return s;
}

// decay weight of key j in a chunk of n valid keys: gamma^(n - 1 - j), and 0 past the end
// (where the power would overflow for gamma = 0)
__device__ __forceinline__ float key_weight(float lg, int n, int j)
{
    return j < n ? decay_pow(lg, n - 1 - j) : 0.f;
}

// One tensor's rows of the next chunk, loaded into registers while the current chunk is
// computed: element e = tid + u NT of the chunk's [ch, width] rows, u below the chunk's count
// per thread (at most PF). The loads are unconditional (rows clamped to the segment's last, the
// element to the chunk's last), so that nothing waits for their data before the chunk is
// staged; staging writes zeros for rows past the end (not features of zero). Used when
// ch width <= PF NT (every head size at the default chunks); otherwise each chunk loads its rows
// when it is staged. Measured on MI355X at B=2 H=16 N=8192 (same-box A/B): d=32 float32 causal
// 316.5 -> 299.8 us and global 140.3 -> 119.8 us, d=32 bf16 global 139.1 -> 133.8 us, d=64 d_v=32
// bf16 causal 546.3 -> 527.8 us, d=32 bf16 causal unchanged. PF = 8 cost the causal kernel half
// its waves per SIMD (129 VGPRs) and slowed it by half.
constexpr int PF = 2;
template <typename T, int NT> struct NextRows {
    float x[PF];
    __device__ __forceinline__ void load(const T *base, int t0, int last, int width, int ch, int tid)
    {
        const int n = ch * width, cnt = (n + NT - 1) / NT; // the same in every thread
#pragma unroll
        for (int u = 0; u < PF; ++u)
            if (u < cnt) {
                const int e = min(tid + u * NT, n - 1), row = min(t0 + e / width, last);
                x[u] = Elem<T>::ld(base, (size_t)row * width + e % width);
            }
    }
    __device__ __forceinline__ void stage(float *dst, int nvalid, int width, int ch, int tid, bool feat,
                                          bool ident) const
    {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int e = tid + u * NT;
            if (e < ch * width)
                dst[e] = e / width < nvalid ? (feat ? feature(x[u], ident) : x[u]) : 0.f;
        }
    }
};

// dynamic LDS carve-up (float32): S [d*dv] | z [d] | Qf [CH*d] | Kf [CH*d] | V [CH*dv] |
// A [CH*CH] | den [CH]
struct Lay {
    int oS, oz, oQ, oK, oV, oA, oden, total;
    __host__ __device__ Lay(int d, int dv, int ch)
    {
        oS = 0;
        oz = oS + d * dv;
        oQ = oz + d;
        oK = oQ + ch * d;
        oV = oK + ch * d;
        oA = oV + ch * dv;
        oden = oA + ch * ch;
        total = oden + ch;
    }
};

template <typename T, int NT>
__global__ __launch_bounds__(NT) void k_agg_valu(const T *__restrict__ k, const T *__restrict__ v,
                                                 float *__restrict__ dstS,
                                                 float *__restrict__ dstz, long sstride,
                                                 long zstride, int N, int d, int dv, int ch,
                                                 int L, int nseg, int P, int flags,
                                                 const float *__restrict__ gamma, int H)
{
    const bool ident = flags & F_IDENTITY;
    extern __shared__ float sm[];
    const Lay lay(d, dv, ch);
    float *sS = sm + lay.oS, *sz = sm + lay.oz, *sK = sm + lay.oK, *sV = sm + lay.oV;
    const int tid = threadIdx.x;
    const int p = blockIdx.x % nseg, bh = blockIdx.x / nseg;
    const int tb = p * L, te = min(N, tb + L);
    const T *kb = k + (size_t)bh * N * d;
    const T *vb = v + (size_t)bh * N * dv;
    const float lg = decay_log2(gamma, bh, H);

    for (int e = tid; e < d * dv; e += NT)
        sS[e] = 0.f;
    for (int f = tid; f < d; f += NT)
        sz[f] = 0.f;
    const bool pf = ch * d <= PF * NT && ch * dv <= PF * NT;
    NextRows<T, NT> nk, nv;
    if (pf && tb < te) {
        nk.load(kb, tb, te - 1, d, ch, tid);
        nv.load(vb, tb, te - 1, dv, ch, tid);
    }
    for (int t0 = tb; t0 < te; t0 += ch) {
        const int nvalid = min(ch, te - t0);
        __syncthreads();
        if (pf) {
            nk.stage(sK, nvalid, d, ch, tid, true, ident);
            nv.stage(sV, nvalid, dv, ch, tid, false, ident);
            const int tn = t0 + ch;
            if (tn < te) {
                nk.load(kb, tn, te - 1, d, ch, tid);
                nv.load(vb, tn, te - 1, dv, ch, tid);
            }
        } else {
            for (int e = tid; e < ch * d; e += NT) {
                const int j = e / d;
                sK[e] = j < nvalid ? feature(Elem<T>::ld(kb, (size_t)(t0 + j) * d + e % d), ident) : 0.f;
            }
            for (int e = tid; e < ch * dv; e += NT) {
                const int j = e / dv;
                sV[e] = j < nvalid ? Elem<T>::ld(vb, (size_t)(t0 + j) * dv + e % dv) : 0.f;
            }
        }
        __syncthreads();
        if (gamma) {
            const float fc = decay_pow(lg, nvalid);
            for (int e = tid; e < d * dv; e += NT) {
                const int f = e / dv, c = e % dv;
                const float s = sum16(ch, [&](int j) { return key_weight(lg, nvalid, j) * sK[j * d + f] * sV[j * dv + c]; });
                sS[e] = fc * sS[e] + s;
            }
            for (int f = tid; f < d; f += NT) {
                const float s = sum16(ch, [&](int j) { return key_weight(lg, nvalid, j) * sK[j * d + f]; });
                sz[f] = fc * sz[f] + s;
            }
        } else {
            for (int e = tid; e < d * dv; e += NT) {
                const int f = e / dv, c = e % dv;
                sS[e] += sum16(ch, [&](int j) { return sK[j * d + f] * sV[j * dv + c]; });
            }
            for (int f = tid; f < d; f += NT) {
                sz[f] += sum16(ch, [&](int j) { return sK[j * d + f]; });
            }
        }
    }
    __syncthreads();
    float *S = dstS + ((long)bh * P + p) * sstride;
    for (int e = tid; e < d * dv; e += NT)
        S[e] = sS[e];
    for (int f = tid; f < d; f += NT)
        dstz[((long)bh * P + p) * zstride + f] = sz[f];
}

template <typename T, bool CAUSAL, int NT>
__global__ __launch_bounds__(NT) void k_out_valu(const T *__restrict__ q, const T *__restrict__ k,
                                                 const T *__restrict__ v, T *__restrict__ out,
                                                 const float *__restrict__ preS,
                                                 const float *__restrict__ prez, long pstride,
                                                 long pzstride, int pslots,
                                                 float *__restrict__ Sout,
                                                 float *__restrict__ zout, int N, int d, int dv,
                                                 int ch, int L, int P, int flags,
                                                 const float *__restrict__ gamma, int H)
{
    extern __shared__ float sm[];
    const bool ident = flags & F_IDENTITY, norm = !(flags & F_UNNORM);
    const Lay lay(d, dv, ch);
    float *sS = sm + lay.oS, *sz = sm + lay.oz, *sQ = sm + lay.oQ, *sK = sm + lay.oK;
    float *sV = sm + lay.oV, *sA = sm + lay.oA, *sden = sm + lay.oden;
    const int tid = threadIdx.x;
    const int p = blockIdx.x % P, bh = blockIdx.x / P;
    const int tb = p * L, te = min(N, tb + L);
    const T *qb = q + (size_t)bh * N * d;
    const T *kb = CAUSAL ? k + (size_t)bh * N * d : nullptr;
    const T *vb = CAUSAL ? v + (size_t)bh * N * dv : nullptr;
    T *ob = out + (size_t)bh * N * dv;
    const float lg = decay_log2(gamma, bh, H);

    const long slot = (long)bh * pslots + min(p, pslots - 1);
    const float *S0 = preS ? preS + slot * pstride : nullptr;
    const float *z0 = preS ? prez + slot * pzstride : nullptr;
    for (int e = tid; e < d * dv; e += NT)
        sS[e] = S0 ? S0[e] : 0.f;
    for (int f = tid; f < d; f += NT)
        sz[f] = z0 ? z0[f] : 0.f;

    const bool pf = ch * d <= PF * NT && ch * dv <= PF * NT;
    NextRows<T, NT> nq, nk, nv;
    if (pf && tb < te) {
        nq.load(qb, tb, te - 1, d, ch, tid);
        if (CAUSAL) {
            nk.load(kb, tb, te - 1, d, ch, tid);
            nv.load(vb, tb, te - 1, dv, ch, tid);
        }
    }
    for (int t0 = tb; t0 < te; t0 += ch) {
        const int nvalid = min(ch, te - t0);
        __syncthreads();
        if (pf) {
            nq.stage(sQ, nvalid, d, ch, tid, true, ident);
            if (CAUSAL) {
                nk.stage(sK, nvalid, d, ch, tid, true, ident);
                nv.stage(sV, nvalid, dv, ch, tid, false, ident);
            }
            const int tn = t0 + ch;
            if (tn < te) {
                nq.load(qb, tn, te - 1, d, ch, tid);
                if (CAUSAL) {
                    nk.load(kb, tn, te - 1, d, ch, tid);
                    nv.load(vb, tn, te - 1, dv, ch, tid);
                }
            }
        } else {
            for (int e = tid; e < ch * d; e += NT) {
                const int j = e / d;
                const size_t gi = (size_t)(t0 + j) * d + e % d;
                sQ[e] = j < nvalid ? feature(Elem<T>::ld(qb, gi), ident) : 0.f;
                if (CAUSAL)
                    sK[e] = j < nvalid ? feature(Elem<T>::ld(kb, gi), ident) : 0.f;
            }
            if (CAUSAL)
                for (int e = tid; e < ch * dv; e += NT) {
                    const int j = e / dv;
                    sV[e] = j < nvalid ? Elem<T>::ld(vb, (size_t)(t0 + j) * dv + e % dv) : 0.f;
                }
        }
        __syncthreads();
        if (CAUSAL)
            for (int e = tid; e < ch * ch; e += NT) {
                const int i = e / ch, j = e % ch;
                const float s = j <= i ? sum16(d, [&](int f) { return sQ[i * d + f] * sK[j * d + f]; }) : 0.f;
                sA[e] = gamma && j <= i ? s * decay_pow(lg, i - j) : s;
            }
        __syncthreads();
        for (int i = tid; i < ch; i += NT) {
            float s = sum16(d, [&](int f) { return sQ[i * d + f] * sz[f]; });
            if (gamma)
                s *= decay_pow(lg, i + 1);
            if (CAUSAL)
                s = sum16(ch, [&](int j) { return sA[i * ch + j]; }, s);
            sden[i] = s;
        }
        __syncthreads();
        for (int e = tid; e < ch * dv; e += NT) {
            const int i = e / dv, c = e % dv;
            if (i >= nvalid)
                continue;
            float s = sum16(d, [&](int f) { return sQ[i * d + f] * sS[f * dv + c]; });
            if (gamma)
                s *= decay_pow(lg, i + 1);
            if (CAUSAL)
                s = sum16(ch, [&](int j) { return sA[i * ch + j] * sV[j * dv + c]; }, s);
            Elem<T>::st(ob, (size_t)(t0 + i) * dv + c, norm ? s / sden[i] : s);
        }
        if (CAUSAL && gamma) {
            __syncthreads();
            const float fc = decay_pow(lg, nvalid);
            for (int e = tid; e < d * dv; e += NT) {
                const int f = e / dv, c = e % dv;
                const float s = sum16(ch, [&](int j) { return key_weight(lg, nvalid, j) * sK[j * d + f] * sV[j * dv + c]; });
                sS[e] = fc * sS[e] + s;
            }
            for (int f = tid; f < d; f += NT) {
                const float s = sum16(ch, [&](int j) { return key_weight(lg, nvalid, j) * sK[j * d + f]; });
                sz[f] = fc * sz[f] + s;
            }
        } else if (CAUSAL) {
            __syncthreads();
            for (int e = tid; e < d * dv; e += NT) {
                const int f = e / dv, c = e % dv;
                sS[e] += sum16(ch, [&](int j) { return sK[j * d + f] * sV[j * dv + c]; });
            }
            for (int f = tid; f < d; f += NT) {
                sz[f] += sum16(ch, [&](int j) { return sK[j * d + f]; });
            }
        }
    }
    if (CAUSAL && Sout && p == P - 1) {
        __syncthreads();
        for (int e = tid; e < d * dv; e += NT)
            Sout[(size_t)bh * d * dv + e] = sS[e];
        for (int f = tid; f < d; f += NT)
            zout[(size_t)bh * d + f] = sz[f];
    }
}

// ---- short sequences ---------------------------------------------------------------------
// The causal form of a sequence of at most SHORT_N tokens evaluated as one chunk, directly:
//   out_i = (phi(q_i)^T S0 + sum_{j <= i} (phi(q_i) . phi(k_j)) v_j)
//           / (phi(q_i) . z0 + sum_{j <= i} phi(q_i) . phi(k_j))
// -- the chunked evaluation with the whole sequence as its one chunk ("Linear Attention: From
// Pairwise Reads to a Recurrent State", section "A recurrence need not force token-serial
// training": the state from before the chunk plus the pairwise reads inside it) -- followed by
// the final state S0 + phi(K)^T V, z0 + phi(K)^T 1. One workgroup of 256 threads per head,
// four per row: thread (i, part) keeps phi(q_i) in registers, forms the scores of the keys
// part, part + 4, ... and accumulates them and their value rows over all value columns, reading
// each key row from LDS together with the other lanes of its wave; the row's four threads then
// add their parts by lane exchange and each stores a quarter of the row. No decay (the decayed
// form keeps the chunked kernel). Against the chunked kernel there are no per-chunk phases and
// barriers. B=1 H=1 N=64 d=16 float32 on MI355X, per call replayed from a graph: 8.1 us (9.7 us
// with one thread per (row, quarter of the value columns) forming every score four times and
// the global loads issued one element per loop step; 13.5 us with four 16-token chunks).
constexpr int SHORT_N = 64;

// elements e .. e + 3 as float32 (e a multiple of 4 and the row 16-byte aligned: one 16-byte
// load for float32, one 8-byte load for bf16)
template <typename T> __device__ __forceinline__ f32x4 ld4(const T *p, size_t e);
template <> __device__ __forceinline__ f32x4 ld4<float>(const float *p, size_t e)
{
    return *reinterpret_cast<const f32x4 *>(p + e);
}
template <> __device__ __forceinline__ f32x4 ld4<bf16_t>(const bf16_t *p, size_t e)
{
    const u32x2 w = *reinterpret_cast<const u32x2 *>(p + e);
    return f32x4{bf_lo(w[0]), bf_hi(w[0]), bf_lo(w[1]), bf_hi(w[1])};
}

template <typename T, int D, int DV>
__global__ __launch_bounds__(SNT) void k_short(const T *__restrict__ q, const T *__restrict__ k,
                                              const T *__restrict__ v, T *__restrict__ out,
                                              const float *__restrict__ S0,
                                              const float *__restrict__ z0,
                                              float *__restrict__ Sout, float *__restrict__ zout,
                                              int N, int flags)
{
    static_assert(SNT == 4 * SHORT_N, "four threads per row");
    constexpr int CW = DV / 4;
    __shared__ __attribute__((aligned(16))) float sK[SHORT_N][D], sV[SHORT_N][DV], sS[D * DV], sz[D];
    const bool ident = flags & F_IDENTITY, norm = !(flags & F_UNNORM);
    const int tid = threadIdx.x, i = tid >> 2, c0 = (tid & 3) * CW;
    const size_t bh = blockIdx.x;
    const T *qb = q + bh * N * D, *kb = k + bh * N * D, *vb = v + bh * N * DV;

    // every global load is issued before any of them is used: four consecutive elements per
    // load, at most two per thread and tensor (the sequence fits one workgroup's pass), then
    // the thread's query row. Issued one element per loop step, each load waited for its data
    // before the next left: 9.5 us of kernel time at N = 64, d = 16 float32 (MI355X trace).
    constexpr int KP = (SHORT_N * D / 4 + SNT - 1) / SNT, VP = (SHORT_N * DV / 4 + SNT - 1) / SNT;
    constexpr int SP = (D * DV / 4 + SNT - 1) / SNT;
    f32x4 kr[KP], vr[VP], sr[SP];
#pragma unroll
    for (int u = 0; u < KP; ++u) {
        const int e = 4 * (tid + u * SNT);
        if (e < N * D)
            kr[u] = ld4(kb, e);
    }
#pragma unroll
    for (int u = 0; u < VP; ++u) {
        const int e = 4 * (tid + u * SNT);
        if (e < N * DV)
            vr[u] = ld4(vb, e);
    }
#pragma unroll
    for (int u = 0; u < SP; ++u) {
        const int e = 4 * (tid + u * SNT);
        if (e < D * DV)
            sr[u] = S0 ? *reinterpret_cast<const f32x4 *>(S0 + bh * D * DV + e) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float zr = tid < D && S0 ? z0[bh * D + tid] : 0.f;
    float qf[D];
    const int ir = min(i, N - 1); // rows past the end compute on the last row and store nothing
#pragma unroll
    for (int f = 0; f < D; f += 4) {
        const f32x4 x = ld4(qb, (size_t)ir * D + f);
#pragma unroll
        for (int c = 0; c < 4; ++c)
            qf[f + c] = feature(x[c], ident);
    }
    // rows N .. SHORT_N - 1 of both arrays hold zeros, so that the final-state sums below run
    // over whole blocks of 16 keys: the extra terms are exact zeros
#pragma unroll
    for (int u = 0; u < KP; ++u) {
        const int e = 4 * (tid + u * SNT);
        if (e < SHORT_N * D)
            *reinterpret_cast<f32x4 *>(&sK[e / D][e % D]) =
                e < N * D ? f32x4{feature(kr[u][0], ident), feature(kr[u][1], ident),
                                  feature(kr[u][2], ident), feature(kr[u][3], ident)}
                          : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < VP; ++u) {
        const int e = 4 * (tid + u * SNT);
        if (e < SHORT_N * DV)
            *reinterpret_cast<f32x4 *>(&sV[e / DV][e % DV]) = e < N * DV ? vr[u] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < SP; ++u) {
        const int e = 4 * (tid + u * SNT);
        if (e < D * DV)
            *reinterpret_cast<f32x4 *>(&sS[e]) = sr[u];
    }
    if (tid < D)
        sz[tid] = zr;
    __syncthreads();

    // the state before the sequence
    float num[CW], den = 0.f;
#pragma unroll
    for (int c = 0; c < CW; ++c)
        num[c] = 0.f;
#pragma unroll
    for (int f = 0; f < D; ++f) {
        den = fmaf(qf[f], sz[f], den);
#pragma unroll
        for (int c = 0; c < CW; ++c)
            num[c] = fmaf(qf[f], sS[f * DV + c0 + c], num[c]);
    }
    // the pairs j <= i (keys past the wave's last row add nothing to any of its rows): the
    // row's four threads (adjacent lanes) take every fourth key each, p, p + 4, ..., over all
    // value columns, so that each score phi(q_i) . phi(k_j) is formed once; their parts are then
    // added in a fixed order (lane pairs, then pairs of pairs: every lane holds the same sums)
    const int part = tid & 3;
    const int jend = min(N, (tid / 64) * 16 + 16);
    float pn[DV], pd = 0.f;
#pragma unroll
    for (int c = 0; c < DV; ++c)
        pn[c] = 0.f;
#pragma unroll 2
    for (int j = part; j < jend; j += 4) {
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int f = 0; f < D; f += 2) {
            a0 = fmaf(qf[f], sK[j][f], a0);
            a1 = fmaf(qf[f + 1], sK[j][f + 1], a1);
        }
        const float a = j <= i ? a0 + a1 : 0.f;
        pd += a;
#pragma unroll
        for (int c = 0; c < DV; ++c)
            pn[c] = fmaf(a, sV[j][c], pn[c]);
    }
    pd += __shfl_xor(pd, 1, 64);
    pd += __shfl_xor(pd, 2, 64);
    den += pd;
#pragma unroll
    for (int c = 0; c < DV; ++c) {
        pn[c] += __shfl_xor(pn[c], 1, 64);
        pn[c] += __shfl_xor(pn[c], 2, 64);
    }
    // this thread's value columns c0 .. c0 + CW - 1 (selected without indexing registers)
#pragma unroll
    for (int c = 0; c < CW; ++c)
        num[c] += part == 0 ? pn[c] : part == 1 ? pn[CW + c] : part == 2 ? pn[2 * CW + c] : pn[3 * CW + c];
    if (i < N)
#pragma unroll
        for (int c = 0; c < CW; ++c)
            Elem<T>::st(out, (bh * N + i) * DV + c0 + c, norm ? num[c] / den : num[c]);
    if (Sout) {
        const int n16 = (N + 15) & ~15;
        for (int e = tid; e < D * DV; e += SNT) {
            const int f = e / DV, c = e % DV;
            float s = sS[e];
            for (int j0 = 0; j0 < n16; j0 += 16)
#pragma unroll
                for (int j = j0; j < j0 + 16; ++j)
                    s = fmaf(sK[j][f], sV[j][c], s);
            Sout[bh * D * DV + e] = s;
        }
        for (int f = tid; f < D; f += SNT) {
            float s = sz[f];
            for (int j0 = 0; j0 < n16; j0 += 16)
#pragma unroll
                for (int j = j0; j < j0 + 16; ++j)
                    s += sK[j][f];
            zout[bh * D + f] = s;
        }
    }
}

} // namespace

template <typename T, int NT>
hipError_t agg_valu_t(int flags, const void *k, const void *v, float *dstS, float *dstz,
                      long sstride, long zstride, int BH, int N, int d, int dv, int chunk, int L,
                      int nseg, int P, const float *gamma, int H, hipStream_t st)
{
    const size_t lds = sizeof(float) * Lay(d, dv, chunk).total;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_agg_valu<T, NT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((k_agg_valu<T, NT>), dim3((unsigned)(BH * nseg)), dim3(NT), lds, st,
                       static_cast<const T *>(k), static_cast<const T *>(v), dstS, dstz, sstride,
                       zstride, N, d, dv, chunk, L, nseg, P, flags, gamma, H);
    return hipGetLastError();
}

hipError_t agg_valu(bool bf16, int flags, const void *k, const void *v, float *dstS, float *dstz,
                    long sstride, long zstride, int BH, int N, int d, int dv, int chunk, int L,
                    int nseg, int P, const float *gamma, int H, hipStream_t st)
{
    const bool big = valu_threads(d, dv) == 1024;
    auto f = bf16 ? (big ? agg_valu_t<bf16_t, 1024> : agg_valu_t<bf16_t, 512>)
                  : (big ? agg_valu_t<float, 1024> : agg_valu_t<float, 512>);
    return f(flags, k, v, dstS, dstz, sstride, zstride, BH, N, d, dv, chunk, L, nseg, P, gamma, H, st);
}

template <typename T, bool CAUSAL, int NT>
hipError_t out_valu_t(int flags, const void *q, const void *k, const void *v, void *out, const float *preS,
                      const float *prez, long pstride, long pzstride, int pslots, float *Sout,
                      float *zout, int BH, int N, int d, int dv, int chunk, int L, int P,
                      const float *gamma, int H, hipStream_t st)
{
    const size_t lds = sizeof(float) * Lay(d, dv, chunk).total;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_out_valu<T, CAUSAL, NT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((k_out_valu<T, CAUSAL, NT>), dim3((unsigned)(BH * P)), dim3(NT), lds, st,
                       static_cast<const T *>(q), static_cast<const T *>(k),
                       static_cast<const T *>(v), static_cast<T *>(out), preS, prez, pstride,
                       pzstride, pslots, Sout, zout, N, d, dv, chunk, L, P, flags, gamma, H);
    return hipGetLastError();
}

hipError_t out_valu(bool bf16, bool causal, int flags, const void *q, const void *k, const void *v,
                    void *out, const float *preS, const float *prez, long pstride,
                    long pzstride, int pslots, float *Sout, float *zout, int BH, int N, int d,
                    int dv, int chunk, int L, int P, const float *gamma, int H, hipStream_t st)
{
    const bool big = valu_threads(d, dv) == 1024;
    auto f = bf16 ? (causal ? (big ? out_valu_t<bf16_t, true, 1024> : out_valu_t<bf16_t, true, 512>)
                            : (big ? out_valu_t<bf16_t, false, 1024> : out_valu_t<bf16_t, false, 512>))
                  : (causal ? (big ? out_valu_t<float, true, 1024> : out_valu_t<float, true, 512>)
                            : (big ? out_valu_t<float, false, 1024> : out_valu_t<float, false, 512>));
    return f(flags, q, k, v, out, preS, prez, pstride, pzstride, pslots, Sout, zout, BH, N, d, dv, chunk,
             L, P, gamma, H, st);
}

bool short_ok(int N, int d, int dv)
{
    return N >= 1 && N <= SHORT_N && (d == 16 || d == 32) && (dv == 16 || dv == 32);
}

hipError_t short_causal(bool bf16, int flags, const void *q, const void *k, const void *v, void *out,
                        const float *S0, const float *z0, float *S, float *z, int BH, int N, int d,
                        int dv, hipStream_t st)
{
    if (!short_ok(N, d, dv))
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)BH), block(SNT);
#define LA_SH(TT, DD, VV)                                                                          \
    if (d == DD && dv == VV) {                                                                     \
        hipLaunchKernelGGL((k_short<TT, DD, VV>), grid, block, 0, st, static_cast<const TT *>(q),    \
                           static_cast<const TT *>(k), static_cast<const TT *>(v),                 \
                           static_cast<TT *>(out), S0, z0, S, z, N, flags);                        \
        return hipGetLastError();                                                                  \
    }
    if (bf16) {
        LA_SH(bf16_t, 16, 16) LA_SH(bf16_t, 16, 32) LA_SH(bf16_t, 32, 16) LA_SH(bf16_t, 32, 32)
    } else {
        LA_SH(float, 16, 16) LA_SH(float, 16, 32) LA_SH(float, 32, 16) LA_SH(float, 32, 32)
    }
#undef LA_SH
    return hipErrorInvalidValue;
}

// Largest dynamic LDS the vector-ALU kernels take (d = d_v = 128, chunk 32): 118,912 bytes.
size_t valu_lds_bytes(int d, int dv, int chunk) { return sizeof(float) * Lay(d, dv, chunk).total; }

} // namespace la
