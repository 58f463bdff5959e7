// k_mfma32.hip -- float32 matrix-core kernels of liblinattn (d = d_v in {64, 128}): the segment
// sums, the causal prefill and the global read, all arithmetic in float32 on
// v_mfma_f32_16x16x4_f32 (the chip's fp32 matrix rate is twice its unpacked vector rate).
//
// The recurrence is the one of "Linear Attention Math", section "The recurrent form: a running
// KV state", grouped by chunk of CH = 32 tokens as in "Linear Attention: From Pairwise Reads to
// a Recurrent State", section "A recurrence need not force token-serial training": with
// Qf = phi(Q_c), Kf = phi(K_c) and the state S, z before the chunk,
//   num = Qf S + mask(Qf Kf^T) V_c,  den = Qf z + rowsum(mask(Qf Kf^T)),  out = num / den,
//   then S += Kf^T V_c, z += colsum(Kf)
// (mask: key <= query). The global read is out = Qf S / Qf z ("Linear Attention Math", section
// "The associativity trick, written out"). The segment sums and the causal kernel also take a
// per-head decay (below, at decayed_values).
//
// Operand layout. A 16x16x4 product takes A[l % 16][k = l / 16] and B[k = l / 16][l % 16] from
// lane l and leaves D[4 (l / 16) + r][l % 16] (r < 4) in lane l (checked on gfx950). A product
// only needs the A and B lanes of one lane group to agree on which k they carry, so the k-th
// product step may give lane group g the feature (or key) 4 g + k of a 16-block. With that
// choice an accumulator tile is itself a B operand: lane (g, c) of the tile of S holds
// S[16 ft + 4 g + r][c], exactly the B value of step r. So the state stays in accumulators, in
// float32, for the whole segment; the scores are built transposed (A^T = Kf Qf^T, key rows) for
// the same reason, so that they are A operands of the product with V without any exchange.
// All other operands are 16-byte LDS reads of four consecutive features or keys.
//
// Causal and global workgroups: D/16 waves, wave w owning the value columns 16 w .. 16 w + 15
// of S, num and out (the segment sums, which only update S, use twice the waves; see A32).
// Causal, per chunk, phase 1: waves 0-3 form partial scores over a quarter of the features each (one
// wave per SIMD), every wave computes Qf S for its columns, the last wave forms Qf z; barrier;
// phase 2: every wave adds the four partial score tiles (in a fixed order), divides, forms
// num += A V and updates its columns of S; the next chunk is staged into the other half of the
// double-buffered LDS; barrier.
#include "la_device.h"
#include "la_launch.h"

namespace la {
namespace {

constexpr int CH = 32;

__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ void st4(float *p, f32x4 x) { *reinterpret_cast<f32x4 *>(p) = x; }

// The hardware exponential (exp2 of x log2 e): relative error about |x| 2^-24 against expf, far
// below the float32 tolerance of the outputs, and 5 % of the causal kernel's time
// (B=2 H=16 N=8192 d=128 on MI355X: 245 -> 234 us).
__device__ __forceinline__ f32x4 phi4(f32x4 x)
{
    return f32x4{phi_fast(x[0]), phi_fast(x[1]), phi_fast(x[2]), phi_fast(x[3])};
}

template <int D> struct C32 {
    static constexpr int NW = D / 16;        // waves
    static constexpr int THREADS = NW * 64;
    static constexpr int NFT = D / 16;       // 16-feature tiles of S
    static constexpr int RS = D + 4;         // row stride (floats) of a row-major chunk array
    static constexpr int TS = CH + 4;        // row stride of the feature-major key array
    static constexpr int Q4 = D / 4;         // 16-byte pieces per row
};

// Chunk staging. Row-major tensors (q, v): piece u is row u / Q4, columns 4 (u % Q4) .. + 3 (a
// wave reads whole rows). Keys: piece u is key u % CH, features 4 (u / CH) .. + 3, so that the
// feature-major copy is written with consecutive keys in consecutive lanes. Rows past the
// segment's end are loaded from its last row (every load in bounds) and staged as zeros.
template <int D, int TH = C32<D>::THREADS> struct Stage {
    using G = C32<D>;
    static constexpr int PER = CH * G::Q4 / TH; // 16-byte pieces of a chunk per thread
    static_assert(PER * TH == CH * G::Q4, "chunk pieces must divide evenly");
    const int tid;
    __device__ Stage(int t) : tid(t) {}
    __device__ void rows(f32x4 (&r)[PER], const float *base, int t0, int n) const
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = tid + i * TH, row = min(u / G::Q4, n - 1);
            r[i] = ld4(base + (size_t)(t0 + row) * D + 4 * (u % G::Q4));
        }
    }
    __device__ void keys(f32x4 (&r)[PER], const float *base, int t0, int n) const
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = tid + i * TH, key = min(u % CH, n - 1);
            r[i] = ld4(base + (size_t)(t0 + key) * D + 4 * (u / CH));
        }
    }
    template <bool PHI> __device__ void put_rows(float *dst, const f32x4 (&r)[PER], int n) const
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = tid + i * TH, row = u / G::Q4;
            const f32x4 x = row < n ? (PHI ? phi4(r[i]) : r[i]) : f32x4{0.f, 0.f, 0.f, 0.f};
            st4(dst + row * G::RS + 4 * (u % G::Q4), x);
        }
    }
    // keys to the feature-major array (and, when rowmaj is given, also row-major)
    template <bool PHI>
    __device__ void put_keys(float *kt, float *rowmaj, const f32x4 (&r)[PER], int n) const
    {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = tid + i * TH, key = u % CH, c4 = u / CH;
            const f32x4 x = key < n ? (PHI ? phi4(r[i]) : r[i]) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j)
                kt[(4 * c4 + j) * G::TS + key] = x[j];
            if (rowmaj)
                st4(rowmaj + key * G::RS + 4 * c4, x);
        }
    }
};

// S += Kf^T V_c for this wave's value columns and NF feature tiles from the feature-major row
// kt (its first feature): step r of key tile kt gives lane group g the key 16 kt + 4 g + r (A:
// Kf^T rows; B: the V values vb). The NF accumulators take turns (feature tile innermost), so
// consecutive products never wait for each other's results.
template <int D, int NF>
__device__ __forceinline__ void update_state(f32x4 (&sacc)[NF], const float *kt,
                                             const float (&vb)[2][4], int li, int g)
{
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        f32x4 a[NF];
#pragma unroll
        for (int ft = 0; ft < NF; ++ft)
            a[ft] = ld4(kt + (16 * ft + li) * C32<D>::TS + 16 * t + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int ft = 0; ft < NF; ++ft)
                sacc[ft] = mma(a[ft][r], vb[t][r], sacc[ft]);
    }
}

// column sum of the chunk's features into z (feature f = thread index, keys in order)
template <int D> __device__ __forceinline__ float key_col_sum(const float *kt, int f)
{
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < CH / 4; ++j) {
        const f32x4 x = ld4(kt + f * C32<D>::TS + 4 * j);
        s += ((x[0] + x[1]) + (x[2] + x[3]));
    }
    return s;
}

// Qf z for the CH queries of a chunk (Qb: row-major features, row stride C32<D>::RS), spread
// over the NW waves of a workgroup: wave w takes queries QPW w .. + QPW - 1, LPQ lanes per query
// each add up their groups of four features, then a fixed shuffle tree. (One wave doing all
// queries sat on the path to the barrier that follows: the float32 causal kernel with 2 D/16
// waves took 232 us at B=2 H=16 N=8192 d=128 that way, 211 us this way.)
template <int D, int NW>
__device__ __forceinline__ void chunk_qz(float *sdz, const float *Qb, const float *sz, int w, int l)
{
    constexpr int QPW = CH / NW, LPQ = 64 / QPW, G = D / (4 * LPQ);
    static_assert(QPW * NW == CH && G * 4 * LPQ == D, "queries and features must divide evenly");
    const int qq = QPW * w + l / LPQ, fg = l % LPQ;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int f = 4 * (fg + LPQ * i);
        const f32x4 x = ld4(Qb + qq * C32<D>::RS + f), zz = ld4(sz + f);
        s = fmaf(x[0], zz[0], fmaf(x[1], zz[1], fmaf(x[2], zz[2], fmaf(x[3], zz[3], s))));
    }
#pragma unroll
    for (int off = LPQ / 2; off > 0; off >>= 1)
        s += __shfl_xor(s, off, 64);
    if (fg == 0)
        sdz[qq] = s;
}

// With a decay gamma (the retention recurrence S_t = gamma S_{t-1} + Kf_t V_t^T of "Linear
// Attention Math", section "The kernel cousins: SSMs and RetNet"), a chunk of n valid keys updates
// S = gamma^n S + sum_j gamma^(n - 1 - j) Kf_j V_j^T (z alike): the V values of the product are
// weighted per key. Keys past the end weigh 0 (their staged rows are zero, and gamma^(n - 1 - j)
// would overflow there for gamma = 0).
__device__ __forceinline__ void decayed_values(float (&vbs)[2][4], const float (&vb)[2][4], float lg,
                                               int n, int g)
{
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = 16 * t + 4 * g + r;
            vbs[t][r] = key < n ? vb[t][r] * decay_pow(lg, n - 1 - key) : 0.f;
        }
}
template <int D>
__device__ __forceinline__ float key_col_sum_decayed(const float *kt, int f, float lg, int n)
{
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < CH / 4; ++j) {
        const f32x4 x = ld4(kt + f * C32<D>::TS + 4 * j);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = 4 * j + i;
            s = fmaf(x[i], key < n ? decay_pow(lg, n - 1 - key) : 0.f, s);
        }
    }
    return s;
}

// ---------------------------------------------------------------------------------------------
// Segment sums dS = Kf^T V, dz = colsum(Kf) over segments 0 .. nseg - 1 of each head (with a
// decay: decayed to the segment's last token).
// Twice the waves of the causal kernel: wave w owns the value columns 16 (w mod D/16) .. + 15 and
// the feature half w div (D/16) of S, so each SIMD runs four waves (measured on MI355X for the
// 2 x 16 x 8192 x 128 float32 sums: 82 us, against 87 us with D/16 waves owning whole columns).
template <int D> struct A32 {
    static constexpr int NCT = D / 16;       // value-column tiles
    static constexpr int NW = 2 * NCT;       // waves
    static constexpr int THREADS = NW * 64;
    static constexpr int NFH = D / 32;       // feature tiles per wave (half of S's rows)
};

template <int D, bool PHI, bool DECAY>
__global__ __launch_bounds__(A32<D>::THREADS) void k_agg32(const float *__restrict__ k,
                                                          const float *__restrict__ v,
                                                          float *__restrict__ dstS,
                                                          float *__restrict__ dstz, long sstride,
                                                          long zstride, int N, int L, int nseg,
                                                          int P, const float *__restrict__ gamma,
                                                          int H)
{
    using G = C32<D>;
    using A = A32<D>;
    using ST = Stage<D, A::THREADS>;
    __shared__ __attribute__((aligned(16))) float sKT[2][D * G::TS];
    __shared__ __attribute__((aligned(16))) float sV[2][CH * G::RS];
    const int tid = threadIdx.x, w = wave_index(), l = tid & 63, li = l & 15, g = l >> 4;
    const int p = blockIdx.x % nseg, bh = blockIdx.x / nseg;
    const int tb = p * L, te = min(N, tb + L), nch = (te - tb + CH - 1) / CH;
    const float *kh = k + (size_t)bh * N * D, *vh = v + (size_t)bh * N * D;
    const int c0 = 16 * (w % A::NCT), f0 = (D / 2) * (w / A::NCT);
    const ST stg(tid);
    const float lg = DECAY ? decay_log2(gamma, bh, H) : 0.f;

    f32x4 sacc[A::NFH];
#pragma unroll
    for (int ft = 0; ft < A::NFH; ++ft)
        sacc[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
    float zr = 0.f;

    f32x4 rk[ST::PER], rv[ST::PER];
    auto load = [&](int cc) {
        const int t0 = tb + min(cc, nch - 1) * CH;
        stg.keys(rk, kh, t0, te - t0);
        stg.rows(rv, vh, t0, te - t0);
    };
    auto put = [&](int b, int cc) {
        const int n = te - (tb + cc * CH);
        stg.template put_keys<PHI>(sKT[b], nullptr, rk, n);
        stg.template put_rows<false>(sV[b], rv, n);
    };
    load(0);
    put(0, 0);
    load(1);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const int b = c & 1;
        const float *kt = sKT[b] + f0 * G::TS;
        float vb[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                vb[t][r] = sV[b][(16 * t + 4 * g + r) * G::RS + c0 + li];
        if (DECAY) {
            const int n = min(CH, te - (tb + c * CH));
            const float gn = decay_pow(lg, n);
            float vbs[2][4];
            decayed_values(vbs, vb, lg, n, g);
#pragma unroll
            for (int ft = 0; ft < A::NFH; ++ft)
                sacc[ft] *= gn;
            update_state<D, A::NFH>(sacc, kt, vbs, li, g);
            if (tid < D)
                zr = fmaf(gn, zr, key_col_sum_decayed<D>(sKT[b], tid, lg, n));
        } else {
            update_state<D, A::NFH>(sacc, kt, vb, li, g);
            if (tid < D)
                zr += key_col_sum<D>(sKT[b], tid);
        }
        if (c + 1 < nch)
            put(b ^ 1, c + 1);
        load(c + 2);
        __syncthreads();
    }
    float *S = dstS + ((long)bh * P + p) * sstride;
#pragma unroll
    for (int ft = 0; ft < A::NFH; ++ft)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[(size_t)(f0 + 16 * ft + 4 * g + r) * D + c0 + li] = sacc[ft][r];
    if (tid < D)
        dstz[((long)bh * P + p) * zstride + tid] = zr;
}

// ---------------------------------------------------------------------------------------------
// Causal outputs of one segment of one head from its prefix state (or zero), and the final
// state from the last segment. F: F_IDENTITY (q, k are the features), F_UNNORM (no division).
template <int D, int F, bool DECAY>
__global__ __launch_bounds__(C32<D>::THREADS) void k_causal32(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    float *__restrict__ out, const float *__restrict__ preS, const float *__restrict__ prez,
    long pstride, long pzstride, float *__restrict__ Sout, float *__restrict__ zout, int N, int L,
    int P, const float *__restrict__ gamma, int H)
{
    using G = C32<D>;
    constexpr bool PHI = !(F & F_IDENTITY), NORM = !(F & F_UNNORM);
    constexpr int NW = G::NW, RS = G::RS, NFT = G::NFT, FQ = D / 4;
    __shared__ __attribute__((aligned(16))) float sQ[2][CH * RS];
    __shared__ __attribute__((aligned(16))) float sK[2][CH * RS];
    __shared__ __attribute__((aligned(16))) float sKT[2][D * G::TS];
    __shared__ __attribute__((aligned(16))) float sV[2][CH * RS];
    __shared__ __attribute__((aligned(16))) float sPart[4][3][64 * 4]; // partial score tiles
    __shared__ float sz[D];
    __shared__ float sdz[CH];

    const int tid = threadIdx.x, w = wave_index(), l = tid & 63, li = l & 15, g = l >> 4;
    const int p = blockIdx.x % P, bh = blockIdx.x / P;
    const int tb = p * L, te = min(N, tb + L), nch = (te - tb + CH - 1) / CH;
    const size_t hoff = (size_t)bh * N * D;
    const float *qh = q + hoff, *kh = k + hoff, *vh = v + hoff;
    float *oh = out + hoff;
    const int c0 = 16 * w;
    const Stage<D> stg(tid);
    const float lg = DECAY ? decay_log2(gamma, bh, H) : 0.f;

    // state before the segment: lane (g, li) of tile ft holds S[16 ft + 4 g + r][c0 + li]
    f32x4 sacc[NFT];
    {
        const float *S0 = preS ? preS + ((long)bh * P + p) * pstride : nullptr;
        const float *z0 = preS ? prez + ((long)bh * P + p) * pzstride : nullptr;
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[ft][r] = S0 ? S0[(size_t)(16 * ft + 4 * g + r) * D + c0 + li] : 0.f;
        if (tid < D)
            sz[tid] = z0 ? z0[tid] : 0.f;
    }

    f32x4 rq[Stage<D>::PER], rk[Stage<D>::PER], rv[Stage<D>::PER];
    auto load = [&](int cc) {
        const int t0 = tb + min(cc, nch - 1) * CH;
        stg.rows(rq, qh, t0, te - t0);
        stg.keys(rk, kh, t0, te - t0);
        stg.rows(rv, vh, t0, te - t0);
    };
    auto put = [&](int b, int cc) {
        const int n = te - (tb + cc * CH);
        stg.template put_rows<PHI>(sQ[b], rq, n);
        stg.template put_keys<PHI>(sKT[b], sK[b], rk, n);
        stg.template put_rows<false>(sV[b], rv, n);
    };
    load(0);
    put(0, 0);
    load(1);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const int b = c & 1;
        const float *Qb = sQ[b], *Kb = sK[b];

        // phase 1. Partial scores A^T[key][query] over features [w D/4, (w + 1) D/4): tiles
        // (key tile, query tile) = (0, 0), (0, 1), (1, 1); keys 16-31 never reach queries 0-15.
        if (w < 4) {
            f32x4 pa[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int fb = w * FQ; fb < (w + 1) * FQ; fb += 16) {
                const f32x4 k0 = ld4(Kb + li * RS + fb + 4 * g), k1 = ld4(Kb + (16 + li) * RS + fb + 4 * g);
                const f32x4 q0 = ld4(Qb + li * RS + fb + 4 * g), q1 = ld4(Qb + (16 + li) * RS + fb + 4 * g);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pa[0] = mma(k0[j], q0[j], pa[0]);
                    pa[1] = mma(k0[j], q1[j], pa[1]);
                    pa[2] = mma(k1[j], q1[j], pa[2]);
                }
            }
#pragma unroll
            for (int t = 0; t < 3; ++t)
                st4(&sPart[w][t][4 * l], pa[t]);
        }
        // num = Qf S for query tiles 0 and 1 (the state before this chunk)
        f32x4 num[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
            const f32x4 a0 = ld4(Qb + li * RS + 16 * ft + 4 * g);
            const f32x4 a1 = ld4(Qb + (16 + li) * RS + 16 * ft + 4 * g);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                num[0] = mma(a0[j], sacc[ft][j], num[0]);
                num[1] = mma(a1[j], sacc[ft][j], num[1]);
            }
        }
        // Qf z for the chunk's queries
        if (NORM)
            chunk_qz<D, NW>(sdz, Qb, sz, w, l);
        __syncthreads();

        // phase 2. Scores: the four partial tiles in order, then the causal mask on the
        // diagonal tiles (lane (g, li) holds keys 4 g + r of query li)
        f32x4 at[3];
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            at[t] = ld4(&sPart[0][t][4 * l]);
#pragma unroll
            for (int ww = 1; ww < 4; ++ww)
                at[t] += ld4(&sPart[ww][t][4 * l]);
        }
        if (DECAY) {
            // key 16 kt + 4 g + r reaches query 16 qt + li with weight gamma^(query - key), keys
            // after the query none; the carried state reaches row i scaled by gamma^(i + 1)
            constexpr int KTI[3] = {0, 0, 1}, QTI[3] = {0, 1, 1};
#pragma unroll
            for (int t = 0; t < 3; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int dq = 16 * QTI[t] + li - (16 * KTI[t] + 4 * g + r);
                    at[t][r] = dq >= 0 ? at[t][r] * decay_pow(lg, dq) : 0.f;
                }
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    num[t][r] *= decay_pow(lg, 16 * t + 4 * g + r + 1);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (4 * g + r > li) {
                    at[0][r] = 0.f;
                    at[2][r] = 0.f;
                }
        }
        float vb[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                vb[t][r] = sV[b][(16 * t + 4 * g + r) * RS + c0 + li];
        // num += A V: step r of key tile t gives lane group g the key 16 t + 4 g + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            num[0] = mma(at[0][r], vb[0][r], num[0]);
            num[1] = mma(at[1][r], vb[0][r], num[1]);
            num[1] = mma(at[2][r], vb[1][r], num[1]);
        }
        // den of query li (tile 0) and 16 + li (tile 1), then moved to the output layout
        // (lane (g, li) holds queries 4 g + r)
        float inv[2][4];
        if (NORM) {
            float d0 = (at[0][0] + at[0][1]) + (at[0][2] + at[0][3]);
            float d1 = ((at[1][0] + at[1][1]) + (at[1][2] + at[1][3])) +
                       ((at[2][0] + at[2][1]) + (at[2][2] + at[2][3]));
            d0 += __shfl_xor(d0, 16, 64);
            d1 += __shfl_xor(d1, 16, 64);
            d0 += __shfl_xor(d0, 32, 64);
            d1 += __shfl_xor(d1, 32, 64);
            const float z0 = DECAY ? sdz[li] * decay_pow(lg, li + 1) : sdz[li];
            const float z1 = DECAY ? sdz[16 + li] * decay_pow(lg, 17 + li) : sdz[16 + li];
            const float i0 = 1.f / (d0 + z0), i1 = 1.f / (d1 + z1);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                inv[0][r] = __shfl(i0, 4 * g + r, 64);
                inv[1][r] = __shfl(i1, 4 * g + r, 64);
            }
        }
        const int t0 = tb + c * CH, n = te - t0;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * t + 4 * g + r;
                if (row < n)
                    oh[(size_t)(t0 + row) * D + c0 + li] = NORM ? num[t][r] * inv[t][r] : num[t][r];
            }
        if (DECAY) {
            const int nk = min(CH, n);
            const float gn = decay_pow(lg, nk);
            float vbs[2][4];
            decayed_values(vbs, vb, lg, nk, g);
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft)
                sacc[ft] *= gn;
            update_state<D, NFT>(sacc, sKT[b], vbs, li, g);
            if (tid < D)
                sz[tid] = fmaf(gn, sz[tid], key_col_sum_decayed<D>(sKT[b], tid, lg, nk));
        } else {
            update_state<D, NFT>(sacc, sKT[b], vb, li, g);
            if (tid < D)
                sz[tid] += key_col_sum<D>(sKT[b], tid);
        }
        if (c + 1 < nch)
            put(b ^ 1, c + 1);
        load(c + 2);
        __syncthreads();
    }
    if (Sout && p == P - 1) {
        float *So = Sout + (size_t)bh * D * D;
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                So[(size_t)(16 * ft + 4 * g + r) * D + c0 + li] = sacc[ft][r];
        if (tid < D)
            zout[(size_t)bh * D + tid] = sz[tid];
    }
}

// The causal kernel with twice the waves (four per SIMD): wave w owns the value columns
// 16 (w mod D/16) .. + 15 and the feature half fh = w div (D/16) of S, and writes the outputs of
// query tile fh. In phase 1 it forms Qf S over its features for both query tiles and leaves
// the other tile's partial in LDS for the wave with the same columns and the other half; in
// phase 2 it adds that partial (features 0 .. D/2 - 1 first), the scores and the division for
// its query tile, and updates its half of S. The scores read K from the feature-major array
// (the row-major copy is left out, so the LDS still holds one workgroup).
template <int D> struct C32H {
    static constexpr int NCT = D / 16;
    static constexpr int NW = 2 * NCT;
    static constexpr int THREADS = NW * 64;
    static constexpr int NFH = D / 32;       // feature tiles per wave
};

template <int D, int F, bool DECAY>
__global__ __launch_bounds__(C32H<D>::THREADS) void k_causal32h(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    float *__restrict__ out, const float *__restrict__ preS, const float *__restrict__ prez,
    long pstride, long pzstride, float *__restrict__ Sout, float *__restrict__ zout, int N, int L,
    int P, const float *__restrict__ gamma, int H)
{
    using G = C32<D>;
    using W2 = C32H<D>;
    using ST = Stage<D, W2::THREADS>;
    constexpr bool PHI = !(F & F_IDENTITY), NORM = !(F & F_UNNORM);
    constexpr int NW = W2::NW, RS = G::RS, TS = G::TS, NFH = W2::NFH, FQ = D / 4;
    __shared__ __attribute__((aligned(16))) float sQ[2][CH * RS];
    __shared__ __attribute__((aligned(16))) float sKT[2][D * TS];
    __shared__ __attribute__((aligned(16))) float sV[2][CH * RS];
    __shared__ __attribute__((aligned(16))) float sPart[4][3][64 * 4]; // partial score tiles
    __shared__ __attribute__((aligned(16))) float sNum[NW][64 * 4];    // partial Qf S handed over
    __shared__ float sz[D];
    __shared__ float sdz[CH];

    const int tid = threadIdx.x, w = wave_index(), l = tid & 63, li = l & 15, g = l >> 4;
    const int fh = w / W2::NCT, c0 = 16 * (w % W2::NCT), f0 = fh * (D / 2);
    const int partner = (w + W2::NCT) % NW;
    const int p = blockIdx.x % P, bh = blockIdx.x / P;
    const int tb = p * L, te = min(N, tb + L), nch = (te - tb + CH - 1) / CH;
    const size_t hoff = (size_t)bh * N * D;
    const float *qh = q + hoff, *kh = k + hoff, *vh = v + hoff;
    float *oh = out + hoff;
    const ST stg(tid);
    const float lg = DECAY ? decay_log2(gamma, bh, H) : 0.f;

    // this wave's part of the state: lane (g, li) of tile ft holds S[f0 + 16 ft + 4 g + r][c0 + li]
    f32x4 sacc[NFH];
    {
        const float *S0 = preS ? preS + ((long)bh * P + p) * pstride : nullptr;
        const float *z0 = preS ? prez + ((long)bh * P + p) * pzstride : nullptr;
#pragma unroll
        for (int ft = 0; ft < NFH; ++ft)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[ft][r] = S0 ? S0[(size_t)(f0 + 16 * ft + 4 * g + r) * D + c0 + li] : 0.f;
        if (tid < D)
            sz[tid] = z0 ? z0[tid] : 0.f;
    }

    f32x4 rq[ST::PER], rk[ST::PER], rv[ST::PER];
    auto load = [&](int cc) {
        const int t0 = tb + min(cc, nch - 1) * CH;
        stg.rows(rq, qh, t0, te - t0);
        stg.keys(rk, kh, t0, te - t0);
        stg.rows(rv, vh, t0, te - t0);
    };
    auto put = [&](int b, int cc) {
        const int n = te - (tb + cc * CH);
        stg.template put_rows<PHI>(sQ[b], rq, n);
        stg.template put_keys<PHI>(sKT[b], nullptr, rk, n);
        stg.template put_rows<false>(sV[b], rv, n);
    };
    load(0);
    put(0, 0);
    load(1);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const int b = c & 1;
        const float *Qb = sQ[b], *KTb = sKT[b];

        // phase 1. Partial scores A^T over features [w D/4, (w + 1) D/4) (waves 0-3, one per
        // SIMD); the key operand comes from the feature-major array, four single reads per block
        if (w < 4) {
            f32x4 pa[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int fb = w * FQ; fb < (w + 1) * FQ; fb += 16) {
                f32x4 k0, k1;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    k0[j] = KTb[(fb + 4 * g + j) * TS + li];
                    k1[j] = KTb[(fb + 4 * g + j) * TS + 16 + li];
                }
                const f32x4 q0 = ld4(Qb + li * RS + fb + 4 * g), q1 = ld4(Qb + (16 + li) * RS + fb + 4 * g);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pa[0] = mma(k0[j], q0[j], pa[0]);
                    pa[1] = mma(k0[j], q1[j], pa[1]);
                    pa[2] = mma(k1[j], q1[j], pa[2]);
                }
            }
#pragma unroll
            for (int t = 0; t < 3; ++t)
                st4(&sPart[w][t][4 * l], pa[t]);
        }
        // Qf S over this wave's features, both query tiles; the other tile's part is handed over
        f32x4 num[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ft = 0; ft < NFH; ++ft) {
            const f32x4 a0 = ld4(Qb + li * RS + f0 + 16 * ft + 4 * g);
            const f32x4 a1 = ld4(Qb + (16 + li) * RS + f0 + 16 * ft + 4 * g);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                num[0] = mma(a0[j], sacc[ft][j], num[0]);
                num[1] = mma(a1[j], sacc[ft][j], num[1]);
            }
        }
        st4(&sNum[w][4 * l], fh ? num[0] : num[1]);
        const f32x4 mine = fh ? num[1] : num[0]; // (only this tile's part lives across the barrier)
        if (NORM)
            chunk_qz<D, NW>(sdz, Qb, sz, w, l);
        __syncthreads();

        // phase 2, query tile fh: Qf S with both feature halves (half 0 first)
        const f32x4 other = ld4(&sNum[partner][4 * l]);
        f32x4 acc = fh ? other + mine : mine + other;
        f32x4 at[3];
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            at[t] = ld4(&sPart[0][t][4 * l]);
#pragma unroll
            for (int ww = 1; ww < 4; ++ww)
                at[t] += ld4(&sPart[ww][t][4 * l]);
        }
        if (DECAY) {
            constexpr int KTI[3] = {0, 0, 1}, QTI[3] = {0, 1, 1};
#pragma unroll
            for (int t = 0; t < 3; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int dq = 16 * QTI[t] + li - (16 * KTI[t] + 4 * g + r);
                    at[t][r] = dq >= 0 ? at[t][r] * decay_pow(lg, dq) : 0.f;
                }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[r] *= decay_pow(lg, 16 * fh + 4 * g + r + 1);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (4 * g + r > li) {
                    at[0][r] = 0.f;
                    at[2][r] = 0.f;
                }
        }
        float vb[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                vb[t][r] = sV[b][(16 * t + 4 * g + r) * RS + c0 + li];
        // num += A V for query tile fh (wave-uniform branch)
        if (fh == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc = mma(at[0][r], vb[0][r], acc);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc = mma(at[1][r], vb[0][r], acc);
                acc = mma(at[2][r], vb[1][r], acc);
            }
        }
        float inv[4];
        if (NORM) {
            float dn = fh ? ((at[1][0] + at[1][1]) + (at[1][2] + at[1][3])) +
                                ((at[2][0] + at[2][1]) + (at[2][2] + at[2][3]))
                          : (at[0][0] + at[0][1]) + (at[0][2] + at[0][3]);
            dn += __shfl_xor(dn, 16, 64);
            dn += __shfl_xor(dn, 32, 64);
            const int qi = 16 * fh + li;
            const float zq = DECAY ? sdz[qi] * decay_pow(lg, qi + 1) : sdz[qi];
            const float iv = 1.f / (dn + zq);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                inv[r] = __shfl(iv, 4 * g + r, 64);
        }
        const int t0 = tb + c * CH, n = te - t0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * fh + 4 * g + r;
            if (row < n)
                oh[(size_t)(t0 + row) * D + c0 + li] = NORM ? acc[r] * inv[r] : acc[r];
        }
        const float *kt = KTb + f0 * TS;
        if (DECAY) {
            const int nk = min(CH, n);
            const float gn = decay_pow(lg, nk);
            float vbs[2][4];
            decayed_values(vbs, vb, lg, nk, g);
#pragma unroll
            for (int ft = 0; ft < NFH; ++ft)
                sacc[ft] *= gn;
            update_state<D, NFH>(sacc, kt, vbs, li, g);
            if (tid < D)
                sz[tid] = fmaf(gn, sz[tid], key_col_sum_decayed<D>(KTb, tid, lg, nk));
        } else {
            update_state<D, NFH>(sacc, kt, vb, li, g);
            if (tid < D)
                sz[tid] += key_col_sum<D>(KTb, tid);
        }
        if (c + 1 < nch)
            put(b ^ 1, c + 1);
        load(c + 2);
        __syncthreads();
    }
    if (Sout && p == P - 1) {
        float *So = Sout + (size_t)bh * D * D;
#pragma unroll
        for (int ft = 0; ft < NFH; ++ft)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                So[(size_t)(f0 + 16 * ft + 4 * g + r) * D + c0 + li] = sacc[ft][r];
        if (tid < D)
            zout[(size_t)bh * D + tid] = sz[tid];
    }
}

// ---------------------------------------------------------------------------------------------
// Global read out = Qf S / Qf z over one segment of rows of one head. The outputs of chunk c
// are stored after the barrier that ends it (Qf z from the last wave is visible there; the
// per-chunk Qf z is double-buffered), so each chunk takes one barrier.
template <int D, int F>
__global__ __launch_bounds__(C32<D>::THREADS) void k_gread32(const float *__restrict__ q,
                                                            float *__restrict__ out,
                                                            const float *__restrict__ S,
                                                            const float *__restrict__ z, int N,
                                                            int L, int P)
{
    using G = C32<D>;
    constexpr bool PHI = !(F & F_IDENTITY), NORM = !(F & F_UNNORM);
    constexpr int NW = G::NW, RS = G::RS, NFT = G::NFT;
    __shared__ __attribute__((aligned(16))) float sQ[2][CH * RS];
    __shared__ __attribute__((aligned(16))) float sz[D];
    __shared__ float sdz[2][CH];

    const int tid = threadIdx.x, w = wave_index(), l = tid & 63, li = l & 15, g = l >> 4;
    const int p = blockIdx.x % P, bh = blockIdx.x / P;
    const int tb = p * L, te = min(N, tb + L), nch = (te - tb + CH - 1) / CH;
    const size_t hoff = (size_t)bh * N * D;
    const float *qh = q + hoff;
    float *oh = out + hoff;
    const int c0 = 16 * w;
    const Stage<D> stg(tid);

    f32x4 sacc[NFT];
    {
        const float *Sh = S + (size_t)bh * D * D;
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[ft][r] = Sh[(size_t)(16 * ft + 4 * g + r) * D + c0 + li];
        if (tid < D)
            sz[tid] = z[(size_t)bh * D + tid];
    }
    f32x4 rq[Stage<D>::PER];
    auto load = [&](int cc) {
        const int t0 = tb + min(cc, nch - 1) * CH;
        stg.rows(rq, qh, t0, te - t0);
    };
    load(0);
    stg.template put_rows<PHI>(sQ[0], rq, te - tb);
    load(1);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const int b = c & 1;
        const float *Qb = sQ[b];
        f32x4 num[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
            const f32x4 a0 = ld4(Qb + li * RS + 16 * ft + 4 * g);
            const f32x4 a1 = ld4(Qb + (16 + li) * RS + 16 * ft + 4 * g);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                num[0] = mma(a0[j], sacc[ft][j], num[0]);
                num[1] = mma(a1[j], sacc[ft][j], num[1]);
            }
        }
        if (NORM)
            chunk_qz<D, NW>(sdz[b], Qb, sz, w, l);
        if (c + 1 < nch)
            stg.template put_rows<PHI>(sQ[b ^ 1], rq, te - (tb + (c + 1) * CH));
        load(c + 2);
        __syncthreads();
        const int t0 = tb + c * CH, n = te - t0;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * t + 4 * g + r;
                if (row < n)
                    oh[(size_t)(t0 + row) * D + c0 + li] = NORM ? num[t][r] / sdz[b][row] : num[t][r];
            }
    }
}

template <int D, int F>
void launch_causal32_f(dim3 grid, hipStream_t st, const float *q, const float *k, const float *v,
                       float *o, const float *preS, const float *prez, long ps, long pzs,
                       float *Sout, float *zout, int N, int L, int P, const float *gamma, int H)
{
    // the decayed form keeps D/16 waves: its extra registers do not fit the 128 of four waves
    // per SIMD (152 bytes per lane spilled at D = 128)
    if (gamma)
        hipLaunchKernelGGL((k_causal32<D, F, true>), grid, dim3(C32<D>::THREADS), 0, st, q, k, v, o, preS, prez, ps, pzs, Sout, zout, N, L, P, gamma, H);
    else
        hipLaunchKernelGGL((k_causal32h<D, F, false>), grid, dim3(C32H<D>::THREADS), 0, st, q, k, v, o, preS, prez, ps, pzs, Sout, zout, N, L, P, gamma, H);
}

template <int D>
void launch_causal32(int flags, dim3 grid, hipStream_t st, const float *q, const float *k,
                     const float *v, float *o, const float *preS, const float *prez, long ps,
                     long pzs, float *Sout, float *zout, int N, int L, int P, const float *gamma,
                     int H)
{
    switch (flags & (F_IDENTITY | F_UNNORM)) {
    case 0: launch_causal32_f<D, 0>(grid, st, q, k, v, o, preS, prez, ps, pzs, Sout, zout, N, L, P, gamma, H); break;
    case F_IDENTITY: launch_causal32_f<D, F_IDENTITY>(grid, st, q, k, v, o, preS, prez, ps, pzs, Sout, zout, N, L, P, gamma, H); break;
    case F_UNNORM: launch_causal32_f<D, F_UNNORM>(grid, st, q, k, v, o, preS, prez, ps, pzs, Sout, zout, N, L, P, gamma, H); break;
    default: launch_causal32_f<D, F_IDENTITY | F_UNNORM>(grid, st, q, k, v, o, preS, prez, ps, pzs, Sout, zout, N, L, P, gamma, H); break;
    }
}

template <int D, bool PHI>
void launch_agg32_f(dim3 grid, hipStream_t st, const float *k, const float *v, float *dstS,
                    float *dstz, long sstride, long zstride, int N, int L, int nseg, int P,
                    const float *gamma, int H)
{
    const dim3 block(A32<D>::THREADS);
    if (gamma)
        hipLaunchKernelGGL((k_agg32<D, PHI, true>), grid, block, 0, st, k, v, dstS, dstz, sstride, zstride, N, L, nseg, P, gamma, H);
    else
        hipLaunchKernelGGL((k_agg32<D, PHI, false>), grid, block, 0, st, k, v, dstS, dstz, sstride, zstride, N, L, nseg, P, gamma, H);
}

template <int D>
void launch_gread32(int flags, dim3 grid, hipStream_t st, const float *q, float *o, const float *S,
                    const float *z, int N, int L, int P)
{
    const dim3 block(C32<D>::THREADS);
    switch (flags & (F_IDENTITY | F_UNNORM)) {
    case 0: hipLaunchKernelGGL((k_gread32<D, 0>), grid, block, 0, st, q, o, S, z, N, L, P); break;
    case F_IDENTITY: hipLaunchKernelGGL((k_gread32<D, F_IDENTITY>), grid, block, 0, st, q, o, S, z, N, L, P); break;
    case F_UNNORM: hipLaunchKernelGGL((k_gread32<D, F_UNNORM>), grid, block, 0, st, q, o, S, z, N, L, P); break;
    default: hipLaunchKernelGGL((k_gread32<D, F_IDENTITY | F_UNNORM>), grid, block, 0, st, q, o, S, z, N, L, P); break;
    }
}

} // namespace

hipError_t agg_mfma32(int D, int flags, const void *k, const void *v, float *dstS, float *dstz,
                      long sstride, long zstride, int BH, int N, int L, int nseg, int P,
                      const float *gamma, int H, hipStream_t st)
{
    const dim3 grid((unsigned)(BH * nseg));
    const auto *kk = static_cast<const float *>(k);
    const auto *vv = static_cast<const float *>(v);
    const bool phi = !(flags & F_IDENTITY);
    if (D == 128) {
        if (phi)
            launch_agg32_f<128, true>(grid, st, kk, vv, dstS, dstz, sstride, zstride, N, L, nseg, P, gamma, H);
        else
            launch_agg32_f<128, false>(grid, st, kk, vv, dstS, dstz, sstride, zstride, N, L, nseg, P, gamma, H);
    } else {
        if (phi)
            launch_agg32_f<64, true>(grid, st, kk, vv, dstS, dstz, sstride, zstride, N, L, nseg, P, gamma, H);
        else
            launch_agg32_f<64, false>(grid, st, kk, vv, dstS, dstz, sstride, zstride, N, L, nseg, P, gamma, H);
    }
    return hipGetLastError();
}

hipError_t causal_mfma32(int D, int flags, const void *q, const void *k, const void *v, void *out,
                         const float *preS, const float *prez, long pstride, long pzstride,
                         float *Sout, float *zout, int BH, int N, int L, int P, const float *gamma,
                         int H, hipStream_t st)
{
    const dim3 grid((unsigned)(BH * P));
    const auto *qq = static_cast<const float *>(q);
    const auto *kk = static_cast<const float *>(k);
    const auto *vv = static_cast<const float *>(v);
    auto *oo = static_cast<float *>(out);
    if (D == 128)
        launch_causal32<128>(flags, grid, st, qq, kk, vv, oo, preS, prez, pstride, pzstride, Sout, zout, N, L, P, gamma, H);
    else
        launch_causal32<64>(flags, grid, st, qq, kk, vv, oo, preS, prez, pstride, pzstride, Sout, zout, N, L, P, gamma, H);
    return hipGetLastError();
}

hipError_t global_read_mfma32(int D, int flags, const void *q, void *out, const float *S,
                              const float *z, int BH, int N, hipStream_t st)
{
    // the read takes its own split: about two workgroups per CU, whole chunks per segment
    const long want = 2 * 256;
    const long pr = (want + BH - 1) / BH;
    const long nch = (N + CH - 1) / CH;
    const int L = (int)((nch + pr - 1) / pr) * CH;
    const int P = (N + L - 1) / L;
    const dim3 grid((unsigned)(BH * P));
    const auto *qq = static_cast<const float *>(q);
    auto *oo = static_cast<float *>(out);
    if (D == 128)
        launch_gread32<128>(flags, grid, st, qq, oo, S, z, N, L, P);
    else
        launch_gread32<64>(flags, grid, st, qq, oo, S, z, N, L, P);
    return hipGetLastError();
}

} // namespace la
