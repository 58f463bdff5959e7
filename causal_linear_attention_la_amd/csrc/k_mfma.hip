// k_mfma.hip -- matrix-core kernels of liblinattn: bf16 inputs, d == d_v = D in {64, 128},
// chunks of C = 64 tokens, 256 threads (4 wave64s) per workgroup, gfx950 MFMA
// v_mfma_f32_16x16x32_bf16 with float32 accumulation.
//
// Chunked causal evaluation (the within-chunk part plus the state carried from earlier chunks,
// as "Linear Attention: From Pairwise Reads to a Recurrent State", section "A recurrence need
// not force token-serial training", describes). For a chunk c of tokens with mapped features
// Qf = phi(Q_c), Kf = phi(K_c) and values V_c, and the state S, z before the chunk:
//   A       = mask_{j <= i}(Qf Kf^T)                     (C x C, inclusive: token i sees itself)
//   num     = A V_c + Qf S,    den = rowsum(A) + Qf z    (the recurrence's read, all rows at once)
//   out     = num / den
//   S, z   += Kf^T V_c, colsum(Kf)                       (the recurrence's write, summed over c)
// which is the recurrence S_i = S_{i-1} + phi(k_i) v_i^T, z_i = z_{i-1} + phi(k_i),
// o_i = phi(q_i)^T S_i / phi(q_i)^T z_i of "Linear Attention Math", section "The recurrent
// form: a running KV state", regrouped by associativity.
//
// MFMA 16x16x32 operand layout used throughout (lane l, li = l % 16, g = l / 16):
//   A operand: row li, k-slots 8g..8g+7      B operand: column li, k-slots 8g..8g+7
//   C/D:       column li, rows 4g..4g+3
// Any per-lane permutation of the k-slots is allowed as long as A and B use the same one; the
// state read uses the permutation {4g..4g+3, 16+4g..16+4g+3}, which is exactly how an
// accumulator pair holds a 32-row block, so the float32 state S never goes through LDS.
//
// Work split inside a workgroup: wave w owns value columns [w*D/4, (w+1)*D/4) of the state S
// (all D feature rows, in accumulators) and of the outputs; for the C x C score block wave w
// computes query rows 16w..16w+15.
#include "la_device.h"
#include "la_launch.h"

namespace la {
namespace {

constexpr int C = 64;   // tokens per chunk
constexpr int NT = 256; // threads per workgroup

template <int D> struct Cfg {
    static constexpr int TM = C * D / (8 * NT); // tokens per loader micro-tile (4 or 2)
    static constexpr int TG = C / TM;           // token groups per chunk
    static constexpr int LA = TG / 4;           // token groups per wave
    static constexpr int QS = D + 8;            // row stride (elements) of sQ, sK
    static constexpr int TS = C + 8;            // row stride of sKT, sVT, sA
    static constexpr int NCT = D / 64;          // 16-wide column tiles owned by one wave
    static constexpr int NFT = D / 16;          // 16-row feature tiles of S
    static constexpr int NKB = D / 32;          // 32-feature k blocks
    static_assert(TM == 2 || TM == 4, "loader micro-tile");
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <typename T> __device__ __forceinline__ T lds(const uint16_t *p)
{
    return *reinterpret_cast<const T *>(p);
}
template <typename T> __device__ __forceinline__ void sts(uint16_t *p, T x)
{
    *reinterpret_cast<T *>(p) = x;
}

// Element index of (row f, token j) in a token-contiguous [D][TS] array. Tokens are grouped
// in 8-byte granules of 4; the granule index is XOR-swizzled by an even value taken from the
// row so that the transposing stores below spread over all LDS banks, while 16-byte reads of
// 8 consecutive tokens (an even granule pair) stay contiguous.
template <int D> __device__ __forceinline__ int tix(int f, int j)
{
    return f * Cfg<D>::TS + ((((j >> 2) ^ ((f >> 3) & 14))) << 2) + (j & 3);
}

// φ applied to 8 packed bf16 values, result rounded to bf16 (nearest even).
__device__ __forceinline__ u32x4 phi8(u32x4 x)
{
    u32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        y[i] = pack_bf2(phi_fast(bf_lo(x[i])), phi_fast(bf_hi(x[i])));
    return y;
}

// Each thread owns a micro-tile of TM consecutive tokens x 8 consecutive features of a
// [C, D] chunk. Within a wave the TM-row groups vary fastest, so one load instruction reads
// whole 2*D-byte rows.
template <int D> struct Tile {
    using K = Cfg<D>;
    int a, b; // token group, feature group
    __device__ explicit Tile(int tid)
    {
        const int w = tid >> 6, l = tid & 63;
        a = K::LA * w + (l % K::LA);
        b = l / K::LA;
    }
    // rows of the chunk starting at `base`, clamped to the chunk's last valid row so every
    // access is in bounds and no load sits in a branch (a load merged with a zero in a branch
    // makes the compiler wait for it right away); rows past nvalid are masked when staged.
    __device__ __forceinline__ void load(u32x4 (&r)[K::TM], const uint16_t *__restrict__ base,
                                         int nvalid) const
    {
#pragma unroll
        for (int i = 0; i < K::TM; ++i) {
            const int row = min(K::TM * a + i, nvalid - 1);
            r[i] = *reinterpret_cast<const u32x4 *>(base + (size_t)row * D + 8 * b);
        }
    }
    __device__ __forceinline__ bool valid(int i, int nvalid) const { return K::TM * a + i < nvalid; }
    // natural [C][QS] layout
    __device__ __forceinline__ void store_rows(uint16_t *s, const u32x4 (&r)[K::TM]) const
    {
#pragma unroll
        for (int i = 0; i < K::TM; ++i)
            sts<u32x4>(s + (K::TM * a + i) * K::QS + 8 * b, r[i]);
    }
    // transposed [D][TS] layout: feature row 8b+e receives the TM tokens of this micro-tile
    __device__ __forceinline__ void store_cols(uint16_t *s, const u32x4 (&r)[K::TM]) const
    {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int sh = 16 * (e & 1);
            uint32_t h[K::TM];
#pragma unroll
            for (int i = 0; i < K::TM; ++i)
                h[i] = (r[i][e >> 1] >> sh) & 0xffffu;
            const int f = 8 * b + e;
            if constexpr (K::TM == 4)
                sts<u32x2>(s + tix<D>(f, 4 * a), u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)});
            else
                sts<uint32_t>(s + tix<D>(f, 2 * a), h[0] | (h[1] << 16));
        }
    }
};

// S += Kf^T V over one chunk for the columns this wave owns. sacc[ft][ct]: rows
// f = 16ft + 4g + r, column cw0 + 16ct + li.
template <int D>
__device__ __forceinline__ void state_update(f32x4 (&sacc)[Cfg<D>::NFT][Cfg<D>::NCT],
                                             const uint16_t *sKT, const uint16_t *sVT, int cw0,
                                             int li, int g)
{
    using K = Cfg<D>;
#pragma unroll
    for (int m = 0; m < C / 32; ++m) {
        bf16x8 bv[K::NCT];
#pragma unroll
        for (int ct = 0; ct < K::NCT; ++ct)
            bv[ct] = lds<bf16x8>(sVT + tix<D>(cw0 + 16 * ct + li, 32 * m + 8 * g));
#pragma unroll
        for (int ft = 0; ft < K::NFT; ++ft) {
            const bf16x8 ak = lds<bf16x8>(sKT + tix<D>(16 * ft + li, 32 * m + 8 * g));
#pragma unroll
            for (int ct = 0; ct < K::NCT; ++ct)
                sacc[ft][ct] = mfma(ak, bv[ct], sacc[ft][ct]);
        }
    }
}

// Column sums of Kf over one chunk (threads 0..2D-1: feature tid/2, half tid%2 of the chunk).
template <int D> __device__ __forceinline__ float kf_colsum_half(const uint16_t *sKT, int tid)
{
    float s = 0.f;
    if (tid < 2 * D) {
        const int f = tid >> 1, h = tid & 1;
#pragma unroll
        for (int i = 0; i < C / 16; ++i) {
            const u32x4 w = lds<u32x4>(sKT + tix<D>(f, (C / 2) * h + 8 * i));
#pragma unroll
            for (int e = 0; e < 4; ++e)
                s += bf_lo(w[e]) + bf_hi(w[e]);
        }
    }
    return s;
}

// bf16 A-operand fragments of S^T for the state read (k = feature, permuted as
// {4g..4g+3, 16+4g..16+4g+3} within each 32-feature block m).
template <int D>
__device__ __forceinline__ void state_frags(bf16x8 (&sf)[Cfg<D>::NCT][Cfg<D>::NKB],
                                            const f32x4 (&sacc)[Cfg<D>::NFT][Cfg<D>::NCT])
{
    using K = Cfg<D>;
#pragma unroll
    for (int ct = 0; ct < K::NCT; ++ct)
#pragma unroll
        for (int m = 0; m < K::NKB; ++m) {
            const f32x4 lo = sacc[2 * m][ct], hi = sacc[2 * m + 1][ct];
            const u32x4 w = {pack_bf2(lo[0], lo[1]), pack_bf2(lo[2], lo[3]), pack_bf2(hi[0], hi[1]),
                             pack_bf2(hi[2], hi[3])};
            sf[ct][m] = __builtin_bit_cast(bf16x8, w);
        }
}

// num^T += S^T Qf^T for the wave's columns and all C query rows. acc[ct][it]: rows (value
// columns) cw0 + 16ct + 4g + r, column (query) 16it + li.
template <int D>
__device__ __forceinline__ void state_read(f32x4 (&acc)[Cfg<D>::NCT][4],
                                           const bf16x8 (&sf)[Cfg<D>::NCT][Cfg<D>::NKB],
                                           const uint16_t *sQ, int li, int g)
{
    using K = Cfg<D>;
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int m = 0; m < K::NKB; ++m) {
            const uint16_t *row = sQ + (16 * it + li) * K::QS + 32 * m + 4 * g;
            const u32x2 q0 = lds<u32x2>(row), q1 = lds<u32x2>(row + 16);
            const bf16x8 bq = __builtin_bit_cast(bf16x8, u32x4{q0[0], q0[1], q1[0], q1[1]});
#pragma unroll
            for (int ct = 0; ct < K::NCT; ++ct)
                acc[ct][it] = mfma(sf[ct][m], bq, acc[ct][it]);
        }
}

// out rows [0, nvalid) of the chunk at `ob`: out = num / den, rounded to bf16.
template <int D>
__device__ __forceinline__ void store_out(const f32x4 (&acc)[Cfg<D>::NCT][4], const float *sden,
                                          uint16_t *__restrict__ ob, int nvalid, int cw0, int li,
                                          int g)
{
    using K = Cfg<D>;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int i = 16 * it + li;
        if (i < nvalid) {
            const float inv = __builtin_amdgcn_rcpf(sden[i]);
#pragma unroll
            for (int ct = 0; ct < K::NCT; ++ct) {
                const f32x4 a = acc[ct][it];
                const u32x2 w = {pack_bf2(a[0] * inv, a[1] * inv), pack_bf2(a[2] * inv, a[3] * inv)};
                *reinterpret_cast<u32x2 *>(ob + (size_t)i * D + cw0 + 16 * ct + 4 * g) = w;
            }
        }
    }
}

// sdi[i] = phi(Q)[i] . z for the C rows of a staged chunk (256 threads: row tid/4, a quarter of
// the features each).
template <int D>
__device__ __forceinline__ void den_inter(float *sdi, const uint16_t *sQ, const float *sz, int tid)
{
    using K = Cfg<D>;
    const int i = tid >> 2, qq = tid & 3;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < D / 32; ++e) {
        const int f = qq * (D / 4) + 8 * e;
        const u32x4 qw = lds<u32x4>(sQ + i * K::QS + f);
#pragma unroll
        for (int h = 0; h < 4; ++h)
            s += bf_lo(qw[h]) * sz[f + 2 * h] + bf_hi(qw[h]) * sz[f + 2 * h + 1];
    }
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    if (qq == 0)
        sdi[i] = s;
}

// ------------------------------------------------------------------------------------------
// Segment sums: dS = phi(K_seg)^T V_seg, dz = colsum phi(K_seg).
template <int D>
__global__ __launch_bounds__(NT) void k_agg(const uint16_t *__restrict__ k,
                                            const uint16_t *__restrict__ v,
                                            float *__restrict__ dstS, float *__restrict__ dstz,
                                            long sstride, long zstride, int N, int L, int nseg,
                                            int P)
{
    using K = Cfg<D>;
    __shared__ __attribute__((aligned(16))) uint16_t sKT[D * K::TS];
    __shared__ __attribute__((aligned(16))) uint16_t sVT[D * K::TS];

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, g = l >> 4;
    const int p = blockIdx.x % nseg, bh = blockIdx.x / nseg;
    const int tb = p * L, te = min(N, tb + L);
    const uint16_t *kb = k + (size_t)bh * N * D;
    const uint16_t *vb = v + (size_t)bh * N * D;
    const int cw0 = w * (D / 4);
    const Tile<D> tile(tid);

    f32x4 sacc[K::NFT][K::NCT];
#pragma unroll
    for (int ft = 0; ft < K::NFT; ++ft)
#pragma unroll
        for (int ct = 0; ct < K::NCT; ++ct)
            sacc[ft][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    float zpart = 0.f;

    u32x4 rk[K::TM], rv[K::TM];
    tile.load(rk, kb + (size_t)tb * D, te - tb);
    tile.load(rv, vb + (size_t)tb * D, te - tb);
    const int tlast = tb + ((te - tb - 1) / C) * C; // first token of the segment's last chunk
    for (int t0 = tb; t0 < te; t0 += C) {
        const int nvalid = min(C, te - t0);
#pragma unroll
        for (int i = 0; i < K::TM; ++i) {
            const bool ok = tile.valid(i, nvalid);
            rk[i] = ok ? phi8(rk[i]) : u32x4{0u, 0u, 0u, 0u};
            rv[i] = ok ? rv[i] : u32x4{0u, 0u, 0u, 0u};
        }
        tile.store_cols(sKT, rk);
        tile.store_cols(sVT, rv);
        __syncthreads();
        {   // prefetch the next chunk (the last chunk again at the end: always in bounds)
            const int tn = min(t0 + C, tlast);
            tile.load(rk, kb + (size_t)tn * D, te - tn);
            tile.load(rv, vb + (size_t)tn * D, te - tn);
        }
        state_update<D>(sacc, sKT, sVT, cw0, li, g);
        zpart += kf_colsum_half<D>(sKT, tid);
        __syncthreads();
    }

    float *S = dstS + ((long)bh * P + p) * sstride;
#pragma unroll
    for (int ft = 0; ft < K::NFT; ++ft)
#pragma unroll
        for (int ct = 0; ct < K::NCT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[(16 * ft + 4 * g + r) * D + cw0 + 16 * ct + li] = sacc[ft][ct][r];
    zpart += __shfl_xor(zpart, 1, 64);
    if (tid < 2 * D && (tid & 1) == 0)
        dstz[((long)bh * P + p) * zstride + (tid >> 1)] = zpart;
}

// ------------------------------------------------------------------------------------------
// Causal outputs of one segment, starting from the state before the segment.
//
// 512 threads in two roles that share every SIMD. Waves 0-3 ("compute") hold the float32 state
// S in accumulators (wave w owns value columns [w*D/4, (w+1)*D/4)) and run the matrix-core
// products of chunk c. Waves 4-7 ("stage") meanwhile prepare chunk c+1 in the other half of the
// double-buffered LDS: they apply phi, write phi(Q), phi(K) row-major and phi(K), V
// token-major, keep the key sum z (float32, LDS) and compute the inter-chunk part of the
// denominators, phi(q_i) . z. Two workgroup barriers per chunk:
//   phase 1  compute: scores A of chunk c (query rows 16w..16w+15), den = rowsum(A) + phi(q).z
//            stage:   z += colsum(phi(K_c)); phi(Q_{c+1}) -> LDS; load Q_{c+2}
//   --- barrier X ---
//   phase 2  compute: num = A V_c + phi(Q_c) S; out = num / den; S += phi(K_c)^T V_c
//            stage:   phi(K_{c+1}), V_{c+1} -> LDS; load K_{c+2}, V_{c+2}; phi(Q_{c+1}) . z
//   --- barrier Y ---
template <int D> struct CausalLds {
    uint16_t sQ[2][C * Cfg<D>::QS];
    uint16_t sK[2][C * Cfg<D>::QS];
    uint16_t sKT[2][D * Cfg<D>::TS];
    uint16_t sVT[2][D * Cfg<D>::TS];
    uint16_t sA[C * Cfg<D>::TS];
    float sz[2][D];  // z before chunk c lives in sz[c & 1]
    float sdi[2][C]; // phi(q_i) . z for chunk c in sdi[c & 1]
    float sden[C];
};

struct CausalArgs {
    const uint16_t *qh, *kh, *vh; // the head's [N, D] rows
    uint16_t *oh;
    const float *S0, *z0;         // state before the segment (null: zero)
    float *Sout, *zout;           // final state of the head (null: not written)
    int tb, te, nch;              // token range of the segment, chunks in it
};

// Compute role (waves 0-3). Barrier sequence: 2 in the prologue, 2 per chunk.
template <int D>
__device__ __forceinline__ void causal_compute(CausalLds<D> &sm, const CausalArgs &a, int w,
                                               int li, int g)
{
    using K = Cfg<D>;
    const int cw0 = w * (D / 4);
    f32x4 sacc[K::NFT][K::NCT];
    bf16x8 sf[K::NCT][K::NKB];
#pragma unroll
    for (int ft = 0; ft < K::NFT; ++ft)
#pragma unroll
        for (int ct = 0; ct < K::NCT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[ft][ct][r] = a.S0 ? a.S0[(16 * ft + 4 * g + r) * D + cw0 + 16 * ct + li] : 0.f;
    state_frags<D>(sf, sacc);
    __syncthreads();
    __syncthreads();

    for (int c = 0; c < a.nch; ++c) {
        const int b = c & 1;
        const int t0 = a.tb + c * C, nvalid = min(C, a.te - t0);
        // phase 1: scores of query rows 16w..16w+15 against keys j <= i; den = rowsum + phi(q).z
        {
            bf16x8 qb[K::NKB];
#pragma unroll
            for (int kk = 0; kk < K::NKB; ++kk)
                qb[kk] = lds<bf16x8>(sm.sQ[b] + (16 * w + li) * K::QS + 32 * kk + 8 * g);
            float rs = 0.f;
            for (int jt = 0; jt <= w; ++jt) {
                f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < K::NKB; ++kk)
                    t = mfma(lds<bf16x8>(sm.sK[b] + (16 * jt + li) * K::QS + 32 * kk + 8 * g), qb[kk], t);
                // t[r] = A[i = 16w + li][j = 16jt + 4g + r]
                if (jt == w) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (4 * g + r > li)
                            t[r] = 0.f;
                }
                const uint32_t p0 = pack_bf2(t[0], t[1]), p1 = pack_bf2(t[2], t[3]);
                sts<u32x2>(sm.sA + (16 * w + li) * K::TS + 16 * jt + 4 * g, u32x2{p0, p1});
                rs += (bf_lo(p0) + bf_hi(p0)) + (bf_lo(p1) + bf_hi(p1));
            }
            if ((w & 1) == 0) // the 32-token block read below also covers j-tile w+1: zero it
                sts<u32x2>(sm.sA + (16 * w + li) * K::TS + 16 * (w + 1) + 4 * g, u32x2{0u, 0u});
            rs += __shfl_xor(rs, 16, 64);
            rs += __shfl_xor(rs, 32, 64);
            if (g == 0)
                sm.sden[16 * w + li] = rs + sm.sdi[b][16 * w + li];
        }
        __syncthreads();
        // phase 2: num^T = V^T A^T + S^T Qf^T for the wave's columns; out; S += Kf^T V
        {
            f32x4 acc[K::NCT][4];
#pragma unroll
            for (int ct = 0; ct < K::NCT; ++ct)
#pragma unroll
                for (int it = 0; it < 4; ++it)
                    acc[ct][it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int it = 0; it < 4; ++it)
#pragma unroll
                for (int m = 0; m <= it / 2; ++m) {
                    const bf16x8 ba = lds<bf16x8>(sm.sA + (16 * it + li) * K::TS + 32 * m + 8 * g);
#pragma unroll
                    for (int ct = 0; ct < K::NCT; ++ct)
                        acc[ct][it] = mfma(lds<bf16x8>(sm.sVT[b] + tix<D>(cw0 + 16 * ct + li, 32 * m + 8 * g)),
                                           ba, acc[ct][it]);
                }
            state_read<D>(acc, sf, sm.sQ[b], li, g);
            store_out<D>(acc, sm.sden, a.oh + (size_t)t0 * D, nvalid, cw0, li, g);
            state_update<D>(sacc, sm.sKT[b], sm.sVT[b], cw0, li, g);
            state_frags<D>(sf, sacc);
        }
        __syncthreads();
    }
    if (a.Sout) {
#pragma unroll
        for (int ft = 0; ft < K::NFT; ++ft)
#pragma unroll
            for (int ct = 0; ct < K::NCT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    a.Sout[(16 * ft + 4 * g + r) * D + cw0 + 16 * ct + li] = sacc[ft][ct][r];
    }
}

// Stage role (waves 4-7, thread index ht = 0..255). Same barrier sequence as the compute role.
template <int D>
__device__ __forceinline__ void causal_stage(CausalLds<D> &sm, const CausalArgs &a, int ht)
{
    using K = Cfg<D>;
    const Tile<D> tile(ht);
    u32x4 rq[K::TM], rk[K::TM], rv[K::TM];
    const int tb = a.tb, te = a.te, nch = a.nch;

    if (ht < D)
        sm.sz[0][ht] = a.z0 ? a.z0[ht] : 0.f;
    // first token of chunk c' (clamped to the last chunk, so prefetches past the end re-read
    // it: every load is in bounds and unconditional)
    auto chunk_t0 = [&](int cc) { return tb + min(cc, nch - 1) * C; };
    tile.load(rq, a.qh + (size_t)tb * D, te - tb);
    tile.load(rk, a.kh + (size_t)tb * D, te - tb);
    tile.load(rv, a.vh + (size_t)tb * D, te - tb);
#pragma unroll
    for (int i = 0; i < K::TM; ++i) {
        const bool ok = tile.valid(i, te - tb);
        rq[i] = ok ? phi8(rq[i]) : u32x4{0u, 0u, 0u, 0u};
        rk[i] = ok ? phi8(rk[i]) : u32x4{0u, 0u, 0u, 0u};
        rv[i] = ok ? rv[i] : u32x4{0u, 0u, 0u, 0u};
    }
    tile.store_rows(sm.sQ[0], rq);
    tile.store_rows(sm.sK[0], rk);
    tile.store_cols(sm.sKT[0], rk);
    tile.store_cols(sm.sVT[0], rv);
    {
        const int tn = chunk_t0(1);
        tile.load(rq, a.qh + (size_t)tn * D, te - tn);
        tile.load(rk, a.kh + (size_t)tn * D, te - tn);
        tile.load(rv, a.vh + (size_t)tn * D, te - tn);
    }
    __syncthreads();
    den_inter<D>(sm.sdi[0], sm.sQ[0], sm.sz[0], ht);
    __syncthreads();

    for (int c = 0; c < nch; ++c) {
        const int b = c & 1, nb = b ^ 1;
        const int t0 = tb + c * C;
        const int n1 = min(C, te - t0 - C); // valid rows of chunk c+1 (if it exists)
        const int tn = chunk_t0(c + 2), nn = te - tn;
        // phase 1: z after chunk c; phi(Q_{c+1}) -> LDS; load Q_{c+2}
        {
            float zs = kf_colsum_half<D>(sm.sKT[b], ht);
            zs += __shfl_xor(zs, 1, 64);
            if (ht < 2 * D && (ht & 1) == 0)
                sm.sz[nb][ht >> 1] = sm.sz[b][ht >> 1] + zs;
            if (c + 1 < nch) {
#pragma unroll
                for (int i = 0; i < K::TM; ++i)
                    rq[i] = tile.valid(i, n1) ? phi8(rq[i]) : u32x4{0u, 0u, 0u, 0u};
                tile.store_rows(sm.sQ[nb], rq);
            }
            tile.load(rq, a.qh + (size_t)tn * D, nn);
        }
        __syncthreads();
        // phase 2: phi(K_{c+1}), V_{c+1} -> LDS; load K_{c+2}, V_{c+2}; phi(Q_{c+1}) . z
        if (c + 1 < nch) {
#pragma unroll
            for (int i = 0; i < K::TM; ++i) {
                const bool ok = tile.valid(i, n1);
                rk[i] = ok ? phi8(rk[i]) : u32x4{0u, 0u, 0u, 0u};
                rv[i] = ok ? rv[i] : u32x4{0u, 0u, 0u, 0u};
            }
            tile.store_rows(sm.sK[nb], rk);
            tile.store_cols(sm.sKT[nb], rk);
            tile.store_cols(sm.sVT[nb], rv);
        }
        tile.load(rk, a.kh + (size_t)tn * D, nn);
        tile.load(rv, a.vh + (size_t)tn * D, nn);
        if (c + 1 < nch)
            den_inter<D>(sm.sdi[nb], sm.sQ[nb], sm.sz[nb], ht);
        __syncthreads();
    }
    if (a.zout && ht < D)
        a.zout[ht] = sm.sz[nch & 1][ht];
}

// ------------------------------------------------------------------------------------------
// Causal outputs of one segment, starting from the state before the segment.
//
// 512 threads in two roles that share every SIMD. Waves 0-3 ("compute") hold the float32 state
// S in accumulators (wave w owns value columns [w*D/4, (w+1)*D/4)) and run the matrix-core
// products of chunk c. Waves 4-7 ("stage") meanwhile prepare chunk c+1 in the other half of the
// double-buffered LDS: they apply phi, write phi(Q), phi(K) row-major and phi(K), V
// token-major, keep the key sum z (float32, LDS) and compute the inter-chunk part of the
// denominators, phi(q_i) . z. Two workgroup barriers per chunk:
//   phase 1  compute: scores A of chunk c (query rows 16w..16w+15), den = rowsum(A) + phi(q).z
//            stage:   z += colsum(phi(K_c)); phi(Q_{c+1}) -> LDS; load Q_{c+2}
//   --- barrier ---
//   phase 2  compute: num = A V_c + phi(Q_c) S; out = num / den; S += phi(K_c)^T V_c
//            stage:   phi(K_{c+1}), V_{c+1} -> LDS; load K_{c+2}, V_{c+2}; phi(Q_{c+1}) . z
//   --- barrier ---
// The roles are wave-uniform, so every wave executes the same sequence of barriers.
template <int D>
__global__ __launch_bounds__(2 * NT) void k_causal(const uint16_t *__restrict__ q,
                                                   const uint16_t *__restrict__ k,
                                                   const uint16_t *__restrict__ v,
                                                   uint16_t *__restrict__ out,
                                                   const float *__restrict__ preS,
                                                   const float *__restrict__ prez, long pstride,
                                                   long pzstride, float *__restrict__ Sout,
                                                   float *__restrict__ zout, int N, int L, int P)
{
    __shared__ __attribute__((aligned(16))) CausalLds<D> sm;
    const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
    const int p = blockIdx.x % P, bh = blockIdx.x / P;
    const size_t hoff = (size_t)bh * N * D;
    CausalArgs a;
    a.qh = q + hoff;
    a.kh = k + hoff;
    a.vh = v + hoff;
    a.oh = out + hoff;
    a.S0 = preS ? preS + ((long)bh * P + p) * pstride : nullptr;
    a.z0 = preS ? prez + ((long)bh * P + p) * pzstride : nullptr;
    const bool last = p == P - 1;
    a.Sout = Sout && last ? Sout + (size_t)bh * D * D : nullptr;
    a.zout = Sout && last ? zout + (size_t)bh * D : nullptr;
    a.tb = p * L;
    a.te = min(N, a.tb + L);
    a.nch = (a.te - a.tb + C - 1) / C;
    if (wave < 4)
        causal_compute<D>(sm, a, wave, l & 15, l >> 4);
    else
        causal_stage<D>(sm, a, tid - NT);
}

// ------------------------------------------------------------------------------------------
// Global read: out = phi(Q) S / phi(Q) z for one segment of tokens of one head.
template <int D>
__global__ __launch_bounds__(NT) void k_gread(const uint16_t *__restrict__ q,
                                              uint16_t *__restrict__ out,
                                              const float *__restrict__ S,
                                              const float *__restrict__ z, int N, int L, int P)
{
    using K = Cfg<D>;
    __shared__ __attribute__((aligned(16))) uint16_t sQ[C * K::QS];
    __shared__ float sz[D];
    __shared__ float sden[C];

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, g = l >> 4;
    const int p = blockIdx.x % P, bh = blockIdx.x / P;
    const int tb = p * L, te = min(N, tb + L);
    const size_t hoff = (size_t)bh * N * D;
    const int cw0 = w * (D / 4);
    const Tile<D> tile(tid);

    bf16x8 sf[K::NCT][K::NKB];
    {
        const float *Sh = S + (size_t)bh * D * D;
#pragma unroll
        for (int ct = 0; ct < K::NCT; ++ct)
#pragma unroll
            for (int m = 0; m < K::NKB; ++m) {
                float x[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    x[r] = Sh[(32 * m + 4 * g + r) * D + cw0 + 16 * ct + li];
                    x[4 + r] = Sh[(32 * m + 16 + 4 * g + r) * D + cw0 + 16 * ct + li];
                }
                const u32x4 wv = {pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]), pack_bf2(x[4], x[5]),
                                  pack_bf2(x[6], x[7])};
                sf[ct][m] = __builtin_bit_cast(bf16x8, wv);
            }
    }
    if (tid < D)
        sz[tid] = z[(size_t)bh * D + tid];

    u32x4 rq[K::TM];
    tile.load(rq, q + hoff + (size_t)tb * D, te - tb);
    const int tlast = tb + ((te - tb - 1) / C) * C;
    for (int t0 = tb; t0 < te; t0 += C) {
        const int nvalid = min(C, te - t0);
#pragma unroll
        for (int i = 0; i < K::TM; ++i)
            rq[i] = tile.valid(i, nvalid) ? phi8(rq[i]) : u32x4{0u, 0u, 0u, 0u};
        tile.store_rows(sQ, rq);
        __syncthreads();
        {
            const int tn = min(t0 + C, tlast);
            tile.load(rq, q + hoff + (size_t)tn * D, te - tn);
        }
        {
            // den[i] = Qf[i] . z: 4 threads per row, D/4 features each
            const int i = tid >> 2, qq = tid & 3;
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < D / 32; ++e) {
                const int f = qq * (D / 4) + 8 * e;
                const u32x4 qw = lds<u32x4>(sQ + i * K::QS + f);
#pragma unroll
                for (int h = 0; h < 4; ++h)
                    s += bf_lo(qw[h]) * sz[f + 2 * h] + bf_hi(qw[h]) * sz[f + 2 * h + 1];
            }
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            if (qq == 0)
                sden[i] = s;
        }
        __syncthreads();
        f32x4 acc[K::NCT][4];
#pragma unroll
        for (int ct = 0; ct < K::NCT; ++ct)
#pragma unroll
            for (int it = 0; it < 4; ++it)
                acc[ct][it] = f32x4{0.f, 0.f, 0.f, 0.f};
        state_read<D>(acc, sf, sQ, li, g);
        store_out<D>(acc, sden, out + hoff + (size_t)t0 * D, nvalid, cw0, li, g);
        __syncthreads();
    }
}

} // namespace

// ------------------------------------------------------------------------------------------
hipError_t agg_mfma(int D, const void *k, const void *v, float *dstS, float *dstz, long sstride,
                    long zstride, int BH, int N, int L, int nseg, int P, hipStream_t st)
{
    const dim3 grid((unsigned)(BH * nseg)), block(NT);
    const auto *kk = static_cast<const uint16_t *>(k);
    const auto *vv = static_cast<const uint16_t *>(v);
    if (D == 128)
        hipLaunchKernelGGL(k_agg<128>, grid, block, 0, st, kk, vv, dstS, dstz, sstride, zstride, N, L, nseg, P);
    else
        hipLaunchKernelGGL(k_agg<64>, grid, block, 0, st, kk, vv, dstS, dstz, sstride, zstride, N, L, nseg, P);
    return hipGetLastError();
}

hipError_t causal_mfma(int D, const void *q, const void *k, const void *v, void *out,
                       const float *preS, const float *prez, long pstride, long pzstride,
                       float *Sout, float *zout, int BH, int N, int L, int P, hipStream_t st)
{
    const dim3 grid((unsigned)(BH * P)), block(2 * NT);
    const auto *qq = static_cast<const uint16_t *>(q);
    const auto *kk = static_cast<const uint16_t *>(k);
    const auto *vv = static_cast<const uint16_t *>(v);
    auto *oo = static_cast<uint16_t *>(out);
    if (D == 128)
        hipLaunchKernelGGL(k_causal<128>, grid, block, 0, st, qq, kk, vv, oo, preS, prez, pstride,
                           pzstride, Sout, zout, N, L, P);
    else
        hipLaunchKernelGGL(k_causal<64>, grid, block, 0, st, qq, kk, vv, oo, preS, prez, pstride,
                           pzstride, Sout, zout, N, L, P);
    return hipGetLastError();
}

hipError_t global_read_mfma(int D, const void *q, void *out, const float *S, const float *z,
                            int BH, int N, int L, int P, hipStream_t st)
{
    const dim3 grid((unsigned)(BH * P)), block(NT);
    const auto *qq = static_cast<const uint16_t *>(q);
    auto *oo = static_cast<uint16_t *>(out);
    if (D == 128)
        hipLaunchKernelGGL(k_gread<128>, grid, block, 0, st, qq, oo, S, z, N, L, P);
    else
        hipLaunchKernelGGL(k_gread<64>, grid, block, 0, st, qq, oo, S, z, N, L, P);
    return hipGetLastError();
}

} // namespace la
