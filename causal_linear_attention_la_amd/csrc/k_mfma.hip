// k_mfma.hip -- matrix-core kernels of liblinattn: bf16 inputs, d == d_v = D in {64, 128},
// chunks of C = 64 tokens, gfx950 MFMA v_mfma_f32_16x16x32_bf16 with float32 accumulation.
// Variants are compile-time parameters of the same kernels: the identity map and the
// unnormalised read (flags), a per-head decay of the carried state (the retention recurrence)
// and positive random features computed in the staging.
//
// Chunked causal evaluation (the within-chunk part plus the state carried from earlier chunks,
// as "Linear Attention: From Pairwise Reads to a Recurrent State", section "A recurrence need
// not force token-serial training", describes). For a chunk c of tokens with mapped features
// Qf = phi(Q_c), Kf = phi(K_c) and values V_c, and the state S, z before the chunk:
//   A       = mask_{j <= i}(Qf Kf^T)                     (C x C, inclusive: token i sees itself)
//   num     = A V_c + Qf S,    den = rowsum(A) + Qf z    (the recurrence's read, all rows at once)
//   out     = num / den
//   S, z   += Kf^T V_c, Kf^T 1                           (the recurrence's write, summed over c)
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
// Chunks live in LDS row-major (token x feature), the layout in which they arrive from HBM.
// Products that contract over features read them directly; products that contract over tokens
// (S += Kf^T V, the key sum Kf^T 1, and A V) take their operands through the LDS transpose read
// ds_read_b64_tr_b16: within each group of 16 lanes, lane j addresses the 8-byte piece at
// (row j/4, columns 4(j%4)..4(j%4)+3) of a 4 x 16 block and receives column j of the block.
#include "la_device.h"
#include "la_launch.h"

namespace la {
namespace {

constexpr int C = 64;   // tokens per chunk
// waves and threads of the global-read kernel: two workgroups of eight waves share a CU (their
// LDS and 128 VGPRs per wave allow it); measured on MI355X, B=1 H=8 N=100000 d=128: 168.8 us
// per global call against 171.6 us with three workgroups of four waves
constexpr int GW = 8, NT = 64 * GW;

template <int D> struct Cfg {
    static constexpr int RS = D + 16;           // row stride (elements) of the chunk arrays
    static constexpr int AS = C * RS + (C / 8 - 1) * 64; // chunk array size (elements)
    static constexpr int TS = C + 16;           // row stride (elements) of the score block
    static constexpr int ZS = D + 16;           // row stride (elements) of the key-sum operand
    static constexpr int NCT = D / 64;          // 16-wide value-column tiles per wave (4 waves)
    static constexpr int NFT = D / 16;          // 16-row feature tiles of S
    static constexpr int NKB = D / 32;          // 32-feature k blocks
    static constexpr int ZFT = NFT / 4;         // feature tiles of z one wave keeps (4 waves)
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Index of the calling wave within its workgroup, as a wave-uniform (scalar) value. Branches on
// it then compile to scalar branches; matrix-core instructions do not honour the EXEC mask, so
// they must never sit under a lane-masked branch.
__device__ __forceinline__ int wave_id()
{
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

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

// LDS layout of the row-major [C][D] chunk arrays. gfx950 LDS has 64 banks of 4 bytes for
// reads and 32 for writes; a 16-byte store is served 8 lanes at a time, an 8-byte read 32
// lanes at a time, and a 16-byte read 16 lanes at a time, grouped as lanes 4q..4q+3 of one
// half-wave whose quad index q has the same bit parity. Layout: rows padded to D + 16 elements,
// a further 64 elements after every 8 rows, and the low bit of the 16-byte granule index
// flipped in rows with bit 3 set. With it, every access below is free of bank conflicts:
//   staging stores (8 lanes = 128 contiguous bytes of one row),
//   16-byte operand reads (16 consecutive rows x one granule per lane group),
//   8-byte reads of 16 consecutive rows x one granule, and the transpose reads
//   (8 consecutive rows x 32 bytes).
template <int D> __device__ __forceinline__ int nix(int row, int col)
{
    return row * Cfg<D>::RS + 64 * (row >> 3) + ((((col >> 3) ^ ((row >> 3) & 1))) << 3) + (col & 7);
}
// For row0 % 16 == 0 and col0 % 16 == 0: nix(row0 + r, col0 + c) == blk(row0, col0) + nix(r, c).
// Every access below splits its address this way into a lane part computed once and a
// compile-time block part that becomes the instruction's immediate offset.
template <int D> __host__ __device__ constexpr int blk(int row0, int col0)
{
    return row0 * (Cfg<D>::RS + 8) + col0;
}

// Operand fragment whose k-slots run over tokens, read with two transpose reads from a
// row-major chunk (tokens x columns): slot 4h + y holds M[row0 + 16h + 4g + y][col0 + li].
// `p` = chunk base + blk(row0, col0) + tr_lane(li, g). (The k-slot order is a permutation of
// the 32 tokens of the block; every product pairs it with an operand in the same order.)
template <int D> __device__ __forceinline__ int tr_lane(int li, int g)
{
    return nix<D>(4 * g + (li >> 2), 4 * (li & 3));
}
template <int D> __device__ __forceinline__ bf16x8 frag_tok(const uint16_t *p)
{
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + blk<D>(16, 0)));
    const i16x8 x = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, x);
}

// Score block: [query row][key], row stride TS = C + 16. Within each 32-key block, key
// 16h + 4q + y is stored at position 8q + 4h + y, so a 16-byte read at position 8g holds the
// keys in the k-slot order of frag_tok (slot 4h + y = key 16h + 4g + y), and one lane's two
// 4-key score pieces of a tile pair form one 16-byte store. The 16-byte granules of rows with
// bit 2 set are swapped in pairs (granule index xor 1): with the stride this makes both the
// score stores (8 lanes per pass) and the A V reads (16 lanes per pass) free of bank conflicts
// (the unswizzled stride C + 8 left every A V read with two-way conflicts).
__device__ __forceinline__ int sa_ix(int row, int kblock, int g)
{
    return row * (C + 16) + 32 * kblock + 8 * (g ^ ((row >> 2) & 1));
}

// phi(x) = ELU(x) + 1 = exp(min(x, 0)) + max(x, 0) on 8 packed bf16 values, rounded to bf16
// (nearest even). min and max are taken on the bit patterns (an integer compare orders floats
// correctly against zero), so no compare/select pair is needed.
__device__ __forceinline__ float phi_bits(uint32_t xb)
{
    const int xi = (int)xb;
    const float neg = __int_as_float(min(xi, 0)), pos = __int_as_float(max(xi, 0));
    return __builtin_amdgcn_exp2f(neg * 1.44269504088896341f) + pos;
}
__device__ __forceinline__ u32x4 phi8(u32x4 x)
{
    u32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        y[i] = pack_bf2(phi_bits(x[i] << 16), phi_bits(x[i] & 0xffff0000u));
    return y;
}

// Staging of one [C, D] chunk by NTH threads: consecutive lanes own consecutive 16-byte feature
// groups of one row (FG lanes per row), so a wave's global load reads whole rows (1 KiB
// contiguous) and 8 lanes of a staging store cover 128 contiguous bytes of one row. Thread t
// owns rows t / FG + RPI * i, i < TM.
template <int D, int NTH = NT> struct Tile {
    static constexpr int FG = D / 8;       // 16-byte feature groups per row
    static constexpr int RPI = NTH / FG;   // chunk rows one staging instruction covers
    static constexpr int TM = C / RPI;     // staging rows per thread
    static_assert(TM >= 1 && TM * RPI == C, "staging tile");
    int a, b;  // first row, feature group
    int lofs;  // LDS offset (elements) of (row a, group b)
    __device__ explicit Tile(int tid) : a(tid / FG), b(tid % FG), lofs(nix<D>(a, 8 * b)) {}
    // rows of the chunk starting at `base` (wave-uniform), clamped to the chunk's last valid row
    // so every access is in bounds and no load sits in a branch (a load merged with a zero in a
    // branch makes the compiler wait for it right away); rows past nvalid are masked when staged.
    // Offsets are 32-bit from the uniform base, so the loads use scalar-base addressing.
    __device__ __forceinline__ void load(u32x4 (&r)[TM], const uint16_t *__restrict__ base,
                                         int nvalid) const
    {
        const char *bb = reinterpret_cast<const char *>(base);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const uint32_t rr = (uint32_t)min(a + RPI * i, nvalid - 1);
            r[i] = *reinterpret_cast<const u32x4 *>(bb + (rr * (uint32_t)(2 * D) + 16u * (uint32_t)b));
        }
    }
    // rows >= nvalid become 0 (phi(K) and V rows of a ragged last chunk must not contribute)
    __device__ __forceinline__ void store(uint16_t *s, const u32x4 (&r)[TM], int nvalid,
                                          bool apply_phi) const
    {
        if (nvalid >= C) { // wave-uniform: a full chunk needs no masking
#pragma unroll
            for (int i = 0; i < TM; ++i)
                sts<u32x4>(s + lofs + blk<D>(RPI * i, 0), apply_phi ? phi8(r[i]) : r[i]);
        } else {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const u32x4 y = apply_phi ? phi8(r[i]) : r[i];
                const bool ok = a + RPI * i < nvalid;
                sts<u32x4>(s + lofs + blk<D>(RPI * i, 0), ok ? y : u32x4{0u, 0u, 0u, 0u});
            }
        }
    }
};

// ---- positive random features in the staging ------------------------------------------
// The random-feature form maps q and k while they are staged: f_r(x) = exp(w_r . x - |x|^2 / 2)
// / sqrt(D) for D projections w_r (W bf16 [D][D], m = d = D; "Linear Attention Math", section
// "Feature maps: elu+1 and positive random features"). A staging wave takes 16 rows of a
// chunk as matrix-core B operands straight from HBM, multiplies them by W held in LDS and
// writes the bf16 features into the chunk array, where the attention reads them as it reads
// phi(Q), phi(K). The work of one chunk of Q (or K) is 4 row tiles x 2 feature halves.
template <int D> struct Rf {
    static constexpr int NKB = D / 32; // k blocks of 32 input features
    static constexpr int TPH = D / 32; // 16-projection tiles per feature half
    static constexpr int GF = D / 8;   // consecutive features one lane group holds in a half
};

// W -> LDS in matrix-core fragment order (the 16 bytes lane l reads for tile mt, k block kk
// sit at ((mt * NKB + kk) * 64 + l) * 16: contiguous, conflict-free 1 KiB reads), with the
// projections placed so that in the product for half h lane group g holds features
// h D/2 + g D/8 .. + D/8 - 1 of its row: projection h D/2 + g D/8 + 4t + j is row 4g + j of tile
// h TPH + t.
template <int D, int NTH>
__device__ __forceinline__ void rf_put_w(uint16_t *sW, const uint16_t *__restrict__ W, int tid)
{
    using R = Rf<D>;
    for (int e = tid; e < D * D / 8; e += NTH) {
        const int p = e / (D / 8), c = e % (D / 8);
        const int h = p / (D / 2), rem = p % (D / 2);
        const int gq = rem / R::GF, t = (rem % R::GF) / 4, j = p % 4;
        const int frag = (h * R::TPH + t) * R::NKB + c / 4, lane = (c % 4) * 16 + 4 * gq + j;
        sts<u32x4>(sW + (frag * 64 + lane) * 8,
                   *reinterpret_cast<const u32x4 *>(W + (size_t)p * D + 8 * c));
    }
}

// Rows 16 rt + li of the chunk at `chunk` (clamped to its last valid row, so every load is in
// bounds) as B operands: k-slots 8g..8g+7 of k block kk.
template <int D>
__device__ __forceinline__ void rf_load(u32x4 (&x)[D / 32], const uint16_t *chunk, int rt, int nvalid,
                                        int li, int g)
{
    const uint32_t r = (uint32_t)min(16 * rt + li, nvalid - 1);
    const char *b = reinterpret_cast<const char *>(chunk);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
        x[kk] = *reinterpret_cast<const u32x4 *>(b + (r * (uint32_t)(2 * D) + 64u * kk + 16u * g));
}

// Features of half h of rows 16 rt + li into the chunk array s (rows >= nvalid become 0).
template <int D>
__device__ __forceinline__ void rf_put(uint16_t *s, const uint16_t *sW, const u32x4 (&x)[D / 32],
                                       int rt, int h, int nvalid, int l, int li, int g)
{
    using R = Rf<D>;
    constexpr float LOG2E = 1.44269504088896341f;
    constexpr float NEG_HALF_LOG2M = D == 128 ? -3.5f : -3.0f; // -log2(sqrt(D))
    float n = 0.f;
#pragma unroll
    for (int kk = 0; kk < R::NKB; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a = bf_lo(x[kk][i]), b = bf_hi(x[kk][i]);
            n = fmaf(a, a, n);
            n = fmaf(b, b, n);
        }
    n += __shfl_xor(n, 16, 64);
    n += __shfl_xor(n, 32, 64);
    // exponent in base 2: (w . x - |x|^2 / 2) log2(e) - log2(D) / 2
    const float bias = fmaf(-0.5f * LOG2E, n, NEG_HALF_LOG2M);
    const int row = 16 * rt + li;
    const bool ok = row < nvalid;
    // the half's TPH tiles as independent accumulation chains, interleaved over k blocks
    f32x4 c[R::TPH];
#pragma unroll
    for (int t = 0; t < R::TPH; ++t)
        c[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < R::NKB; ++kk) {
        bf16x8 wa[R::TPH];
#pragma unroll
        for (int t = 0; t < R::TPH; ++t)
            wa[t] = lds<bf16x8>(sW + (((h * R::TPH + t) * R::NKB + kk) * 64 + l) * 8);
#pragma unroll
        for (int t = 0; t < R::TPH; ++t)
            c[t] = mfma(wa[t], __builtin_bit_cast(bf16x8, x[kk]), c[t]);
    }
#pragma unroll
    for (int s2 = 0; s2 < R::TPH / 2; ++s2) {
        uint32_t o[4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            float e[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                e[j] = __builtin_amdgcn_exp2f(fmaf(c[2 * s2 + hh][j], LOG2E, bias));
            o[2 * hh] = pack_bf2(e[0], e[1]);
            o[2 * hh + 1] = pack_bf2(e[2], e[3]);
        }
        sts<u32x4>(s + nix<D>(row, h * (D / 2) + g * R::GF + 8 * s2),
                   ok ? u32x4{o[0], o[1], o[2], o[3]} : u32x4{0u, 0u, 0u, 0u});
    }
}

// The staging work of one wave for a chunk of Q or K: its row tile (wave % 4) and its feature
// half (NW = 8 staging waves: wave / 4) or both halves (NW = 4).
template <int D, int NW>
__device__ __forceinline__ void rf_put_share(uint16_t *s, const uint16_t *sW, const u32x4 (&x)[D / 32],
                                             int sw, int nvalid, int l)
{
    const int li = l & 15, g = l >> 4;
    if (NW == 8) {
        rf_put<D>(s, sW, x, sw & 3, sw >> 2, nvalid, l, li, g);
    } else {
        rf_put<D>(s, sW, x, sw & 3, 0, nvalid, l, li, g);
        rf_put<D>(s, sW, x, sw & 3, 1, nvalid, l, li, g);
    }
}

// An offset hidden from the compiler. The 8-byte state-read pieces of one lane sit 32 or 64
// bytes apart; with their offsets visible the compiler merges them into ds_read2_b64, which
// gfx950 serves with bank conflicts that separate 8-byte reads do not have. Reads off distinct
// hidden bases cannot be merged (same-base reads below are >= 4 KiB apart, out of its range).
__device__ __forceinline__ int hidden(int x)
{
    asm volatile("" : "+v"(x));
    return x;
}

// bf16 A-operand fragment of S^T for the state read: value-column tile ct, 32-feature block m,
// k = feature permuted as {4g..4g+3, 16+4g..16+4g+3} -- exactly the rows an accumulator pair
// (feature tiles 2m, 2m+1) holds in this lane.
template <int D, int NCT>
__device__ __forceinline__ bf16x8 state_frag(const f32x4 (&sacc)[Cfg<D>::NFT][NCT], int ct, int m)
{
    const f32x4 lo = sacc[2 * m][ct], hi = sacc[2 * m + 1][ct];
    const u32x4 w = {pack_bf2(lo[0], lo[1]), pack_bf2(lo[2], lo[3]), pack_bf2(hi[0], hi[1]),
                     pack_bf2(hi[2], hi[3])};
    return __builtin_bit_cast(bf16x8, w);
}

// num^T += S^T Qf^T for the wave's value columns and all C query rows, with S the state in
// sacc (float32, rounded to bf16 fragments here). acc[ct][it]: rows (value columns)
// cw0 + 16ct + 4g + r, column (query) 16it + li. `q` = Qf chunk base + nix(li, 4g).
template <int D, int NCT>
__device__ __forceinline__ void state_read(f32x4 (&acc)[NCT][4], const f32x4 (&sacc)[Cfg<D>::NFT][NCT],
                                           const uint16_t *q)
{
    using K = Cfg<D>;
#pragma unroll
    for (int m = 0; m < K::NKB; ++m) {
        bf16x8 sf[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            sf[ct] = state_frag<D, NCT>(sacc, ct, m);
        const uint16_t *q0b = q + hidden(32 * m), *q1b = q + hidden(32 * m + 16);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const u32x2 q0 = lds<u32x2>(q0b + blk<D>(16 * it, 0));
            const u32x2 q1 = lds<u32x2>(q1b + blk<D>(16 * it, 0));
            const bf16x8 bq = __builtin_bit_cast(bf16x8, u32x4{q0[0], q0[1], q1[0], q1[1]});
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                acc[ct][it] = mfma(sf[ct], bq, acc[ct][it]);
        }
    }
}

// S += Kf^T V over one chunk for the NCT value-column tiles of this wave. sacc[ft][ct]: rows
// f = 16ft + 4g + r, column 16ct + li of the wave's columns. `k` = Kf chunk base + tr_lane,
// `v` = V chunk base + (first column of the wave) + tr_lane.
template <int D, int NCT>
__device__ __forceinline__ void state_update(f32x4 (&sacc)[Cfg<D>::NFT][NCT], const uint16_t *k,
                                             const uint16_t *v)
{
    using K = Cfg<D>;
#pragma unroll
    for (int m = 0; m < C / 32; ++m) {
        bf16x8 bv[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            bv[ct] = frag_tok<D>(v + blk<D>(32 * m, 16 * ct));
#pragma unroll
        for (int ft = 0; ft < K::NFT; ++ft) {
            const bf16x8 ak = frag_tok<D>(k + blk<D>(32 * m, 16 * ft));
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                sacc[ft][ct] = mfma(ak, bv[ct], sacc[ft][ct]);
        }
    }
}

// z += Kf^T 1 for ZT feature tiles (every column of a zacc tile holds the same sum).
// `k` = Kf chunk base + (first feature of the tiles) + tr_lane.
template <int D, int ZT>
__device__ __forceinline__ void key_sum(f32x4 (&zacc)[ZT], const uint16_t *k)
{
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
#pragma unroll
    for (int m = 0; m < C / 32; ++m)
#pragma unroll
        for (int zt = 0; zt < ZT; ++zt)
            zacc[zt] = mfma(frag_tok<D>(k + blk<D>(32 * m, 16 * zt)), ones, zacc[zt]);
}

// ---- decay of the carried state (the retention recurrence S_t = gamma S_{t-1} + ...) ------
// gamma^n = exp2(n lg) with lg = decay_log2 (log2(gamma) clamped to -1000, so gamma = 0 gives 1
// for n = 0 and 0 for n > 0 without an infinity; NaN for a negative or NaN gamma).
__device__ __forceinline__ float decay_lg(const float *gamma, int bh, int H)
{
    return decay_log2(gamma, bh, H);
}
__device__ __forceinline__ float dpow(float lg, int n) { return __builtin_amdgcn_exp2f(lg * (float)n); }

// Token weights gamma^(nvalid - 1 - tok) of 32-token block m in the k-slot order of frag_tok:
// slot 4h + y is token 32m + 16h + 4g + y. Tokens past nvalid (zero rows) get weight 1.
__device__ __forceinline__ void tok_weights(float (&wt)[8], float lg, int nvalid, int m, int g)
{
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int y = 0; y < 4; ++y)
            wt[4 * h + y] = dpow(lg, max(nvalid - 1 - (32 * m + 16 * h + 4 * g + y), 0));
}

__device__ __forceinline__ bf16x8 scale_frag(bf16x8 x, const float (&w)[8])
{
    const u32x4 u = __builtin_bit_cast(u32x4, x);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = pack_bf2(bf_lo(u[i]) * w[2 * i], bf_hi(u[i]) * w[2 * i + 1]);
    return __builtin_bit_cast(bf16x8, o);
}

// S = gamma^nvalid S + Kf^T diag(w) V and z = gamma^nvalid z + Kf^T w over one chunk, with
// the token weights w of tok_weights: the chunk's tokens decayed to its last one.
template <int D, int NCT, int ZT>
__device__ __forceinline__ void state_update_decay(f32x4 (&sacc)[Cfg<D>::NFT][NCT], f32x4 (&zacc)[ZT],
                                                   const uint16_t *k, const uint16_t *v,
                                                   const uint16_t *kz, float lg, int nvalid, int g)
{
    using K = Cfg<D>;
    const float fc = dpow(lg, nvalid);
#pragma unroll
    for (int ft = 0; ft < K::NFT; ++ft)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            sacc[ft][ct] *= fc;
#pragma unroll
    for (int zt = 0; zt < ZT; ++zt)
        zacc[zt] *= fc;
#pragma unroll
    for (int m = 0; m < C / 32; ++m) {
        float wt[8];
        tok_weights(wt, lg, nvalid, m, g);
        bf16x8 bv[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            bv[ct] = scale_frag(frag_tok<D>(v + blk<D>(32 * m, 16 * ct)), wt);
#pragma unroll
        for (int ft = 0; ft < K::NFT; ++ft) {
            const bf16x8 ak = frag_tok<D>(k + blk<D>(32 * m, 16 * ft));
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                sacc[ft][ct] = mfma(ak, bv[ct], sacc[ft][ct]);
        }
        const u32x4 wb = {pack_bf2(wt[0], wt[1]), pack_bf2(wt[2], wt[3]), pack_bf2(wt[4], wt[5]),
                          pack_bf2(wt[6], wt[7])};
#pragma unroll
        for (int zt = 0; zt < ZT; ++zt)
            zacc[zt] = mfma(frag_tok<D>(kz + blk<D>(32 * m, 16 * zt)), __builtin_bit_cast(bf16x8, wb), zacc[zt]);
    }
}

// out rows [0, nvalid) of the chunk at `ob`: out = num / den, rounded to bf16.
// The denominator of row i is sden[i] (+ sden2[i] when given); NORM = false stores num itself
// (the unnormalised form) and reads no denominator.
template <int D, int NCT, bool NORM = true>
__device__ __forceinline__ void store_out(const f32x4 (&acc)[NCT][4], const float *sden,
                                          const float *sden2, uint16_t *__restrict__ ob, int nvalid,
                                          int cw0, int li, int g)
{
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int i = 16 * it + li;
        if (i < nvalid) {
            const float inv = NORM ? __builtin_amdgcn_rcpf(sden2 ? sden[i] + sden2[i] : sden[i]) : 1.f;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const f32x4 a = acc[ct][it];
                const u32x2 w = {pack_bf2(a[0] * inv, a[1] * inv), pack_bf2(a[2] * inv, a[3] * inv)};
                *reinterpret_cast<u32x2 *>(ob + (size_t)i * D + cw0 + 16 * ct + 4 * g) = w;
            }
        }
    }
}

template <int D, int NCT, int ZT>
__device__ __forceinline__ void zero_acc(f32x4 (&sacc)[Cfg<D>::NFT][NCT], f32x4 (&zacc)[ZT])
{
#pragma unroll
    for (int ft = 0; ft < Cfg<D>::NFT; ++ft)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            sacc[ft][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int zt = 0; zt < ZT; ++zt)
        zacc[zt] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// ------------------------------------------------------------------------------------------
// Segment sums: dS = phi(K_seg)^T V_seg, dz = phi(K_seg)^T 1. One wave per 16 value columns of
// S (and per 16 features of z), D/16 waves; every wave also stages 1/(D/16) of the next chunk
// into the other half of a double-buffered LDS before running the matrix-core update on the
// current one (one barrier per chunk). The wave count is what keeps enough loads in flight
// when each CU runs a single workgroup.
template <int D> struct AggCfg {
    static constexpr int NW = D / 16;
    static constexpr int THREADS = NW * 64;
};

template <int D, bool PHI, bool DECAY, bool RF>
__global__ __launch_bounds__(AggCfg<D>::THREADS) void k_agg(const uint16_t *__restrict__ k,
                                                           const uint16_t *__restrict__ v,
                                                           float *__restrict__ dstS,
                                                           float *__restrict__ dstz, long sstride,
                                                           long zstride, int N, int L, int nseg,
                                                           int P, const float *__restrict__ gamma,
                                                           int H, const uint16_t *__restrict__ W,
                                                           const float *__restrict__ S0,
                                                           const float *__restrict__ z0)
{
    using K = Cfg<D>;
    using TL = Tile<D, AggCfg<D>::THREADS>;
    // double-buffered chunks; single-buffered with the random-feature map (its W takes
    // 32 KiB of LDS): measured on MI355X, two barriers per chunk over 71 KiB beat one barrier
    // per chunk over 110 KiB there (the staging of a random-feature chunk is matrix work of
    // its own, and it overlaps better with the other workgroups than within one)
    constexpr int NB = RF ? 1 : 2;
    __shared__ __attribute__((aligned(16))) uint16_t sK[NB][K::AS];
    __shared__ __attribute__((aligned(16))) uint16_t sV[NB][K::AS];
    __shared__ __attribute__((aligned(16))) uint16_t sW[RF ? D * D : 8];

    const int tid = threadIdx.x, w = wave_id(), l = tid & 63, li = l & 15, g = l >> 4;
    const int p = blockIdx.x % nseg, bh = blockIdx.x / nseg;
    const int tb = p * L, te = min(N, tb + L);
    const int nch = (te - tb + C - 1) / C;
    const uint16_t *kb = k + (size_t)bh * N * D;
    const uint16_t *vb = v + (size_t)bh * N * D;
    const int cw0 = 16 * w;
    const int trl = tr_lane<D>(li, g);
    const TL tile(tid);
    auto chunk_t0 = [&](int cc) { return tb + min(cc, nch - 1) * C; };
    const float lg = DECAY ? decay_lg(gamma, bh, H) : 0.f;

    f32x4 sacc[K::NFT][1];
    f32x4 zacc[1];
    zero_acc<D, 1, 1>(sacc, zacc);
    if (S0 && p == 0) {
        // the head's initial state into slot nseg, where the causal kernel reads it (so the
        // final state may overwrite S0 there)
        const f32x4 *src = reinterpret_cast<const f32x4 *>(S0 + (size_t)bh * D * D);
        f32x4 *dst = reinterpret_cast<f32x4 *>(dstS + ((long)bh * P + nseg) * sstride);
        for (int i = tid; i < D * D / 4; i += AggCfg<D>::THREADS)
            dst[i] = src[i];
        if (tid < D / 4)
            reinterpret_cast<f32x4 *>(dstz + ((long)bh * P + nseg) * zstride)[tid] =
                reinterpret_cast<const f32x4 *>(z0 + (size_t)bh * D)[tid];
    }

    // K staging: phi (or as given) through the tile map, or random features (RF) with each
    // wave taking its row tile and feature half of every chunk
    u32x4 rk[RF ? D / 32 : TL::TM], rv[TL::TM];
    auto load_k = [&](const uint16_t *base, int nvalid) {
        if constexpr (RF)
            rf_load<D>(rk, base, w & 3, nvalid, li, g);
        else
            tile.load(rk, base, nvalid);
    };
    auto put_k = [&](uint16_t *dst, int nvalid) {
        if constexpr (RF)
            rf_put_share<D, AggCfg<D>::NW>(dst, sW, rk, w, nvalid, l);
        else
            tile.store(dst, rk, nvalid, PHI);
    };
    if (RF) {
        rf_put_w<D, AggCfg<D>::THREADS>(sW, W, tid);
        __syncthreads();
    }
    auto update = [&](int b, int c) {
        if (DECAY) {
            state_update_decay<D, 1, 1>(sacc, zacc, sK[b] + trl, sV[b] + cw0 + trl, sK[b] + cw0 + trl,
                                        lg, min(C, te - (tb + c * C)), g);
        } else {
            state_update<D, 1>(sacc, sK[b] + trl, sV[b] + cw0 + trl);
            key_sum<D, 1>(zacc, sK[b] + cw0 + trl);
        }
    };
    if constexpr (RF) {
        // single buffer: sum chunk c, then stage chunk c + 1 (two barriers per chunk)
        load_k(kb + (size_t)tb * D, te - tb);
        tile.load(rv, vb + (size_t)tb * D, te - tb);
        put_k(sK[0], te - tb);
        tile.store(sV[0], rv, te - tb, false);
        {
            const int tn = chunk_t0(1);
            load_k(kb + (size_t)tn * D, te - tn);
            tile.load(rv, vb + (size_t)tn * D, te - tn);
        }
        __syncthreads();
        for (int c = 0; c < nch; ++c) {
            update(0, c);
            __syncthreads();
            if (c + 1 < nch) {
                const int n1 = min(C, te - (tb + (c + 1) * C));
                put_k(sK[0], n1);
                tile.store(sV[0], rv, n1, false);
            }
            const int tn = chunk_t0(c + 2);
            load_k(kb + (size_t)tn * D, te - tn);
            tile.load(rv, vb + (size_t)tn * D, te - tn);
            __syncthreads();
        }
    } else {
        // Double-buffered LDS and two register sets: at the top of iteration c, chunk c is in
        // LDS buffer c & 1, chunk c + 1 is loading into register set (c + 1) & 1 and set c & 1
        // is free. The loads of chunk c + 2 go out first, so they are in flight while chunk c + 1
        // is staged (wait, phi, LDS stores) and chunk c is summed: the loads never wait behind
        // the staging. (Issuing them after the staging left each workgroup with no load in
        // flight for the length of its staging, measured on MI355X: 27.3 us for the sums of the
        // 2 x 16 x 8192 x 128 prefill against 19.7 us for a plain read of the same bytes.)
        constexpr int TM = TL::TM;
        u32x4 k0[TM], v0[TM], k1[TM], v1[TM];
        auto ld = [&](u32x4 (&rkk)[TM], u32x4 (&rvv)[TM], int cc) {
            const int tn = chunk_t0(cc);
            tile.load(rkk, kb + (size_t)tn * D, te - tn);
            tile.load(rvv, vb + (size_t)tn * D, te - tn);
        };
        auto put = [&](int bsel, const u32x4 (&rkk)[TM], const u32x4 (&rvv)[TM], int n) {
            tile.store(sK[bsel], rkk, n, PHI);
            tile.store(sV[bsel], rvv, n, false);
        };
        ld(k0, v0, 0);
        put(0, k0, v0, te - tb);
        ld(k1, v1, 1);
        __syncthreads();
        auto step = [&](int c, u32x4 (&fk)[TM], u32x4 (&fv)[TM], const u32x4 (&nk)[TM],
                        const u32x4 (&nv)[TM]) {
            ld(fk, fv, c + 2);
            if (c + 1 < nch)
                put((c & 1) ^ 1, nk, nv, min(C, te - (tb + (c + 1) * C)));
            update(c & 1, c);
            __syncthreads();
        };
        for (int c = 0; c < nch; c += 2) {
            step(c, k0, v0, k1, v1);
            if (c + 1 < nch)
                step(c + 1, k1, v1, k0, v0);
        }
    }

    float *S = dstS + ((long)bh * P + p) * sstride;
#pragma unroll
    for (int ft = 0; ft < K::NFT; ++ft)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[(16 * ft + 4 * g + r) * D + cw0 + li] = sacc[ft][0][r];
    if (li == 0) {
        float *z = dstz + ((long)bh * P + p) * zstride;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            z[cw0 + 4 * g + r] = zacc[0][r];
    }
}

// ------------------------------------------------------------------------------------------
// Causal kernel geometry: NCW = D/16 compute waves, each owning 16 value columns of S and one
// 16-feature tile of z, plus NSW stage waves. Staging (three tensors per chunk, phi on two of
// them) is the longer role per chunk at d = 128, so it gets as many waves as the register
// budget of 16 waves per CU allows.
template <int D> struct CausalCfg {
    static constexpr int NCW = D / 16;
    static constexpr int NSW = D == 128 ? 8 : 4;
    static constexpr int STAGE_THREADS = NSW * 64;
    static constexpr int THREADS = (NCW + NSW) * 64;
};

template <int D> struct CausalLds {
    uint16_t sQ[2][Cfg<D>::AS]; // phi(Q), double-buffered (read in both phases)
    uint16_t sK[2][Cfg<D>::AS]; // phi(K), double-buffered (read in both phases)
    uint16_t sV[Cfg<D>::AS];    // V, read only in phase 2
    uint16_t sA[C * Cfg<D>::TS];
    // key sum before the chunk being computed, as the A operand of phi(Q) z: row 0 = bf16(z),
    // row 1 = bf16(z - row 0) (together ~16 significant bits), row 2 = 0 (read by lanes 2..15)
    uint16_t szA[3][Cfg<D>::ZS];
    float srs[C];          // rowsum(A) per query row of the chunk
    float sqz[C];          // phi(q) . z per query row of the chunk
};

struct CausalArgs {
    const uint16_t *qh, *kh, *vh; // the head's [N, D] rows
    uint16_t *oh;
    const float *S0, *z0;         // state before the segment (null: zero, or formed from pre)
    float *Sout, *zout;           // final state of the head (null: not written)
    int tb, te, nch;              // token range of the segment, chunks in it
    float lg;                     // log2 of the head's decay (0: none)
    // the state before the segment formed from the head's segment sums (pre non-null): slots
    // of pe floats (S, then z), the sums of segments 0..np-1 and the initial state in slot ini
    // (-1: zero state)
    const float *pre;
    long pe;
    int np, ini, L;
};

// The state before a segment from the head's segment sums: the sums of segments 0..np-1, each
// decayed over the whole segments after it (gamma^(L (np - 1 - t)) for segment t; no weight
// without a decay), plus the initial state decayed over all np of them -- the recurrence of the
// state over segments ("Linear Attention: From Pairwise Reads to a Recurrent State", section "A
// recurrence need not force token-serial training"; with the decay, "Linear Attention Math",
// section "The kernel cousins: SSMs and RetNet") unrolled. The walk runs from the newest slot
// down, so that at each step the workgroups of a head read different slots: each slot comes
// from memory once, for the workgroup right after it, and from the L2 for the later ones (the
// head's workgroups share an XCD). Each lane reads the 4 NFT floats of S it holds in the
// accumulators (rows 16 ft + 4 g + r of column 16 w + li) and 4 of z.
template <int D, bool DECAY>
__device__ __forceinline__ void prefix_state(f32x4 (&sacc)[Cfg<D>::NFT][1], f32x4 (&zacc)[1],
                                             const CausalArgs &a, int w, int li, int g, int L)
{
    constexpr int NFT = Cfg<D>::NFT, NX = 4 * NFT + 4;
    const int cw0 = 16 * w;
    auto ld = [&](float (&x)[NX], int t) {
        const float *s = a.pre + (size_t)t * a.pe;
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                x[4 * ft + r] = s[(16 * ft + 4 * g + r) * D + cw0 + li];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            x[4 * NFT + r] = s[D * D + cw0 + 4 * g + r];
    };
    // run += weight * x (the first term is taken as it is)
    auto add = [&](const float (&x)[NX], bool first, float wt) {
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[ft][0][r] = first ? (DECAY ? x[4 * ft + r] * wt : x[4 * ft + r])
                                       : (DECAY ? fmaf(x[4 * ft + r], wt, sacc[ft][0][r])
                                                : sacc[ft][0][r] + x[4 * ft + r]);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            zacc[0][r] = first ? (DECAY ? x[4 * NFT + r] * wt : x[4 * NFT + r])
                               : (DECAY ? fmaf(x[4 * NFT + r], wt, zacc[0][r])
                                        : zacc[0][r] + x[4 * NFT + r]);
    };
    // step j: slot np - 1 - j, decayed over the j segments after it; then the initial state.
    // One slot is in flight per lane: a second one gains nothing measurable (the last segment's
    // workgroup reads P - 1 slots, 448 KiB at d = 128 and P = 8, and it is these bytes through
    // the one CU that take the time, measured on MI355X) and spills with the decay.
    const int ns = a.np + (a.ini >= 0 ? 1 : 0);
    for (int j = 0; j < ns; ++j) {
        float x[NX];
        ld(x, j < a.np ? a.np - 1 - j : a.ini);
        add(x, j == 0, DECAY ? decay_pow(a.lg, j * L) : 1.f);
    }
}

// Writes the wave's 16 features of z (rows 4g..4g+3 of its tile; lane li == 0 of each group)
// into the key-sum operand rows: bf16(z) and bf16(z - bf16(z)).
template <int D>
__device__ __forceinline__ void put_z(CausalLds<D> &sm, const f32x4 &z, int w, int li, int g)
{
    if (li == 0) {
        const uint32_t h0 = pack_bf2(z[0], z[1]), h1 = pack_bf2(z[2], z[3]);
        const uint32_t l0 = pack_bf2(z[0] - bf_lo(h0), z[1] - bf_hi(h0));
        const uint32_t l1 = pack_bf2(z[2] - bf_lo(h1), z[3] - bf_hi(h1));
        sts<u32x2>(&sm.szA[0][16 * w + 4 * g], u32x2{h0, h1});
        sts<u32x2>(&sm.szA[1][16 * w + 4 * g], u32x2{l0, l1});
    }
}

// Compute role (waves 0..NCW-1). Wave w owns value columns [16w, 16w+16) of S and the key-sum
// features [16w, 16w+16). Barrier sequence: 1 in the prologue, 2 per chunk. NORM = false (the
// unnormalised form) skips the denominator: no row sums of A and no phi(q) . z, while z is
// still accumulated as part of the state.
template <int D, bool NORM, bool DECAY>
__device__ __forceinline__ void causal_compute(CausalLds<D> &sm, const CausalArgs &a, int w,
                                               int li, int g)
{
    using K = Cfg<D>;
    constexpr int NCW = CausalCfg<D>::NCW;
    const int cw0 = 16 * w;
    // per-lane LDS offsets of the access patterns (elements)
    const int trl = tr_lane<D>(li, g); // transpose reads
    const int opl = nix<D>(li, 8 * g); // 16-byte operand reads, rows 16t + li
    const int sql = nix<D>(li, 4 * g); // 8-byte state-read pieces, rows 16t + li
    f32x4 sacc[K::NFT][1];
    f32x4 zacc[1];
    zero_acc<D, 1, 1>(sacc, zacc);
    if (a.pre) {
        prefix_state<D, DECAY>(sacc, zacc, a, w, li, g, a.L);
    } else if (a.S0) {
#pragma unroll
        for (int ft = 0; ft < K::NFT; ++ft)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sacc[ft][0][r] = a.S0[(16 * ft + 4 * g + r) * D + cw0 + li];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            zacc[0][r] = a.z0[16 * w + 4 * g + r];
    }
    put_z<D>(sm, zacc[0], w, li, g);
    if (w == 0)
        for (int i = threadIdx.x; i < D / 8; i += 64)
            sts<u32x4>(&sm.szA[2][8 * i], u32x4{0u, 0u, 0u, 0u});
    __syncthreads();

    // phase-1 jobs: waves 0-3 compute the scores of query rows 16w..16w+15; the waves that
    // compute phi(q) . z for rows 16(w%4).. are waves 4-7 (D = 128) or the same waves (D = 64)
    const bool scores = w < 4;
    const bool qz = NORM && (NCW == 8 ? w >= 4 : true);
    const int iw = w & 3;
    for (int c = 0; c < a.nch; ++c) {
        const int b = c & 1;
        const int t0 = a.tb + c * C, nvalid = min(C, a.te - t0);
        const uint16_t *sQ = sm.sQ[b], *sK = sm.sK[b];
        // ---- phase 1
        // every compute wave reads the carried state for its value columns here (phi(Q_c) and
        // S are ready): phase 2, with the within-chunk product, the output and the state
        // update, is the longer phase of the two (measured on MI355X: the compute waves arrive
        // last at its barrier, the stage waves at phase 1's), so this work is moved out of it.
        // The decayed form keeps it in phase 2, where its registers fit without spilling.
        f32x4 acc[1][4];
#pragma unroll
        for (int it = 0; it < 4; ++it)
            acc[0][it] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (!DECAY)
            state_read<D, 1>(acc, sacc, sQ + sql);
        if (scores) {
            bf16x8 qb[K::NKB];
#pragma unroll
            for (int kk = 0; kk < K::NKB; ++kk)
                qb[kk] = lds<bf16x8>(sQ + opl + blk<D>(16 * w, 32 * kk));
            float rs = 0.f;
            // key tiles 2mp and 2mp + 1 (the second one is all zero past the diagonal tile)
            for (int mp = 0; 2 * mp <= w; ++mp) {
                uint32_t pk[4];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int jt = 2 * mp + h;
                    f32x4 t = {0.f, 0.f, 0.f, 0.f};
                    if (jt <= w) { // wave-uniform
#pragma unroll
                        for (int kk = 0; kk < K::NKB; ++kk)
                            t = mfma(lds<bf16x8>(sK + opl + blk<D>(16 * jt, 32 * kk)), qb[kk], t);
                    }
                    // t[r] = A[i = 16w + li][j = 16jt + 4g + r]
                    if (jt == w) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (4 * g + r > li)
                                t[r] = 0.f;
                    }
                    if (DECAY && jt <= w) {
                        // A[i][j] *= gamma^(i - j) for j <= i (the decay mask)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int lag = 16 * (w - jt) + li - 4 * g - r;
                            t[r] = lag >= 0 ? t[r] * dpow(a.lg, lag) : 0.f;
                        }
                    }
                    pk[2 * h] = pack_bf2(t[0], t[1]);
                    pk[2 * h + 1] = pack_bf2(t[2], t[3]);
                    if (NORM)
                        rs += (bf_lo(pk[2 * h]) + bf_hi(pk[2 * h])) + (bf_lo(pk[2 * h + 1]) + bf_hi(pk[2 * h + 1]));
                }
                sts<u32x4>(sm.sA + sa_ix(16 * w + li, mp, g), u32x4{pk[0], pk[1], pk[2], pk[3]});
            }
            if (NORM) {
                rs += __shfl_xor(rs, 16, 64);
                rs += __shfl_xor(rs, 32, 64);
                if (g == 0)
                    sm.srs[16 * w + li] = rs;
            }
        }
        if (qz) {
            // phi(Q) z for query rows 16iw..: one matrix-core product per 32 features with
            // A = the key-sum rows (lane li reads row min(li, 2)); C rows 0 and 1 hold the
            // two parts of the sum for the lane's query
            const uint16_t *za = &sm.szA[li < 2 ? li : 2][8 * g];
            f32x4 cz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < K::NKB; ++kk)
                cz = mfma(lds<bf16x8>(za + 32 * kk), lds<bf16x8>(sQ + opl + blk<D>(16 * iw, 32 * kk)), cz);
            if (g == 0) // the carried key sum reaches query row i decayed by gamma^(i + 1)
                sm.sqz[16 * iw + li] = (cz[0] + cz[1]) * (DECAY ? dpow(a.lg, 16 * iw + li + 1) : 1.f);
        }
        __syncthreads();
        // ---- phase 2: num^T += V^T A^T for the wave's columns; out; S, z += Kf^T [V 1]
        {
            if (DECAY) {
                // the carried state reaches query row i decayed by gamma^(i + 1): read it
                // first and scale the rows before the within-chunk part is added
                state_read<D, 1>(acc, sacc, sQ + sql);
#pragma unroll
                for (int it = 0; it < 4; ++it)
                    acc[0][it] *= dpow(a.lg, 16 * it + li + 1);
            }
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const bf16x8 av = frag_tok<D>(sm.sV + cw0 + trl + blk<D>(32 * m, 0));
#pragma unroll
                for (int it = 2 * m; it < 4; ++it) {
                    const bf16x8 ba = lds<bf16x8>(sm.sA + sa_ix(16 * it + li, m, g));
                    acc[0][it] = mfma(av, ba, acc[0][it]);
                }
            }
            store_out<D, 1, NORM>(acc, sm.srs, sm.sqz, a.oh + (size_t)t0 * D, nvalid, cw0, li, g);
            if (DECAY) {
                state_update_decay<D, 1, 1>(sacc, zacc, sK + trl, sm.sV + cw0 + trl, sK + 16 * w + trl,
                                            a.lg, nvalid, g);
            } else {
                state_update<D, 1>(sacc, sK + trl, sm.sV + cw0 + trl);
                key_sum<D, 1>(zacc, sK + 16 * w + trl);
            }
            if (NORM)
                put_z<D>(sm, zacc[0], w, li, g);
        }
        __syncthreads();
    }
    if (a.Sout) {
#pragma unroll
        for (int ft = 0; ft < K::NFT; ++ft)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                a.Sout[(16 * ft + 4 * g + r) * D + cw0 + li] = sacc[ft][0][r];
        if (li == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                a.zout[16 * w + 4 * g + r] = zacc[0][r];
        }
    }
}

// Stage role (the NSW waves after the compute waves, thread index ht). Same barrier sequence
// as the compute role. PHI = false stages q and k as given (already mapped features).
template <int D, bool PHI, bool RF>
__device__ __forceinline__ void causal_stage(CausalLds<D> &sm, const uint16_t *sW, const CausalArgs &a,
                                             int ht)
{
    using TL = Tile<D, CausalCfg<D>::STAGE_THREADS>;
    constexpr int NSW = CausalCfg<D>::NSW;
    const TL tile(ht);
    // q and k in the tile map (phi or as given), or as B operands of the random-feature
    // product (RF: stage wave sw takes row tile sw % 4 and its feature half)
    u32x4 rq[RF ? D / 32 : TL::TM], rk[RF ? D / 32 : TL::TM], rv[TL::TM];
    const int sw = ht >> 6, l = ht & 63;
    auto load_qk = [&](u32x4 (&r)[RF ? D / 32 : TL::TM], const uint16_t *base, int nvalid) {
        if constexpr (RF)
            rf_load<D>(r, base, sw & 3, nvalid, l & 15, l >> 4);
        else
            tile.load(r, base, nvalid);
    };
    auto put_qk = [&](uint16_t *dst, const u32x4 (&r)[RF ? D / 32 : TL::TM], int nvalid) {
        if constexpr (RF)
            rf_put_share<D, NSW>(dst, sW, r, sw, nvalid, l);
        else
            tile.store(dst, r, nvalid, PHI);
    };
    const int tb = a.tb, te = a.te, nch = a.nch;
    // first token of chunk c' (clamped to the last chunk, so prefetches past the end re-read
    // it: every load is in bounds and unconditional)
    auto chunk_t0 = [&](int cc) { return tb + min(cc, nch - 1) * C; };

    load_qk(rq, a.qh + (size_t)tb * D, te - tb);
    load_qk(rk, a.kh + (size_t)tb * D, te - tb);
    tile.load(rv, a.vh + (size_t)tb * D, te - tb);
    put_qk(sm.sQ[0], rq, te - tb);
    put_qk(sm.sK[0], rk, te - tb);
    {
        const int tn = chunk_t0(1);
        load_qk(rq, a.qh + (size_t)tn * D, te - tn);
        load_qk(rk, a.kh + (size_t)tn * D, te - tn);
    }
    __syncthreads();

    for (int c = 0; c < nch; ++c) {
        const int nb = (c & 1) ^ 1;
        const int t0 = tb + c * C;
        const int n0 = min(C, te - t0);     // valid rows of chunk c
        const int n1 = min(C, te - t0 - C); // valid rows of chunk c+1 (if it exists)
        // phase 1: V_c -> LDS, load V_{c+1}; phi(Q_{c+1}) -> LDS, load Q_{c+2}
        tile.store(sm.sV, rv, n0, false);
        {
            const int tn = chunk_t0(c + 1);
            tile.load(rv, a.vh + (size_t)tn * D, te - tn);
        }
        if (c + 1 < nch)
            put_qk(sm.sQ[nb], rq, n1);
        {
            const int tn = chunk_t0(c + 2);
            load_qk(rq, a.qh + (size_t)tn * D, te - tn);
        }
        __syncthreads();
        // phase 2: phi(K_{c+1}) -> LDS, load K_{c+2}
        if (c + 1 < nch)
            put_qk(sm.sK[nb], rk, n1);
        {
            const int tn = chunk_t0(c + 2);
            load_qk(rk, a.kh + (size_t)tn * D, te - tn);
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------------------------------
// Causal outputs of one segment, starting from the state before the segment: one slot of preS,
// prez per segment, or (PM_SUMS) the head's segment sums, which the compute waves add up
// (prefix_state) while the stage waves load and stage the segment's first chunks.
//
// Two roles share every SIMD. D/16 "compute" waves hold the float32 state S and key sum z in
// accumulators (16 value columns of S and 16 features of z each) and run the matrix-core
// products of chunk c. NSW "stage" waves load the next chunks from HBM, apply phi and store
// them row-major into LDS. Two barriers per chunk:
//   phase 1  compute: num = phi(Q_c) S (all compute waves, their value columns); scores A of
//                     chunk c (waves 0-3: query rows 16w..16w+15), rowsum(A) and phi(q) . z
//                     per query row
//            stage:   V_c -> LDS, load V_{c+1}; phi(Q_{c+1}) -> LDS, load Q_{c+2}
//   --- barrier ---
//   phase 2  compute: num += A V_c; out = num / den; S, z += phi(K_c)^T [V_c 1]
//            stage:   phi(K_{c+1}) -> LDS, load K_{c+2}
//   --- barrier ---
// (with a decay, num = phi(Q_c) S is read in phase 2, scaled per row, before A V_c is added)
// Roles are chosen by the wave-uniform wave index, so every wave executes the same sequence of
// barriers. F: variant flags (F_IDENTITY: q, k are already features; F_UNNORM: no denominator).
// RF: q and k are mapped to positive random features by W while staged (one more barrier,
// after W is copied into LDS).
template <int D, int F, bool DECAY, bool RF>
__global__ __launch_bounds__(CausalCfg<D>::THREADS) void k_causal(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    uint16_t *__restrict__ out, const float *__restrict__ preS, const float *__restrict__ prez,
    long pstride, long pzstride, float *__restrict__ Sout, float *__restrict__ zout, int N, int L,
    int P, const float *__restrict__ gamma, int H, const uint16_t *__restrict__ W, int pm)
{
    constexpr int NCW = CausalCfg<D>::NCW;
    __shared__ __attribute__((aligned(16))) CausalLds<D> sm;
    __shared__ __attribute__((aligned(16))) uint16_t sW[RF ? D * D : 8];
    const int tid = threadIdx.x, wave = wave_id(), l = tid & 63;
    // block order: segment-minor, or (PM_XCD, the head count a multiple of 8) every segment of
    // a head on the same XCD -- consecutive workgroups go to the eight XCDs in turn -- so that
    // the head's segment sums, read by all of its workgroups, are fetched into one L2
    int p, bh;
    if (pm & PM_XCD) {
        const int x = blockIdx.x & 7, y = blockIdx.x >> 3;
        p = y % P;
        bh = x + 8 * (y / P);
    } else {
        p = blockIdx.x % P;
        bh = blockIdx.x / P;
    }
    const size_t hoff = (size_t)bh * N * D;
    CausalArgs a;
    a.qh = q + hoff;
    a.kh = k + hoff;
    a.vh = v + hoff;
    a.oh = out + hoff;
    a.pre = nullptr;
    a.S0 = a.z0 = nullptr;
    if (pm & PM_SUMS) {
        // preS: the workspace of segment sums (pstride floats per slot, P slots per head)
        a.pre = preS + (long)bh * P * pstride;
        a.pe = pstride;
        a.np = p;
        a.ini = (pm & PM_INIT) ? P - 1 : -1;
        a.L = L;
    } else if (preS) {
        a.S0 = preS + ((long)bh * P + p) * pstride;
        a.z0 = prez + ((long)bh * P + p) * pzstride;
    }
    const bool last = p == P - 1;
    a.Sout = Sout && last ? Sout + (size_t)bh * D * D : nullptr;
    a.zout = Sout && last ? zout + (size_t)bh * D : nullptr;
    a.tb = p * L;
    a.te = min(N, a.tb + L);
    a.nch = (a.te - a.tb + C - 1) / C;
    a.lg = DECAY ? decay_lg(gamma, bh, H) : 0.f;
    if (RF) {
        rf_put_w<D, CausalCfg<D>::THREADS>(sW, W, tid);
        __syncthreads();
    }
    if (wave < NCW)
        causal_compute<D, !(F & F_UNNORM), DECAY>(sm, a, wave, l & 15, l >> 4);
    else
        causal_stage<D, !(F & F_IDENTITY), RF>(sm, sW, a, tid - NCW * 64);
}

// ------------------------------------------------------------------------------------------
// Global read: out = phi(Q) S / phi(Q) z for one segment of tokens of one head (F as for
// k_causal). The workgroup copies S (bf16, in matrix-core fragment order) and z into LDS once;
// after that each wave works alone on groups of RT 16-row tiles of the segment (groups w,
// w + GW, ...) with no further barrier. A wave loads its rows of Q straight from HBM as the B
// operands of num^T = S^T phi(Q)^T (lane li holds row li; the next group's rows load while the
// current one is computed), applies phi in registers, takes phi(q) . z for its row from the
// same registers,
// and writes the 16 x D output tile to a wave-private LDS tile that it stores as whole rows
// (1 KiB per store instruction). (The earlier form staged Q through LDS with two barriers per
// chunk and stored 64-byte pieces of 16 rows per instruction.)
template <int D> struct GreadCfg {
    static constexpr int NKB = D / 32;   // 32-feature k blocks
    static constexpr int NCT = D / 16;   // 16-column value tiles
    static constexpr int OS = D + 4;     // row stride (elements) of a wave's output tile
};

// (at most 128 VGPRs: four waves per SIMD, so two workgroups share a CU)
template <int D, int F, int RT = 2>
__global__ __launch_bounds__(NT, 2) void k_gread(const uint16_t *__restrict__ q,
                                              uint16_t *__restrict__ out,
                                              const float *__restrict__ S,
                                              const float *__restrict__ z, int N, int L, int P)
{
    using G = GreadCfg<D>;
    constexpr int NKB = G::NKB, NCT = G::NCT, OS = G::OS, LPR = D / 8, RPI = 64 / LPR;
    constexpr bool PHI = !(F & F_IDENTITY), NORM = !(F & F_UNNORM);
    __shared__ __attribute__((aligned(16))) uint16_t sS[D * D];      // S^T fragments
    __shared__ __attribute__((aligned(16))) uint16_t sT[GW][16 * OS]; // per-wave output tiles
    __shared__ float sz[D];

    const int tid = threadIdx.x, w = wave_id(), l = tid & 63, li = l & 15, g = l >> 4;
    const int p = blockIdx.x % P, bh = blockIdx.x / P;
    const int tb = p * L, te = min(N, tb + L);
    const size_t hoff = (size_t)bh * N * D;

    const int ntile = (te - tb + 15) / 16, ngrp = (ntile + RT - 1) / RT;
    // B operand of tile t: row tb + 16 t + li (clamped to the segment's last row: every load is
    // in bounds), features 32 kb + 8 g .. + 7; a group is RT consecutive tiles (tiles past the
    // segment's end load its last tile again and store nothing)
    auto ldq = [&](u32x4 (&r)[NKB], int t) {
        const int row = min(tb + 16 * t + li, te - 1);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
            r[kb] = *reinterpret_cast<const u32x4 *>(q + hoff + (size_t)row * D + 32 * kb + 8 * g);
    };
    auto ldg = [&](u32x4 (&r)[RT][NKB], int gi) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            ldq(r[rt], min(gi * RT + rt, ntile - 1));
    };
    // the wave's first group is requested before S, so both loads are in flight together
    u32x4 qa[RT][NKB], qn[RT][NKB];
    ldg(qa, w);

    // S^T -> LDS: fragment fr = ct * NKB + kb, lane ll = lli + 16 lg holds S[32 kb + 8 lg + j]
    // [16 ct + lli], j < 8 (the A operand: row = value column, k-slots = 8 features). Item u
    // is the 8 x 4 block of S at rows 8 rg .. + 7 (rg = 4 kb + lg), columns 4 c4 .. + 3: eight
    // 16-byte row loads, all of a thread's items issued before any is converted, then four
    // whole fragment entries.
    {
        constexpr int NU = D * D / 32, NI = (NU + NT - 1) / NT;
        const float *Sh = S + (size_t)bh * D * D;
        f32x4 x[NI][8];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int u = tid + i * NT, rg = u / (D / 4), c4 = u % (D / 4);
            if (u < NU)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    x[i][j] = *reinterpret_cast<const f32x4 *>(Sh + (size_t)(8 * rg + j) * D + 4 * c4);
        }
        if (tid < D)
            sz[tid] = z[(size_t)bh * D + tid];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int u = tid + i * NT, rg = u / (D / 4), c4 = u % (D / 4);
            if (u < NU)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int col = 4 * c4 + c, ct = col / 16, lli = col % 16;
                    const int kb = rg / 4, lg = rg % 4;
                    sts<u32x4>(sS + ((ct * NKB + kb) * 64 + lli + 16 * lg) * 8,
                               u32x4{pack_bf2(x[i][0][c], x[i][1][c]), pack_bf2(x[i][2][c], x[i][3][c]),
                                     pack_bf2(x[i][4][c], x[i][5][c]), pack_bf2(x[i][6][c], x[i][7][c])});
                }
        }
    }
    __syncthreads();

    if (w >= ngrp)
        return;
    uint16_t *tile = sT[w];
    // a 16-row tile of outputs back as whole rows (this wave's LDS only: its accesses stay in
    // order), with non-temporal stores: the outputs (as many bytes as q) are not left dirty in
    // the caches, where the next call's segment sums would find their write-back in the way of
    // their reads (measured on MI355X for B=1 H=8 N=100000 d=128: 189 -> 174 us per call)
    auto put_rows = [&](int t) {
        const int r0 = tb + 16 * t;
#pragma unroll
        for (int i = 0; i < 16 / RPI; ++i) {
            const int row = RPI * i + l / LPR, col = 8 * (l % LPR);
            const u32x4 x = lds<u32x4>(tile + row * OS + col);
            if (r0 + row < te)
                __builtin_nontemporal_store(x, reinterpret_cast<u32x4 *>(out + hoff + (size_t)(r0 + row) * D + col));
        }
    };
    for (int gi = w; gi < ngrp; gi += GW) {
        ldg(qn, min(gi + GW, ngrp - 1)); // next group (a re-read of the last one at the end)
        bf16x8 qb[RT][NKB];
        float inv[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float den = 0.f;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const u32x4 y = PHI ? phi8(qa[rt][kb]) : qa[rt][kb];
                qb[rt][kb] = __builtin_bit_cast(bf16x8, y);
                if (NORM) {
                    const float4 z0 = *reinterpret_cast<const float4 *>(sz + 32 * kb + 8 * g);
                    const float4 z1 = *reinterpret_cast<const float4 *>(sz + 32 * kb + 8 * g + 4);
                    const float zz[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
                    for (int h = 0; h < 4; ++h)
                        den = fmaf(bf_lo(y[h]), zz[2 * h], fmaf(bf_hi(y[h]), zz[2 * h + 1], den));
                }
            }
            inv[rt] = 1.f;
            if (NORM) {
                den += __shfl_xor(den, 16, 64);
                den += __shfl_xor(den, 32, 64);
                inv[rt] = __builtin_amdgcn_rcpf(den);
            }
        }
        // every S fragment read from LDS feeds the group's RT tiles; the first tile goes to the
        // wave's LDS tile at once, the others wait in registers as packed bf16
        u32x2 later[RT - 1][NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            f32x4 c[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                c[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const bf16x8 a = lds<bf16x8>(sS + ((ct * NKB + kb) * 64 + l) * 8);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    c[rt] = mfma(a, qb[rt][kb], c[rt]);
            }
            // c[rt][r] = num[query row li of tile rt][value column 16 ct + 4 g + r]
            sts<u32x2>(tile + li * OS + 16 * ct + 4 * g,
                       u32x2{pack_bf2(c[0][0] * inv[0], c[0][1] * inv[0]),
                             pack_bf2(c[0][2] * inv[0], c[0][3] * inv[0])});
#pragma unroll
            for (int rt = 1; rt < RT; ++rt)
                later[rt - 1][ct] = u32x2{pack_bf2(c[rt][0] * inv[rt], c[rt][1] * inv[rt]),
                                          pack_bf2(c[rt][2] * inv[rt], c[rt][3] * inv[rt])};
            // (the loop is unrolled for the register array above; without this fence the
            // scheduler hoists every S fragment read of the group and spills)
            __builtin_amdgcn_sched_barrier(0);
        }
        put_rows(gi * RT);
#pragma unroll
        for (int rt = 1; rt < RT; ++rt) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                sts<u32x2>(tile + li * OS + 16 * ct + 4 * g, later[rt - 1][ct]);
            put_rows(gi * RT + rt);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                qa[rt][kb] = qn[rt][kb];
    }
}

// ------------------------------------------------------------------------------------------
// Host dispatch over the compile-time variants. Every kernel is instantiated for D in {64, 128}
// and each variant flag it uses.
template <int D, int F> void launch_causal(dim3 grid, hipStream_t st, const uint16_t *q,
                                           const uint16_t *k, const uint16_t *v, uint16_t *o,
                                           const float *preS, const float *prez, long ps, long pzs,
                                           int pm, float *Sout, float *zout, int N, int L, int P,
                                           const float *gamma, int H)
{
    const uint16_t *W = nullptr;
    if (gamma)
        hipLaunchKernelGGL((k_causal<D, F, true, false>), grid, dim3(CausalCfg<D>::THREADS), 0, st, q,
                           k, v, o, preS, prez, ps, pzs, Sout, zout, N, L, P, gamma, H, W, pm);
    else
        hipLaunchKernelGGL((k_causal<D, F, false, false>), grid, dim3(CausalCfg<D>::THREADS), 0, st, q,
                           k, v, o, preS, prez, ps, pzs, Sout, zout, N, L, P, gamma, H, W, pm);
}

template <int D> void launch_causal_f(int flags, dim3 grid, hipStream_t st, const uint16_t *q,
                                      const uint16_t *k, const uint16_t *v, uint16_t *o,
                                      const float *preS, const float *prez, long ps, long pzs,
                                      int pm, float *Sout, float *zout, int N, int L, int P,
                                      const float *gamma, int H)
{
    switch (flags & (F_IDENTITY | F_UNNORM)) {
    case 0: launch_causal<D, 0>(grid, st, q, k, v, o, preS, prez, ps, pzs, pm, Sout, zout, N, L, P, gamma, H); break;
    case 1: launch_causal<D, 1>(grid, st, q, k, v, o, preS, prez, ps, pzs, pm, Sout, zout, N, L, P, gamma, H); break;
    case 2: launch_causal<D, 2>(grid, st, q, k, v, o, preS, prez, ps, pzs, pm, Sout, zout, N, L, P, gamma, H); break;
    default: launch_causal<D, 3>(grid, st, q, k, v, o, preS, prez, ps, pzs, pm, Sout, zout, N, L, P, gamma, H); break;
    }
}

template <int D> void launch_gread_f(int flags, dim3 grid, hipStream_t st, const uint16_t *q,
                                     uint16_t *o, const float *S, const float *z, int N, int L, int P)
{
    switch (flags & (F_IDENTITY | F_UNNORM)) {
    case 0: hipLaunchKernelGGL((k_gread<D, 0>), grid, dim3(NT), 0, st, q, o, S, z, N, L, P); break;
    case 1: hipLaunchKernelGGL((k_gread<D, 1>), grid, dim3(NT), 0, st, q, o, S, z, N, L, P); break;
    case 2: hipLaunchKernelGGL((k_gread<D, 2>), grid, dim3(NT), 0, st, q, o, S, z, N, L, P); break;
    default: hipLaunchKernelGGL((k_gread<D, 3>), grid, dim3(NT), 0, st, q, o, S, z, N, L, P); break;
    }
}

template <int D, bool PHI> void launch_agg(dim3 grid, hipStream_t st, const uint16_t *k,
                                           const uint16_t *v, float *dstS, float *dstz, long ss,
                                           long zs, int N, int L, int nseg, int P,
                                           const float *gamma, int H, const float *S0,
                                           const float *z0)
{
    const uint16_t *W = nullptr;
    if (gamma)
        hipLaunchKernelGGL((k_agg<D, PHI, true, false>), grid, dim3(AggCfg<D>::THREADS), 0, st, k, v,
                           dstS, dstz, ss, zs, N, L, nseg, P, gamma, H, W, S0, z0);
    else
        hipLaunchKernelGGL((k_agg<D, PHI, false, false>), grid, dim3(AggCfg<D>::THREADS), 0, st, k, v,
                           dstS, dstz, ss, zs, N, L, nseg, P, gamma, H, W, S0, z0);
}

template <int D> void launch_agg_f(int flags, dim3 grid, hipStream_t st, const uint16_t *k,
                                   const uint16_t *v, float *dstS, float *dstz, long ss, long zs,
                                   int N, int L, int nseg, int P, const float *gamma, int H,
                                   const float *S0, const float *z0)
{
    if (flags & F_IDENTITY)
        launch_agg<D, false>(grid, st, k, v, dstS, dstz, ss, zs, N, L, nseg, P, gamma, H, S0, z0);
    else
        launch_agg<D, true>(grid, st, k, v, dstS, dstz, ss, zs, N, L, nseg, P, gamma, H, S0, z0);
}

} // namespace

hipError_t agg_mfma(int D, int flags, const void *k, const void *v, float *dstS, float *dstz,
                    long sstride, long zstride, int BH, int N, int L, int nseg, int P,
                    const float *gamma, int H, const float *S0, const float *z0, hipStream_t st)
{
    if (S0 && (!z0 || nseg >= P))
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)(BH * nseg));
    const auto *kk = static_cast<const uint16_t *>(k);
    const auto *vv = static_cast<const uint16_t *>(v);
    if (D == 128)
        launch_agg_f<128>(flags, grid, st, kk, vv, dstS, dstz, sstride, zstride, N, L, nseg, P, gamma,
                          H, S0, z0);
    else
        launch_agg_f<64>(flags, grid, st, kk, vv, dstS, dstz, sstride, zstride, N, L, nseg, P, gamma,
                         H, S0, z0);
    return hipGetLastError();
}

// The prefix modes' preconditions (see la_launch.h).
static bool pm_ok(int pm, int D, const float *preS, const float *prez, long ps, long pzs, int BH)
{
    if (!(pm & PM_SUMS))
        return pm == 0;
    return preS && prez == preS + (long)D * D && ps == pzs && ps >= (long)D * D + D &&
           (!(pm & PM_XCD) || BH % 8 == 0);
}

hipError_t causal_mfma(int D, int flags, const void *q, const void *k, const void *v, void *out,
                       const float *preS, const float *prez, long pstride, long pzstride, int pm,
                       float *Sout, float *zout, int BH, int N, int L, int P, const float *gamma,
                       int H, hipStream_t st)
{
    if (!pm_ok(pm, D, preS, prez, pstride, pzstride, BH))
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)(BH * P));
    const auto *qq = static_cast<const uint16_t *>(q);
    const auto *kk = static_cast<const uint16_t *>(k);
    const auto *vv = static_cast<const uint16_t *>(v);
    auto *oo = static_cast<uint16_t *>(out);
    if (D == 128)
        launch_causal_f<128>(flags, grid, st, qq, kk, vv, oo, preS, prez, pstride, pzstride, pm, Sout,
                             zout, N, L, P, gamma, H);
    else
        launch_causal_f<64>(flags, grid, st, qq, kk, vv, oo, preS, prez, pstride, pzstride, pm, Sout,
                            zout, N, L, P, gamma, H);
    return hipGetLastError();
}

hipError_t agg_rf_mfma(int D, const void *k, const void *v, const void *W, float *dstS, float *dstz,
                       long sstride, long zstride, int BH, int N, int L, int nseg, int P,
                       const float *S0, const float *z0, hipStream_t st)
{
    if (S0 && (!z0 || nseg >= P))
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)(BH * nseg));
    const auto *kk = static_cast<const uint16_t *>(k);
    const auto *vv = static_cast<const uint16_t *>(v);
    const auto *ww = static_cast<const uint16_t *>(W);
    const float *gamma = nullptr;
    if (D == 128)
        hipLaunchKernelGGL((k_agg<128, false, false, true>), grid, dim3(AggCfg<128>::THREADS), 0, st,
                           kk, vv, dstS, dstz, sstride, zstride, N, L, nseg, P, gamma, 1, ww, S0, z0);
    else
        hipLaunchKernelGGL((k_agg<64, false, false, true>), grid, dim3(AggCfg<64>::THREADS), 0, st,
                           kk, vv, dstS, dstz, sstride, zstride, N, L, nseg, P, gamma, 1, ww, S0, z0);
    return hipGetLastError();
}

hipError_t causal_rf_mfma(int D, int flags, const void *q, const void *k, const void *v,
                          const void *W, void *out, const float *preS, const float *prez,
                          long pstride, long pzstride, int pm, float *Sout, float *zout, int BH,
                          int N, int L, int P, hipStream_t st)
{
    if (!pm_ok(pm, D, preS, prez, pstride, pzstride, BH))
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)(BH * P));
    const auto *qq = static_cast<const uint16_t *>(q);
    const auto *kk = static_cast<const uint16_t *>(k);
    const auto *vv = static_cast<const uint16_t *>(v);
    const auto *ww = static_cast<const uint16_t *>(W);
    auto *oo = static_cast<uint16_t *>(out);
    const float *gamma = nullptr;
#define LA_RFC(DD, FF)                                                                          \
    hipLaunchKernelGGL((k_causal<DD, FF, false, true>), grid, dim3(CausalCfg<DD>::THREADS), 0, st, \
                       qq, kk, vv, oo, preS, prez, pstride, pzstride, Sout, zout, N, L, P, gamma, 1, \
                       ww, pm)
    const bool unnorm = flags & F_UNNORM;
    if (D == 128) {
        if (unnorm)
            LA_RFC(128, F_UNNORM);
        else
            LA_RFC(128, 0);
    } else {
        if (unnorm)
            LA_RFC(64, F_UNNORM);
        else
            LA_RFC(64, 0);
    }
#undef LA_RFC
    return hipGetLastError();
}

hipError_t global_read_mfma(int D, int flags, const void *q, void *out, const float *S,
                            const float *z, int BH, int N, int L, int P, hipStream_t st)
{
    // the read needs no segment sums, so it takes its own split: about two workgroups per CU
    // (as many as fit), 16-row tiles of the sequence
    {
        const long want = 2 * 256;
        if ((long)BH * P < want) {
            const long pr = (want + BH - 1) / BH;
            const int Lr = (int)(((N + pr - 1) / pr + 15) / 16 * 16);
            L = Lr;
            P = (N + Lr - 1) / Lr;
        }
    }
    const dim3 grid((unsigned)(BH * P));
    const auto *qq = static_cast<const uint16_t *>(q);
    auto *oo = static_cast<uint16_t *>(out);
    if (D == 128)
        launch_gread_f<128>(flags, grid, st, qq, oo, S, z, N, L, P);
    else
        launch_gread_f<64>(flags, grid, st, qq, oo, S, z, N, L, P);
    return hipGetLastError();
}

} // namespace la
